"""HIP path vs the fp64 oracle at the full sizes of the six large packs (the last one split-KV), in the launch
configuration the benchmark times (one plan, one forward launch, ring merges, one backward
launch over the whole pack).

The oracle cannot redo a whole pack in a test's time, so each (segment, head) is compared on
rows the oracle computes one by one:
  * O, LSE and dQ on sampled query rows of EVERY (segment, head): first, last and uniformly
    drawn rows, Q_SAMPLES of them per head (LONG_Q_SAMPLES on sequences longer than
    LONG_TOKENS, i.e. the 497,760-token shard of the long pack);
  * dK and dV on sampled key rows, which need every query row's LSE_i and D_i = dO_i . O_i:
    - segments of up to 4,096 tokens: every head, the oracle redoing the head in full;
    - 32,760-token sequences: two heads per segment, redone in full;
    - the 75,600-token shard of the mixed pack and the 497,760-token shard of the long pack
      (all 5 heads of each): LSE and D of every query row from
      tests/golden/long_rows_<pack>.npz, written by tests/golden/make_long_rows.py, which
      calls only the oracle (checked against the sha256 of this run's bf16 inputs before
      use). On the 75,600-token shard half of the sampled keys lie at tokens >= 52,557, whose
      dK/dV rows sit past 2^31 bytes of the fp32 gradient tensors;
  * ring partials of the KV-split pack on sampled rows of every part, and the group's final
    rows merged once more by zl_lse_merge (the one-group call, through pointer offsets).
Properties that hold at any size are checked on every (segment, head) of the GPU output:
  * sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (softmax shift invariance, rows of P sum to 1);
  * every covered output row was written (the buffers start as NaN).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_harness as H
from tests.golden import make_long_rows as LR

pytestmark = [pytest.mark.gpu, H.requires_gpu]

Q_SAMPLES = 8            # query rows per (segment, head)
DEEP_Q_SAMPLES = 32      # ... on the heads whose dK/dV are also checked
LONG_TOKENS = 100_000
LONG_Q_SAMPLES = 256     # query rows per head of sequences longer than LONG_TOKENS
K_SAMPLES = 32
CACHED_K_SAMPLES = 256
FULL_REDO_TOKENS = 4096  # segments up to this many tokens get dK/dV on every head
FULL_HEAD_LIMIT = 32760 * 32760  # Lq * Lkv of the largest head the oracle redoes in full
ROW_2GB = (1 << 31) // (128 * 4)  # first fp32 d=128 row past 2^31 bytes


def _views(pack, t, side):
    """Per-sequence [tokens, heads, d] views of a packed tensor."""
    lens = pack.seq_q if side == "q" else pack.seq_kv
    out, off = [], 0
    for l, h in zip(lens, pack.heads):
        out.append(t[off:off + l * h].view(l, h, *t.shape[1:]))
        off += l * h
    return out


def _check_invariants(pack, out, do_dev):
    dks, dvs, dos = _views(pack, out["dk"], "kv"), _views(pack, out["dv"], "kv"), _views(pack, do_dev, "q")
    worst_k = worst_v = 0.0
    for (s, h0, h1, q0, q1, k0, k1, part) in pack.segments:
        if part >= 0:
            continue
        dk = dks[s][k0:k1, h0:h1].double()
        dv = dvs[s][k0:k1, h0:h1].double()
        dsum = dos[s][q0:q1, h0:h1].double().sum(0)
        rk = (dk.sum(0).norm(dim=-1) / dk.norm(dim=(0, 2))).max().item()
        rv = ((dv.sum(0) - dsum).norm(dim=-1) / dv.norm(dim=(0, 2))).max().item()
        worst_k, worst_v = max(worst_k, rk), max(worst_v, rv)
    print(f"  invariants: max |sum dK| / |dK| = {worst_k:.2e}, max |sum dV - sum dO| / |dV| = {worst_v:.2e}", flush=True)
    assert worst_k < 2e-2 and worst_v < 2e-2


def _cached_rows(pack, ins):
    """Oracle LSE and D per query row of the cached long heads: {(seq, head): (lse, d)}."""
    path = LR.path_for(pack.name)
    if pack.name not in LR.TARGETS:
        return {}
    assert os.path.exists(path), f"{path} is missing: run tests/golden/make_long_rows.py {pack.name}"
    z = np.load(path, allow_pickle=False)
    s = int(z["seq"])
    assert str(z["pack"]) == pack.name and int(z["seed"]) == pack.seed
    out = {}
    for h in (int(x) for x in z["heads"]):
        sha = LR.digest(LR.head_rows(pack, ins, s, h))
        for key, val in sha.items():
            assert str(z[f"sha_{key}_{h}"]) == val, f"cached rows of head {h} were made from other {key} inputs"
        out[(s, h)] = (z[f"lse_{h}"].astype(np.float64), z[f"d_{h}"].astype(np.float64))
    return out


def _key_sample(n, count, rng, tok_hi=None):
    """Sampled key positions; with tok_hi, half of them at or after tok_hi."""
    if tok_hi is None or tok_hi >= n:
        return H.sample(n, count, rng)
    lo = H.sample(tok_hi, count // 2, rng)
    hi = tok_hi + rng.choice(n - tok_hi, size=count - count // 2, replace=False)
    return np.unique(np.concatenate([lo, hi, [n - 1]]))


class _Acc:
    def __init__(self):
        self.got, self.ref = {}, {}

    def add(self, name, got, ref):
        self.got.setdefault(name, []).append(np.asarray(got, dtype=np.float64))
        self.ref.setdefault(name, []).append(np.asarray(ref, dtype=np.float64))

    def check(self):
        for n in self.got:
            H.assert_close(n, np.concatenate(self.got[n]), np.concatenate(self.ref[n]))


def _check_sampled(pack, ins, out, seed):
    rng = np.random.default_rng(seed)
    tau = pack.softmax_scale()
    lay = oracle.PackLayout(pack.seq_q, pack.seq_kv, pack.heads)
    cached = _cached_rows(pack, ins)
    acc = _Acc()
    groups = {}
    n_heads_checked = 0
    for si, seg in enumerate(pack.segments):
        s, h0, h1, q0, q1, k0, k1, part = seg
        if part >= 0:
            groups.setdefault((s, q0, q1, h0, h1), []).append(seg)
            continue
        lq, lk = q1 - q0, k1 - k0
        deep = {h0 + (si + j * 7) % (h1 - h0) for j in range(2)}
        for h in range(h0, h1):
            n_heads_checked += 1
            qi_all = lay.q_index(s, q0, q1, h)
            ki_all = lay.kv_index(s, k0, k1, h)
            k = H.f64(ins["k"][ki_all])
            v = H.f64(ins["v"][ki_all])
            full_redo = lq <= FULL_REDO_TOKENS or (h in deep and lq * lk <= FULL_HEAD_LIMIT)
            nq = LONG_Q_SAMPLES if lq > LONG_TOKENS else DEEP_Q_SAMPLES if full_redo else Q_SAMPLES
            sel = H.sample(lq, nq, rng)
            qs = qi_all[sel]
            qq, dd = H.f64(ins["q"][qs]), H.f64(ins["do"][qs])
            o_r, l_r = oracle.head_forward(qq, k, v, tau)
            dq_r, _, _ = oracle.head_backward(qq, k, v, o_r, l_r, dd, tau)
            acc.add("o", H.f64(out["o"][qs]), o_r)
            acc.add("lse", H.f64(out["lse"][qs]), l_r)
            acc.add("dq", H.f64(out["dq"][qs]), dq_r)
            if (s, h) in cached and (q0, q1, k0, k1) == (0, pack.seq_q[s], 0, pack.seq_kv[s]):
                # dK/dV from the cached per-row LSE and D of the whole head
                l_all, d_all = cached[(s, h)]
                first_2g = max(0, -(-(ROW_2GB - lay.kv_off[s] - h) // pack.heads[s]))  # first token past 2^31 B
                ks = _key_sample(lk, CACHED_K_SAMPLES if lq > LONG_TOKENS else 64, rng,
                                 tok_hi=first_2g if first_2g < lk else None)
                qa, da = H.f64(ins["q"][qi_all]), H.f64(ins["do"][qi_all])
                _, dk_r, dv_r = oracle.head_backward_delta(qa, k[ks], v[ks], l_all, d_all, da, tau)
                name = "dk/dv rows past 2^31 B" if (ki_all[ks] >= ROW_2GB).any() else "dk/dv cached"
                print(f"  seq {s} head {h}: {len(ks)} keys from cached rows ({name}), "
                      f"{int((ki_all[ks] >= ROW_2GB).sum())} past 2^31 B", flush=True)
                acc.add("dk", H.f64(out["dk"][ki_all[ks]]), dk_r)
                acc.add("dv", H.f64(out["dv"][ki_all[ks]]), dv_r)
            elif full_redo:
                qa, da = H.f64(ins["q"][qi_all]), H.f64(ins["do"][qi_all])
                o_all, l_all = oracle.head_forward(qa, k, v, tau)
                ks = H.sample(lk, K_SAMPLES, rng)
                _, dk_r, dv_r = oracle.head_backward(qa, k[ks], v[ks], o_all, l_all, da, tau)
                acc.add("dk", H.f64(out["dk"][ki_all[ks]]), dk_r)
                acc.add("dv", H.f64(out["dv"][ki_all[ks]]), dv_r)
    for key, segs in groups.items():
        s, q0, q1, h0, h1 = key
        segs.sort(key=lambda x: x[7])
        k0, k1 = min(x[5] for x in segs), max(x[6] for x in segs)
        g = [gg for gg in out["plan"].groups if gg["seq"] == s and gg["o_row"] == lay.q_off[s] + q0 * pack.heads[s]][0]
        full_heads = {h0, h0 + (h1 - h0) // 2, h1 - 1}
        for h in range(h0, h1):
            n_heads_checked += 1
            qi_all = lay.q_index(s, q0, q1, h)
            ki_all = lay.kv_index(s, k0, k1, h)
            k, v = H.f64(ins["k"][ki_all]), H.f64(ins["v"][ki_all])
            if h in full_heads:
                qa, da = H.f64(ins["q"][qi_all]), H.f64(ins["do"][qi_all])
                o_all, l_all = oracle.head_forward(qa, k, v, tau)  # unsplit: what the merge must give
                sel = H.sample(len(qi_all), DEEP_Q_SAMPLES, rng)
                o_s, l_s, qq, dd = o_all[sel], l_all[sel], qa[sel], da[sel]
                ks = H.sample(len(ki_all), K_SAMPLES, rng)
                _, dk_r, dv_r = oracle.head_backward(qa, k[ks], v[ks], o_all, l_all, da, tau)
                acc.add("dk", H.f64(out["dk"][ki_all[ks]]), dk_r)
                acc.add("dv", H.f64(out["dv"][ki_all[ks]]), dv_r)
            else:
                sel = H.sample(len(qi_all), Q_SAMPLES, rng)
                qq, dd = H.f64(ins["q"][qi_all[sel]]), H.f64(ins["do"][qi_all[sel]])
                o_s, l_s = oracle.head_forward(qq, k, v, tau)
            dq_r, _, _ = oracle.head_backward(qq, k, v, o_s, l_s, dd, tau)
            for n, r in (("o", o_s), ("lse", l_s), ("dq", dq_r)):
                acc.add(n, H.f64(out[n][qi_all[sel]]), r)
            if "o_merged" in out:  # the same rows merged again by zl_lse_merge
                acc.add("o (zl_lse_merge)", H.f64(out["o_merged"][qi_all[sel]]), o_s)
                acc.add("lse (zl_lse_merge)", H.f64(out["lse_merged"][qi_all[sel]]), l_s)
            # every part's normalised partial on the sampled query rows
            for seg in segs:
                b, pk0, pk1 = seg[7], seg[5], seg[6]
                pki = lay.kv_index(s, pk0, pk1, h)
                po, pl = oracle.head_forward(qq, H.f64(ins["k"][pki]), H.f64(ins["v"][pki]), tau)
                slab = g["part_row"] + b * g["n_rows"] + sel.astype(np.int64) * (h1 - h0) + (h - h0)
                acc.add("o_part", H.f64(out["o_part"][slab]), po)
                acc.add("lse_part", H.f64(out["lse_part"][slab]), pl)
    print(f"  compared sampled rows on {n_heads_checked} (segment, head) pairs", flush=True)
    acc.check()


def _merge_again(out, pack):
    """Merge every ring group of the pack once more with zl_lse_merge into fresh buffers (groups
    over all stored heads: contiguous rows), so that the one-group call is checked at full size."""
    z = H.zl()
    plan = out["plan"]
    if not plan.groups:
        return
    o2 = torch.full_like(out["o"], float("nan"))
    l2 = torch.full_like(out["lse"], float("nan"))
    for g in plan.groups:
        assert g["head_end"] - g["head_begin"] == g["n_heads"]
        pr, r0, n = g["part_row"], g["o_row"], g["n_rows"]
        z.lse_merge(g["n_parts"], n, pack.d, out["o_part"][pr:], out["lse_part"][pr:], o2[r0:r0 + n], l2[r0:r0 + n])
    torch.cuda.synchronize()
    out["o_merged"], out["lse_merged"] = o2, l2


@pytest.mark.parametrize("name", ["image", "mixed", "ring", "long", "shard", "head1"])
def test_full_size(name):
    pack = W.config(name)
    print(f"[case] {name}: {len(pack.segments)} segments, q rows {pack.q_rows()}, kv rows {pack.kv_rows()}", flush=True)
    ins = W.draw(pack)
    out = H.run_pack(pack, ins)
    for n in ("o", "lse", "dq"):
        assert not torch.isnan(out[n]).any(), f"{n}: a covered row was not written"
    for n in ("dk", "dv"):
        assert not torch.isnan(out[n]).any(), f"{n}: a covered row was not written"
    _merge_again(out, pack)
    _check_invariants(pack, out, ins["do"].to(out["o"].device))
    _check_sampled(pack, ins, out, seed=pack.seed)


def test_full_size_d64():
    """d_head 64 at scale: 4 x 8192 tokens at 8 heads and one 32,760-token sequence at 2 heads,
    in the benchmark's launch configuration, checked on sampled rows like the packs above."""
    pack = W.whole_pack("wide64", [8192] * 4 + [32760], [8] * 4 + [2], 64, 9)
    print(f"[case] wide64: {len(pack.segments)} segments, q rows {pack.q_rows()}", flush=True)
    ins = W.draw(pack)
    out = H.run_pack(pack, ins)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert not torch.isnan(out[n]).any(), f"{n}: a covered row was not written"
    _check_invariants(pack, out, ins["do"].to(out["o"].device))
    _check_sampled(pack, ins, out, seed=pack.seed)
