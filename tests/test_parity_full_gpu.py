"""HIP path vs the fp64 oracle at the full sizes of the six large packs (the last one split-KV), in the launch
configuration the benchmark times (one plan, one forward launch, ring merges, one backward
launch over the whole pack).

The oracle cannot redo a whole pack in a test's time, so each (segment, head) checked is
compared on sampled rows the oracle computes one by one:
  * O, LSE and dQ on sampled query rows (each needs one pass over the segment's keys);
  * dK and dV on sampled key rows of segments whose full head the oracle can redo (it needs
    every query row's LSE and O), i.e. up to 32760 x 32760 per head;
  * ring partials of the KV-split pack on sampled rows of every part.
Properties that hold at any size are checked on every (segment, head) of the GPU output:
  * sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (softmax shift invariance, rows of P sum to 1);
  * every covered output row was written (the buffers start as NaN).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]

Q_SAMPLES = 32
K_SAMPLES = 32
FULL_HEAD_LIMIT = 32760 * 32760  # Lq * Lkv of the largest head the oracle redoes in full


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


def _check_sampled(pack, ins, out, seed):
    rng = np.random.default_rng(seed)
    tau = pack.softmax_scale()
    lay = oracle.PackLayout(pack.seq_q, pack.seq_kv, pack.heads)
    q64 = {n: ins[n] for n in ("q", "k", "v", "do")}
    got = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    ref = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    groups = {}
    for si, seg in enumerate(pack.segments):
        s, h0, h1, q0, q1, k0, k1, part = seg
        if part >= 0:
            groups.setdefault((s, q0, q1, h0, h1), []).append(seg)
            continue
        n_heads = 2 if (q1 - q0) <= 4096 else 1
        heads = [h0 + (si + j * 7) % (h1 - h0) for j in range(n_heads)]
        for h in sorted(set(heads)):
            qi_all = lay.q_index(s, q0, q1, h)
            ki_all = lay.kv_index(s, k0, k1, h)
            k = H.f64(q64["k"][ki_all])
            v = H.f64(q64["v"][ki_all])
            qs = qi_all[H.sample(len(qi_all), Q_SAMPLES, rng)]
            qq, dd = H.f64(q64["q"][qs]), H.f64(q64["do"][qs])
            o_r, l_r = oracle.head_forward(qq, k, v, tau)
            dq_r, _, _ = oracle.head_backward(qq, k, v, o_r, l_r, dd, tau)
            for n, r in (("o", o_r), ("lse", l_r), ("dq", dq_r)):
                got[n].append(H.f64(out[n][qs]))
                ref[n].append(r)
            if (q1 - q0) * (k1 - k0) <= FULL_HEAD_LIMIT:
                qa, da = H.f64(q64["q"][qi_all]), H.f64(q64["do"][qi_all])
                o_all, l_all = oracle.head_forward(qa, k, v, tau)
                ks = H.sample(len(ki_all), K_SAMPLES, rng)
                _, dk_r, dv_r = oracle.head_backward(qa, k[ks], v[ks], o_all, l_all, da, tau)
                got["dk"].append(H.f64(out["dk"][ki_all[ks]]))
                got["dv"].append(H.f64(out["dv"][ki_all[ks]]))
                ref["dk"].append(dk_r)
                ref["dv"].append(dv_r)
    for key, segs in groups.items():
        s, q0, q1, h0, h1 = key
        segs.sort(key=lambda x: x[7])
        k0, k1 = min(x[5] for x in segs), max(x[6] for x in segs)
        g = [gg for gg in out["plan"].groups if gg["seq"] == s and gg["o_row"] == lay.q_off[s] + q0 * pack.heads[s]][0]
        for h in (h0, h0 + (h1 - h0) // 2, h1 - 1):
            qi_all = lay.q_index(s, q0, q1, h)
            ki_all = lay.kv_index(s, k0, k1, h)
            k, v = H.f64(q64["k"][ki_all]), H.f64(q64["v"][ki_all])
            qa, da = H.f64(q64["q"][qi_all]), H.f64(q64["do"][qi_all])
            o_all, l_all = oracle.head_forward(qa, k, v, tau)  # unsplit: what the merge must give
            sel = H.sample(len(qi_all), Q_SAMPLES, rng)
            dq_r, _, _ = oracle.head_backward(qa[sel], k, v, o_all[sel], l_all[sel], da[sel], tau)
            for n, r in (("o", o_all[sel]), ("lse", l_all[sel]), ("dq", dq_r)):
                got[n].append(H.f64(out[n][qi_all[sel]]))
                ref[n].append(r)
            ks = H.sample(len(ki_all), K_SAMPLES, rng)
            _, dk_r, dv_r = oracle.head_backward(qa, k[ks], v[ks], o_all, l_all, da, tau)
            got["dk"].append(H.f64(out["dk"][ki_all[ks]]))
            got["dv"].append(H.f64(out["dv"][ki_all[ks]]))
            ref["dk"].append(dk_r)
            ref["dv"].append(dv_r)
            # every part's normalised partial on the sampled query rows
            for seg in segs:
                b, pk0, pk1 = seg[7], seg[5], seg[6]
                pki = lay.kv_index(s, pk0, pk1, h)
                po, pl = oracle.head_forward(qa[sel], H.f64(q64["k"][pki]), H.f64(q64["v"][pki]), tau)
                slab = g["part_row"] + b * g["n_rows"] + sel.astype(np.int64) * pack.heads[s] + (h - h0)
                got.setdefault("o_part", []).append(H.f64(out["o_part"][slab]))
                got.setdefault("lse_part", []).append(H.f64(out["lse_part"][slab]))
                ref.setdefault("o_part", []).append(po)
                ref.setdefault("lse_part", []).append(pl)
    for n in got:
        if got[n]:
            H.assert_close(n, np.concatenate(got[n]), np.concatenate(ref[n]))


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
