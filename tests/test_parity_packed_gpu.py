"""QKV-packed layout (the buffer a QKV-packed all-to-all delivers: per sequence
[tokens][Q, K, V][heads][d], and the same for dQ, dK, dV) vs the planar layout.

The kernels only address rows differently, so the packed run must reproduce the planar run bit
for bit: O, LSE, every ring partial and, unpacked, dQ, dK and dV, with untouched rows left
untouched. The planar run is itself checked against the fp64 oracle. Covers whole sequences,
head subsets, a query range, a ring group and split-KV items at d_head 64 and 128, and the
seeded random packs whose sequences have equal query and key lengths.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_harness as H
from tests import random_packs as R

pytestmark = [pytest.mark.gpu, H.requires_gpu]


def _pack_qkv(pack, q, k, v):
    """Per sequence, [L, nh, d] x 3 -> [L, 3, nh, d], sequences one after another."""
    out, off = [], 0
    for L, nh in zip(pack.seq_q, pack.heads):
        parts = [t[off:off + L * nh].view(L, nh, -1) for t in (q, k, v)]
        out.append(torch.stack(parts, dim=1).reshape(3 * L * nh, -1))
        off += L * nh
    return torch.cat(out).contiguous()


def _unpack(pack, t):
    qs, ks, vs, off = [], [], [], 0
    for L, nh in zip(pack.seq_q, pack.heads):
        x = t[off:off + 3 * L * nh].view(L, 3, nh, -1)
        qs.append(x[:, 0].reshape(L * nh, -1))
        ks.append(x[:, 1].reshape(L * nh, -1))
        vs.append(x[:, 2].reshape(L * nh, -1))
        off += 3 * L * nh
    return torch.cat(qs), torch.cat(ks), torch.cat(vs)


def _same(name, a, b):
    """Bit-for-bit equality (NaN fills included), compared where the tensors live."""
    nan_a, nan_b = torch.isnan(a), torch.isnan(b)
    assert torch.equal(nan_a, nan_b), f"{name}: written rows differ"
    assert torch.equal(torch.nan_to_num(a), torch.nan_to_num(b)), f"{name}: values differ"


def _packed_matches(pack, ins, planar, rows=None):
    """Run `pack` in the QKV-packed layout (forward items of `rows` query rows, or the plan's
    choice) and compare every output with the planar run bit for bit."""
    z = H.zl()
    dev = torch.device("cuda:0")
    d = pack.d
    plan = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, d, qkv_packed=True, item_rows=rows)
    assert plan.info["fwd_rows"] == planar["plan"].info["fwd_rows"]
    info = plan.info
    assert info["qkv_rows"] == 3 * info["q_rows"]
    qkv = _pack_qkv(pack, ins["q"].to(dev), ins["k"].to(dev), ins["v"].to(dev))
    do = ins["do"].to(dev)
    nan = float("nan")
    o = torch.full((info["q_rows"], d), nan, dtype=torch.float32, device=dev)
    lse = torch.full((info["q_rows"],), nan, dtype=torch.float32, device=dev)
    o, lse, o_part, lse_part = z.attn_fwd(plan, qkv, qkv, qkv, o=o, lse=lse)
    if info["n_groups"]:
        z.merge_groups(plan, o_part, lse_part, o, lse)
    dqkv = torch.full((info["qkv_rows"], d), nan, dtype=torch.float32, device=dev)
    z.attn_bwd(plan, qkv, qkv, qkv, o, lse, do, dq=dqkv, dk=dqkv, dv=dqkv)
    torch.cuda.synchronize()
    _same("o", o, planar["o"])
    _same("lse", lse, planar["lse"])
    if planar["o_part"] is not None:
        _same("o_part", o_part, planar["o_part"])
        _same("lse_part", lse_part, planar["lse_part"])
    dq, dk, dv = _unpack(pack, dqkv)
    _same("dq", dq, planar["dq"])
    _same("dk", dk, planar["dk"])
    _same("dv", dv, planar["dv"])


CASES = {
    "mixed_segments": (
        (200, 333, 700, 5000), (4, 4, 2, 1),
        ((0, 0, 4, 0, 200, 0, 200, -1),
         (1, 1, 3, 0, 333, 0, 333, -1), (1, 0, 1, 17, 290, 0, 333, -1),
         (2, 0, 2, 0, 300, 0, 350, 0), (2, 0, 2, 0, 300, 350, 700, 1),
         (3, 0, 1, 0, 5000, 0, 5000, -1))),
}


@pytest.mark.parametrize("rows", [None, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_packed_matches_planar_bitwise(d, rows):
    lens, heads, seg = CASES["mixed_segments"]
    pack = W.Pack(f"packed{d}", lens, lens, heads, seg, d, 90 + d)
    ins = W.draw(pack)
    print(f"[case] packed vs planar d={d} item_rows={rows or 'plan'}", flush=True)
    planar = H.run_pack(pack, ins, item_rows=rows)
    assert planar["plan"].info["split_tiles"] > 0
    ref = H.oracle_pack(pack, ins)
    H.compare_full(pack, ins, planar, ref)
    _packed_matches(pack, ins, planar, rows)


def test_packed_rejects_distinct_pointers():
    z = H.zl()
    dev = torch.device("cuda:0")
    plan = z.Plan((64,), (64,), (1,), ((0, 0, 1, 0, 64, 0, 64, -1),), 64, qkv_packed=True)
    qkv = torch.zeros(3 * 64, 64, dtype=torch.bfloat16, device=dev)
    other = torch.zeros(3 * 64, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(z.ZlError, match="q == k == v"):
        z.attn_fwd(plan, qkv, other, qkv)


PACKED_SEEDS = tuple(seed for seed in R.SEEDS if R.random_pack(seed).seq_q == R.random_pack(seed).seq_kv)


@pytest.mark.parametrize("seed", PACKED_SEEDS)
def test_random_packs_packed_match_planar(seed):
    """The seeded random packs whose sequences have equal query and key lengths (ring groups with
    out-of-order parts, head subsets, query ranges, split items), packed vs planar bit for bit."""
    pack = R.random_pack(seed)
    ins = W.draw(pack)
    print(f"[case] packed vs planar {pack.name} d={pack.d} seqs={pack.seq_q} heads={pack.heads}", flush=True)
    planar = H.run_pack(pack, ins)
    _packed_matches(pack, ins, planar)


def test_packed_matches_planar_at_full_size():
    """The mixed image-video pack in the QKV-packed layout: 4.3 M query rows, so the packed bf16
    buffer (3.3 GB) and the packed fp32 gradients (6.6 GB) are addressed past 2^31 bytes; every
    output bit for bit against the planar run (itself checked against the oracle at full size)."""
    pack = W.config("mixed")
    ins = W.draw(pack)
    print(f"[case] packed vs planar, mixed pack: {pack.q_rows()} rows", flush=True)
    planar = H.run_pack(pack, ins)
    assert 3 * pack.q_rows() * pack.d * 2 > 2 ** 31
    _packed_matches(pack, ins, planar)
