"""Running-merge forward (zl_attn_fwd_accumulate) vs the fp64 oracle.

Ring accumulation: each call folds one key/value block of a query chunk into the running
(O, LSE) at the chunk's rows. After the last block, in any order, the rows must hold
attention over the whole key range, element by element within the usual tolerance; after
the first block they must hold that block's own result. Covers d_head 64 and 128, blocks of
one key and of ragged lengths, two ring groups folded in the same calls, whole segments
written in the same launch, and the seeded random packs that hold ring groups.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_harness as H
from tests import random_packs as R

pytestmark = [pytest.mark.gpu, H.requires_gpu]

SEQ_Q = (150, 77, 100)
SEQ_KV = (333, 77, 300)
HEADS = (3, 3, 2)
BLOCKS0 = ((0, 1), (1, 64), (64, 200), (200, 333))  # sequence 0: queries [0,150), 3 heads
BLOCKS2 = ((0, 150), (150, 300))                    # sequence 2: queries [20,100), 2 heads
WHOLE1 = (1, 0, 3, 0, 77, 0, 77, -1)


def _oracle(d, segs, ins):
    q, k, v = (H.f64(ins[n]) for n in ("q", "k", "v"))
    scale = 1.0 / np.sqrt(d)
    return oracle.pack_forward(SEQ_Q, SEQ_KV, HEADS, segs, d, scale, q, k, v)


def _rows(lay, s, q0, q1, h0, h1):
    return np.concatenate([lay.q_index(s, q0, q1, h) for h in range(h0, h1)])


@pytest.mark.parametrize("d,order,rows", [(64, (2, 0, 3, 1), None), (128, (0, 1, 2, 3), None),
                                          (128, (3, 2, 1, 0), None), (64, (1, 3, 0, 2), 256),
                                          (128, (2, 1, 3, 0), 256)])
def test_ring_blocks_folded_one_call_at_a_time(d, order, rows):
    """rows: the forward item size (256 forces the 8-wave forward; None is the plan's choice)."""
    z = H.zl()
    dev = torch.device("cuda:0")
    pack = W.Pack(f"acc{d}", SEQ_Q, SEQ_KV, HEADS, (WHOLE1,), d, 31 + d)
    ins = W.draw(pack)
    q, k, v = (ins[n].to(dev) for n in ("q", "k", "v"))
    lay = oracle.PackLayout(SEQ_Q, SEQ_KV, HEADS)
    rows0 = _rows(lay, 0, 0, 150, 0, 3)
    rows2 = _rows(lay, 2, 20, 100, 0, 2)
    n_q = int(lay.q_off[-1])
    o = torch.full((n_q, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((n_q,), float("nan"), dtype=torch.float32, device=dev)
    lse[torch.as_tensor(np.concatenate([rows0, rows2]), device=dev)] = float("-inf")
    print(f"[case] accumulate d={d} order={order} item_rows={rows or 'plan'}", flush=True)
    for i, b in enumerate(order):
        segs = [(0, 0, 3, 0, 150, BLOCKS0[b][0], BLOCKS0[b][1], 0)]
        if i < len(BLOCKS2):
            segs.append((2, 0, 2, 20, 100, BLOCKS2[i][0], BLOCKS2[i][1], 0))
        if i == 0:
            segs.append(WHOLE1)
        plan = z.Plan(SEQ_Q, SEQ_KV, HEADS, tuple(segs), d, item_rows=rows)
        z.attn_fwd_accumulate(plan, q, k, v, o, lse)
        if i == 0:
            torch.cuda.synchronize()
            first = _oracle(d, [(0, 0, 3, 0, 150, BLOCKS0[b][0], BLOCKS0[b][1], -1)], ins)
            H.assert_close("first block O", H.f64(o)[rows0], first["o"][rows0])
            H.assert_close("first block LSE", H.f64(lse)[rows0], first["lse"][rows0])
    torch.cuda.synchronize()
    ref = _oracle(d, [(0, 0, 3, 0, 150, 0, 333, -1), WHOLE1, (2, 0, 2, 20, 100, 0, 300, -1)], ins)
    go, gl = H.f64(o), H.f64(lse)
    cov = ~np.isnan(ref["lse"])
    assert cov.sum() == len(rows0) + len(rows2) + 77 * 3
    H.assert_close("O", go[cov], ref["o"][cov])
    H.assert_close("LSE", gl[cov], ref["lse"][cov])
    assert np.isnan(go[~cov]).all() and np.isnan(gl[~cov]).all(), "rows no segment covers were written"


def test_whole_segments_match_plain_forward_bit_for_bit():
    """With no ring part in the plan the running-merge forward is the plain forward."""
    z = H.zl()
    dev = torch.device("cuda:0")
    pack = W.tiny()
    ins = W.draw(pack)
    q, k, v = (ins[n].to(dev) for n in ("q", "k", "v"))
    plan = H.make_plan(pack)
    n_q = plan.info["q_rows"]
    print("[case] accumulate vs plain forward, tiny pack", flush=True)
    o1, l1, _, _ = z.attn_fwd(plan, q, k, v)
    o2 = torch.zeros((n_q, pack.d), dtype=torch.float32, device=dev)
    l2 = torch.zeros((n_q,), dtype=torch.float32, device=dev)
    z.attn_fwd_accumulate(plan, q, k, v, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
def test_head_subset_group_folded(d):
    """A ring group over heads [1,3) of 4: each fold lands at the subset's strided rows and
    leaves the other heads' rows untouched."""
    z = H.zl()
    dev = torch.device("cuda:0")
    seq_q, seq_kv, heads = (140,), (230,), (4,)
    blocks = ((0, 64), (64, 65), (65, 230))
    pack = W.Pack(f"acc_sub{d}", seq_q, seq_kv, heads, ((0, 1, 3, 0, 140, 0, 230, -1),), d, 41 + d)
    ins = W.draw(pack)
    q, k, v = (ins[n].to(dev) for n in ("q", "k", "v"))
    lay = oracle.PackLayout(seq_q, seq_kv, heads)
    rows = _rows(lay, 0, 0, 140, 1, 3)
    n_q = int(lay.q_off[-1])
    o = torch.full((n_q, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((n_q,), float("nan"), dtype=torch.float32, device=dev)
    lse[torch.as_tensor(rows, device=dev)] = float("-inf")
    print(f"[case] accumulate head subset d={d}", flush=True)
    for b in (1, 2, 0):
        plan = z.Plan(seq_q, seq_kv, heads, ((0, 1, 3, 0, 140, blocks[b][0], blocks[b][1], 0),), d)
        z.attn_fwd_accumulate(plan, q, k, v, o, lse)
    torch.cuda.synchronize()
    qf, kf, vf = (H.f64(ins[n]) for n in ("q", "k", "v"))
    ref = oracle.pack_forward(seq_q, seq_kv, heads, [(0, 1, 3, 0, 140, 0, 230, -1)], d, 1.0 / np.sqrt(d), qf, kf, vf)
    go, gl = H.f64(o), H.f64(lse)
    cov = ~np.isnan(ref["lse"])
    assert cov.sum() == len(rows)
    H.assert_close("O", go[cov], ref["o"][cov])
    H.assert_close("LSE", gl[cov], ref["lse"][cov])
    assert np.isnan(go[~cov]).all() and np.isnan(gl[~cov]).all(), "rows outside the head subset were written"


ACC_SEEDS = tuple(seed for seed in R.SEEDS if any(sg[7] >= 0 for sg in R.random_pack(seed).segments))


@pytest.mark.parametrize("seed", ACC_SEEDS)
def test_random_packs_folded_part_by_part(seed):
    """The seeded random packs with ring groups, forward by running merge: launch b folds part b
    of every group (renumbered part 0 of a one-part plan) into O and LSE, whole segments go with
    launch 0, and every row starts at LSE = -inf. After the last launch every covered row must
    hold the oracle's merged result."""
    z = H.zl()
    dev = torch.device("cuda:0")
    pack = R.random_pack(seed)
    ins = W.draw(pack)
    q, k, v = (ins[n].to(dev) for n in ("q", "k", "v"))
    n_q = pack.q_rows()
    o = torch.full((n_q, pack.d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((n_q,), float("-inf"), dtype=torch.float32, device=dev)
    n_launch = 1 + max(sg[7] for sg in pack.segments)
    print(f"[case] running merge {pack.name} d={pack.d} launches={n_launch}", flush=True)
    for b in range(n_launch):
        segs = tuple(sg[:7] + (0,) for sg in pack.segments if sg[7] == b)
        if b == 0:
            segs += tuple(sg for sg in pack.segments if sg[7] < 0)
        plan = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, segs, pack.d)
        z.attn_fwd_accumulate(plan, q, k, v, o, lse)
    torch.cuda.synchronize()
    ref = H.oracle_pack(pack, ins)
    cov = ~np.isnan(ref["lse"])
    H.assert_close("O", H.f64(o)[cov], ref["o"][cov])
    H.assert_close("LSE", H.f64(lse)[cov], ref["lse"][cov])
