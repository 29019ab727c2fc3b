"""HIP path vs the fp64 oracle on packs the oracle finishes in seconds, element by element.

Covers: the tiny 3-sequence pack (d_head 64), ragged lengths around the tile sizes, head
subsets (Ulysses shards), query ranges (all-gather shards), ring groups with uneven parts
including a one-key part, ring groups over head subsets, peaked and drifting-max softmax inputs, and untouched rows.

Packs this small get 128-row forward items from the plan; the cases marked ``rows`` run again
with 256-row items forced (the 8-wave forward kernel, which the plan picks for deep queues), so
that both forward instances meet the oracle on ragged tails, subsets and ring parts.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]


ROWS = pytest.mark.parametrize("rows", [None, 256])


def _run(pack, ins=None, stress=False, rows=None):
    ins = W.draw(pack) if ins is None else ins
    print(f"[case] {pack.name} d={pack.d} seqs={pack.seq_q}/{pack.seq_kv} segs={len(pack.segments)} "
          f"item_rows={rows or 'plan'}", flush=True)
    out = H.run_pack(pack, ins, item_rows=rows)
    ref = H.oracle_pack(pack, ins)
    H.compare_full(pack, ins, out, ref, scaled_max_abs=stress)
    return out, ref


@ROWS
def test_tiny_pack_full(rows):
    _run(W.tiny(), rows=rows)


@ROWS
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_lengths(d, rows):
    lens = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300]
    pack = W.whole_pack(f"ragged{d}", lens, [2] * len(lens), d, 11)
    _run(pack, rows=rows)


@ROWS
@pytest.mark.parametrize("d", [64, 128])
def test_head_subsets_and_query_ranges(d, rows):
    seg = (
        (0, 0, 4, 0, 200, 0, 200, -1),      # whole, 4 heads
        (1, 1, 3, 0, 333, 0, 333, -1),      # Ulysses-style head subset [1,3)
        (1, 0, 1, 17, 290, 0, 333, -1),     # query range of head 0
        (1, 3, 4, 0, 129, 5, 300, -1),      # query and key ranges of head 3
        (2, 0, 2, 0, 45, 0, 700, -1),       # short queries, long keys
    )
    pack = W.Pack(f"subsets{d}", (200, 333, 45), (200, 333, 700), (4, 4, 2), seg, d, 12)
    _run(pack, rows=rows)


def test_ring_group_shrunk():
    """The ring KV-split shard at reduced size: 300 queries vs 2400 keys in 8 blocks, 4 heads."""
    pack = W.ring_pack("ring_small", 300, 2400, 8, 4, 128, 13)
    _run(pack)


@ROWS
def test_ring_group_uneven_parts(rows):
    seg = ((0, 0, 3, 0, 150, 0, 1, 2), (0, 0, 3, 0, 150, 1, 64, 0), (0, 0, 3, 0, 150, 64, 200, 1),
           (0, 0, 3, 0, 150, 200, 333, 3), (1, 0, 3, 0, 77, 0, 77, -1))
    pack = W.Pack("ring_uneven", (150, 77), (333, 77), (3, 3), seg, 128, 14)
    _run(pack, rows=rows)


def test_two_ring_groups_and_whole():
    # two query chunks of different sequences, each a two-part ring group, plus a whole one
    seg = ((0, 0, 2, 0, 100, 0, 150, 0), (0, 0, 2, 0, 100, 150, 300, 1),
           (1, 0, 2, 0, 156, 0, 100, 0), (1, 0, 2, 0, 156, 100, 300, 1),
           (2, 0, 2, 0, 90, 0, 90, -1))
    pack = W.Pack("two_rings", (100, 156, 90), (300, 300, 90), (2, 2, 2), seg, 64, 15)
    _run(pack)


@ROWS
@pytest.mark.parametrize("d", [64, 128])
def test_head_subset_ring_groups(d, rows):
    """Composed placements (Ulysses heads x ring keys): groups over head subsets, merged in
    one launch into strided O rows; rows of the subset heads outside the groups stay untouched."""
    seg = ((0, 0, 2, 0, 200, 0, 100, 0), (0, 0, 2, 0, 200, 100, 260, 1),
           (0, 2, 5, 0, 130, 0, 1, 0), (0, 2, 5, 0, 130, 1, 77, 1), (0, 2, 5, 0, 130, 77, 260, 2),
           (0, 5, 6, 0, 200, 0, 260, -1),
           (1, 1, 3, 5, 90, 0, 45, 1), (1, 1, 3, 5, 90, 45, 90, 0))
    pack = W.Pack(f"head_subset_rings{d}", (200, 90), (260, 90), (6, 3), seg, d, 18)
    _run(pack, rows=rows)


@ROWS
def test_peaked_softmax(rows):
    """Queries scaled by 8: nearly one-hot rows of P, large running-max changes."""
    pack = W.whole_pack("peaked", [257, 1000], [2, 2], 128, 16)
    ins = W.draw(pack)
    ins["q"] = (ins["q"].float() * 8).to(torch.bfloat16)
    _run(pack, ins, stress=True, rows=rows)


@ROWS
def test_drifting_max(rows):
    """Key norms grow along the sequence, so the running max changes in every key block."""
    pack = W.whole_pack("drift", [640, 1100], [2, 1], 128, 17)
    ins = W.draw(pack)
    n_k = ins["k"].shape[0]
    ramp = torch.linspace(0.25, 3.0, n_k).unsqueeze(1)
    ins["k"] = (ins["k"].float() * ramp).to(torch.bfloat16)
    _run(pack, ins, stress=True, rows=rows)


def test_block_diagonal_separation_bitwise():
    """Changing one sequence's K/V leaves every other sequence's outputs bit for bit."""
    pack = W.whole_pack("sep", [100, 300, 77], [2, 2, 2], 128, 18)
    ins = W.draw(pack)
    a = H.run_pack(pack, ins)
    ins2 = {k: v.clone() for k, v in ins.items()}
    k0, k1 = 100 * 2, 100 * 2 + 300 * 2
    ins2["k"][k0:k1] = (ins2["k"][k0:k1].float() + 0.5).to(torch.bfloat16)
    ins2["v"][k0:k1] = (ins2["v"][k0:k1].float() - 1.0).to(torch.bfloat16)
    b = H.run_pack(pack, ins2)
    q_other = np.r_[0:200, 800:800 + 154]
    for n in ("o", "lse"):
        assert torch.equal(a[n][q_other].cpu(), b[n][q_other].cpu()), n
    for n in ("dk", "dv"):  # written once per row, no atomics: bitwise too
        assert torch.equal(a[n][q_other].cpu(), b[n][q_other].cpu()), n
    assert not torch.equal(a["o"][200:800].cpu(), b["o"][200:800].cpu())


@ROWS
def test_bitwise_reproducible(rows):
    """No atomics on data: two runs of the same pack give identical bits (ring group included)."""
    seg = ((0, 0, 2, 0, 300, 0, 200, 0), (0, 0, 2, 0, 300, 200, 500, 1), (1, 0, 3, 0, 129, 0, 129, -1))
    pack = W.Pack("repro", (300, 129), (500, 129), (2, 3), seg, 128, 19)
    ins = W.draw(pack)
    a = H.run_pack(pack, ins, item_rows=rows)
    b = H.run_pack(pack, ins, item_rows=rows)
    for n in ("o", "lse", "dq", "dk", "dv", "o_part", "lse_part"):
        assert torch.equal(a[n].cpu(), b[n].cpu()), n
