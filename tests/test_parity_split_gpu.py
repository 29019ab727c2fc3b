"""Split-KV forward (items cut into key pieces, merged by the last piece) vs the fp64 oracle.

Packs with few long items make the plan cut every forward item into key pieces; the result
must match the oracle element by element as an unsplit forward does, for final segments,
ring parts (partials in the slab, then the plan merge) and the running merge, with ragged
piece tails, at d_head 64 and 128. The backward runs on the split forward's O and LSE. The
whole-sequence and ring cases run with both forward item sizes (the pieces of a 256-row item
use 256-row slots of the split workspace).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]


def _run(pack, rows=None):
    ins = W.draw(pack)
    print(f"[case] {pack.name} d={pack.d} seqs={pack.seq_q}/{pack.seq_kv} segs={len(pack.segments)} "
          f"item_rows={rows or 'plan'}", flush=True)
    out = H.run_pack(pack, ins, item_rows=rows)
    assert out["plan"].info["split_tiles"] > 0, "the pack was meant to be split"
    ref = H.oracle_pack(pack, ins)
    H.compare_full(pack, ins, out, ref)
    return out, ref, ins


@pytest.mark.parametrize("rows", [None, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_split_whole_sequences(d, rows):
    seg = ((0, 0, 1, 0, 4100, 0, 4100, -1), (1, 0, 2, 0, 700, 0, 2500, -1), (2, 0, 2, 0, 90, 0, 90, -1))
    _run(W.Pack(f"split_whole{d}", (4100, 700, 90), (4100, 2500, 90), (1, 2, 2), seg, d, 51 + d), rows)


@pytest.mark.parametrize("rows", [None, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_split_ring_parts(d, rows):
    """Ring parts long enough to be split: each part's pieces merge into its slab rows, then
    the plan merge combines the parts."""
    seg = ((0, 0, 2, 0, 333, 0, 2100, 1), (0, 0, 2, 0, 333, 2100, 6000, 0), (1, 1, 2, 0, 150, 0, 3000, -1))
    _run(W.Pack(f"split_ring{d}", (333, 150), (6000, 3000), (2, 2), seg, d, 61 + d), rows)


def test_split_matches_unsplit_plan():
    """The same pack with and without split-KV: both within the oracle tolerance of the
    oracle and of each other. They are not closer to each other than to the oracle: P is
    rounded to bf16 relative to each piece's own running max, so the two round differently."""
    z = H.zl()
    dev = torch.device("cuda:0")
    seg = ((0, 0, 2, 0, 500, 0, 5000, -1),)
    pack = W.Pack("split_vs_unsplit", (500,), (5000,), (2,), seg, 128, 71)
    ins = W.draw(pack)
    q, k, v = (ins[n].to(dev) for n in ("q", "k", "v"))
    print("[case] split vs unsplit plan", flush=True)
    outs = []
    for split in (True, False):
        plan = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, split=split)
        assert (plan.info["split_tiles"] > 0) == split
        o, lse, _, _ = z.attn_fwd(plan, q, k, v)
        outs.append((H.f64(o), H.f64(lse)))
    torch.cuda.synchronize()
    ref = H.oracle_pack(pack, ins)
    for (o, lse) in outs:
        H.assert_close("O", o, ref["o"])
        H.assert_close("LSE", lse, ref["lse"])
    H.assert_close("O split vs unsplit", outs[0][0], outs[1][0])
    H.assert_close("LSE split vs unsplit", outs[0][1], outs[1][1])


@pytest.mark.parametrize("d", [64, 128])
def test_split_running_merge(d):
    """Running merge of ring blocks whose items are split: the last piece of each item folds
    the merged block result into the running O/LSE."""
    z = H.zl()
    dev = torch.device("cuda:0")
    seq_q, seq_kv, heads = (260,), (7000,), (1,)
    blocks = ((0, 2600), (2600, 2700), (2700, 7000))
    pack = W.Pack(f"split_acc{d}", seq_q, seq_kv, heads, ((0, 0, 1, 0, 260, 0, 7000, -1),), d, 81 + d)
    ins = W.draw(pack)
    q, k, v = (ins[n].to(dev) for n in ("q", "k", "v"))
    o = torch.full((260, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((260,), float("-inf"), dtype=torch.float32, device=dev)
    print(f"[case] split running merge d={d}", flush=True)
    n_split = 0
    for b in (2, 0, 1):
        plan = z.Plan(seq_q, seq_kv, heads, ((0, 0, 1, 0, 260, blocks[b][0], blocks[b][1], 0),), d)
        n_split += plan.info["split_tiles"]
        z.attn_fwd_accumulate(plan, q, k, v, o, lse)
    torch.cuda.synchronize()
    assert n_split > 0
    ref = H.oracle_pack(pack, ins)
    H.assert_close("O", H.f64(o), ref["o"])
    H.assert_close("LSE", H.f64(lse), ref["lse"])


def _dq_split_run(pack):
    ins = W.draw(pack)
    print(f"[case] {pack.name} d={pack.d} seqs={pack.seq_q}/{pack.seq_kv} segs={len(pack.segments)}", flush=True)
    out = H.run_pack(pack, ins)
    assert out["plan"].info["dq_split_tiles"] > 0, "the dQ queue was meant to be split"
    ref = H.oracle_pack(pack, ins)
    H.compare_full(pack, ins, out, ref)
    return out, ins


@pytest.mark.parametrize("d", [64, 128])
def test_dq_split_whole_sequence(d):
    """One head of 5000 tokens: 40 dQ items, each cut into pieces of its 79 key blocks (the
    last one ragged); the last piece of each item adds the pieces' partials."""
    pack = W.Pack(f"dq_split{d}", (5000,), (5000,), (1,), ((0, 0, 1, 0, 5000, 0, 5000, -1),), d, 91 + d)
    _dq_split_run(pack)


@pytest.mark.parametrize("d", [64, 128])
def test_dq_split_ring_chain(d):
    """A ring group of three uneven parts: the dQ items walk the parts' key blocks as one chain and
    their pieces cut it across part boundaries (ragged blocks at every part's end)."""
    seg = ((0, 0, 2, 0, 333, 0, 1900, 0), (0, 0, 2, 0, 333, 1900, 4100, 1), (0, 0, 2, 0, 333, 4100, 6000, 2))
    _dq_split_run(W.Pack(f"dq_split_ring{d}", (333,), (6000,), (2,), seg, d, 95 + d))


def test_dq_split_reproducible_and_close_to_unsplit():
    """Pieces are added in piece order, so split dQ, dK and dV are bitwise the same on every run
    whatever piece finishes last; they match the unsplit plan's within the oracle tolerance (the
    summation order differs)."""
    z = H.zl()
    dev = torch.device("cuda:0")
    pack = W.Pack("dq_split_repro", (3000,), (3000,), (2,), ((0, 0, 2, 0, 3000, 0, 3000, -1),), 128, 97)
    ins = W.draw(pack)
    q, k, v, do = (ins[n].to(dev) for n in ("q", "k", "v", "do"))
    print("[case] dQ split: reproducible, close to unsplit", flush=True)
    grads = []
    for split in (True, True, False):
        plan = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, split=split)
        assert (plan.info["dq_split_tiles"] > 0) == split and (plan.info["kv_split_tiles"] > 0) == split
        o, lse, _, _ = z.attn_fwd(plan, q, k, v)
        grads.append(z.attn_bwd(plan, q, k, v, o, lse, do))
    torch.cuda.synchronize()
    ref = H.oracle_pack(pack, ins)
    for i, name in enumerate(("dq", "dk", "dv")):
        assert torch.equal(grads[0][i], grads[1][i]), f"split {name} differs between two runs"
        for g in grads:
            H.assert_close(name, H.f64(g[i]), ref[name])
        H.assert_close(f"{name} split vs unsplit", H.f64(grads[0][i]), H.f64(grads[2][i]))


@pytest.mark.parametrize("d", [64, 128])
def test_dkdv_split_many_queries(d):
    """Few keys, many queries: the dK/dV items (128 keys each) loop over 47 query blocks of 64
    rows (the last one ragged) and are cut into runs of them; the last piece of each item adds
    the partial dK and dV. dV sums over 3000 queries, so its rows' magnitudes are well above 1:
    each element's max-abs bound scales with its own row's magnitude (rel-L2 unchanged)."""
    pack = W.Pack(f"kv_split{d}", (3000,), (500,), (2,), ((0, 0, 2, 0, 3000, 0, 500, -1),), d, 101 + d)
    ins = W.draw(pack)
    print(f"[case] {pack.name} d={pack.d} seqs={pack.seq_q}/{pack.seq_kv}", flush=True)
    out = H.run_pack(pack, ins)
    assert out["plan"].info["kv_split_tiles"] > 0, "the dK/dV queue was meant to be split"
    H.compare_full(pack, ins, out, H.oracle_pack(pack, ins), row_scaled=True)


@pytest.mark.parametrize("name", ["dq_split_repro", "ring_group"])
def test_staged_backward_matches_one_call(name):
    """The pre-pass, dK/dV and dQ launched by three calls on one workspace (the way the
    benchmark times them) give the same bits as one call: the pre-pass alone sets both queues'
    counters, the split counters and the row values the later launches read. Cases: one head of
    3,000 tokens (dQ and dK/dV queues cut into pieces) and a ring group with a whole sequence."""
    z = H.zl()
    dev = torch.device("cuda:0")
    if name == "dq_split_repro":
        pack = W.Pack(name, (3000,), (3000,), (2,), ((0, 0, 2, 0, 3000, 0, 3000, -1),), 128, 97)
    else:
        seg = ((0, 0, 2, 0, 300, 0, 200, 0), (0, 0, 2, 0, 300, 200, 500, 1), (1, 0, 3, 0, 129, 0, 129, -1))
        pack = W.Pack(name, (300, 129), (500, 129), (2, 3), seg, 128, 19)
    ins = W.draw(pack)
    q, k, v, do = (ins[n].to(dev) for n in ("q", "k", "v", "do"))
    print(f"[case] staged backward: {name}", flush=True)
    plan = H.make_plan(pack)
    if name == "dq_split_repro":
        assert plan.info["dq_split_tiles"] > 0 and plan.info["kv_split_tiles"] > 0
    o, lse, o_part, lse_part = z.attn_fwd(plan, q, k, v)
    if plan.info["n_groups"]:
        z.merge_groups(plan, o_part, lse_part, o, lse)
    one = z.attn_bwd(plan, q, k, v, o, lse, do)
    info = plan.info
    nan = lambda rows: torch.full((rows, pack.d), float("nan"), device=dev)
    dq, dk, dv = nan(info["q_rows"]), nan(info["kv_rows"]), nan(info["kv_rows"])
    ws = torch.empty(info["ws_bwd"], dtype=torch.uint8, device=dev)
    for stage in (z.BWD_PRE, z.BWD_DKDV, z.BWD_DQ):
        z.attn_bwd(plan, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, stages=stage)
    torch.cuda.synchronize()
    for n, a, b in zip(("dq", "dk", "dv"), one, (dq, dk, dv)):
        assert torch.equal(torch.isnan(a), torch.isnan(b)), n
        assert torch.equal(torch.nan_to_num(a), torch.nan_to_num(b)), f"{n}: staged calls differ from one call"
