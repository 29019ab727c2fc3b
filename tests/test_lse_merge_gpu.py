"""zl_lse_merge on the GPU against the oracle's merge (Zellige page §II-B: ring attention
accumulates the output over key blocks; merging normalised partials by their log-sum-exps is
exact).

Inputs are seeded synthetic partial slabs (``workloads.draw_partials``), the same fp32 values
on both sides. Cases: d 64 and 128; 1 to 8 parts; parts with LSE = -inf and rows whose parts
are all -inf (the merge gives O = 0, LSE = -inf there); row counts that are not a multiple of
the rows one workgroup handles per pass (8 at d 128, 16 at d 64); the ring shard's slab at full
size (9,450 tokens x 40 heads = 378,000 rows x 8 parts, d 128); and the documented use on one
group of a plan, through pointer offsets into larger buffers.

Tolerance: the target's bar (max-abs 2e-2, rel-L2 5e-3) and a tighter one that fp32 arithmetic
on fp32 inputs meets: every weight exp(LSE_b - LSE) carries a relative error of a few ulp (the
exponential, the logarithm of a sum of at most 8 terms, one subtraction of values near 10,
whose ulp is 1e-6), so each output is within about 1e-5 of its magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]

TIGHT = 1e-5


def _run(n_parts, n_rows, d, seed, empty_frac=0.0, empty_rows=0):
    print(f"[case] lse_merge parts {n_parts} rows {n_rows} d {d} seed {seed} empty {empty_frac}/{empty_rows}",
          flush=True)
    z = H.zl()
    ins = W.draw_partials(n_parts, n_rows, d, seed, empty_frac, empty_rows)
    dev = torch.device("cuda:0")
    o_part = ins["o_part"].to(dev)
    lse_part = ins["lse_part"].to(dev)
    o = torch.full((n_rows, d), float("nan"), device=dev)
    lse = torch.full((n_rows,), float("nan"), device=dev)
    z.lse_merge(n_parts, n_rows, d, o_part, lse_part, o, lse)
    torch.cuda.synchronize()
    return ins, o.cpu().double().numpy(), lse.cpu().double().numpy()


def _check(ins, o, lse, chunk=1 << 16):
    lp = ins["lse_part"].double().numpy()
    op = ins["o_part"]
    n_rows = lp.shape[1]
    dead = np.isneginf(lp).all(axis=0)
    # rows whose parts are all -inf: O = 0 exactly and LSE = -inf
    assert np.isneginf(lse[dead]).all(), "an all -inf row did not get LSE = -inf"
    assert (o[dead] == 0).all(), "an all -inf row did not get O = 0"
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for r0 in range(0, n_rows, chunk):  # the merge is row-wise: the oracle runs on row chunks
        r1 = min(n_rows, r0 + chunk)
        mo, ml = oracle.lse_merge(op[:, r0:r1].double().numpy(), lp[:, r0:r1])
        live = ~dead[r0:r1]
        got_o.append(o[r0:r1][live])
        ref_o.append(mo[live])
        got_l.append(lse[r0:r1][live])
        ref_l.append(ml[live])
    go, ro, gl, rl = (np.concatenate(x) for x in (got_o, ref_o, got_l, ref_l))
    H.assert_close("o", go, ro)
    H.assert_close("lse", gl, rl)
    H.assert_close("o (fp32 bound)", go, ro, max_abs=TIGHT * max(1.0, float(np.abs(ro).max(initial=0))),
                   rel_l2=TIGHT)
    H.assert_close("lse (fp32 bound)", gl, rl, max_abs=TIGHT * max(1.0, float(np.abs(rl).max(initial=0))),
                   rel_l2=TIGHT)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_parts", [1, 2, 3, 5, 8])
def test_lse_merge_parts(d, n_parts):
    ins, o, lse = _run(n_parts, 1001 + 3 * n_parts, d, seed=100 + n_parts + d)
    _check(ins, o, lse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_rows", [1, 7, 9, 17, 4099])
def test_lse_merge_ragged_rows_and_empty_parts(d, n_rows):
    ins, o, lse = _run(4, n_rows, d, seed=200 + n_rows, empty_frac=0.3, empty_rows=min(3, n_rows))
    _check(ins, o, lse)


def test_lse_merge_single_part_is_identity():
    """One part: O and LSE come back as they went in (weight exp(0) = 1), bit for bit."""
    ins, o, lse = _run(1, 777, 128, seed=301, empty_frac=0.1)
    lp = ins["lse_part"][0].double().numpy()
    live = ~np.isneginf(lp)
    assert np.array_equal(lse[live], lp[live])
    assert np.array_equal(o[live], ins["o_part"][0].double().numpy()[live])


def test_lse_merge_ring_shard_full_size():
    """The ring shard's slab at full size: 9,450 query tokens x 40 heads = 378,000 rows, 8 parts,
    d 128 (1.55 GB of partials), every row compared."""
    ins, o, lse = _run(8, 9450 * 40, 128, seed=4, empty_frac=0.01, empty_rows=5)
    _check(ins, o, lse)


def test_lse_merge_on_a_plan_group():
    """The documented use on one group of a plan: pointer offsets into the slab and into O/LSE
    (views of larger buffers), a group that covers every stored head of its sequence, next to a
    whole sequence whose rows must stay untouched."""
    z = H.zl()
    pack = W.Pack("merge_group", (300, 500), (300, 1200), (3, 4),
                  ((0, 0, 3, 0, 300, 0, 300, -1),) + tuple((1, 0, 4, 0, 500, 400 * b, 400 * (b + 1), b)
                                                           for b in range(3)), 128, 31)
    plan = H.make_plan(pack)
    info = plan.info
    assert info["n_groups"] == 1
    g = plan.groups[0]
    n_parts, n_rows, d = g["n_parts"], g["n_rows"], pack.d
    ins = W.draw_partials(n_parts, n_rows, d, seed=32, empty_frac=0.05)
    dev = torch.device("cuda:0")
    o_part = torch.full((info["part_rows"] + 5, d), float("nan"), device=dev)
    lse_part = torch.full((info["part_rows"] + 5,), float("nan"), device=dev)
    pr = g["part_row"]
    o_part[pr:pr + n_parts * n_rows] = ins["o_part"].reshape(-1, d).to(dev)
    lse_part[pr:pr + n_parts * n_rows] = ins["lse_part"].reshape(-1).to(dev)
    o = torch.full((info["q_rows"], d), float("nan"), device=dev)
    lse = torch.full((info["q_rows"],), float("nan"), device=dev)
    r0 = g["o_row"]
    z.lse_merge(n_parts, n_rows, d, o_part[pr:], lse_part[pr:], o[r0:r0 + n_rows], lse[r0:r0 + n_rows])
    torch.cuda.synchronize()
    og, lg = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.isnan(og[:r0]).all() and np.isnan(lg[:r0]).all(), "rows outside the group were written"
    _check(ins, og[r0:r0 + n_rows], lg[r0:r0 + n_rows])


def test_binding_rejects_bad_merge_buffers():
    """dtype and device errors are raised before anything is launched."""
    z = H.zl()
    dev = torch.device("cuda:0")
    good = dict(o_part=torch.zeros(2 * 10 * 64, device=dev), lse_part=torch.zeros(20, device=dev),
                o=torch.zeros(640, device=dev), lse=torch.zeros(10, device=dev))
    for name in good:
        bad = dict(good)
        bad[name] = good[name].to(torch.bfloat16)
        with pytest.raises(TypeError):
            z.lse_merge(2, 10, 64, **bad)
        bad[name] = good[name].cpu()
        with pytest.raises(ValueError):
            z.lse_merge(2, 10, 64, **bad)
