"""zl_attn_bwd_noalloc (the backward with the library's fixed device scratch, for callers that
cannot allocate) against zl_attn_bwd with a caller workspace: the same kernels run on the same
inputs, so the gradients must agree bit for bit (which meets the parity bar a fortiori; the
bar is asserted too). Two calls in a row, the second on a smaller pack, show that what the
first call left in the shared array does not leak into the second. A plan needing more scratch
than the array holds is rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]


def _case(pack):
    """Forward once, then the backward through both entry points on the same inputs."""
    z = H.zl()
    dev = torch.device("cuda:0")
    print(f"[case] noalloc {pack.name}: q rows {pack.q_rows()}", flush=True)
    plan = H.make_plan(pack)
    info = plan.info
    assert info["ws_bwd"] <= z.NOALLOC_SCRATCH_BYTES
    ins = W.draw(pack)
    q, k, v, do = (ins[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse, o_part, lse_part = z.attn_fwd(plan, q, k, v)
    if info["n_groups"]:
        z.merge_groups(plan, o_part, lse_part, o, lse)
    # rows no segment covers stay untouched on both sides: both start as NaN
    nan = lambda rows: torch.full((rows, pack.d), float("nan"), device=dev)
    ref = z.attn_bwd(plan, q, k, v, o, lse, do, dq=nan(info["q_rows"]), dk=nan(info["kv_rows"]),
                     dv=nan(info["kv_rows"]))
    got = z.attn_bwd_noalloc(plan, q, k, v, o, lse, do, nan(info["q_rows"]), nan(info["kv_rows"]),
                             nan(info["kv_rows"]))
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        gh, rh = H.f64(g), H.f64(r)
        same = (gh == rh) | (np.isnan(gh) & np.isnan(rh))
        assert same.all(), f"{name}: noalloc differs from the workspace backward in {int((~same).sum())} values"
        cov = ~np.isnan(rh[:, 0])
        H.assert_close(name, gh[cov], rh[cov])
    return info


def test_noalloc_matches_workspace_backward_twice():
    # first call: whole sequences, a head subset, a ring group and a split head (large scratch)
    segs = ((0, 0, 8, 0, 1024, 0, 1024, -1), (1, 0, 8, 0, 1024, 0, 1024, -1), (2, 2, 5, 0, 3000, 0, 3000, -1),
            (3, 0, 4, 0, 700, 0, 900, 0), (3, 0, 4, 0, 700, 900, 2000, 1), (4, 0, 1, 0, 2100, 0, 2100, -1))
    big = W.Pack("noalloc_big", (1024, 1024, 3000, 700, 2100), (1024, 1024, 3000, 2000, 2100), (8, 8, 5, 4, 1),
                 segs, 128, 41)
    info_big = _case(big)
    # second call, smaller: the tiny pack (d 64), reusing the array the first call filled
    info_small = _case(W.tiny())
    assert info_small["ws_bwd"] < info_big["ws_bwd"]


def test_noalloc_rejects_plans_beyond_the_array():
    """One head of 8,192 tokens splits its dQ and dK/dV items into 256 pieces each, whose
    partials need 64.07 MiB, more than the 64 MiB array: the call fails with a clear error
    before any launch, and leaves the outputs as they were."""
    z = H.zl()
    dev = torch.device("cuda:0")
    pack = W.Pack("noalloc_too_big", (8192,), (8192,), (1,), ((0, 0, 1, 0, 8192, 0, 8192, -1),), 128, 42)
    plan = H.make_plan(pack)
    assert plan.info["ws_bwd"] > z.NOALLOC_SCRATCH_BYTES
    ins = W.draw(pack)
    q, k, v, do = (ins[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.zeros(8192, 128, device=dev)
    lse = torch.zeros(8192, device=dev)
    dq, dk, dv = (torch.full((8192, 128), 7.0, device=dev) for _ in range(3))
    with pytest.raises(z.ZlError) as e:
        z.attn_bwd_noalloc(plan, q, k, v, o, lse, do, dq, dk, dv)
    assert e.value.status == -2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in (dq, dk, dv))
