"""Plans built with ZL_PLAN_DEFERRED_UPLOAD and uploaded with zl_plan_upload into caller memory on
the caller's stream: the per-rank lowering of a step (Zellige page §IV-D) without a device
allocation or a wait for the device.

* The uploaded plan runs the same kernels on the same tables as a plan built the usual way, so
  every output matches bit for bit (the usual plan is checked against the oracle elsewhere).
* A deferred plan refuses to run before its upload, and uploads once.
* Plans built and uploaded one after another reuse the pinned staging once its copy is done.
* Building and uploading a plan while the GPU is busy does not wait for the queued work.
"""
import time

import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]

SEGS = ((0, 1, 3, 0, 96, 0, 96, -1), (1, 0, 2, 0, 70, 0, 100, 0), (1, 0, 2, 0, 70, 100, 257, 1),
        (2, 0, 1, 0, 2100, 0, 2100, -1))
PACK = W.Pack("upload", (96, 70, 2100), (96, 257, 2100), (4, 2, 1), SEGS, 128, 17)


def _step(plan, ins, dev):
    z = H.zl()
    q, k, v, do = (ins[n].to(dev) for n in ("q", "k", "v", "do"))
    info = plan.info
    o = torch.full((info["q_rows"], PACK.d), float("nan"), device=dev)
    lse = torch.full((info["q_rows"],), float("nan"), device=dev)
    o, lse, o_part, lse_part = z.attn_fwd(plan, q, k, v, o=o, lse=lse)
    z.merge_groups(plan, o_part, lse_part, o, lse)
    nan = lambda rows: torch.full((rows, PACK.d), float("nan"), device=dev)
    dq, dk, dv = z.attn_bwd(plan, q, k, v, o, lse, do, dq=nan(info["q_rows"]), dk=nan(info["kv_rows"]),
                            dv=nan(info["kv_rows"]))
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _same(a, b):
    for n in a:
        x, y = a[n], b[n]
        assert torch.equal(torch.isnan(x), torch.isnan(y)), n
        assert torch.equal(torch.nan_to_num(x), torch.nan_to_num(y)), f"{n} differs from the usual plan"


def test_deferred_plan_matches_usual_plan():
    z = H.zl()
    dev = torch.device("cuda:0")
    print("[case] deferred upload vs usual plan", flush=True)
    ins = W.draw(PACK)
    ref = _step(H.make_plan(PACK), ins, dev)
    plan = z.Plan(PACK.seq_q, PACK.seq_kv, PACK.heads, PACK.segments, PACK.d, deferred=True)
    assert plan.info["dev_bytes"] > 0 and plan.info["split_tiles"] > 0
    q = ins["q"].to(dev)
    with pytest.raises(z.ZlError) as e:  # not uploaded yet
        z.attn_fwd(plan, q, ins["k"].to(dev), ins["v"].to(dev))
    assert "zl_plan_upload" in str(e.value)
    plan.upload()
    with pytest.raises(z.ZlError):  # once per plan
        plan.upload()
    _same(_step(plan, ins, dev), ref)


def test_uploads_reuse_staging_and_plans_outlive_none():
    """Several deferred plans built, uploaded, run and destroyed in turn (the staging of an earlier
    upload is reused once its copy has completed); each still matches the usual plan."""
    z = H.zl()
    dev = torch.device("cuda:0")
    ins = W.draw(PACK)
    ref = _step(H.make_plan(PACK), ins, dev)
    for i in range(4):
        plan = z.Plan(PACK.seq_q, PACK.seq_kv, PACK.heads, PACK.segments, PACK.d, deferred=True)
        plan.upload()
        _same(_step(plan, ins, dev), ref)
        plan.close()


def test_deferred_build_does_not_wait_for_the_device():
    """With about 200 ms of matrix products queued on the current stream, building and
    uploading the mixed pack's plan returns in host time only (a few ms), long before the queued
    work ends."""
    z = H.zl()
    dev = torch.device("cuda:0")
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        a @ a
    torch.cuda.synchronize()
    per = (time.perf_counter() - t0) / 5
    n = max(40, int(0.2 / max(per, 1e-6)))  # about 200 ms of queued work
    pack = W.config("mixed")
    for _ in range(n):
        a @ a
    t0 = time.perf_counter()
    plan = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, deferred=True)
    plan.upload()
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    total_ms = (time.perf_counter() - t0) * 1e3
    print(f"  deferred build + upload of the mixed pack's plan: {host_ms:.2f} ms on the host, "
          f"queued work drained {total_ms:.1f} ms after the start", flush=True)
    assert host_ms < 0.25 * total_ms and host_ms < 25.0
