"""A whole step (forward, ring merge, backward) captured in a HIP graph and replayed.

Every launch of the path is a kernel on the caller's stream (queue counters and split-KV
counters are cleared by kernels, not memsets), so the step can be captured once and replayed.
Each replay follows eager work that overwrites every output with NaN, and must reproduce the
eager step bit for bit. Also: one plan run on two streams at once with separate workspaces
gives the single-stream result.
"""
import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]

SEG = ((0, 0, 4, 0, 200, 0, 200, -1),
       (1, 0, 2, 0, 300, 0, 1500, 0), (1, 0, 2, 0, 300, 1500, 3000, 1),
       (2, 0, 1, 0, 5000, 0, 5000, -1))
PACK = W.Pack("graph", (200, 300, 5000), (200, 3000, 5000), (4, 2, 1), SEG, 128, 77)


def _buffers(plan, dev):
    info, d = plan.info, plan.d
    f = lambda *shape: torch.empty(*shape, dtype=torch.float32, device=dev)
    return {"o": f(info["q_rows"], d), "lse": f(info["q_rows"]), "o_part": f(info["part_rows"], d),
            "lse_part": f(info["part_rows"]), "dq": f(info["q_rows"], d), "dk": f(info["kv_rows"], d),
            "dv": f(info["kv_rows"], d),
            "ws_f": torch.empty(info["ws_fwd"], dtype=torch.uint8, device=dev),
            "ws_b": torch.empty(info["ws_bwd"], dtype=torch.uint8, device=dev)}


def _step(z, plan, t, b, stream=None):
    z.attn_fwd(plan, t["q"], t["k"], t["v"], o=b["o"], lse=b["lse"], o_part=b["o_part"], lse_part=b["lse_part"],
               workspace=b["ws_f"], stream=stream)
    z.merge_groups(plan, b["o_part"], b["lse_part"], b["o"], b["lse"], stream=stream)
    z.attn_bwd(plan, t["q"], t["k"], t["v"], b["o"], b["lse"], t["do"], dq=b["dq"], dk=b["dk"], dv=b["dv"],
               workspace=b["ws_b"], stream=stream)


OUTS = ("o", "lse", "o_part", "lse_part", "dq", "dk", "dv")


def test_captured_step_replays_bitwise():
    z = H.zl()
    dev = torch.device("cuda:0")
    ins = W.draw(PACK)
    t = {n: ins[n].to(dev) for n in ("q", "k", "v", "do")}
    plan = H.make_plan(PACK)
    assert plan.info["split_tiles"] > 0 and plan.info["n_groups"] == 1
    b = _buffers(plan, dev)
    print("[case] graph capture of a whole step", flush=True)
    _step(z, plan, t, b)
    torch.cuda.synchronize()
    eager = {n: b[n].clone() for n in OUTS}
    ref = H.oracle_pack(PACK, ins)
    H.assert_close("o (eager)", H.f64(eager["o"]), ref["o"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        _step(z, plan, t, b)
    torch.cuda.synchronize()
    for rep in range(3):
        for n in OUTS:
            b[n].fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(b[n], eager[n]), f"replay {rep}: {n} differs from the eager step"


def test_one_plan_on_two_streams():
    z = H.zl()
    dev = torch.device("cuda:0")
    ins = W.draw(PACK)
    t = {n: ins[n].to(dev) for n in ("q", "k", "v", "do")}
    plan = H.make_plan(PACK)
    print("[case] one plan, two streams", flush=True)
    b0 = _buffers(plan, dev)
    _step(z, plan, t, b0)
    torch.cuda.synchronize()
    b1, b2 = _buffers(plan, dev), _buffers(plan, dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        _step(z, plan, t, b1, stream=s1)
    with torch.cuda.stream(s2):
        _step(z, plan, t, b2, stream=s2)
    torch.cuda.synchronize()
    for n in OUTS:
        assert torch.equal(b1[n], b0[n]) and torch.equal(b2[n], b0[n]), f"{n} differs across streams"
