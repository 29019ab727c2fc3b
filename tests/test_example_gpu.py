"""The usage example in the binding's module docstring runs as written, and its ring-merged
output equals whole-sequence attention of the same inputs (within the parity bar): the docs
cannot drift from the API."""
import pytest
import torch

from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]


def _example_code(z) -> str:
    doc = z.__doc__
    block = doc.split("d_head 128::", 1)[1]
    lines = [l[4:] for l in block.splitlines() if l.startswith("    ")]
    return "\n".join(lines)


def test_docstring_example_runs_and_matches_whole_attention():
    z = H.zl()
    code = _example_code(z)
    assert "zl.attn_bwd" in code and "zl.merge_groups" in code
    print("[case] binding docstring example", flush=True)
    torch.manual_seed(0)
    env = {}
    exec(compile(code, "zl-docstring-example", "exec"), env)
    torch.cuda.synchronize()
    plan, q, k, v, do = env["plan"], env["q"], env["k"], env["v"], env["do"]
    o, lse, dq, dk, dv = env["o"], env["lse"], env["dq"], env["dk"], env["dv"]
    # the same inputs through a plan that keeps the second sequence whole
    whole = z.Plan([1024, 4096], [1024, 4096], [24, 24],
                   [(0, 0, 24, 0, 1024, 0, 1024, -1), (1, 0, 24, 0, 4096, 0, 4096, -1)], 128)
    o2, lse2, _, _ = z.attn_fwd(whole, q, k, v)
    dq2, dk2, dv2 = z.attn_bwd(whole, q, k, v, o2, lse2, do)
    torch.cuda.synchronize()
    for name, a, b in (("o", o, o2), ("lse", lse, lse2), ("dq", dq, dq2), ("dk", dk, dk2), ("dv", dv, dv2)):
        H.assert_close(f"{name} ring-merged vs whole", H.f64(a), H.f64(b))
