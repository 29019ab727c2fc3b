"""Scheduler check on the GPU: every work item of every queue is taken by exactly one workgroup.

The three persistent kernels pull items from per-XCD queues with one atomic per take and steal
from the other queues once their own is empty (the lowering of a rank-local schedule into one
launch, Zellige page §IV-D). A plan built with ZL_PLAN_COUNT_VISITS counts, per item, the
workgroups that took it. Covering every output row (the NaN fills of the parity tests) shows
"at least once"; the counters show "exactly once", which the split items rely on: their
last-piece counters finish only if every piece runs once.

Packs: the mixed image-video pack (the benchmark's), many tiny images (2,000 whole sequences of
1 to 130 tokens at 2 heads: thousands of one-block items in every queue, most of them taken by
atomics and stealing), one head of a 32,760-token video (forward
and dQ items split into pieces), one head of 8,192 tokens (forward, dQ and dK/dV items split),
the ring shard (dQ items walking 8-part key chains), and a few-item pack (512 + 2,048 tokens,
one head each), unsplit and split. In the few-item pack the 512-token sequence's four forward
items share one queue chunk. The grid is one workgroup per item, and the queues are uneven:
queue 0 holds more items than it has home workgroups, and other queues hold fewer. So the
workgroups take static first items, find their home queue short, and take the rest by stealing
after the one-round-trip counter check. The counting plan's outputs must also equal a plain plan's bit for bit: the items and
their order are the same, and every output is written once by one workgroup.
"""
import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu, H.requires_gpu]


def _run(plan, pack, ins, dev):
    z = H.zl()
    info = plan.info
    q, k, v, do = (ins[n].to(dev) for n in ("q", "k", "v", "do"))
    ws_f = torch.zeros(info["ws_fwd"], dtype=torch.uint8, device=dev)
    ws_b = torch.zeros(info["ws_bwd"], dtype=torch.uint8, device=dev)
    o, lse, o_part, lse_part = z.attn_fwd(plan, q, k, v, workspace=ws_f)
    if info["n_groups"]:
        z.merge_groups(plan, o_part, lse_part, o, lse)
    dq, dk, dv = z.attn_bwd(plan, q, k, v, o, lse, do, workspace=ws_b)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, ws_f, ws_b


def _many_pack():
    """2,000 whole sequences of 1 to 130 tokens (the tile-edge lengths among them), 2 heads, d 128."""
    import numpy as np
    rng = np.random.default_rng(12)
    lens = [int(x) for x in rng.integers(1, 131, size=2000)]
    lens[:8] = [1, 2, 63, 64, 65, 127, 128, 129]
    return W.whole_pack("many", lens, [2] * len(lens), 128, 12)


def _pack(name):
    if name == "many":
        return _many_pack()
    if name == "head8k":  # one head of 8,192 tokens: forward, dQ and dK/dV items all split
        return W.Pack("head8k", (8192,), (8192,), (1,), ((0, 0, 1, 0, 8192, 0, 8192, -1),), 128, 8)
    if name.startswith("few"):  # 20 forward items in 17 queue chunks
        return W.Pack("few", (512, 2048), (512, 2048), (1, 1),
                      ((0, 0, 1, 0, 512, 0, 512, -1), (1, 0, 1, 0, 2048, 0, 2048, -1)), 128, 9)
    return W.config(name)


@pytest.mark.parametrize("name", ["mixed", "many", "head1", "head8k", "ring", "few", "few_nosplit"])
def test_every_item_taken_exactly_once(name):
    z = H.zl()
    pack = _pack(name)
    split = name != "few_nosplit"
    print(f"[case] visits {name}", flush=True)
    dev = torch.device("cuda:0")
    ins = W.draw(pack)
    plan = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, pack.scale, count_visits=True,
                  split=split)
    info = plan.info
    if name == "few_nosplit":  # uneven queues: queue 0 has more items than home workgroups
        bounds = plan.queues(0)
        sizes = [b - a for a, b in zip(bounds, bounds[1:])]
        homes = [(info["fwd_tiles"] - k + 7) // 8 for k in range(8)]
        assert sizes[0] > homes[0] and any(n < h for n, h in zip(sizes, homes)), (sizes, homes)
    if name == "head1":
        assert info["split_tiles"] > 0 and info["dq_split_tiles"] > 0
    if name == "head8k":
        assert info["split_tiles"] > 0 and info["dq_split_tiles"] > 0 and info["kv_split_tiles"] > 0
    out, ws_f, ws_b = _run(plan, pack, ins, dev)
    counts = plan.visits(ws_f, ws_b)
    for key, n_items in (("fwd", info["fwd_tiles"]), ("dkdv", info["bwd_tiles"]), ("dq", info["dq_tiles"])):
        c = counts[key]
        assert c.numel() == n_items
        print(f"  {key}: {n_items} items, visits min {int(c.min())} max {int(c.max())}", flush=True)
        assert bool((c == 1).all()), f"{key}: items taken {int((c == 0).sum())} x never, {int((c > 1).sum())} x more than once"
    # the same plan without counters gives the same bits
    plain = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, pack.scale, split=split)
    ref, _, _ = _run(plain, pack, ins, dev)
    for n in out:
        assert torch.equal(out[n], ref[n]), f"{n}: the counting plan's output differs from the plain plan's"
    # a second forward + backward on the same workspaces: the launches clear the counters
    out2, _, _ = _run(plan, pack, ins, dev)
    counts = plan.visits(ws_f, ws_b)
    assert all(bool((c == 1).all()) for c in counts.values())


def test_many_tiny_sequences_match_the_oracle():
    """The many-tiny-images pack element by element against the oracle: every row of all 2,000
    sequences, uncovered rows none."""
    pack = _many_pack()
    ins = W.draw(pack)
    print(f"[case] many: {len(pack.seq_q)} sequences, {sum(pack.seq_q)} tokens", flush=True)
    out = H.run_pack(pack, ins)
    info = out["plan"].info
    print(f"  items: fwd {info['fwd_tiles']}, dK/dV {info['bwd_tiles']}, dQ {info['dq_tiles']}", flush=True)
    H.compare_full(pack, ins, out, H.oracle_pack(pack, ins))
