"""Benchmark: attention forward+backward TFLOP/s on the mixed image-video pack, one GPU.

One step is one pass of the whole path over the pack: the forward launch, the exact merge
of every ring group (the mixed pack has none), and the backward launch (pre-pass + main
kernel). Inputs, outputs and workspaces are allocated and resident in HBM before the timed
region; nothing is allocated inside it.

FLOPs follow the metric's convention: 4*Lq*Lkv*d per (segment, head) forward, 2.5x that
backward. Prints one JSON line; with --json-out also writes it to a file.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixed] [--no-cpu-baseline] [--ring-fold]
                    [--no-split] [--graph] [--power]

With --graph the step is captured once in a HIP graph and the K timed steps are replays of
it (per-kernel times still come from event-bracketed eager steps run before them). With --power
the host samples socket power and graphics clocks (amd-smi) while the queued timed steps run.
    python bench.py --price-table [--price-reps R] [--json-out FILE]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s on mixed image-video pack; % of bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CUs x 4 SIMDs x 1024 flop/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0

WORKLOAD_TEXT = {
    "tiny": "tiny pack: 64, 256, 1024 tokens x 4 heads, d_head 64",
    "image": "image-only pack: 24 x 1024 + 8 x 4096 tokens, 24 heads, d_head 128",
    "mixed": "mixed image-video pack: 16 x 1024 + 4 x 4096 + 2 x 32760 tokens at 40 heads, plus the 5-head "
             "Ulysses shard of a 75600-token video; d_head 128, non-causal",
    "ring": "ring KV-split shard: 9450 queries vs 75600 keys in 8 parts + LSE merge, 40 heads, d_head 128",
    "long": "long-video share: 5 heads of a 497760-token sequence + 8 x 4096 tokens at 40 heads, d_head 128",
    "shard": "Ulysses share of one 32760-token video: 5 of 40 heads at full length, d_head 128",
    "head1": "one head of a 32760-token video at full length, d_head 128 (forward split over keys)",
}


def cpu_baseline(pack, ins, budget_s: float = 12.0) -> dict:
    """Time the fp64 oracle on a bounded sample of the pack's segment heads (host cores).

    One head per distinct segment shape, query rows cut to 1024, forward + backward against
    all of the segment's keys; the shapes are cycled over further heads until about
    ``budget_s`` seconds of oracle work have run. Throughput = flops computed / time.
    """
    import torch
    import oracle

    lay = oracle.PackLayout(pack.seq_q, pack.seq_kv, pack.heads)
    tau = pack.softmax_scale()
    f64 = lambda t: t.to(dtype=torch.float64).numpy()
    seen, shapes = set(), []
    for (s, h0, h1, q0, q1, k0, k1, part) in pack.segments:
        if (q1 - q0, k1 - k0) not in seen:
            seen.add((q1 - q0, k1 - k0))
            shapes.append((s, h0, h1, q0, min(q1, q0 + 1024), k0, k1))
    flops, t_used, done = 0.0, 0.0, {}
    for rnd in range(64):
        for (s, h0, h1, q0, q1, k0, k1) in shapes:
            h = h0 + rnd % (h1 - h0)
            qi, ki = lay.q_index(s, q0, q1, h), lay.kv_index(s, k0, k1, h)
            q, k, v, do = f64(ins["q"][qi]), f64(ins["k"][ki]), f64(ins["v"][ki]), f64(ins["do"][qi])
            t0 = time.perf_counter()
            o, lse = oracle.head_forward(q, k, v, tau)
            oracle.head_backward(q, k, v, o, lse, do, tau)
            t_used += time.perf_counter() - t0
            flops += 3.5 * 4.0 * (q1 - q0) * (k1 - k0) * pack.d
            key = f"{q1 - q0}x{k1 - k0}"
            done[key] = done.get(key, 0) + 1
        if t_used > budget_s:
            break
    threads = int(os.environ.get("OPENBLAS_NUM_THREADS", os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    desc = ", ".join(f"{n} x ({k})" for k, n in done.items())
    return {"value": round(flops / t_used / 1e12, 4), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 numpy oracle, fwd+bwd of (segment, head) samples, query rows cut to 1024 "
                      f"(queries x keys): {desc}; {flops / 1e12:.3f} TFLOP in {t_used:.1f} s"}


KERNEL_SOURCES = [os.path.join(ROOT, "coalesced_varlen_attention_amd", "csrc", f)
                  for f in ("zl_fwd.hip", "zl_bwd.hip", "zl_device.hpp", "zl_internal.h")] + [
    os.path.join(ROOT, "coalesced_varlen_attention_amd", "build.py")]  # compile flags shape the kernels too


def _code_only(path: str) -> bytes:
    """The source without comments and with whitespace runs collapsed, so that an edit of
    comments alone leaves the hash (and the counters stored under it) valid."""
    import io
    import re
    import tokenize
    with open(path) as fh:
        text = fh.read()
    if path.endswith(".py"):
        toks = [t for t in tokenize.generate_tokens(io.StringIO(text).readline) if t.type != tokenize.COMMENT]
        text = " ".join(t.string for t in toks if t.string.strip())
    else:  # C++: drop // and /* */ comments, keep string literals (inline assembly)
        pat = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)
        text = pat.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
        text = " ".join(text.split())
    return text.encode()


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(_code_only(f))
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, config: str):
    """HBM bytes per launch of ``kernel`` from the committed counter summary, if it was taken
    on the current kernel sources (else None: the counters no longer describe this code)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    ent = rec.get(config, {}).get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent


def calibrate_copy(gib: float = 2.0, reps: int = 3) -> int:
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 4, "reps": reps}), flush=True)
    return 0


# Placement options of one sequence on `degree` ranks, as one rank's local attention share
# (Zellige §IV-A, Table II): whole (1,1,1); Ulysses (1,h,1) keeps H/h heads at full length;
# ring (1,1,k) keeps L/k queries against the L keys in k blocks, accumulated block by block;
# all-gather (q,1,1) keeps L/q queries against all L keys; composed (1,h,k) both.
PRICE_BUCKETS = (1024, 4096, 9450, 32760, 75600)
PRICE_CONFIGS = (("whole", 1, 1, 1), ("ulysses", 2, 1, 1), ("ulysses", 4, 1, 1), ("ulysses", 8, 1, 1),
                 ("ring", 1, 2, 1), ("ring", 1, 4, 1), ("ring", 1, 8, 1), ("allgather", 1, 1, 2),
                 ("allgather", 1, 1, 4), ("allgather", 1, 1, 8), ("ulysses_ring", 2, 2, 1),
                 ("ulysses_ring", 4, 2, 1), ("ulysses_ring", 2, 4, 1))
PRICE_HEADS = 40


def price_table(reps: int, out_path) -> int:
    """Per-rank attention prices P_{b,theta} of this engine (Zellige §IV-B): forward and
    backward time of one rank's local share of a bucket-length sequence under each placement
    option, on this GPU, communication excluded. The ring forward runs as the ring executor
    computes it, one running-merge launch per arriving key block; its backward is one launch
    over all blocks. Also reports the launch floor: the same calls on a 64-token sequence."""
    import torch
    import workloads as W
    import coalesced_varlen_attention_amd as zl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d, H = 128, PRICE_HEADS

    def measure(L, h, k, qd):
        heads = H // h
        lq = L // (k * qd)                      # this rank's queries
        blocks = [(b * L // k, (b + 1) * L // k) for b in range(k)]
        segs = tuple((0, 0, heads, 0, lq, b0, b1, b if k > 1 else -1) for b, (b0, b1) in enumerate(blocks))
        pack = W.Pack("price", (lq,), (L,), (heads,), segs, d, 11)
        full = zl.Plan(pack.seq_q, pack.seq_kv, pack.heads, segs, d)
        steps = [zl.Plan(pack.seq_q, pack.seq_kv, pack.heads, (sg[:7] + (0,),), d) for sg in segs] if k > 1 else [full]
        info = full.info
        g = torch.Generator(device=dev)
        g.manual_seed(L * 64 + h * 8 + k + qd)
        rnd = lambda rows: torch.randn(rows, d, generator=g, device=dev).to(torch.bfloat16)
        q, kk, v, do = rnd(info["q_rows"]), rnd(info["kv_rows"]), rnd(info["kv_rows"]), rnd(info["q_rows"])
        o = torch.empty(info["q_rows"], d, device=dev)
        lse = torch.empty(info["q_rows"], device=dev)
        dq = torch.empty(info["q_rows"], d, device=dev)
        dk = torch.empty(info["kv_rows"], d, device=dev)
        dv = torch.empty(info["kv_rows"], d, device=dev)
        ws_f = torch.empty(max(p.info["ws_fwd"] for p in steps), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(info["ws_bwd"], dtype=torch.uint8, device=dev)

        def fwd():
            if k > 1:
                lse.fill_(float("-inf"))
                for p in steps:
                    zl.attn_fwd_accumulate(p, q, kk, v, o, lse, workspace=ws_f)
            else:
                zl.attn_fwd(full, q, kk, v, o=o, lse=lse, workspace=ws_f)

        def bwd():
            zl.attn_bwd(full, q, kk, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws_b)

        fwd(); bwd()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        f_ms = b_ms = 0.0
        for _ in range(reps):
            ev[0].record(); fwd(); ev[1].record(); bwd(); ev[2].record()
            torch.cuda.synchronize()
            f_ms += ev[0].elapsed_time(ev[1]) / reps
            b_ms += ev[1].elapsed_time(ev[2]) / reps
        return f_ms, b_ms, 3.5 * info["fwd_flops"]

    floor_f, floor_b, _ = measure(64, 1, 1, 1)
    rows = []
    for L in PRICE_BUCKETS:
        for (name, h, k, qd) in PRICE_CONFIGS:
            f_ms, b_ms, flops = measure(L, h, k, qd)
            row = {"bucket_tokens": L, "config": name, "theta_qhk": [qd, h, k], "degree": qd * h * k,
                   "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "price_ms": round(f_ms + b_ms, 4),
                   "net_price_ms": round(f_ms + b_ms - floor_f - floor_b, 4),
                   "tflops": round(flops / ((f_ms + b_ms) * 1e-3) / 1e12, 1)}
            rows.append(row)
            print(json.dumps(row), flush=True)
    head = {"launch_floor_ms": round(floor_f + floor_b, 4), "heads": H, "d_head": d, "reps": reps}
    print(json.dumps(head), flush=True)
    if out_path:
        with open(out_path, "w") as fh:
            fh.write(json.dumps(head) + "\n")
            for r in rows:
                fh.write(json.dumps(r) + "\n")
    return 0


def start_power_sampler(period_s: float = 0.5):
    """Sample socket power and graphics clocks (`amd-smi metric -p -c --json`) on a background
    thread while the GPU runs the queued timed steps. Returns a function that stops the sampler
    and summarises the samples; call it after the timed region, so that the region's wall clock
    never waits for a sample in flight."""
    import subprocess
    import threading
    watts, mhz = [], []
    stop = threading.Event()

    def run():
        while not stop.is_set():
            try:
                out = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                     timeout=10).stdout
                gpu = json.loads(out[out.index("{"):])["gpu_data"][0]
                w = float(gpu["power"]["socket_power"]["value"])
                clk = [float(v["clk"]["value"]) for k, v in gpu["clock"].items()
                       if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                if not stop.is_set():  # a sample that ends after the timed steps is not theirs
                    watts.append(w)
                    if clk:
                        mhz.append(sum(clk) / len(clk))
            except Exception:
                pass
            stop.wait(period_s)

    thread = threading.Thread(target=run, daemon=True)
    thread.start()

    def finish() -> dict:
        stop.set()
        thread.join(timeout=15)
        if not watts:
            return {"samples": 0}
        return {"samples": len(watts), "socket_w_mean": round(sum(watts) / len(watts), 1), "socket_w_max": max(watts),
                "gfx_mhz_mean": round(sum(mhz) / len(mhz), 1) if mhz else None,
                "source": "amd-smi metric -p -c, sampled during the timed steps"}

    return finish


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="mixed", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--calibrate-copy", action="store_true", help="run only a 2 GiB device copy (counter scale)")
    ap.add_argument("--no-split", action="store_true", help="build the plan without split-KV of forward items")
    ap.add_argument("--item-rows", type=int, choices=(128, 256), default=None,
                    help="fix the forward and dQ item sizes (default: the plan's choice)")
    ap.add_argument("--ring-fold", action="store_true",
                    help="forward ring groups block by block with the running merge (one launch per ring "
                         "block, folding into O/LSE) instead of one launch plus the LSE merge")
    ap.add_argument("--price-table", action="store_true",
                    help="print per-rank attention prices for every bucket x placement option (one JSON line each)")
    ap.add_argument("--price-reps", type=int, default=3)
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph (launch-bound packs)")
    ap.add_argument("--power", action="store_true",
                    help="sample socket power and graphics clocks (amd-smi) while the timed steps run")
    args = ap.parse_args()
    if args.calibrate_copy:
        return calibrate_copy()
    if args.price_table:
        return price_table(args.price_reps, args.json_out)
    if args.gpus != 1:
        print(f"bench.py: the library runs one GPU's share on one GPU (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding is a design, not a measured path", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    import coalesced_varlen_attention_amd as zl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pack = W.config(args.config)
    # Plan build: the first build in the process also loads the library's kernels; a per-batch
    # engine pays the warm figure (the median of five later builds, each destroyed after),
    # reported beside it. Neither is in the step.
    build = lambda: zl.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, pack.scale,
                            split=not args.no_split, item_rows=args.item_rows)
    t0 = time.perf_counter()
    plan = build()
    plan_ms = (time.perf_counter() - t0) * 1e3
    warm, destroy = [], []
    for _ in range(5):
        t0 = time.perf_counter()
        plan_warm = build()
        warm.append((time.perf_counter() - t0) * 1e3)
        t0 = time.perf_counter()
        plan_warm.close()
        destroy.append((time.perf_counter() - t0) * 1e3)
    plan_warm_ms = statistics.median(warm)
    plan_destroy_ms = statistics.median(destroy)
    info = plan.info
    ins = W.draw(pack)
    q, k, v, do = (ins[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty(info["q_rows"], pack.d, dtype=torch.float32, device=dev)
    lse = torch.empty(info["q_rows"], dtype=torch.float32, device=dev)
    o_part = torch.empty(max(1, info["part_rows"]), pack.d, dtype=torch.float32, device=dev)
    lse_part = torch.empty(max(1, info["part_rows"]), dtype=torch.float32, device=dev)
    dq = torch.empty(info["q_rows"], pack.d, dtype=torch.float32, device=dev)
    dk = torch.empty(info["kv_rows"], pack.d, dtype=torch.float32, device=dev)
    dv = torch.empty(info["kv_rows"], pack.d, dtype=torch.float32, device=dev)
    ws_f = torch.empty(info["ws_fwd"], dtype=torch.uint8, device=dev)
    ws_b = torch.empty(info["ws_bwd"], dtype=torch.uint8, device=dev)
    has_groups = info["n_groups"] > 0
    stream = torch.cuda.current_stream()
    fold_plans = []
    if args.ring_fold:
        if not has_groups:
            print(f"bench.py: --ring-fold needs a pack with ring groups ({args.config} has none)", file=sys.stderr)
            return 2
        # Ring step b sees only block b of every group (renumbered part 0); whole segments go
        # with the first step.
        n_steps = max(g["n_parts"] for g in plan.groups)
        for b in range(n_steps):
            segs = tuple(sg[:7] + (0,) for sg in pack.segments if sg[7] == b)
            if b == 0:
                segs += tuple(sg for sg in pack.segments if sg[7] < 0)
            fold_plans.append(zl.Plan(pack.seq_q, pack.seq_kv, pack.heads, segs, pack.d, pack.scale,
                                      split=not args.no_split, item_rows=args.item_rows))
        ws_f = torch.empty(max(fp.info["ws_fwd"] for fp in fold_plans), dtype=torch.uint8, device=dev)
    group_rows = [(g["o_row"], g["n_rows"]) for g in plan.groups]
    # The exact merge of ring partials: zl_lse_merge per group when every group covers all of its
    # sequence's stored heads (its O/LSE rows are then contiguous), else zl_plan_merge (one launch
    # for every group, head subsets at their strided rows).
    lse_merge_calls = None
    if has_groups and all(g["head_end"] - g["head_begin"] == g["n_heads"] for g in plan.groups):
        lse_merge_calls = [(g["n_parts"], g["n_rows"], o_part[g["part_row"]:], lse_part[g["part_row"]:],
                            o[g["o_row"]:g["o_row"] + g["n_rows"]], lse[g["o_row"]:g["o_row"] + g["n_rows"]])
                           for g in plan.groups]

    def merge():
        if lse_merge_calls is not None:
            for (n_parts, n_rows, op, lp, oo, ll) in lse_merge_calls:
                zl.lse_merge(n_parts, n_rows, pack.d, op, lp, oo, ll)
        else:
            zl.merge_groups(plan, o_part, lse_part, o, lse)

    def forward():
        if fold_plans:
            for r0, n in group_rows:
                lse[r0:r0 + n].fill_(float("-inf"))
            for fp in fold_plans:
                zl.attn_fwd_accumulate(fp, q, k, v, o, lse, workspace=ws_f)
        else:
            zl.attn_fwd(plan, q, k, v, o=o, lse=lse, o_part=o_part if has_groups else None,
                        lse_part=lse_part if has_groups else None, workspace=ws_f)

    def step(ev=None):
        """One step. With `ev` (six events) the backward runs as its three stage launches with an
        event around each; without, as one call."""
        if ev is None:
            forward()
            if has_groups and not fold_plans:
                merge()
            zl.attn_bwd(plan, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws_b)
            return
        ev[0].record(stream)
        forward()
        ev[1].record(stream)
        if has_groups and not fold_plans:
            merge()
        ev[2].record(stream)
        zl.attn_bwd(plan, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws_b, stages=zl.BWD_PRE)
        ev[3].record(stream)
        zl.attn_bwd(plan, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws_b, stages=zl.BWD_DKDV)
        ev[4].record(stream)
        zl.attn_bwd(plan, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws_b, stages=zl.BWD_DQ)
        ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    # A per-batch plan built and uploaded while a step runs (ZL_PLAN_DEFERRED_UPLOAD: host time
    # only, no device allocation and no wait for the queued step).
    step()
    t0 = time.perf_counter()
    plan_next = zl.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, pack.scale,
                        split=not args.no_split, item_rows=args.item_rows, deferred=True)
    plan_next.upload()
    plan_deferred_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    plan_next.close()
    # Per-kernel durations come from HIP events on the launch stream inside the timed region, on
    # a tenth of the steps (at least one, spread evenly): a timing event costs the GPU a few us,
    # which on a 0.07 ms step would be a third of the step.
    n_inst = max(1, args.steps // 10)
    every = args.steps // n_inst
    instrumented = [j * every + every // 2 for j in range(n_inst)]
    events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(6)] for i in instrumented}
    torch.cuda.synchronize()
    finish_power = start_power_sampler() if args.power else None
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    smi = finish_power() if finish_power else None
    if args.graph:
        # Capture on a side stream (the library launches on the current stream, which the
        # capture makes the side stream), then time replays on the default stream.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    avg = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in events.values()) / len(events)
    per_step = sorted(e[0].elapsed_time(e[5]) for e in events.values())
    fwd_ms, merge_ms, pre_ms, dkdv_ms, dq_ms = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4), avg(4, 5)
    bwd_ms = pre_ms + dkdv_ms + dq_ms
    ms_per_step = wall * 1e3 / args.steps
    # HBM bytes the streaming launches must move: the merge reads every part's O and LSE of a
    # group's rows and writes one O and LSE per row; the pre-pass reads dO (bf16), O and LSE of
    # every covered row and writes -D and -LSE/tau.
    merge_bytes = sum(g["n_rows"] * (g["n_parts"] + 1) * (4 * pack.d + 4) for g in plan.groups)
    covered = sum((q1 - q0) * (h1 - h0) for (s_, h0, h1, q0, q1, k0, k1, part) in pack.segments if part <= 0)
    pre_bytes = covered * (2 * pack.d + 4 * pack.d + 4 + 8)
    flops_step = 3.5 * info["fwd_flops"]
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    # Per-kernel work in the method's own flops (the metric's convention: the backward's 2.5
    # forward units are dV and dP (1.0), dK (0.5) and dQ (0.5) on top of the recomputed S (0.5)):
    # forward 1.0 fwd_flops; dK/dV kernel 2.0 (S, dP, dV, dK); dQ kernel 0.5 (its dQ product; its
    # second S and dP are recomputation). The flops each kernel executes on the matrix cores are
    # reported beside them: forward 1.0, dK/dV 2.0, dQ 1.5 (S, dP, dQ).
    f = info["fwd_flops"]
    kernels = {
        "fwd_kernel": {"ms": fwd_ms, "flops": f, "exec_flops": f},
        "dkdv_kernel": {"ms": dkdv_ms, "flops": 2.0 * f, "exec_flops": 2.0 * f},
        "dq_kernel": {"ms": dq_ms, "flops": 0.5 * f, "exec_flops": 1.5 * f},
    }
    tf = lambda flops, ms: flops / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    for kname, kv in kernels.items():
        kv["tflops"] = tf(kv["flops"], kv["ms"])
        kv["exec_tflops"] = tf(kv["exec_flops"], kv["ms"])
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dk_ = kernels[dom]
    roof = {"bound": "mfma", "kernel": f"{dom}<{pack.d}>", "achieved": round(dk_["tflops"], 2),
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(dk_["tflops"] / BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "flops_basis": "algorithmic (metric convention): fwd 1.0, dK/dV 2.0, dQ 0.5 forward units",
            "per_kernel": {n: {"ms": round(kv["ms"], 3), "tflops": round(kv["tflops"], 1),
                               "frac": round(kv["tflops"] / BF16_PEAK_TFLOPS, 4),
                               "exec_mfma_tflops": round(kv["exec_tflops"], 1),
                               "exec_mfma_frac": round(kv["exec_tflops"] / BF16_PEAK_TFLOPS, 4)}
                           for n, kv in kernels.items()},
            "bwd_alg_frac": round(tf(2.5 * f, bwd_ms) / BF16_PEAK_TFLOPS, 4),
            "step_frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    traffic = stored_traffic(dom, args.config)
    if traffic is not None:
        roof["traffic"] = traffic["bytes_per_launch"]
        roof["traffic_source"] = traffic["source"]
    line = {"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": WORKLOAD_TEXT[args.config], "pack": args.config,
                       "fwd_bwd_tflop_per_step": round(flops_step / 1e12, 3),
                       "pct_of_bf16_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
                       "fwd_ms": round(fwd_ms, 3), "merge_ms": round(merge_ms, 3), "bwd_ms": round(bwd_ms, 3),
                       "bwd_pre_ms": round(pre_ms, 3), "bwd_dkdv_ms": round(dkdv_ms, 3), "bwd_dq_ms": round(dq_ms, 3),
                       "plan_build_ms": round(plan_ms, 2), "plan_build_warm_ms": round(plan_warm_ms, 2),
                       "plan_destroy_ms": round(plan_destroy_ms, 2),
                       "plan_build_deferred_during_step_ms": round(plan_deferred_ms, 2),
                       "parallelism": "none (1 GPU)",
                       "bwd_pre_gbs": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1) if pre_ms > 0 else None,
                       "merge_gbs": (round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1)
                                     if merge_bytes and merge_ms > 0 and not fold_plans else None),
                       "launch": "HIP graph replay" if args.graph else "eager",
                       "step_ms_events": {"median": round(per_step[len(per_step) // 2], 3),
                                          "min": round(per_step[0], 3), "max": round(per_step[-1], 3)},
                       "ring_forward": (f"running merge, {len(fold_plans)} launches" if fold_plans
                                        else ("partials + zl_lse_merge" if lse_merge_calls is not None
                                              else "partials + zl_plan_merge") if has_groups else "none"),
                       "item_rows": {"fwd": info["fwd_rows"], "dq": info["dq_rows"]},
                       "split_kv": {"fwd_items_split": info["split_tiles"], "pieces": info["split_pieces"],
                                    "dq_items_split": info["dq_split_tiles"], "dq_pieces": info["dq_split_pieces"],
                                    "dkdv_items_split": info["kv_split_tiles"], "dkdv_pieces": info["kv_split_pieces"]}},
            "roofline": roof}
    if smi is not None:
        line["config"]["power"] = smi
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pack, ins)
    text = json.dumps(line)
    print(text, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as fh:
            fh.write(text + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
