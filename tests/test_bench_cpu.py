"""CPU checks of bench.py's bookkeeping (no GPU): every workload it names is a pack of the
workloads module whose FLOP count matches the metric's convention, and the committed HBM-traffic
record is used only while the kernel sources still hash to the value it was taken on."""
import json

import bench
import workloads as W


def test_every_bench_workload_is_a_pack():
    for name in bench.WORKLOAD_TEXT:
        pack = W.config(name)
        assert pack.segments and pack.d in (64, 128)
        # 14 * Lq * Lkv * d per (segment, head): forward 4x, backward 2.5x the forward
        assert abs(pack.flops_fwd_bwd() - 3.5 * pack.flops_fwd()) < 1e-6 * pack.flops_fwd_bwd()


def test_mixed_pack_flops_are_the_metric_denominator():
    assert abs(W.config("mixed").flops_fwd_bwd() / 1e12 - 211.079) < 1e-3


def test_traffic_record_follows_the_source_hash(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    rec = {"mixed": {"dkdv_kernel": {"bytes_per_launch": 123, "source_hash": h, "source": "test"}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("dkdv_kernel", "mixed")["bytes_per_launch"] == 123
    assert bench.stored_traffic("dq_kernel", "mixed") is None
    rec["mixed"]["dkdv_kernel"]["source_hash"] = "0" * 16
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("dkdv_kernel", "mixed") is None

