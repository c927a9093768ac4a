"""Host-side checks of bench.py's bookkeeping (no GPU): the stored counter readings are keyed by the
workloads the bench runs and the kernels it times, and each names sources that exist."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_inputs as mi  # noqa: E402


def test_measured_traffic_keys_are_bench_workloads_and_kinds():
    for (name, kind), rec in bench.MEASURED_TRAFFIC.items():
        assert name in mi.WORKLOADS, name
        assert kind in ("experts", "gate_up", "down"), kind
        # the kind the bench times for that workload
        one = bench.one_launch_experts(mi.WORKLOADS[name])
        assert (kind == "experts") == one, (name, kind)
        for src in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, src)), src
        assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0


def test_measured_traffic_is_null_once_a_source_changes(tmp_path, monkeypatch):
    (name, kind), rec = next(iter(bench.MEASURED_TRAFFIC.items()))
    # a copy of the tree's sources with one byte changed in the first source
    for src in rec["sources"]:
        dst = tmp_path / src
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, src), "rb").read())
    first = tmp_path / rec["sources"][0]
    first.write_bytes(first.read_bytes() + b"\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(name, kind) is None
    assert bench.measured_traffic("no_such_workload", kind) is None
