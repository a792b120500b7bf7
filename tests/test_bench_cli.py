"""bench.py's command line on the CPU: more than one GPU is refused with a message (this
path needs no collective and runs on one GPU); the argument defaults are the documented
ones."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_defaults():
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse_args()
    finally:
        sys.argv = old
    assert (a.gpus, a.workload, a.partition_size, a.graph, a.cold) == (1, "high_concurrency",
                                                                       None, False, False)
    assert a.append_in_pass == "auto"
    assert a.steps * 0.25e-3 < 60   # the default timed region stays well under a minute
    assert a.settle_seconds == 0.3  # untimed steps before the warmup: the clocks settle


def test_settle_runs_until_its_time_is_up():
    """settle() runs the step in groups of 8, synchronizing after each group, until the
    given wall time has passed (and not at all for 0 s)."""
    sys.path.insert(0, ROOT)
    import bench

    class FakeTorch:
        class cuda:
            syncs = 0

            @staticmethod
            def synchronize():
                FakeTorch.cuda.syncs += 1

    calls = []
    bench.settle(lambda: calls.append(1), FakeTorch, 0.0)
    assert calls == [] and FakeTorch.cuda.syncs == 0
    bench.settle(lambda: calls.append(1), FakeTorch, 0.02)
    assert len(calls) >= 8 and len(calls) % 8 == 0
    assert FakeTorch.cuda.syncs == len(calls) // 8


def test_traffic_records_are_consistent():
    """Each committed counter record's bytes follow from its own readings and scales, and
    its scales from its calibration copies (512 MiB moved each way per copy)."""
    import json
    import re
    sys.path.insert(0, ROOT)
    import bench
    assert set(bench.TRAFFIC_FILES) >= {"high_concurrency", "long_context", "qwen_gqa"}
    for workload, path in bench.TRAFFIC_FILES.items():
        info = json.load(open(path))
        kib = (info["fetch_size_kib_per_launch"] * info["fetch_scale"]
               + info["write_size_kib_per_launch"] * info["write_scale"])
        assert abs(kib * 1024 - info["bytes_per_launch"]) < 2048, workload
        ratio = info["bytes_per_launch"] / info["algorithmic_bytes_per_launch"]
        assert abs(ratio - info["traffic_over_algorithmic"]) < 1e-4, workload
        fetch = re.search(r"FETCH_SIZE ([\d. /]+) KiB", info["calibration"]).group(1)
        readings = [float(x) for x in fetch.split("/")]
        assert abs(524288.0 * len(readings) / sum(readings) - info["fetch_scale"]) < 1e-4, workload
        assert info["partition_size"] >= 0 and info["seed"] == 0
        assert len(info["kernel_source_sha256"]) == 64
