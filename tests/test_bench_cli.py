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
