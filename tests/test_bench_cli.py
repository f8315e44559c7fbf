"""bench.py's command line on the CPU: --gpus N with N > 1 exits with a message (the library
runs on one GPU; the attention would shard over heads with no communication) before touching
a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU" in r.stderr + r.stdout
    assert not r.stdout.strip().startswith("{")   # no metric line
