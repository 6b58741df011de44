"""bench.py command line: the one-GPU contract (CPU only)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                          "--warmup", "1"], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0
    assert "one GPU" in res.stderr + res.stdout
    assert res.stdout.strip() == "" or not res.stdout.strip().startswith("{")   # no bench line
