"""The benchmark's command-line contract on the host: requests it cannot
serve end with a message and a non-zero status before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_shard_count_must_divide_the_kv_heads():
    r = run_bench("--shard-heads", "3")
    assert r.returncode == 2
    assert "does not divide the 8 KV heads" in r.stderr
    assert r.stdout == ""
