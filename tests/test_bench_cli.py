"""bench.py rejects what it cannot measure before it touches a GPU: more than
one GPU, an unknown workload, and a context override that is not a fixed
length above the BF16 sink + recent window."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_unknown_workload_is_refused():
    r = _bench("--workload", "no-such-workload")
    assert r.returncode == 2 and "unknown workload" in r.stderr


def test_context_override_needs_a_fixed_length_above_the_bf16_regions():
    assert _bench("--context", "132").returncode == 2                                   # = sink + recent
    assert _bench("--workload", "qwen3-8b-b28-ragged", "--context", "4096").returncode == 2  # ragged lengths
