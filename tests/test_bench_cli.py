"""bench.py's refusals, checked on the CPU: they happen before any GPU call."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300, env=e)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _bench(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "asked for 4" in r.stderr


def test_dtype_on_a_named_decode_workload_is_refused():
    r = _bench("--workload", "long4_128k", "--dtype", "bf16", "--no-cpu-baseline")
    assert r.returncode != 0 and "--shape" in r.stderr and r.stdout == ""


def test_fp32_on_a_multi_token_workload_is_refused():
    r = _bench("--workload", "verify32_q4", "--dtype", "f32", "--no-cpu-baseline")
    assert r.returncode != 0 and "f16 or bf16" in r.stderr and r.stdout == ""
