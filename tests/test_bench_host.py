"""bench.py's host-side contract, without a GPU: the one-GPU guard and the host facts that the
CPU baseline reports."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_flop_convention():
    b = _bench_module()
    # 4*S*S*d per (b, h) for the forward, halved for causal: the headline workload's 17.592 TFLOP.
    assert abs(b.causal_flops(2, 32, 32768, 128) - 2 * 32 * 4 * 32768 * 32768 * 128 / 2) < 1
    assert abs(b.causal_flops(2, 32, 32768, 128) / 1e12 - 17.592) < 1e-3


def test_host_facts():
    b = _bench_module()
    facts = b._host_facts()
    assert facts["affinity_cores"] == len(os.sched_getaffinity(0))
    assert isinstance(facts["cpu_model"], str) and facts["cpu_model"]
    assert isinstance(facts["blas"], list)
