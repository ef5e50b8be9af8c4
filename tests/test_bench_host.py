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


def test_smi_metric_parse():
    """The amd-smi CSV reader takes socket power and the per-XCD shader clocks (not their limits), skips
    repeated headers, blank lines and rows whose power is not a number."""
    b = _bench_module()
    hdr = "gpu,socket_power,gfx_voltage,gfx_0_clk,gfx_0_min_clk,gfx_0_max_clk,gfx_1_clk,gfx_1_min_clk,mem_0_clk"
    text = "\n".join([hdr, "0,250,N/A,157,142,2400,158,142,2000", "", hdr, "0,1343,N/A,1894,500,2400,1787,500,2000",
                      "0,N/A,N/A,1,2,3,4,5,6", "0,1350,N/A,1900"])
    assert b.parse_smi_metric_csv(text) == [(250.0, [157.0, 158.0]), (1343.0, [1894.0, 1787.0])]
    assert b.parse_smi_metric_csv("") == []
