"""Negative controls for the full-size parity checks, on the CPU.

At long context the outputs are small (|O| ~ 1e-2), so the absolute bounds
alone would pass some wrong results.  Here mistakes a kernel could make are
planted in the fp64 oracle (never in GPU code), the mistaken results go
through the same checks the GPU tests use (tests.gpu_util.verify and
sum_rule), and each must fail; the correct result, rounded as a bf16 kernel
would round it, must pass.  The shape is a reduced copy of the 128K shard's
structure: one head, d = 128, a query shard of 256 at the end of 8192 causal
keys that arrive in 16 chunks of 512; a grouped-head case covers the head
mapping.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import row0_pin, sum_rule, verify

D, SQ, SK, CH = 128, 256, 8192, 512
QPOS = SK - SQ
C = 1.0 / math.sqrt(D)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(2024)
    q, k, v, do = (_bf16(rng.standard_normal(s)) for s in ((SQ, D), (SK, D), (SK, D), (SQ, D)))
    O, L = oracle.attention_head(q, k, v, C, True, QPOS, 0)
    dq, dk, dv = oracle.attention_backward_head(q, k, v, O, do, L, C, True, QPOS, 0)
    ref = {"O": O, "LSE": L, "dQ": dq, "dK": dk, "dV": dv}
    return (q, k, v, do), ref


def _kernel_like(res):
    """What a correct kernel returns: bf16 outputs, fp32 LSE."""
    return {n: (_f32(x) if n == "LSE" else _bf16(x)) for n, x in res.items()}


def test_correct_result_passes(case):
    (q, k, v, do), ref = case
    got = _kernel_like(ref)
    verify("correct", got, ref)
    assert sum_rule("dK", got["dK"][None], 0.0) < 1e-2
    assert sum_rule("dV", got["dV"][None], do.sum(0)[None]) < 1e-2


def test_zeroed_output_fails(case):
    _, ref = case
    got = _kernel_like(ref)
    got["O"] = np.zeros_like(got["O"])
    with pytest.raises(AssertionError):
        verify("zero O", got, ref)


def test_zeroed_gradients_fail(case):
    (q, k, v, do), ref = case
    for name in ("dK", "dV"):
        got = _kernel_like(ref)
        got[name] = np.zeros_like(got[name])
        with pytest.raises(AssertionError):
            verify(f"zero {name}", got, ref)
    assert sum_rule("zero dV", np.zeros((1, SK, D)), do.sum(0)[None]) > 1e-2


def test_dropped_chunk_fails(case):
    (q, k, v, do), ref = case
    parts = [oracle.attention_head(q, k[a:a + CH], v[a:a + CH], C, True, QPOS, a) for a in range(0, SK, CH)]
    merged = oracle.merge(parts[:5] + parts[6:])
    got = _kernel_like(ref)
    got["O"], got["LSE"] = _bf16(merged[0]), _f32(merged[1])
    with pytest.raises(AssertionError):
        verify("dropped chunk", got, ref)


def test_chunk_local_lse_in_backward_fails(case):
    (q, k, v, do), ref = case
    got = _kernel_like(ref)
    dq = np.zeros_like(ref["dQ"])
    dk, dv = np.zeros_like(ref["dK"]), np.zeros_like(ref["dV"])
    for a in range(0, SK, CH):
        kc, vc = k[a:a + CH], v[a:a + CH]
        Oc, Lc = oracle.attention_head(q, kc, vc, C, True, QPOS, a)  # the chunk's own statistics
        g = oracle.attention_backward_head(q, kc, vc, Oc, do, Lc, C, True, QPOS, a)
        dq += g[0]
        dk[a:a + CH], dv[a:a + CH] = g[1], g[2]
    got["dQ"], got["dK"], got["dV"] = _bf16(dq), _bf16(dk), _bf16(dv)
    with pytest.raises(AssertionError):
        verify("chunk-local LSE", got, ref)


def test_causal_off_by_one_fails(case):
    (q, k, v, do), ref = case
    # Diagonal hidden: key j visible to query i only when r_j < p_i, i.e. r_j <= p_i - 1.
    # In the shard the diagonal is one key among ~8000, and here the relative
    # Frobenius error of O (about 1.35e-2 against 1e-2) is what catches it; at the
    # full shard size it weighs less still, so the suite relies on the checks below.
    O, L = oracle.attention_head(q, k, v, C, True, QPOS - 1, 0)
    g = oracle.attention_backward_head(q, k, v, O, do, L, C, True, QPOS - 1, 0)
    got = _kernel_like({"O": O, "LSE": L, "dQ": g[0], "dK": g[1], "dV": g[2]})
    with pytest.raises(AssertionError):
        verify("causal off by one", got, ref)


def test_causal_off_by_one_fails_row0_pin():
    # Causal self-attention (the 32K workload's structure): with the diagonal
    # hidden, query 0 sees no key, so O_0 = 0 and LSE_0 = -inf, which the row-0
    # pin rejects on every (b, h), and the row's finite pattern differs.
    rng = np.random.default_rng(8)
    q, k, v = (_bf16(rng.standard_normal((64, D))) for _ in range(3))
    O, L = oracle.attention_head(q, k, v, C, True, 0, 0)
    row0_pin(_bf16(O[0]), v[0], _f32(L[0]), q[0], k[0], C)  # the correct result passes
    Ow, Lw = oracle.attention_head(q, k, v, C, True, -1, 0)
    with pytest.raises(AssertionError):
        row0_pin(_bf16(Ow[0]), v[0], _f32(Lw[0]), q[0], k[0], C)
    with pytest.raises(AssertionError):
        verify("off by one", {"O": _bf16(Ow), "LSE": _f32(Lw)}, {"O": O, "LSE": L})


def test_interleaved_gqa_mapping_fails():
    rng = np.random.default_rng(7)
    Hq, Hkv, S = 4, 2, 2048
    q = _bf16(rng.standard_normal((1, S, Hq, D)))
    k, v = (_bf16(rng.standard_normal((1, S, Hkv, D))) for _ in range(2))
    O, L = oracle.attention(q, k, v, C, True)
    # Query head h reading key/value head h % Hkv instead of h // (Hq / Hkv).
    wrong = [oracle.attention_head(q[0, :, h], k[0, :, h % Hkv], v[0, :, h % Hkv], C, True) for h in range(Hq)]
    failed = 0
    for h in range(Hq):
        try:
            verify(f"interleaved GQA head {h}", {"O": _bf16(wrong[h][0]), "LSE": _f32(wrong[h][1])},
                   {"O": O[0, :, h], "LSE": L[0, h]})
        except AssertionError:
            failed += 1
    # Heads 0 and 3 map to the same key/value head either way; 1 and 2 do not.
    assert failed == 2
