"""Tiny-shape sweep on the GPU: forward and backward against the oracle for every pair of query and
key lengths in {1, 17, 64, 65, 255} x {1, 2, 63, 129, 255} (one row, one ragged tile, exact tiles,
one past a tile, many tiles), causal and not.  Causal cases end-align the queries with the keys
(q_pos0 = Sk - Sq when Sk >= Sq), so rows see one key, a diagonal tile or every key; with more queries
than keys the first rows see no key at all.  head_dim alternates between 64 and 128, GQA group 2."""

import itertools
import math

import pytest
import torch

import oracle
from exact_blockwise_attention_attn_amd import binding as B
from tests.gpu_util import check, log, seq_tensor

pytestmark = pytest.mark.gpu

O_TOL, G_TOL, L_TOL = 1e-2, 2e-2, 1e-3
SQ = (1, 17, 64, 65, 255)
SK = (1, 2, 63, 129, 255)
CASES = [(sq, sk, causal, 64 if i % 2 else 128, bool(i % 3 == 0))
         for i, (sq, sk, causal) in enumerate(itertools.product(SQ, SK, (False, True)))]


@pytest.mark.parametrize("case", CASES, ids=["-".join(str(x) for x in c) for c in CASES])
def test_sweep_fwd_bwd(case):
    sq, sk, causal, d, balanced = case
    qp = max(0, sk - sq) if causal else 0
    hq, hkv = 4, 2
    log(f"sweep Sq={sq} Sk={sk} causal={causal} d={d} q_pos0={qp} balanced={balanced}")
    q, qh = seq_tensor(120, 0, 1, sq, hq, d, "bf16")
    k, kh = seq_tensor(120, 1, 1, sk, hkv, d, "bf16")
    v, vh = seq_tensor(120, 2, 1, sk, hkv, d, "bf16")
    do, doh = seq_tensor(120, 3, 1, sq, hq, d, "bf16")
    scale = 1 / math.sqrt(d)
    O_ref, L_ref = oracle.attention(qh, kh, vh, scale, causal, qp, 0)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qh, kh, vh, O_ref, doh, L_ref, scale, causal, qp, 0)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, hq, sq), float("nan"), dtype=torch.float32, device="cuda")
    B.attn_fwd_partial(q, k, v, o, lse, q_pos0=qp, causal=causal, balanced=balanced)
    dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    dq_acc = torch.full((1, sq, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.attn_bwd_workspace_size(1, hq, sq), dtype=torch.uint8, device="cuda")
    B.attn_bwd(q, k, v, o, do, lse, ws, dq_acc, dk, dv, dq=dq, q_pos0=qp, causal=causal, compute_delta=True,
               dq_overwrite=True, finalize_dq=True, balanced=balanced)
    torch.cuda.synchronize()
    check("O", o, O_ref, O_TOL, scale_by_max=True)
    check("LSE", lse, L_ref, L_TOL)
    check("dQ", dq, dq_ref, G_TOL, scale_by_max=True)
    check("dK", dk, dk_ref, G_TOL, scale_by_max=True)
    check("dV", dv, dv_ref, G_TOL, scale_by_max=True)
