"""Scalar pure-Python forward and backward for tiny inputs (a pin for the NumPy oracle).

TEST INFRASTRUCTURE ONLY.  Uses only ``math`` and Python floats (IEEE double),
with ``math.fsum`` for every sum, and walks the definition one scalar at a time:
no vectorisation and no shared helpers with ``attention.py``.
"""

from __future__ import annotations

import math


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def forward(q, k, v, scale, causal=False, q_pos0=0, k_pos0=0):
    """q, k, v as nested lists [[...], ...]; returns (O rows, LSE list)."""
    O, LSE = [], []
    dv = len(v[0]) if v else 0
    for i, qi in enumerate(q):
        vis = [j for j in range(len(k)) if (not causal) or (k_pos0 + j <= q_pos0 + i)]
        if not vis:
            O.append([0.0] * dv)
            LSE.append(-math.inf)
            continue
        s = {j: scale * _dot(qi, k[j]) for j in vis}
        m = max(s.values())
        tot = math.fsum(math.exp(s[j] - m) for j in vis)
        lse = m + math.log(tot)
        p = {j: math.exp(s[j] - lse) for j in vis}
        O.append([math.fsum(p[j] * v[j][t] for j in vis) for t in range(dv)])
        LSE.append(lse)
    return O, LSE


def backward(q, k, v, do, scale, causal=False, q_pos0=0, k_pos0=0):
    """Gradients of sum(dO * O) by the chain rule through softmax, one scalar at a time.

    Independent of the saved-statistics form: P is rebuilt here from scratch
    and D_i = sum_j P_ij (dO_i . v_j) is used (equal to dO_i . O_i).
    """
    n_q, n_k, d, dv = len(q), len(k), len(q[0]), len(v[0])
    P = [[0.0] * n_k for _ in range(n_q)]
    for i in range(n_q):
        vis = [j for j in range(n_k) if (not causal) or (k_pos0 + j <= q_pos0 + i)]
        if not vis:
            continue
        s = {j: scale * _dot(q[i], k[j]) for j in vis}
        m = max(s.values())
        tot = math.fsum(math.exp(s[j] - m) for j in vis)
        for j in vis:
            P[i][j] = math.exp(s[j] - m) / tot
    dP = [[_dot(do[i], v[j]) for j in range(n_k)] for i in range(n_q)]
    # dL/ds_ij = P_ij (dP_ij - sum_t P_it dP_it)   (Jacobian of a softmax row)
    dS = []
    for i in range(n_q):
        avg = math.fsum(P[i][t] * dP[i][t] for t in range(n_k))
        dS.append([P[i][j] * (dP[i][j] - avg) for j in range(n_k)])
    dq = [[scale * math.fsum(dS[i][j] * k[j][t] for j in range(n_k)) for t in range(d)] for i in range(n_q)]
    dk = [[scale * math.fsum(dS[i][j] * q[i][t] for i in range(n_q)) for t in range(d)] for j in range(n_k)]
    dvv = [[math.fsum(P[i][j] * do[i][t] for i in range(n_q)) for t in range(dv)] for j in range(n_k)]
    return dq, dk, dvv
