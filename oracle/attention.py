"""Plain fp64 definitions of forward, merge, backward and decode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation for one (batch, head): query i sits at global position
p_i = q_pos0 + i, key j at r_j = k_pos0 + j.  Without a causal mask every key
is visible; with it, key j is visible to query i iff r_j <= p_i (the diagonal
is visible).  With c the softmax scale:

    s_ij   = c * q_i . k_j
    LSE_i  = ln sum_{j visible} exp(s_ij)          (-inf if nothing is visible)
    P_ij   = exp(s_ij - LSE_i) for visible j, else 0
    O_i    = sum_j P_ij v_j                         (0 if nothing is visible)

The scale multiplies the scores before the softmax and the row log-sum-exp is
taken of the scaled scores in natural log: the pages print no formula, and this
is the plain reading of "exact softmax attention".

Rows are independent, so large inputs are processed in blocks of rows purely to
bound memory; sums over rows (dK, dV) are then accumulated block by block.
"""

from __future__ import annotations

import numpy as np

_BLOCK_ELEMS = 1 << 25  # fp64 score elements per row block (256 MiB)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible_mask(S_q: int, S_k: int, causal: bool, q_pos0: int = 0, k_pos0: int = 0) -> np.ndarray:
    """Boolean [S_q, S_k]: True where key j is visible to query i.

    Causal visibility compares absolute positions, so a query shard that sits
    at a global offset sees every key at or before its own position (the
    sequence-sharded setting of the BurstAttention and DistFlashAttn pages).
    """
    if not causal:
        return np.ones((S_q, S_k), dtype=bool)
    p = q_pos0 + np.arange(S_q, dtype=np.int64)
    r = k_pos0 + np.arange(S_k, dtype=np.int64)
    return r[None, :] <= p[:, None]


def _row_blocks(S_q: int, S_k: int):
    rows = max(1, _BLOCK_ELEMS // max(1, S_k))
    for r0 in range(0, S_q, rows):
        yield r0, min(S_q, r0 + rows)


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Masked row softmax of scores s: returns (P, LSE) in fp64."""
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    any_vis = np.isfinite(m)
    m_safe = np.where(any_vis, m, 0.0)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 on masked entries
    l = np.sum(e, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(any_vis, m_safe + np.log(l), -np.inf)
        P = np.where(any_vis[:, None], e / np.where(any_vis, l, 1.0)[:, None], 0.0)
    return P, lse


def attention_head(q, k, v, scale: float, causal: bool = False, q_pos0: int = 0, k_pos0: int = 0):
    """Exact attention of one head: q [S_q, d], k [S_k, d], v [S_k, d_v] -> (O [S_q, d_v], LSE [S_q]).

    This is the "local attention" that the BurstAttention page has every device
    compute on its own share; with k, v a chunk and k_pos0 its global offset it
    is one partial result.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    S_q, S_k = q.shape[0], k.shape[0]
    O = np.zeros((S_q, v.shape[1]), dtype=np.float64)
    LSE = np.full((S_q,), -np.inf, dtype=np.float64)
    if S_q == 0 or S_k == 0:
        return O, LSE
    for r0, r1 in _row_blocks(S_q, S_k):
        s = scale * (q[r0:r1] @ k.T)
        vis = visible_mask(r1 - r0, S_k, causal, q_pos0 + r0, k_pos0)
        P, lse = _softmax_rows(s, vis)
        O[r0:r1] = P @ v
        LSE[r0:r1] = lse
    return O, LSE


def _kv_head(h: int, H_q: int, H_kv: int) -> int:
    # Grouped heads: query heads g*G .. g*G+G-1 share key/value head g (G = H_q / H_kv).
    return h // (H_q // H_kv)


def attention(q, k, v, scale: float, causal: bool = False, q_pos0: int = 0, k_pos0: int = 0, heads=None):
    """Batched exact attention.

    q [B, S_q, H_q, d], k/v [B, S_k, H_kv, d] -> O [B, S_q, H_q, d_v], LSE [B, H_q, S_q].
    ``heads`` optionally restricts the computation to a list of query heads (other
    heads stay O = 0, LSE = -inf); it exists so tests can sample heads of large inputs.
    """
    B, S_q, H_q, _ = q.shape
    H_kv = k.shape[2]
    O = np.zeros((B, S_q, H_q, v.shape[3]), dtype=np.float64)
    LSE = np.full((B, H_q, S_q), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in (range(H_q) if heads is None else heads):
            g = _kv_head(h, H_q, H_kv)
            O[b, :, h], LSE[b, h] = attention_head(q[b, :, h], k[b, :, g], v[b, :, g], scale, causal, q_pos0, k_pos0)
    return O, LSE


def merge(parts):
    """Log-sum-exp weighted merge of partial results over disjoint key sets.

    ``parts`` is a sequence of (O_c, LSE_c) with O_c [..., d] and LSE_c [...].
    With m = max_c LSE_c:  LSE = m + ln sum_c exp(LSE_c - m),  O = sum_c exp(LSE_c - LSE) O_c.
    A part with LSE_c = -inf contributes nothing; if every part is -inf the
    result is O = 0, LSE = -inf.  This is the aggregation of local results into
    the global one on the BurstAttention page and the reduction that the Tree
    Attention page performs over sequence chunks.
    """
    parts = [(_f64(o), _f64(l)) for o, l in parts]
    lses = np.stack([l for _, l in parts])
    m = np.max(lses, axis=0)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    w = np.exp(lses - m_safe[None])  # exp(-inf) = 0
    tot = np.sum(w, axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(live, m_safe + np.log(np.where(live, tot, 1.0)), -np.inf)
    O = np.zeros_like(parts[0][0])
    for (o, l) in parts:
        coef = np.where(live, np.exp(l - np.where(live, lse, 0.0)), 0.0)
        O = O + coef[..., None] * o
    return O, lse


def merge_tree(parts):
    """Binary-tree merge: adjacent pairs (2i, 2i+1) at each level until one remains.

    The Tree Attention page reduces partial results up a tree; because the
    merge is associative the result equals ``merge(parts)``.  An odd element at
    a level is carried to the next level unchanged.
    """
    level = list(parts)
    while len(level) > 1:
        nxt = [merge(level[i:i + 2]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    o, l = level[0]
    return _f64(o), _f64(l)


def attention_backward_head(q, k, v, o, do, lse, scale: float, causal: bool = False,
                            q_pos0: int = 0, k_pos0: int = 0, delta=None):
    """Gradients of sum(dO * O) for one head, from the saved O and row LSE.

    With P_ij = exp(s_ij - LSE_i) on visible pairs and D_i = sum_t dO_it O_it:

        dV_j  = sum_i P_ij dO_i
        dP_ij = dO_i . v_j
        dS_ij = P_ij (dP_ij - D_i)
        dQ_i  = c sum_j dS_ij k_j
        dK_j  = c sum_i dS_ij q_i

    When k, v are one chunk of the keys and (o, lse) are the final merged
    output and row LSE, the returned dQ is that chunk's additive contribution
    and dK, dV are the chunk's slices of the full gradients: the DistFlashAttn
    page's point that the backward needs the saved statistics, not a re-run of
    the forward.  ``delta`` (D) may be passed in; it is computed from o and do
    otherwise.
    """
    q, k, v, o, do, lse = map(_f64, (q, k, v, o, do, lse))
    S_q, S_k = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if S_q == 0 or S_k == 0:
        return dq, dk, dv
    D = np.sum(do * o, axis=1) if delta is None else _f64(delta)
    for r0, r1 in _row_blocks(S_q, S_k):
        s = scale * (q[r0:r1] @ k.T)
        vis = visible_mask(r1 - r0, S_k, causal, q_pos0 + r0, k_pos0)
        live = np.isfinite(lse[r0:r1])
        lse_safe = np.where(live, lse[r0:r1], 0.0)
        P = np.where(vis & live[:, None], np.exp(np.where(vis, s, -np.inf) - lse_safe[:, None]), 0.0)
        dP = do[r0:r1] @ v.T
        dS = P * (dP - D[r0:r1, None])
        dv += P.T @ do[r0:r1]
        dq[r0:r1] = scale * (dS @ k)
        dk += scale * (dS.T @ q[r0:r1])
    return dq, dk, dv


def attention_backward(q, k, v, o, do, lse, scale: float, causal: bool = False,
                       q_pos0: int = 0, k_pos0: int = 0, heads=None):
    """Batched backward; shapes as in ``attention``.  Returns dq, dk, dv.

    With grouped heads, dK/dV of a key/value head sum the contributions of the
    query heads that share it.  ``heads`` restricts to a list of query heads.
    """
    B, S_q, H_q, _ = q.shape
    H_kv = k.shape[2]
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in (range(H_q) if heads is None else heads):
            g = _kv_head(h, H_q, H_kv)
            a, bk, bv = attention_backward_head(q[b, :, h], k[b, :, g], v[b, :, g], o[b, :, h], do[b, :, h],
                                                lse[b, h], scale, causal, q_pos0, k_pos0)
            dq[b, :, h] += a
            dk[b, :, g] += bk
            dv[b, :, g] += bv
    return dq, dk, dv


def decode(q, k_cache, v_cache, scale: float, seqlens=None, pairs=None):
    """Single-token decode over a KV cache with grouped heads.

    q [B, H_q, d], k_cache/v_cache [B, L, H_kv, d] -> O [B, H_q, d], LSE [B, H_q].
    The query attends every cached key 0..seqlens[b]-1 (all L when seqlens is
    None); no causal mask applies.  This is the decode setting of the Lean
    Attention and Tree Attention pages.  ``pairs`` optionally restricts the
    computation to a list of (b, h_q).
    """
    B, H_q, d = q.shape
    L, H_kv = k_cache.shape[1], k_cache.shape[2]
    O = np.zeros((B, H_q, v_cache.shape[3]), dtype=np.float64)
    LSE = np.full((B, H_q), -np.inf, dtype=np.float64)
    todo = [(b, h) for b in range(B) for h in range(H_q)] if pairs is None else pairs
    for b, h in todo:
        n = L if seqlens is None else int(seqlens[b])
        g = _kv_head(h, H_q, H_kv)
        o, l = attention_head(_f64(q[b, h])[None, :], k_cache[b, :n, g], v_cache[b, :n, g], scale)
        O[b, h], LSE[b, h] = o[0], l[0]
    return O, LSE
