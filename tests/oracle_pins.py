"""Pins for the fp64 oracle: each takes an implementation namespace and raises on mismatch.

The same pins run on the real oracle (``test_oracle_pins.py``) and on mutated
copies of it with one planted mistake each (``test_oracle_mutants.py``), which
shows that every plausible mistake fails at least one pin.  None of them
compares the oracle with a retyped copy of its own formula: they use closed
forms, invariants, finite differences, scalar brute force and library routines
(PyTorch's scaled_dot_product_attention and autograd, SciPy's logsumexp).

``impl`` must provide attention_head, attention, merge, merge_tree,
attention_backward_head and decode with the oracle's signatures.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb), f"{what}: finite pattern differs"
    assert np.array_equal(a[~fa], b[~fb]), f"{what}: non-finite values differ"
    if fa.any():
        err = np.max(np.abs(a[fa] - b[fb]) / (atol + rtol * np.maximum(1.0, np.abs(b[fb]))))
        assert err <= 1.0, f"{what}: error {err:.3g} x tolerance"


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# (S_q, S_k, d, causal, q_pos0, k_pos0): covers full, diagonal, offset and fully masked rows
TINY_CASES = [
    (5, 7, 3, False, 0, 0),
    (6, 6, 4, True, 0, 0),
    (4, 9, 2, True, 5, 0),   # shard after some keys: rows see 6..9 keys
    (7, 5, 3, True, 0, 3),   # rows 0..2 see nothing
    (3, 4, 1, True, 0, 10),  # everything masked
    (1, 8, 5, False, 0, 0),
]


def pin_brute_forward(impl):
    rng = np.random.default_rng(11)
    for (sq, sk, d, causal, qp, kp) in TINY_CASES:
        q, k, v = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, d + 1)
        c = 0.7
        O, L = impl.attention_head(q, k, v, c, causal, qp, kp)
        Ob, Lb = brute.forward(q.tolist(), k.tolist(), v.tolist(), c, causal, qp, kp)
        _close(O, Ob, 1e-12, 1e-14, f"fwd O vs brute {sq, sk, d, causal, qp, kp}")
        _close(L, Lb, 1e-12, 1e-14, f"fwd LSE vs brute {sq, sk, d, causal, qp, kp}")


def pin_golden_two_keys(impl):
    with open(os.path.join(GOLDEN, "two_key_hand_example.json")) as f:
        g = json.load(f)
    O, L = impl.attention_head(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), g["scale"])
    _close(O, g["O"], 1e-14, 0, "golden O")
    _close(L, g["LSE"], 1e-14, 0, "golden LSE")


def pin_closed_forms(impl):
    rng = np.random.default_rng(12)
    d = 6
    # A query whose only visible key is key 0: O is v_0 and LSE is c q.k_0.
    q, k, v = _rand(rng, 4, d), _rand(rng, 4, d), _rand(rng, 4, d)
    O, L = impl.attention_head(q, k, v, 0.3, True, 17, 17)
    _close(O[0], v[0], 1e-15, 0, "single visible key O")
    _close(L[0], 0.3 * float(np.dot(q[0], k[0])), 1e-14, 0, "single visible key LSE")
    # Zero queries: uniform weights over the visible keys, so O is their mean and
    # LSE = ln(count).  Row i of a shard at offset 3 sees keys 0..3+i.
    k, v = _rand(rng, 12, d), _rand(rng, 12, d)
    O, L = impl.attention_head(np.zeros((6, d)), k, v, 0.9, True, 3, 0)
    for i in range(6):
        n = 4 + i
        _close(L[i], math.log(n), 1e-14, 0, f"LSE of zero query row {i}")
        _close(O[i], v[:n].mean(axis=0), 1e-13, 1e-15, f"mean of visible values row {i}")
    # Identical keys give uniform weights whatever q is.
    k = np.tile(_rand(rng, 1, d), (9, 1))
    v = _rand(rng, 9, d)
    O, L = impl.attention_head(_rand(rng, 3, d), k, v, 0.5)
    _close(O, np.tile(v.mean(axis=0), (3, 1)), 1e-13, 1e-15, "identical keys")
    # Nothing visible: O = 0 and LSE = -inf.
    O, L = impl.attention_head(_rand(rng, 3, d), _rand(rng, 5, d), _rand(rng, 5, d), 0.5, True, 0, 10)
    assert np.all(O == 0) and np.all(L == -np.inf), "fully masked rows"
    # Large scale: the softmax becomes a hard argmax.
    q, k, v = _rand(rng, 5, d), _rand(rng, 11, d), _rand(rng, 11, d)
    O, _ = impl.attention_head(q, k, v, 2000.0)
    _close(O, v[np.argmax(q @ k.T, axis=1)], 0, 1e-9, "hard argmax")


def pin_library_sdpa(impl):
    """PyTorch's scaled_dot_product_attention (fp64, CPU) and SciPy's logsumexp."""
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp

    rng = np.random.default_rng(13)
    for (sq, sk, d, causal, qp, kp) in [(33, 47, 8, False, 0, 0), (40, 40, 16, True, 0, 0),
                                        (21, 64, 8, True, 50, 0), (64, 31, 4, True, 40, 20)]:
        q, k, v = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, d)
        c = 1.0 / math.sqrt(d)
        mask = np.ones((sq, sk), bool)
        if causal:
            mask = (kp + np.arange(sk))[None, :] <= (qp + np.arange(sq))[:, None]
        assert mask.any(axis=1).all()
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            attn_mask=torch.from_numpy(mask)[None], scale=c)[0].numpy()
        O, L = impl.attention_head(q, k, v, c, causal, qp, kp)
        _close(O, ref, 1e-12, 1e-14, f"O vs SDPA {sq, sk, causal, qp, kp}")
        scores = np.where(mask, (q @ k.T) * c, -np.inf)
        _close(L, logsumexp(scores, axis=1), 1e-12, 1e-14, "LSE vs scipy logsumexp")
    # Grouped heads through the batched entry point, against SDPA's enable_gqa.
    B, S, Hq, Hkv, d = 2, 19, 8, 2, 8
    q, k, v = _rand(rng, B, S, Hq, d), _rand(rng, B, 23, Hkv, d), _rand(rng, B, 23, Hkv, d)
    O, L = impl.attention(q, k, v, 0.4)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).transpose(1, 2), torch.from_numpy(k).transpose(1, 2),
        torch.from_numpy(v).transpose(1, 2), scale=0.4, enable_gqa=True).transpose(1, 2).numpy()
    _close(O, ref, 1e-12, 1e-14, "GQA O vs SDPA")


def pin_invariants(impl):
    rng = np.random.default_rng(14)
    d = 5
    q, k, v = _rand(rng, 8, d), _rand(rng, 13, d), _rand(rng, 13, d)
    c = 0.6
    O, L = impl.attention_head(q, k, v, c, True, 6, 0)
    # Shifting every key by u leaves O unchanged and moves LSE by c q.u.
    u = _rand(rng, d)
    O2, L2 = impl.attention_head(q, k + u, v, c, True, 6, 0)
    _close(O2, O, 1e-12, 1e-13, "key shift O")
    _close(L2, L + c * (q @ u), 1e-12, 1e-13, "key shift LSE")
    # Changing keys/values that no query sees changes nothing (positions > 6 + 7 = 13 do not exist;
    # key j is hidden from row i when j > 6 + i, so keys 7.. are hidden from row 0).
    k3, v3 = k.copy(), v.copy()
    k3[7:] = _rand(rng, 6, d) * 5
    v3[7:] = _rand(rng, 6, d) * 5
    O3, L3 = impl.attention_head(q[:1], k3, v3, c, True, 6, 0)
    _close(O3, O[:1], 1e-13, 1e-15, "hidden keys O")
    _close(L3, L[:1], 1e-13, 1e-15, "hidden keys LSE")
    # Without a mask, permuting key/value pairs changes nothing.
    perm = rng.permutation(13)
    O4, L4 = impl.attention_head(q, k[perm], v[perm], c)
    O5, L5 = impl.attention_head(q, k, v, c)
    _close(O4, O5, 1e-12, 1e-14, "key permutation O")
    _close(L4, L5, 1e-12, 1e-14, "key permutation LSE")
    # Rows of P sum to one: with every value equal to 1 the output is 1.
    O6, _ = impl.attention_head(q, k, np.ones((13, 3)), c, True, 6, 0)
    _close(O6, np.ones((8, 3)), 1e-13, 0, "rows of P sum to 1")


def _chunks(sk, sizes):
    out, j = [], 0
    for s in sizes:
        out.append((j, j + s))
        j += s
    assert j == sk
    return out


def pin_merge(impl):
    rng = np.random.default_rng(15)
    # The fp32 workload's structure (256 keys in 4 chunks of 64) plus uneven,
    # causal and fully masked chunks.
    for (sq, sk, d, causal, qp, sizes) in [(256, 256, 64, False, 0, [64] * 4),
                                           (40, 100, 8, True, 60, [10, 30, 1, 59]),
                                           (16, 64, 4, True, 0, [16, 16, 16, 16]),
                                           (8, 48, 4, True, 8, [8, 8, 32])]:
        q, k, v = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, d)
        c = 1 / math.sqrt(d)
        O, L = impl.attention_head(q, k, v, c, causal, qp, 0)
        parts = [impl.attention_head(q, k[a:b], v[a:b], c, causal, qp, a) for a, b in _chunks(sk, sizes)]
        for name, (Om, Lm) in [("sequential", impl.merge(parts)),
                               ("reversed", impl.merge(parts[::-1])),
                               ("tree", impl.merge_tree(parts)),
                               ("pairwise fold", _fold(impl, parts))]:
            _close(Om, O, 1e-12, 1e-13, f"merge {name} O {sq, sk, sizes}")
            _close(Lm, L, 1e-12, 1e-13, f"merge {name} LSE {sq, sk, sizes}")
    # 64 splits of a long row reduced by the binary tree equal the unsplit row.
    q, k, v = _rand(rng, 3, 8), _rand(rng, 64 * 16, 8), _rand(rng, 64 * 16, 8)
    O, L = impl.attention_head(q, k, v, 0.35)
    parts = [impl.attention_head(q, k[16 * i:16 * i + 16], v[16 * i:16 * i + 16], 0.35) for i in range(64)]
    Om, Lm = impl.merge_tree(parts)
    _close(Om, O, 1e-12, 1e-13, "64-way tree O")
    _close(Lm, L, 1e-12, 1e-13, "64-way tree LSE")
    # Odd counts are carried through the tree.
    Om, Lm = impl.merge_tree(parts[:7])
    Os, Ls = impl.merge(parts[:7])
    _close(Om, Os, 1e-12, 1e-13, "odd tree O")
    _close(Lm, Ls, 1e-12, 1e-13, "odd tree LSE")
    # The empty partial (0, -inf) is the identity; all-empty stays empty.
    o1, l1 = _rand(rng, 5, 3), _rand(rng, 5)
    e = (np.zeros((5, 3)), np.full(5, -np.inf))
    Om, Lm = impl.merge([e, (o1, l1), e])
    _close(Om, o1, 1e-15, 0, "identity O")
    _close(Lm, l1, 1e-15, 0, "identity LSE")
    Om, Lm = impl.merge([e, e])
    assert np.all(Om == 0) and np.all(Lm == -np.inf), "all-empty merge"
    # Closed form for two equal parts: O unchanged, LSE + ln 2.
    Om, Lm = impl.merge([(o1, l1), (o1, l1)])
    _close(Om, o1, 1e-14, 1e-15, "equal parts O")
    _close(Lm, l1 + math.log(2), 1e-14, 0, "equal parts LSE")


def _fold(impl, parts):
    acc = parts[0]
    for p in parts[1:]:
        acc = impl.merge([acc, p])
    return acc


def _loss(impl, q, k, v, do, c, causal, qp, kp):
    O, _ = impl.attention_head(q, k, v, c, causal, qp, kp)
    return float(np.sum(O * do))


def pin_fd_grad(impl):
    """Central finite differences (h = 1e-6) of sum(dO * O) with respect to every input."""
    rng = np.random.default_rng(16)
    for (sq, sk, d, causal, qp, kp) in [(5, 7, 3, True, 2, 0), (4, 6, 4, False, 0, 0), (6, 5, 2, True, 0, 2)]:
        q, k, v, do = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, d), _rand(rng, sq, d)
        c = 0.8
        O, L = impl.attention_head(q, k, v, c, causal, qp, kp)
        dq, dk, dv = impl.attention_backward_head(q, k, v, O, do, L, c, causal, qp, kp)
        h = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                fp = _loss(impl, q, k, v, do, c, causal, qp, kp)
                x[idx] = old - h
                fm = _loss(impl, q, k, v, do, c, causal, qp, kp)
                x[idx] = old
                num[idx] = (fp - fm) / (2 * h)
            _close(g, num, 1e-6, 1e-8, f"finite-difference d{name} {sq, sk, causal, qp, kp}")


def pin_brute_backward(impl):
    rng = np.random.default_rng(17)
    for (sq, sk, d, causal, qp, kp) in TINY_CASES[:4]:
        q, k, v, do = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, d), _rand(rng, sq, d)
        c = 0.45
        O, L = impl.attention_head(q, k, v, c, causal, qp, kp)
        got = impl.attention_backward_head(q, k, v, O, do, L, c, causal, qp, kp)
        ref = brute.backward(q.tolist(), k.tolist(), v.tolist(), do.tolist(), c, causal, qp, kp)
        for name, a, b in zip("qkv", got, ref):
            _close(a, b, 1e-11, 1e-13, f"d{name} vs brute {sq, sk, causal, qp, kp}")


def pin_torch_autograd(impl):
    """Gradients against PyTorch autograd through SDPA (fp64, CPU)."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(18)
    for (sq, sk, d, causal, qp) in [(24, 40, 8, True, 16), (32, 32, 16, False, 0)]:
        q, k, v, do = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, d), _rand(rng, sq, d)
        c = 1 / math.sqrt(d)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        mask = torch.ones(sq, sk, dtype=torch.bool)
        if causal:
            mask = (torch.arange(sk)[None, :] <= (qp + torch.arange(sq))[:, None])
        out = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mask[None], scale=c)[0]
        out.backward(torch.from_numpy(do))
        O, L = impl.attention_head(q, k, v, c, causal, qp, 0)
        got = impl.attention_backward_head(q, k, v, O, do, L, c, causal, qp, 0)
        for name, a, t in zip("qkv", got, (tq, tk, tv)):
            _close(a, t.grad.numpy(), 1e-11, 1e-13, f"d{name} vs autograd {sq, sk, causal}")


def pin_chunked_backward(impl):
    """Per-chunk backward with the final LSE: dQ contributions add up, dK/dV are slices."""
    rng = np.random.default_rng(19)
    sq, sk, d, qp = 24, 60, 4, 30
    q, k, v, do = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, d), _rand(rng, sq, d)
    c = 0.5
    O, L = impl.attention_head(q, k, v, c, True, qp, 0)
    dq, dk, dv = impl.attention_backward_head(q, k, v, O, do, L, c, True, qp, 0)
    acc = np.zeros_like(dq)
    for a, b in _chunks(sk, [20, 5, 15, 20]):
        a_q, a_k, a_v = impl.attention_backward_head(q, k[a:b], v[a:b], O, do, L, c, True, qp, a)
        acc += a_q
        _close(a_k, dk[a:b], 1e-12, 1e-14, "chunk dK slice")
        _close(a_v, dv[a:b], 1e-12, 1e-14, "chunk dV slice")
    _close(acc, dq, 1e-12, 1e-14, "sum of chunk dQ")


def pin_sum_rules(impl):
    rng = np.random.default_rng(20)
    sq, sk, d, qp, kp = 30, 50, 6, 10, 15
    q, k, v, do = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, d), _rand(rng, sq, d)
    c = 0.4
    O, L = impl.attention_head(q, k, v, c, True, qp, kp)
    dq, dk, dv = impl.attention_backward_head(q, k, v, O, do, L, c, True, qp, kp)
    live = np.isfinite(L)
    assert not live.all() and live.any()
    # Softmax is shift invariant per row, so sum_j dS_ij = 0 and sum_j dK_j = 0.
    _close(dk.sum(axis=0), np.zeros(d), 0, 1e-12, "sum of dK")
    # Rows of P sum to 1, so sum_j dV_j = sum over rows that see a key of dO_i.
    _close(dv.sum(axis=0), do[live].sum(axis=0), 1e-12, 1e-12, "sum of dV")
    # Rows that see nothing get no gradient.
    assert np.all(dq[~live] == 0), "dQ of masked rows"


def pin_energy_gradient(impl):
    """The gradient of LSE_i with respect to q_i is c sum_j P_ij k_j (the scalar
    energy of the Tree Attention abstract), i.e. c times attention with v = k."""
    rng = np.random.default_rng(21)
    q, k = _rand(rng, 4, 5), _rand(rng, 9, 5)
    c, h = 0.7, 1e-6
    _, L = impl.attention_head(q, k, k, c, True, 5, 0)
    expect, _ = impl.attention_head(q, k, k, c, True, 5, 0)
    num = np.zeros_like(q)
    for idx in np.ndindex(q.shape):
        old = q[idx]
        q[idx] = old + h
        lp = impl.attention_head(q, k, k, c, True, 5, 0)[1][idx[0]]
        q[idx] = old - h
        lm = impl.attention_head(q, k, k, c, True, 5, 0)[1][idx[0]]
        q[idx] = old
        num[idx] = (lp - lm) / (2 * h)
    _close(num, c * expect, 1e-6, 1e-9, "dLSE/dq")


def pin_decode(impl):
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(22)
    B, Hq, Hkv, L, d = 3, 8, 2, 37, 8
    q, kc, vc = _rand(rng, B, Hq, d), _rand(rng, B, L, Hkv, d), _rand(rng, B, L, Hkv, d)
    O, LSE = impl.decode(q, kc, vc, 0.3)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None], torch.from_numpy(kc).transpose(1, 2),
        torch.from_numpy(vc).transpose(1, 2), scale=0.3, enable_gqa=True)[:, :, 0].numpy()
    _close(O, ref, 1e-12, 1e-14, "decode O vs SDPA")
    # Consecutive grouping: with constant values per kv head, head h reads the constant of h // 4.
    vconst = np.broadcast_to(np.arange(Hkv, dtype=np.float64)[None, None, :, None], (B, L, Hkv, d)).copy()
    O, _ = impl.decode(q, kc, vconst, 0.3)
    _close(O[:, :, 0], np.broadcast_to((np.arange(Hq) // (Hq // Hkv)).astype(np.float64), (B, Hq)),
           1e-14, 1e-15, "GQA head mapping")
    # Sequence lengths truncate the cache; a zero query makes LSE = ln(len).
    lens = np.array([1, 20, 37])
    O, LSE = impl.decode(np.zeros_like(q), kc, vc, 0.3, seqlens=lens)
    for b in range(B):
        _close(LSE[b], np.full(Hq, math.log(lens[b])), 1e-14, 0, "decode LSE = ln(len)")
        _close(O[b, 0], vc[b, :lens[b], 0].mean(axis=0), 1e-13, 1e-15, "decode mean")


def pin_gqa_backward(impl):
    """The batched backward with grouped heads: dK/dV of a key/value head sum the
    contributions of every query head of its group, and query head h reads key/value
    head h // (H_q / H_kv).  Checked against PyTorch autograd through SDPA with
    enable_gqa (fp64, CPU), and against the scalar brute force run per query head on
    its own key/value head and summed by hand over each group."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(23)
    for (B, sq, sk, Hq, Hkv, d, causal, qp) in [(2, 9, 13, 6, 2, 4, True, 5), (1, 7, 7, 4, 4, 3, False, 0),
                                                 (1, 6, 10, 8, 2, 4, True, 2)]:
        q, k, v = _rand(rng, B, sq, Hq, d), _rand(rng, B, sk, Hkv, d), _rand(rng, B, sk, Hkv, d)
        do = _rand(rng, B, sq, Hq, d)
        c = 0.6
        O, L = impl.attention(q, k, v, c, causal, qp, 0)
        got = impl.attention_backward(q, k, v, O, do, L, c, causal, qp, 0)
        # Autograd through SDPA, heads-major layout [B, H, S, d].
        tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy(), requires_grad=True) for x in (q, k, v))
        mask = torch.ones(sq, sk, dtype=torch.bool)
        if causal:
            mask = torch.arange(sk)[None, :] <= (qp + torch.arange(sq))[:, None]
        out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=c, enable_gqa=True)
        out.backward(torch.from_numpy(do.transpose(0, 2, 1, 3).copy()))
        for name, a, t in zip("qkv", got, (tq, tk, tv)):
            _close(a, t.grad.numpy().transpose(0, 2, 1, 3), 1e-11, 1e-13, f"GQA d{name} vs autograd {Hq, Hkv}")
        # Scalar brute force per query head, summed over each group by hand.
        G = Hq // Hkv
        ref = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
        for b in range(B):
            for h in range(Hq):
                g = h // G
                bq, bk, bv = brute.backward(q[b, :, h].tolist(), k[b, :, g].tolist(), v[b, :, g].tolist(),
                                            do[b, :, h].tolist(), c, causal, qp, 0)
                ref[0][b, :, h] = bq
                ref[1][b, :, g] += np.array(bk)
                ref[2][b, :, g] += np.array(bv)
        for name, a, r in zip("qkv", got, ref):
            _close(a, r, 1e-11, 1e-13, f"GQA d{name} vs brute per head {Hq, Hkv}")
        # A subset of query heads gives exactly their share: the other heads' dQ stays 0.
        sub = impl.attention_backward(q, k, v, O, do, L, c, causal, qp, 0, heads=[0, Hq - 1])
        _close(sub[0][:, :, [0, Hq - 1]], got[0][:, :, [0, Hq - 1]], 1e-15, 0, "GQA head subset dQ")
        assert np.all(sub[0][:, :, 1:Hq - 1] == 0), "GQA head subset leaves other heads"


ALL_PINS = [
    pin_brute_forward,
    pin_golden_two_keys,
    pin_closed_forms,
    pin_library_sdpa,
    pin_invariants,
    pin_merge,
    pin_fd_grad,
    pin_brute_backward,
    pin_torch_autograd,
    pin_chunked_backward,
    pin_sum_rules,
    pin_energy_gradient,
    pin_decode,
    pin_gqa_backward,
]
