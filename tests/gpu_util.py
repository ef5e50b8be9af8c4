"""Helpers for GPU parity tests: seeded inputs on both sides and tolerance checks.

The GPU receives bf16 bit patterns; the oracle receives their exact fp64 upcast,
so input quantisation is not counted as error.

The checks (check, rel_fro, sum_rule, verify) take torch tensors or numpy arrays
and need no GPU: the negative controls in test_checker_controls.py feed them
mistaken oracle outputs on the CPU to show that they fail.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from seeded_inputs import bf16_bits_to_f32, normal_bf16, normal_f32


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def seq_tensor(wid: int, tid: int, b: int, s: int, h: int, d: int, dtype: str):
    """Seeded [b, s, h, d] tensor: (device tensor, fp64 host copy of the same values)."""
    if dtype == "bf16":
        bits = normal_bf16(wid, tid, b, (s, h, d))
        host = bf16_bits_to_f32(bits).astype(np.float64)
        dev = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        return dev, host
    x = np.stack([normal_f32(wid, tid, i, (s, h, d)) for i in range(b)]) if b else np.zeros((0, s, h, d), np.float32)
    return torch.from_numpy(x).cuda(), x.astype(np.float64)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def check(name: str, got, ref, atol: float, *, scale_by_max: bool = False):
    """Max-abs check; the bound is atol, or atol * max(1, max|ref|) when scale_by_max.

    With scale_by_max the relative Frobenius error over the finite entries must
    also stay below atol (skipped when the reference is all zero): the scaled
    absolute bound alone is loose where |ref| is large, and the relative bound
    catches a wrong result that stays small.
    Non-finite entries (e.g. LSE = -inf of rows that see no key) must match exactly.
    Returns (max-abs error, rms of the reference).
    """
    got = to_np(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    fg, fr = np.isfinite(got), np.isfinite(ref)
    bad = np.argwhere(fg != fr)
    assert bad.size == 0, f"{name}: finite pattern differs at {bad[:5].tolist()} (got {got[tuple(bad[0])]})"
    assert np.array_equal(got[~fg], ref[~fr]), f"{name}: non-finite values differ"
    if not fr.any():
        return 0.0, 0.0
    diff = np.abs(got[fr] - ref[fr])
    err = float(diff.max())
    mx = float(np.abs(ref[fr]).max())
    tol = atol * max(1.0, mx) if scale_by_max else atol
    rms = float(np.sqrt(np.mean(ref[fr] ** 2)))
    log(f"  {name}: max|err| {err:.3e} (tol {tol:.1e}) max|ref| {mx:.3e} rms(ref) {rms:.3e}")
    assert err <= tol, f"{name}: max abs error {err:.4e} > {tol:.1e} (max|ref| {mx:.3e})"
    if scale_by_max and rms > 0.0:
        rel = float(np.linalg.norm(got[fr] - ref[fr]) / np.linalg.norm(ref[fr]))
        log(f"  {name}: relative Frobenius error {rel:.3e} (tol {atol:.1e})")
        assert rel <= atol, f"{name}: relative Frobenius error {rel:.4e} > {atol:.1e}"
    return err, rms


# Absolute bounds and relative Frobenius bounds of the full-size checks.
BOUNDS = {"O": 1e-2, "LSE": 1e-3, "dQ": 2e-2, "dK": 2e-2, "dV": 2e-2}
REL_BOUNDS = {"O": 1e-2, "dQ": 2e-2, "dK": 2e-2, "dV": 2e-2}


def rel_fro(got, ref) -> float:
    """||got - ref||_F / ||ref||_F: about 2^-9 for correct bf16 results, 1 for an all-zero output."""
    got = to_np(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def sum_rule(name: str, grads, target) -> float:
    """max over (b, h, d) of |sum_j g_j - target| / sum_j |g_j|, sums over the sequence axis 1.

    Softmax shift invariance gives sum_j dK_j = 0 (target 0); rows of P summing
    to one give sum_j dV_j = the sum of dO over rows that see a key.
    """
    if isinstance(grads, torch.Tensor):
        s, a = grads.double().sum(1), grads.double().abs().sum(1)
        t = target.double() if isinstance(target, torch.Tensor) else target
        r = ((s - t).abs() / a.clamp_min(1e-30)).max().item()
    else:
        g = np.asarray(grads, dtype=np.float64)
        s, a = g.sum(1), np.abs(g).sum(1)
        r = float((np.abs(s - np.asarray(target, dtype=np.float64)) / np.maximum(a, 1e-30)).max())
    log(f"  sum rule {name}: max |sum - target| / sum|.| = {r:.3e}")
    return r


def verify(tag: str, got: dict, ref: dict) -> None:
    """The full-size parity checks of one slice (one (b, h), or sampled rows).

    For every name in ref (O, LSE, dQ, dK, dV): the absolute bound on every
    entry (non-finite entries must match exactly) and, for O and the gradients,
    the relative Frobenius error, which catches outputs that are small enough
    at long context to pass the absolute bound while wrong (all zero, say).
    """
    for name, r in ref.items():
        check(f"{tag} {name}", got[name], r, BOUNDS[name])
        if name in REL_BOUNDS:
            e = rel_fro(got[name], r)
            log(f"  {tag} {name} relative Frobenius error {e:.3e}")
            assert e < REL_BOUNDS[name], f"{tag} {name}: relative Frobenius error {e:.3e} >= {REL_BOUNDS[name]}"


def row0_pin(o0, v0, lse0, q0, k0, scale) -> None:
    """Causal self-attention: query 0 sees only key 0, so O_0 = v_0 exactly (the
    softmax weight is exactly 1) and LSE_0 = scale * q_0 . k_0.  Arrays are
    [..., d] for o0, v0, q0, k0 and [...] for lse0 (any leading shape)."""
    o0 = to_np(o0) if isinstance(o0, torch.Tensor) else np.asarray(o0, dtype=np.float64)
    v0 = to_np(v0) if isinstance(v0, torch.Tensor) else np.asarray(v0, dtype=np.float64)
    assert np.array_equal(o0, v0), "row 0 must equal v_0 exactly"
    lse_ref = np.einsum("...d,...d->...", np.asarray(q0, dtype=np.float64), np.asarray(k0, dtype=np.float64)) * scale
    check("LSE row 0", lse0, lse_ref, BOUNDS["LSE"])
