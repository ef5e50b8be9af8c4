"""Helpers for GPU parity tests: seeded inputs on both sides and tolerance checks.

The GPU receives bf16 bit patterns; the oracle receives their exact fp64 upcast,
so input quantisation is not counted as error.
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
    return err, rms
