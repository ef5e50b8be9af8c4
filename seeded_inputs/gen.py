"""Seeded N(0,1) draws and bfloat16 rounding (round-to-nearest-even)."""

from __future__ import annotations

import concurrent.futures as _cf

import numpy as np

TENSOR_Q = 0
TENSOR_K = 1
TENSOR_V = 2
TENSOR_DO = 3


def _rng(workload_id: int, tensor_id: int, b: int) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(tensor_id), int(b)])


def normal_f32(workload_id: int, tensor_id: int, b: int, shape) -> np.ndarray:
    """N(0,1) float32 samples for batch slice ``b`` of one tensor."""
    return _rng(workload_id, tensor_id, b).standard_normal(tuple(shape), dtype=np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns uint16 bits.

    Inputs here are finite normal draws, so NaN/Inf handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_bits(workload_id: int, tensor_id: int, b: int, shape) -> np.ndarray:
    """bf16 bit patterns of one seeded batch slice."""
    return round_to_bf16(normal_f32(workload_id, tensor_id, b, shape))


def normal_bf16(workload_id: int, tensor_id: int, batch: int, slice_shape, threads: int = 8):
    """All batch slices of one tensor as bf16 bits, shape ``[batch, *slice_shape]``.

    Slices are drawn in parallel threads (NumPy releases the GIL while
    filling); each slice still comes from its own seed, so the result does not
    depend on the thread count.
    """
    out = np.empty((batch,) + tuple(slice_shape), dtype=np.uint16)

    def fill(b):
        out[b] = normal_bf16_bits(workload_id, tensor_id, b, slice_shape)

    if batch == 1 or threads <= 1:
        for b in range(batch):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(min(threads, batch)) as ex:
            list(ex.map(fill, range(batch)))
    return out
