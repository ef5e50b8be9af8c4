"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module holds no attention arithmetic: it draws N(0,1) samples from a
seeded NumPy generator, rounds them to bfloat16 with round-to-nearest-even and
describes the five workloads (shapes, chunking, offsets).  Both sides of a
parity check receive the same bits: the GPU as bf16 bit patterns, the fp64
oracle as their exact upcast.

Seeding: ``numpy.random.default_rng([workload_id, tensor_id, b])`` per batch
slice ``b``, with tensor ids Q=0, K=1, V=2, dO=3; each slice is drawn in the
C order of its layout (``[S, H, d]`` for sequence tensors, ``[H, d]`` for a
decode query).
"""

from .gen import (  # noqa: F401
    TENSOR_Q,
    TENSOR_K,
    TENSOR_V,
    TENSOR_DO,
    bf16_bits_to_f32,
    normal_bf16,
    normal_bf16_bits,
    normal_f32,
    round_to_bf16,
)
from .configs import TREE_DECODE, VARLEN_PACKED, WORKLOADS, Workload, tree_nodes  # noqa: F401
