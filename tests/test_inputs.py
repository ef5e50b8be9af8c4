"""Seeded input generator: determinism, bf16 rounding, distribution."""

import numpy as np
import torch

from seeded_inputs import (WORKLOADS, bf16_bits_to_f32, normal_bf16, normal_bf16_bits, normal_f32,
                           round_to_bf16)


def test_same_seed_same_bits():
    a = normal_bf16_bits(5, 1, 0, (64, 4, 16))
    b = normal_bf16_bits(5, 1, 0, (64, 4, 16))
    assert np.array_equal(a, b)
    c = normal_bf16_bits(5, 1, 1, (64, 4, 16))
    d = normal_bf16_bits(5, 2, 0, (64, 4, 16))
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_threaded_batch_equals_per_slice():
    full = normal_bf16(4, 2, 5, (33, 2, 8), threads=4)
    for b in range(5):
        assert np.array_equal(full[b], normal_bf16_bits(4, 2, b, (33, 2, 8)))


def test_rne_matches_torch_cast():
    x = normal_f32(9, 0, 0, (1 << 16,)) * np.float32(37.0)
    # Add exact ties (lower 16 bits = 0x8000) to exercise round-half-to-even.
    ties = (np.arange(1024, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32) * np.float32(1.0)])
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_widening_is_exact():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(bf16_bits_to_f32(bits), ref)


def test_distribution():
    x = bf16_bits_to_f32(normal_bf16_bits(2, 3, 0, (1 << 18,)))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def test_workload_table():
    w = WORKLOADS["shard_fwd_128k"]
    assert (w.S_q, w.S_k, w.chunk, w.q_pos0) == (4096, 131072, 4096, 65536)
    d = WORKLOADS["decode_gqa_128k"]
    assert d.H_q // d.H_kv == 4 and d.chunk == 2048
    c = WORKLOADS["causal_fwdbwd_32k"]
    assert c.chunk == 2048 and c.balanced
