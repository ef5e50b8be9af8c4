"""The C ABI used from a plain C program (exact_blockwise_attention_attn_amd/examples/c_forward.c, built by
build.py with the system C compiler): its forward of seeded inputs equals the Python binding's call on
the same inputs bit for bit, and the oracle to the forward tolerances."""

import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from exact_blockwise_attention_attn_amd import binding as B
from exact_blockwise_attention_attn_amd import build
from tests.gpu_util import check, log

pytestmark = pytest.mark.gpu

Bn, S, H, D = 1, 300, 2, 128


def example_bits(t):
    """The C program's inputs: a 32-bit hash of (tensor, index) mapped to [-1, 1) and cut to bf16."""
    i = np.arange(Bn * S * H * D, dtype=np.uint32)
    x = (i * np.uint32(2654435761)) ^ np.uint32(((t + 1) * 0x9E3779B9) & 0xFFFFFFFF)
    x ^= x >> np.uint32(16)
    x *= np.uint32(0x7FEB352D)
    x ^= x >> np.uint32(15)
    x *= np.uint32(0x846CA68B)
    x ^= x >> np.uint32(16)
    f = (x >> np.uint32(8)).astype(np.float32) / np.float32(8388608.0) - np.float32(1.0)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16).reshape(Bn, S, H, D)


def test_c_program_matches_binding(tmp_path):
    log("C ABI from a C program")
    assert os.path.exists(build.C_EXAMPLE_PATH), "build.py builds the C example with the library"
    out = tmp_path / "c_forward.bin"
    r = subprocess.run([build.C_EXAMPLE_PATH, str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    data = np.fromfile(out, dtype=np.float32)
    n = Bn * S * H * D
    o_c, l_c = data[:n].reshape(Bn, S, H, D), data[n:].reshape(Bn, H, S)
    bits = [example_bits(t) for t in range(3)]
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda() for b in bits)
    o = torch.empty((Bn, S, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((Bn, H, S), dtype=torch.float32, device="cuda")
    B.attn_fwd_partial(q, k, v, o, lse, causal=True, balanced=True)
    torch.cuda.synchronize()
    assert np.array_equal(o.cpu().numpy(), o_c) and np.array_equal(lse.cpu().numpy(), l_c)
    qh, kh, vh = ((b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64) for b in bits)
    O_ref, L_ref = oracle.attention(qh, kh, vh, 1 / math.sqrt(D), True, 0, 0)
    check("C program O", o_c, O_ref, 1e-2, scale_by_max=True)
    check("C program LSE", l_c, L_ref, 1e-3)
