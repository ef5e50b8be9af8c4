"""attn_decode_splitkv_noalloc against attn_decode_splitkv, through the C ABI.

The allocation-free entry point runs the same kernels with the split partials
in the library's fixed per-device scratch instead of a caller's workspace, so
its outputs must equal the workspace form's bit for bit.  Two calls in a row,
the second smaller (the scratch then still holds the first call's partials
beyond the second's), plus a head_dim 64 call.
"""

import numpy as np
import pytest
import torch

from exact_blockwise_attention_attn_amd import binding as B
from seeded_inputs import normal_bf16
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _bf16(wid, tid, b, shape):
    bits = normal_bf16(wid, tid, b, shape)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _both(Bn, Hq, Hkv, L, D, n_splits, lens, wid):
    q = _bf16(wid, 0, Bn, (Hq, D))
    kc, vc = _bf16(wid, 1, Bn, (L, Hkv, D)), _bf16(wid, 2, Bn, (L, Hkv, D))
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    o_ref = torch.empty((Bn, Hq, D), dtype=torch.bfloat16, device="cuda")
    l_ref = torch.empty((Bn, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.attn_decode_workspace_size(Bn, Hq, D, n_splits), dtype=torch.uint8, device="cuda")
    B.attn_decode_splitkv(q, kc, vc, o_ref, l_ref, ws, n_splits=n_splits, seqlens=sl)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    B.attn_decode_splitkv_noalloc(q, kc, vc, o, lse, n_splits=n_splits, seqlens=sl)
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


CALLS = [
    # (B, H_q, H_kv, L, D, n_splits, seqlens): the first call fills most of the scratch.
    (16, 32, 8, 20000, 128, 64, [20000 - 1250 * i for i in range(16)]),
    (2, 8, 2, 3000, 128, 16, None),
    (3, 16, 4, 5000, 64, 32, [5000, 1, 0]),
]


def test_noalloc_matches_workspace_form_two_calls_in_a_row():
    for i, (Bn, Hq, Hkv, L, D, ns, lens) in enumerate(CALLS):
        log(f"noalloc decode call {i}: B={Bn} H_q={Hq} H_kv={Hkv} L={L} D={D} splits={ns} seqlens={lens is not None}")
        o, lse, o_ref, l_ref = _both(Bn, Hq, Hkv, L, D, ns, lens, 40 + i)
        assert torch.equal(o, o_ref), f"call {i}: O differs from attn_decode_splitkv"
        assert torch.equal(lse.isfinite(), l_ref.isfinite())
        assert torch.equal(lse[l_ref.isfinite()], l_ref[l_ref.isfinite()]), f"call {i}: LSE differs"


def test_noalloc_rejects_oversize():
    q = torch.zeros((16, 32, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((16, 256, 8, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((16, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((16, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(B.AttnError) as e:
        B.attn_decode_splitkv_noalloc(q, kc, kc, o, lse, n_splits=128)
    assert e.value.status == B.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == 0), "a rejected call must leave the outputs untouched"
