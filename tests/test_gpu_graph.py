"""A whole step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every compute entry point enqueues only kernels on the caller's stream (no
allocation, no memset, no synchronisation), so a captured sequence of calls
replays to the eager results bit for bit.  The replays are separated by eager
work and synchronisations, the outputs are poisoned with NaN before each
replay, and the inputs are rewritten in place between replays (a replay must
read the new values, not captured ones).
"""

import pytest
import torch

from exact_blockwise_attention_attn_amd import binding as B
from exact_blockwise_attention_attn_amd import shard
from tests.gpu_util import log, seq_tensor

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    log("HIP graph capture: forward, backward, merge, split-KV decode (stream-K and allocation-free)")
    Bn, S, Hq, Hkv, D = 1, 320, 4, 2, 128
    (q, _), (k, _), (v, _), (do, _) = (seq_tensor(121, t, Bn, S, h, D, "bf16")
                                       for t, h in ((0, Hq), (1, Hkv), (2, Hkv), (3, Hq)))
    (q2, _), (k2, _) = seq_tensor(122, 0, Bn, S, Hq, D, "bf16"), seq_tensor(122, 1, Bn, S, Hkv, D, "bf16")
    o, lse = torch.empty_like(q), torch.empty((Bn, Hq, S), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dq_acc = torch.empty((Bn, S, Hq, D), dtype=torch.float32, device="cuda")
    ws = shard.bwd_workspace(Bn, Hq, S, "cuda")
    # Merge: two partials over the two key halves, merged by the tree.
    o_parts = torch.empty((2, Bn, S, Hq, D), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((2, Bn, Hq, S), dtype=torch.float32, device="cuda")
    om, lm = torch.empty((Bn, S, Hq, D), dtype=torch.bfloat16, device="cuda"), torch.empty_like(lse)
    # Decode: the last query row of each head over the cache k, v with uneven lengths (stream-K).
    sl = torch.tensor([S - 17], dtype=torch.int32, device="cuda")
    od, ld = torch.empty((Bn, Hq, D), dtype=torch.bfloat16, device="cuda"), torch.empty((Bn, Hq), device="cuda")
    od2, ld2 = torch.empty_like(od), torch.empty_like(ld)
    dws = torch.empty(B.attn_decode_workspace_size(Bn, Hq, D, 8), dtype=torch.uint8, device="cuda")
    qd = torch.empty((Bn, Hq, D), dtype=torch.bfloat16, device="cuda")
    outs = (o, lse, dq, dk, dv, dq_acc, om, lm, od, ld, od2, ld2)

    def step():
        shard.causal_attention_forward(q, k, v, o=o, lse=lse)
        shard.causal_attention_backward(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, dq_acc=dq_acc, workspace=ws)
        half = S // 2
        B.attn_fwd_partial(q, k[:, :half], v[:, :half], o_parts[0], l_parts[0], causal=True)
        B.attn_fwd_partial(q, k[:, half:], v[:, half:], o_parts[1], l_parts[1], k_pos0=half, causal=True)
        B.attn_merge_lse(o_parts, l_parts, om, lm, tree=True)
        qd.copy_(q[:, -1])
        B.attn_decode_splitkv(qd, k, v, od, ld, dws, n_splits=8, seqlens=sl)
        B.attn_decode_splitkv_noalloc(qd, k, v, od2, ld2, n_splits=8, seqlens=sl)

    def eager():
        step()
        torch.cuda.synchronize()
        return [t.clone() for t in outs]

    ref = eager()  # also makes every one-time lookup (scratch address, CU count) before capture
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        if r == 2:  # new inputs in place: the replays must see them
            q.copy_(q2)
            k.copy_(k2)
            ref = eager()
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outs)):
            assert torch.equal(a, b), (r, i)
        # Eager work between replays on the same buffers' neighbours.
        shard.causal_attention_forward(q2, k2, v)
        torch.cuda.synchronize()
    assert not torch.isnan(ref[0]).any() and torch.isfinite(ref[8].float()).all()
