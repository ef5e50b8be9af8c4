"""The same calls with every launch serialised by the runtime (AMD_SERIALIZE_KERNEL=3: wait before and
after each kernel; HIP_LAUNCH_BLOCKING=1: each launch blocks the host) give the same bits as the normal
asynchronous run.  A kernel that read something an earlier launch had not finished writing, or depended
on two launches overlapping, would differ between the two.  The serialised run is a child process, since
the runtime reads these variables when it starts.
"""

import os
import subprocess
import sys
import tempfile

import pytest
import torch

from exact_blockwise_attention_attn_amd import binding as B
from exact_blockwise_attention_attn_amd import shard
from tests.gpu_util import log, seq_tensor

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def step_outputs():
    """Forward, backward, chunk-table forward and backward, merge, stream-K decode and tree decode on
    seeded inputs; returns every output on the host."""
    Bn, S, Hq, Hkv, D = 2, 333, 4, 2, 128
    q, _ = seq_tensor(140, 0, Bn, S, Hq, D, "bf16")
    k, _ = seq_tensor(140, 1, Bn, S, Hkv, D, "bf16")
    v, _ = seq_tensor(140, 2, Bn, S, Hkv, D, "bf16")
    do, _ = seq_tensor(140, 3, Bn, S, Hq, D, "bf16")
    out = {}
    out["o"], out["lse"] = shard.causal_attention_forward(q, k, v)
    out["dq"], out["dk"], out["dv"] = shard.causal_attention_backward(q, k, v, out["o"], do, out["lse"])
    ks, vs, pos = [k[:, :100], k[:, 100:200], k[:, 200:]], [v[:, :100], v[:, 100:200], v[:, 200:]], [0, 100, 200]
    oc, lc = torch.empty_like(q), torch.empty_like(out["lse"])
    B.attn_fwd_chunks(q, ks, vs, oc, lc, chunk_pos0=pos, causal=True)
    dks, dvs = [torch.empty_like(x) for x in ks], [torch.empty_like(x) for x in vs]
    dqc = torch.empty_like(q)
    dq_acc = torch.empty((Bn, S, Hq, D), dtype=torch.float32, device="cuda")
    ws = shard.bwd_workspace(Bn, Hq, S, "cuda")
    B.attn_bwd_chunks(q, ks, vs, oc, do, lc, ws, dq_acc, dks, dvs, chunk_pos0=pos, dq=dqc, causal=True,
                      compute_delta=True, dq_overwrite=True, finalize_dq=True)
    out.update(oc=oc, lc=lc, dqc=dqc, dk0=dks[0], dk2=dks[2], dv1=dvs[1])
    o_parts = torch.empty((2, Bn, S, Hq, D), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((2, Bn, Hq, S), dtype=torch.float32, device="cuda")
    B.attn_fwd_partial(q, k[:, :150], v[:, :150], o_parts[0], l_parts[0], causal=True)
    B.attn_fwd_partial(q, k[:, 150:], v[:, 150:], o_parts[1], l_parts[1], k_pos0=150, causal=True)
    out["om"], out["lm"] = torch.empty_like(q), torch.empty_like(out["lse"])
    B.attn_merge_lse(o_parts, l_parts, out["om"], out["lm"], tree=True)
    qd = q[:, -1].contiguous()
    out["od"], out["ld"] = torch.empty_like(qd), torch.empty((Bn, Hq), dtype=torch.float32, device="cuda")
    dws = torch.empty(B.attn_decode_workspace_size(Bn, Hq, D, 16), dtype=torch.uint8, device="cuda")
    sl = torch.tensor([S, 7], dtype=torch.int32, device="cuda")
    B.attn_decode_splitkv(qd, k, v, out["od"], out["ld"], dws, n_splits=16, seqlens=sl)
    nodes = [(0, 200, 0, 4), (200, 60, 0, 2), (260, 73, 2, 4)]
    ks_, kl_, qb_, qe_ = zip(*nodes)
    qt, kt, vt = q[0, :4].contiguous(), k[0], v[0]
    need = B.attn_decode_tree_workspace_size(qt, kt, kv_start=ks_, kv_len=kl_, q_begin=qb_, q_end=qe_)
    tws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out["ot"], out["lt"] = torch.empty_like(qt), torch.empty((4, Hq), dtype=torch.float32, device="cuda")
    B.attn_decode_tree(qt, kt, vt, out["ot"], out["lt"], tws, kv_start=ks_, kv_len=kl_, q_begin=qb_, q_end=qe_)
    torch.cuda.synchronize()
    return {name: t.cpu() for name, t in out.items()}


def test_serialized_launches_same_bits():
    log("serialised launches (AMD_SERIALIZE_KERNEL=3, HIP_LAUNCH_BLOCKING=1) against the asynchronous run")
    ref = step_outputs()
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "serialized.pt")
        code = ("import sys, torch; sys.path.insert(0, %r); from tests.test_gpu_serialized import step_outputs; "
                "torch.save(step_outputs(), %r)") % (ROOT, path)
        env = dict(os.environ, AMD_SERIALIZE_KERNEL="3", HIP_LAUNCH_BLOCKING="1")
        r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        got = torch.load(path, weights_only=True)
    assert sorted(got) == sorted(ref)
    for name in ref:
        assert torch.equal(ref[name], got[name]), name
