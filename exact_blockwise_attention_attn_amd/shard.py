"""Chunked drivers over the C ABI: one device's share of a sequence-sharded attention.

These functions only sequence calls to libattn (every step of the arithmetic
runs in the HIP kernels) and allocate the buffers they need with PyTorch.

* ``shard_forward``: a query shard attends keys that arrive chunk by chunk in
  order (the ring/BurstAttention setting); each chunk's partial is merged into a
  running fp32 (O, LSE) by the kernel's accumulate epilogue, and the last live
  chunk also writes the bf16 output.  Chunks no query can see are skipped: their
  partial is the merge identity.
* ``shard_forward_partials``: the same, but every live chunk writes its own
  partial and one ``attn_merge_lse`` call merges them (sequential order).
* ``shard_backward``: dK/dV per chunk and dQ accumulated over chunks from the
  saved final (O, LSE), without re-running the forward.
* ``causal_attention_forward`` / ``causal_attention_backward``: causal
  self-attention over a whole sequence in one call each, with the balanced
  schedule that pairs early and late query (key) tiles.
"""

from __future__ import annotations

import torch

from . import binding as B


def _chunk_visible(q_pos0: int, sq: int, k_pos0: int, causal: bool) -> bool:
    # Some query sees some key of the chunk iff the chunk's first key is not after the last query.
    return (not causal) or (k_pos0 <= q_pos0 + sq - 1)


def chunk_bounds(sk: int, chunk: int):
    return [(c, min(c + chunk, sk)) for c in range(0, sk, chunk)]


def shard_forward(q, k, v, chunk, *, q_pos0=0, k_pos0=0, causal=False, scale=0.0, stream=None,
                  o_run=None, lse=None, o_out=None):
    """Returns (o_out bf16-or-input-dtype [B,Sq,H,D], lse fp32 [B,H,Sq], o_run fp32)."""
    b, sq, hq, d = q.shape
    sk = k.shape[1]
    dev = q.device
    o_run = torch.empty((b, sq, hq, d), dtype=torch.float32, device=dev) if o_run is None else o_run
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device=dev) if lse is None else lse
    if o_out is None:
        o_out = torch.empty((b, sq, hq, d), dtype=torch.bfloat16, device=dev) if q.dtype == torch.bfloat16 else None
    chunks = [(a, e) for a, e in chunk_bounds(sk, chunk) if _chunk_visible(q_pos0, sq, k_pos0 + a, causal)]
    if not chunks:
        chunks = [(0, 0)]  # nothing visible: one call writes the identity
    for idx, (a, e) in enumerate(chunks):
        last = idx == len(chunks) - 1
        B.attn_fwd_partial(q, k[:, a:e], v[:, a:e], o_run, lse, q_pos0=q_pos0, k_pos0=k_pos0 + a, causal=causal,
                           scale=scale, accumulate=idx > 0, o_final=o_out if last else None, stream=stream)
    return (o_out if o_out is not None else o_run), lse, o_run


def shard_forward_fused(q, k, v, chunk, *, q_pos0=0, k_pos0=0, causal=False, scale=0.0, stream=None,
                        o_out=None, lse=None):
    """The same result as shard_forward in one launch over the chunk table (bf16 only).

    k and v are split into views of `chunk` keys; the kernel keeps each query's
    running (O, LSE) on chip across the chunks.  Returns (o_out, lse).
    """
    b, sq, hq, d = q.shape
    sk = k.shape[1]
    dev = q.device
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device=dev) if lse is None else lse
    o_out = torch.empty((b, sq, hq, d), dtype=q.dtype, device=dev) if o_out is None else o_out
    bounds = chunk_bounds(sk, chunk)
    B.attn_fwd_chunks(q, [k[:, a:e] for a, e in bounds], [v[:, a:e] for a, e in bounds], o_out, lse,
                      chunk_pos0=[k_pos0 + a for a, _ in bounds], q_pos0=q_pos0, causal=causal, scale=scale,
                      stream=stream)
    return o_out, lse


def shard_forward_partials(q, k, v, chunk, *, q_pos0=0, k_pos0=0, causal=False, scale=0.0, tree=False,
                           stream=None):
    """Per-chunk partials into a stacked fp32 buffer, then one merge call.  Returns (o, lse, parts)."""
    b, sq, hq, d = q.shape
    sk = k.shape[1]
    dev = q.device
    chunks = [(a, e) for a, e in chunk_bounds(sk, chunk) if _chunk_visible(q_pos0, sq, k_pos0 + a, causal)]
    n = max(1, len(chunks))
    o_parts = torch.empty((n, b, sq, hq, d), dtype=torch.float32, device=dev)
    lse_parts = torch.empty((n, b, hq, sq), dtype=torch.float32, device=dev)
    if not chunks:
        chunks = [(0, 0)]
    for i, (a, e) in enumerate(chunks):
        B.attn_fwd_partial(q, k[:, a:e], v[:, a:e], o_parts[i], lse_parts[i], q_pos0=q_pos0, k_pos0=k_pos0 + a,
                           causal=causal, scale=scale, stream=stream)
    out_dtype = torch.bfloat16 if q.dtype == torch.bfloat16 else torch.float32
    o = torch.empty((b, sq, hq, d), dtype=out_dtype, device=dev)
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device=dev)
    B.attn_merge_lse(o_parts, lse_parts, o, lse, tree=tree, stream=stream)
    return o, lse, (o_parts, lse_parts)


def bwd_workspace(batch, heads_q, seqlen_q, device):
    """A statistics workspace for attn_bwd (uint8, 256-byte aligned by the caching allocator)."""
    n = B.attn_bwd_workspace_size(batch, heads_q, seqlen_q)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def shard_backward(q, k, v, o, dout, lse, chunk, *, q_pos0=0, k_pos0=0, causal=False, scale=0.0, stream=None,
                   dq=None, dk=None, dv=None, dq_acc=None, workspace=None):
    """Gradients for a query shard whose keys come in chunks.  Returns (dq, dk, dv)."""
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty((b, sk, hkv, d), dtype=q.dtype, device=dev) if dk is None else dk
    dv = torch.empty((b, sk, hkv, d), dtype=q.dtype, device=dev) if dv is None else dv
    dq_acc = torch.empty((b, sq, hq, d), dtype=torch.float32, device=dev) if dq_acc is None else dq_acc
    workspace = bwd_workspace(b, hq, sq, dev) if workspace is None else workspace
    bounds = chunk_bounds(sk, chunk) or [(0, 0)]
    live = [i for i, (a, _) in enumerate(bounds) if _chunk_visible(q_pos0, sq, k_pos0 + a, causal)]
    first_dq = live[0] if live else 0
    last_dq = live[-1] if live else 0
    for i, (a, e) in enumerate(bounds):
        B.attn_bwd(q, k[:, a:e], v[:, a:e], o, dout, lse, workspace, dq_acc, dk[:, a:e], dv[:, a:e], dq=dq,
                   q_pos0=q_pos0, k_pos0=k_pos0 + a, causal=causal, scale=scale, compute_delta=i == 0,
                   dq_overwrite=i == first_dq, finalize_dq=i == last_dq, stream=stream)
    return dq, dk, dv


def shard_backward_fused(q, k, v, o, dout, lse, chunk, *, q_pos0=0, k_pos0=0, causal=False, scale=0.0,
                         stream=None, dq=None, dk=None, dv=None, dq_acc=None, workspace=None):
    """The same gradients as shard_backward from one call over the chunk table (bf16 only).

    k, v, dk and dv are split into views of `chunk` keys; dK/dV of every chunk
    come from one kernel launch, and dQ is summed over the chunks on chip and
    written once.  Returns (dq, dk, dv).
    """
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty((b, sk, hkv, d), dtype=q.dtype, device=dev) if dk is None else dk
    dv = torch.empty((b, sk, hkv, d), dtype=q.dtype, device=dev) if dv is None else dv
    dq_acc = torch.empty((b, sq, hq, d), dtype=torch.float32, device=dev) if dq_acc is None else dq_acc
    workspace = bwd_workspace(b, hq, sq, dev) if workspace is None else workspace
    bounds = chunk_bounds(sk, chunk)
    views = lambda t: [t[:, a:e] for a, e in bounds]  # noqa: E731
    B.attn_bwd_chunks(q, views(k), views(v), o, dout, lse, workspace, dq_acc, views(dk), views(dv),
                      chunk_pos0=[k_pos0 + a for a, _ in bounds], dq=dq, q_pos0=q_pos0, causal=causal, scale=scale,
                      compute_delta=True, dq_overwrite=True, finalize_dq=True, balanced=causal, stream=stream)
    return dq, dk, dv


def causal_attention_forward(q, k, v, *, scale=0.0, balanced=True, o=None, lse=None, stream=None):
    b, s, hq, d = q.shape
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((b, hq, s), dtype=torch.float32, device=q.device) if lse is None else lse
    B.attn_fwd_partial(q, k, v, o, lse, causal=True, scale=scale, balanced=balanced, stream=stream)
    return o, lse


def causal_attention_backward(q, k, v, o, dout, lse, *, scale=0.0, balanced=True, stream=None,
                              dq=None, dk=None, dv=None, dq_acc=None, workspace=None):
    b, s, hq, d = q.shape
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dq_acc = torch.empty((b, s, hq, d), dtype=torch.float32, device=dev) if dq_acc is None else dq_acc
    workspace = bwd_workspace(b, hq, s, dev) if workspace is None else workspace
    B.attn_bwd(q, k, v, o, dout, lse, workspace, dq_acc, dk, dv, dq=dq, causal=True, scale=scale, compute_delta=True,
               dq_overwrite=True, finalize_dq=True, balanced=balanced, stream=stream)
    return dq, dk, dv
