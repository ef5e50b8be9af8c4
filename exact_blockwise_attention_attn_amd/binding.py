"""Thin ctypes binding of libattn (include/attn.h).

Argument marshalling only: each function takes PyTorch tensors (device memory
and the current stream are PyTorch's), checks nothing beyond what is needed to
fill the C argument struct, and calls the C entry point of the same name.  All
arithmetic happens in the HIP kernels.  A nonzero status raises ``AttnError``
carrying ``attn_last_error()``.

The library is loaded from the package directory; if it has not been built
yet it is built once.  There is no fallback: without the library every call
raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

c_i32, c_u32, c_i64, c_f32, c_vp = ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
I64x3 = c_i64 * 3
I64x2 = c_i64 * 2

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE = 3
ATTN_ERR_HIP = 4
ATTN_ERR_NONFINITE = 5
ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1
ATTN_FWD_ACCUMULATE = 1 << 0
ATTN_FWD_BALANCED = 1 << 1
ATTN_MERGE_SEQUENTIAL = 0
ATTN_MERGE_TREE = 1
ATTN_BWD_COMPUTE_DELTA = 1 << 0
ATTN_BWD_DQ_OVERWRITE = 1 << 1
ATTN_BWD_FINALIZE_DQ = 1 << 2
ATTN_BWD_BALANCED = 1 << 3
ATTN_BWD_DETERMINISTIC = 1 << 4


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("dtype", c_u32),
        ("batch", c_i32), ("heads_q", c_i32), ("heads_kv", c_i32),
        ("seqlen_q", c_i32), ("seqlen_k", c_i32), ("head_dim", c_i32),
        ("q", c_vp), ("q_stride", I64x3),
        ("k", c_vp), ("k_stride", I64x3),
        ("v", c_vp), ("v_stride", I64x3),
        ("o", c_vp), ("o_stride", I64x3), ("o_dtype", c_u32),
        ("lse", c_vp),
        ("o_final", c_vp), ("o_final_stride", I64x3),
        ("q_pos0", c_i64), ("k_pos0", c_i64),
        ("causal", c_i32), ("scale", c_f32), ("flags", c_u32),
        ("cu_seqlens_q", c_vp), ("cu_seqlens_k", c_vp),
    ]


class FwdChunksArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("dtype", c_u32),
        ("batch", c_i32), ("heads_q", c_i32), ("heads_kv", c_i32), ("seqlen_q", c_i32), ("head_dim", c_i32),
        ("n_chunks", c_i32),
        ("q", c_vp), ("q_stride", I64x3),
        ("k_chunks", ctypes.POINTER(c_vp)), ("v_chunks", ctypes.POINTER(c_vp)),
        ("chunk_len", ctypes.POINTER(c_i32)), ("chunk_pos0", ctypes.POINTER(c_i64)),
        ("k_stride", I64x3), ("v_stride", I64x3),
        ("chunk_k_bstride", ctypes.POINTER(c_i64)), ("chunk_v_bstride", ctypes.POINTER(c_i64)),
        ("o", c_vp), ("o_stride", I64x3), ("o_dtype", c_u32),
        ("lse", c_vp),
        ("o_final", c_vp), ("o_final_stride", I64x3),
        ("q_pos0", c_i64),
        ("causal", c_i32), ("scale", c_f32), ("flags", c_u32),
    ]


class MergeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("n_parts", c_i32),
        ("batch", c_i32), ("seqlen", c_i32), ("heads", c_i32), ("head_dim", c_i32),
        ("o_parts", c_vp), ("o_part_stride", c_i64), ("o_stride", I64x3),
        ("lse_parts", c_vp), ("lse_part_stride", c_i64),
        ("o_out", c_vp), ("o_out_stride", I64x3), ("o_out_dtype", c_u32),
        ("lse_out", c_vp), ("mode", c_u32),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("dtype", c_u32),
        ("batch", c_i32), ("heads_q", c_i32), ("heads_kv", c_i32),
        ("seqlen_q", c_i32), ("seqlen_k", c_i32), ("head_dim", c_i32),
        ("q", c_vp), ("q_stride", I64x3),
        ("k", c_vp), ("k_stride", I64x3),
        ("v", c_vp), ("v_stride", I64x3),
        ("o", c_vp), ("o_stride", I64x3),
        ("dout", c_vp), ("do_stride", I64x3),
        ("lse", c_vp), ("workspace", c_vp), ("workspace_bytes", ctypes.c_size_t), ("dq_acc", c_vp),
        ("dq", c_vp), ("dq_stride", I64x3),
        ("dk", c_vp), ("dk_stride", I64x3),
        ("dv", c_vp), ("dv_stride", I64x3),
        ("q_pos0", c_i64), ("k_pos0", c_i64),
        ("causal", c_i32), ("scale", c_f32), ("flags", c_u32),
        ("cu_seqlens_q", c_vp), ("cu_seqlens_k", c_vp),
    ]


class BwdChunksArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("dtype", c_u32),
        ("batch", c_i32), ("heads_q", c_i32), ("heads_kv", c_i32), ("seqlen_q", c_i32), ("head_dim", c_i32),
        ("n_chunks", c_i32),
        ("q", c_vp), ("q_stride", I64x3),
        ("o", c_vp), ("o_stride", I64x3),
        ("dout", c_vp), ("do_stride", I64x3),
        ("lse", c_vp), ("workspace", c_vp), ("workspace_bytes", ctypes.c_size_t), ("dq_acc", c_vp),
        ("dq", c_vp), ("dq_stride", I64x3),
        ("k_chunks", ctypes.POINTER(c_vp)), ("v_chunks", ctypes.POINTER(c_vp)),
        ("dk_chunks", ctypes.POINTER(c_vp)), ("dv_chunks", ctypes.POINTER(c_vp)),
        ("chunk_len", ctypes.POINTER(c_i32)), ("chunk_pos0", ctypes.POINTER(c_i64)),
        ("k_stride", I64x3), ("v_stride", I64x3), ("dk_stride", I64x3), ("dv_stride", I64x3),
        ("chunk_k_bstride", ctypes.POINTER(c_i64)), ("chunk_v_bstride", ctypes.POINTER(c_i64)),
        ("chunk_dk_bstride", ctypes.POINTER(c_i64)), ("chunk_dv_bstride", ctypes.POINTER(c_i64)),
        ("q_pos0", c_i64),
        ("causal", c_i32), ("scale", c_f32), ("flags", c_u32),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32),
        ("batch", c_i32), ("heads_q", c_i32), ("heads_kv", c_i32), ("head_dim", c_i32),
        ("cache_len", c_i64),
        ("q", c_vp), ("q_stride", I64x2),
        ("k_cache", c_vp), ("k_stride", I64x3),
        ("v_cache", c_vp), ("v_stride", I64x3),
        ("seqlens", c_vp), ("n_splits", c_i32), ("scale", c_f32),
        ("o", c_vp), ("o_stride", I64x2),
        ("lse", c_vp),
        ("workspace", c_vp), ("workspace_bytes", ctypes.c_size_t),
    ]


class DecodeTreeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32),
        ("n_queries", c_i32), ("heads_q", c_i32), ("heads_kv", c_i32), ("head_dim", c_i32),
        ("n_nodes", c_i32), ("cache_len", c_i64),
        ("q", c_vp), ("q_stride", I64x2),
        ("k_cache", c_vp), ("k_stride", I64x2),
        ("v_cache", c_vp), ("v_stride", I64x2),
        ("kv_start", ctypes.POINTER(c_i64)), ("kv_len", ctypes.POINTER(c_i32)),
        ("q_begin", ctypes.POINTER(c_i32)), ("q_end", ctypes.POINTER(c_i32)),
        ("scale", c_f32),
        ("o", c_vp), ("o_stride", I64x2),
        ("lse", c_vp),
        ("workspace", c_vp), ("workspace_bytes", ctypes.c_size_t),
    ]


EXPORTED = [
    "attn_fwd_partial",
    "attn_fwd_chunks",
    "attn_merge_lse",
    "attn_bwd",
    "attn_bwd_chunks",
    "attn_decode_splitkv",
    "attn_decode_splitkv_noalloc",
    "attn_decode_tree",
    "attn_decode_tree_workspace_size",
    "attn_bwd_workspace_size",
    "attn_decode_workspace_size",
    "attn_status_string",
    "attn_last_error",
    "attn_abi_version",
]

_lib = None
_lock = threading.Lock()


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def lib_path() -> str:
    """The in-tree libattn.so, or the library named by ATTN_LIBRARY (e.g. the host-ASan build)."""
    return os.environ.get("ATTN_LIBRARY") or _build.LIB_PATH


def load(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load libattn.so (building it first if it does not exist)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            if not build_if_missing:
                raise FileNotFoundError(f"{path} is not built")
            _build.build()
        lib = ctypes.CDLL(path)
        for name, argt in (("attn_fwd_partial", [ctypes.POINTER(FwdArgs), c_vp]),
                           ("attn_fwd_chunks", [ctypes.POINTER(FwdChunksArgs), c_vp]),
                           ("attn_merge_lse", [ctypes.POINTER(MergeArgs), c_vp]),
                           ("attn_bwd", [ctypes.POINTER(BwdArgs), c_vp]),
                           ("attn_bwd_chunks", [ctypes.POINTER(BwdChunksArgs), c_vp]),
                           ("attn_decode_splitkv", [ctypes.POINTER(DecodeArgs), c_vp]),
                           ("attn_decode_splitkv_noalloc", [ctypes.POINTER(DecodeArgs), c_vp]),
                           ("attn_decode_tree", [ctypes.POINTER(DecodeTreeArgs), c_vp])):
            fn = getattr(lib, name)
            fn.argtypes = argt
            fn.restype = ctypes.c_int
        lib.attn_bwd_workspace_size.argtypes = [c_i32, c_i32, c_i32]
        lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
        lib.attn_decode_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32]
        lib.attn_decode_workspace_size.restype = ctypes.c_size_t
        lib.attn_decode_tree_workspace_size.argtypes = [ctypes.POINTER(DecodeTreeArgs)]
        lib.attn_decode_tree_workspace_size.restype = ctypes.c_size_t
        lib.attn_status_string.argtypes = [ctypes.c_int]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_abi_version.argtypes = []
        lib.attn_abi_version.restype = ctypes.c_int
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != ATTN_OK:
        msg = load().attn_last_error().decode()
        raise AttnError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float32:
        return ATTN_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _strides3(t: torch.Tensor | None):
    if t is None:
        return I64x3(0, 0, 0)
    assert t.dim() == 4, "expected a [B, S, H, D] tensor"
    if t.numel() == 0:  # nothing is read or written; strides of empty views are arbitrary
        return I64x3(0, 0, 0)
    assert t.stride(3) == 1, "expected a unit innermost stride"
    return I64x3(t.stride(0), t.stride(1), t.stride(2))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def attn_abi_version() -> int:
    return load().attn_abi_version()


def attn_status_string(status: int) -> str:
    return load().attn_status_string(status).decode()


def attn_last_error() -> str:
    return load().attn_last_error().decode()


def attn_bwd_workspace_size(batch: int, heads_q: int, seqlen_q: int) -> int:
    return load().attn_bwd_workspace_size(batch, heads_q, seqlen_q)


def attn_decode_workspace_size(batch: int, heads_q: int, head_dim: int, n_splits: int) -> int:
    return load().attn_decode_workspace_size(batch, heads_q, head_dim, n_splits)


def _tree_args(q, k_cache, v_cache, o, lse, workspace, kv_start, kv_len, q_begin, q_end, scale):
    n = len(kv_start)
    assert len(kv_len) == n and len(q_begin) == n and len(q_end) == n
    a = DecodeTreeArgs()
    a.struct_size = ctypes.sizeof(DecodeTreeArgs)
    a.n_queries, a.heads_q, a.head_dim = q.shape
    a.heads_kv = k_cache.shape[1]
    a.n_nodes = n
    a.cache_len = k_cache.shape[0]
    a.q, a.q_stride = _ptr(q), I64x2(q.stride(0), q.stride(1))
    a.k_cache, a.k_stride = _ptr(k_cache), I64x2(k_cache.stride(0), k_cache.stride(1))
    if v_cache is not None:
        a.v_cache, a.v_stride = _ptr(v_cache), I64x2(v_cache.stride(0), v_cache.stride(1))
    a.kv_start = (c_i64 * max(n, 1))(*[int(x) for x in kv_start])
    a.kv_len = (c_i32 * max(n, 1))(*[int(x) for x in kv_len])
    a.q_begin = (c_i32 * max(n, 1))(*[int(x) for x in q_begin])
    a.q_end = (c_i32 * max(n, 1))(*[int(x) for x in q_end])
    a.scale = float(scale)
    if o is not None:
        a.o, a.o_stride = _ptr(o), I64x2(o.stride(0), o.stride(1))
    a.lse = _ptr(lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a


def attn_decode_tree_workspace_size(q, k_cache, *, kv_start, kv_len, q_begin, q_end) -> int:
    """Workspace bytes attn_decode_tree needs for this tree (0 if the node lists are invalid)."""
    a = _tree_args(q, k_cache, None, None, None, None, kv_start, kv_len, q_begin, q_end, 0.0)
    return load().attn_decode_tree_workspace_size(ctypes.byref(a))


def attn_decode_tree(q, k_cache, v_cache, o, lse, workspace, *, kv_start, kv_len, q_begin, q_end, scale=0.0,
                     stream=None) -> None:
    """q [n_q, Hq, D], packed caches [L, Hkv, D] bf16, node lists (host ints) -> o [n_q, Hq, D], lse [n_q, Hq]."""
    assert q.stride(2) == 1 and k_cache.stride(2) == 1 and v_cache.stride(2) == 1 and o.stride(2) == 1
    a = _tree_args(q, k_cache, v_cache, o, lse, workspace, kv_start, kv_len, q_begin, q_end, scale)
    _check(load().attn_decode_tree(ctypes.byref(a), _stream(stream)))


def attn_fwd_partial(q, k, v, o, lse, *, q_pos0=0, k_pos0=0, causal=False, scale=0.0,
                     accumulate=False, balanced=False, o_final=None, stream=None) -> None:
    """q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D], o [B,Sq,Hq,D] (fp32 or bf16), lse fp32 [B,Hq,Sq]."""
    a = FwdArgs()
    a.struct_size = ctypes.sizeof(FwdArgs)
    a.dtype = _dtype_code(q)
    a.batch, a.seqlen_q, a.heads_q, a.head_dim = q.shape
    a.seqlen_k, a.heads_kv = k.shape[1], k.shape[2]
    a.q, a.q_stride = _ptr(q), _strides3(q)
    a.k, a.k_stride = _ptr(k), _strides3(k)
    a.v, a.v_stride = _ptr(v), _strides3(v)
    a.o, a.o_stride, a.o_dtype = _ptr(o), _strides3(o), _dtype_code(o)
    a.lse = _ptr(lse)
    a.o_final, a.o_final_stride = _ptr(o_final), _strides3(o_final)
    a.q_pos0, a.k_pos0 = int(q_pos0), int(k_pos0)
    a.causal = int(bool(causal))
    a.scale = float(scale)
    a.flags = (ATTN_FWD_ACCUMULATE if accumulate else 0) | (ATTN_FWD_BALANCED if balanced else 0)
    _check(load().attn_fwd_partial(ctypes.byref(a), _stream(stream)))


def attn_fwd_chunks(q, k_chunks, v_chunks, o, lse, *, chunk_pos0, q_pos0=0, causal=False, scale=0.0,
                    accumulate=False, balanced=False, o_final=None, stream=None) -> None:
    """Forward of q over a list of key/value chunks ([B, len_c, Hkv, D] bf16 each, common strides), one launch."""
    n = len(k_chunks)
    assert len(v_chunks) == n and len(chunk_pos0) == n
    a = FwdChunksArgs()
    a.struct_size = ctypes.sizeof(FwdChunksArgs)
    a.dtype = _dtype_code(q)
    a.batch, a.seqlen_q, a.heads_q, a.head_dim = q.shape
    a.heads_kv = k_chunks[0].shape[2] if n else q.shape[2]
    a.n_chunks = n
    a.q, a.q_stride = _ptr(q), _strides3(q)
    kp = (c_vp * max(n, 1))(*[_ptr(k) for k in k_chunks])
    vp = (c_vp * max(n, 1))(*[_ptr(v) for v in v_chunks])
    ln = (c_i32 * max(n, 1))(*[k.shape[1] for k in k_chunks])
    ps = (c_i64 * max(n, 1))(*[int(x) for x in chunk_pos0])
    a.k_chunks, a.v_chunks, a.chunk_len, a.chunk_pos0 = kp, vp, ln, ps
    live = [k for k in k_chunks if k.shape[1] > 0]
    a.k_stride = _strides3(live[0]) if live else I64x3(0, 0, 0)
    live_v = [v for v in v_chunks if v.shape[1] > 0]
    a.v_stride = _strides3(live_v[0]) if live_v else I64x3(0, 0, 0)
    for k in live:
        assert tuple(k.stride()[1:3]) == tuple(a.k_stride)[1:], "key chunks must share sequence and head strides"
    for v in live_v:
        assert tuple(v.stride()[1:3]) == tuple(a.v_stride)[1:], "value chunks must share sequence and head strides"
    kbs = (c_i64 * max(n, 1))(*[k.stride(0) if k.numel() else 0 for k in k_chunks])
    vbs = (c_i64 * max(n, 1))(*[v.stride(0) if v.numel() else 0 for v in v_chunks])
    a.chunk_k_bstride, a.chunk_v_bstride = kbs, vbs
    a.o, a.o_stride, a.o_dtype = _ptr(o), _strides3(o), _dtype_code(o)
    a.lse = _ptr(lse)
    a.o_final, a.o_final_stride = _ptr(o_final), _strides3(o_final)
    a.q_pos0 = int(q_pos0)
    a.causal = int(bool(causal))
    a.scale = float(scale)
    a.flags = (ATTN_FWD_ACCUMULATE if accumulate else 0) | (ATTN_FWD_BALANCED if balanced else 0)
    _check(load().attn_fwd_chunks(ctypes.byref(a), _stream(stream)))


def attn_merge_lse(o_parts, lse_parts, o_out, lse_out, *, tree=False, stream=None) -> None:
    """o_parts fp32 [n,B,S,H,D], lse_parts fp32 [n,B,H,S] -> o_out [B,S,H,D], lse_out [B,H,S]."""
    n, B, S, H, D = o_parts.shape
    assert o_parts.stride(4) == 1 and lse_parts.is_contiguous()
    a = MergeArgs()
    a.struct_size = ctypes.sizeof(MergeArgs)
    a.n_parts, a.batch, a.seqlen, a.heads, a.head_dim = n, B, S, H, D
    a.o_parts, a.o_part_stride = _ptr(o_parts), o_parts.stride(0)
    a.o_stride = I64x3(o_parts.stride(1), o_parts.stride(2), o_parts.stride(3))
    a.lse_parts, a.lse_part_stride = _ptr(lse_parts), lse_parts.stride(0)
    a.o_out, a.o_out_stride, a.o_out_dtype = _ptr(o_out), _strides3(o_out), _dtype_code(o_out)
    a.lse_out = _ptr(lse_out)
    a.mode = ATTN_MERGE_TREE if tree else ATTN_MERGE_SEQUENTIAL
    _check(load().attn_merge_lse(ctypes.byref(a), _stream(stream)))


def attn_merge_lse_pair(o_a, lse_a, o_b, lse_b, o_out, lse_out, *, tree=False, stream=None) -> None:
    """Two partials in separate buffers (fp32 o [B,S,H,D] with equal strides, lse [B,H,S] contiguous), merged
    as parts 0 (a) and 1 (b): the part strides are the buffers' distance in elements, negative if b lies
    below a."""
    assert o_a.dtype == o_b.dtype == torch.float32 and o_a.shape == o_b.shape and o_a.stride() == o_b.stride()
    assert lse_a.shape == lse_b.shape and lse_a.is_contiguous() and lse_b.is_contiguous()
    do, dl = o_b.data_ptr() - o_a.data_ptr(), lse_b.data_ptr() - lse_a.data_ptr()
    assert do % 4 == 0 and dl % 4 == 0
    B, S, H, D = o_a.shape
    a = MergeArgs()
    a.struct_size = ctypes.sizeof(MergeArgs)
    a.n_parts, a.batch, a.seqlen, a.heads, a.head_dim = 2, B, S, H, D
    a.o_parts, a.o_part_stride = _ptr(o_a), do // 4
    a.o_stride = I64x3(o_a.stride(0), o_a.stride(1), o_a.stride(2))
    a.lse_parts, a.lse_part_stride = _ptr(lse_a), dl // 4
    a.o_out, a.o_out_stride, a.o_out_dtype = _ptr(o_out), _strides3(o_out), _dtype_code(o_out)
    a.lse_out = _ptr(lse_out)
    a.mode = ATTN_MERGE_TREE if tree else ATTN_MERGE_SEQUENTIAL
    _check(load().attn_merge_lse(ctypes.byref(a), _stream(stream)))


def attn_bwd(q, k, v, o, dout, lse, workspace, dq_acc, dk, dv, *, dq=None, q_pos0=0, k_pos0=0, causal=False,
             scale=0.0, compute_delta=False, dq_overwrite=False, finalize_dq=False, balanced=False,
             deterministic=False, stream=None) -> None:
    """Backward for one key chunk; see include/attn.h for the contract."""
    a = BwdArgs()
    a.struct_size = ctypes.sizeof(BwdArgs)
    a.dtype = _dtype_code(q)
    a.batch, a.seqlen_q, a.heads_q, a.head_dim = q.shape
    a.seqlen_k, a.heads_kv = k.shape[1], k.shape[2]
    a.q, a.q_stride = _ptr(q), _strides3(q)
    a.k, a.k_stride = _ptr(k), _strides3(k)
    a.v, a.v_stride = _ptr(v), _strides3(v)
    a.o, a.o_stride = _ptr(o), _strides3(o)
    a.dout, a.do_stride = _ptr(dout), _strides3(dout)
    a.lse, a.dq_acc = _ptr(lse), _ptr(dq_acc)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.dq, a.dq_stride = _ptr(dq), _strides3(dq)
    a.dk, a.dk_stride = _ptr(dk), _strides3(dk)
    a.dv, a.dv_stride = _ptr(dv), _strides3(dv)
    a.q_pos0, a.k_pos0 = int(q_pos0), int(k_pos0)
    a.causal = int(bool(causal))
    a.scale = float(scale)
    a.flags = ((ATTN_BWD_COMPUTE_DELTA if compute_delta else 0) | (ATTN_BWD_DQ_OVERWRITE if dq_overwrite else 0)
               | (ATTN_BWD_FINALIZE_DQ if finalize_dq else 0) | (ATTN_BWD_BALANCED if balanced else 0)
               | (ATTN_BWD_DETERMINISTIC if deterministic else 0))
    _check(load().attn_bwd(ctypes.byref(a), _stream(stream)))


def _chunk_strides(ts, what):
    """Shared (batch, seq, head) strides of the non-empty chunks, and a host array of per-chunk batch strides."""
    n = len(ts)
    live = [x for x in ts if x.shape[1] > 0]
    st = _strides3(live[0]) if live else I64x3(0, 0, 0)
    for x in live:
        assert tuple(x.stride()[1:3]) == tuple(st)[1:], f"{what} chunks must share sequence and head strides"
    bs = (c_i64 * max(n, 1))(*[x.stride(0) if x.numel() else 0 for x in ts])
    return st, bs


def attn_bwd_chunks(q, k_chunks, v_chunks, o, dout, lse, workspace, dq_acc, dk_chunks, dv_chunks, *,
                    chunk_pos0, dq=None, q_pos0=0, causal=False, scale=0.0, compute_delta=False,
                    dq_overwrite=False, finalize_dq=False, balanced=False, deterministic=False,
                    stream=None) -> None:
    """Backward of q over a list of key/value chunks ([B, len_c, Hkv, D] bf16 each), dK/dV per chunk; see include/attn.h."""
    n = len(k_chunks)
    assert len(v_chunks) == n and len(dk_chunks) == n and len(dv_chunks) == n and len(chunk_pos0) == n
    for k, v, dk, dv in zip(k_chunks, v_chunks, dk_chunks, dv_chunks):
        assert k.shape == v.shape == dk.shape == dv.shape, "chunk tensors and their gradients must match in shape"
    a = BwdChunksArgs()
    a.struct_size = ctypes.sizeof(BwdChunksArgs)
    a.dtype = _dtype_code(q)
    a.batch, a.seqlen_q, a.heads_q, a.head_dim = q.shape
    a.heads_kv = k_chunks[0].shape[2] if n else q.shape[2]
    a.n_chunks = n
    a.q, a.q_stride = _ptr(q), _strides3(q)
    a.o, a.o_stride = _ptr(o), _strides3(o)
    a.dout, a.do_stride = _ptr(dout), _strides3(dout)
    a.lse, a.dq_acc = _ptr(lse), _ptr(dq_acc)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.dq, a.dq_stride = _ptr(dq), _strides3(dq)
    arr = lambda ts: (c_vp * max(n, 1))(*[_ptr(x) for x in ts])  # noqa: E731
    a.k_chunks, a.v_chunks, a.dk_chunks, a.dv_chunks = arr(k_chunks), arr(v_chunks), arr(dk_chunks), arr(dv_chunks)
    a.chunk_len = (c_i32 * max(n, 1))(*[k.shape[1] for k in k_chunks])
    a.chunk_pos0 = (c_i64 * max(n, 1))(*[int(x) for x in chunk_pos0])
    a.k_stride, a.chunk_k_bstride = _chunk_strides(k_chunks, "key")
    a.v_stride, a.chunk_v_bstride = _chunk_strides(v_chunks, "value")
    a.dk_stride, a.chunk_dk_bstride = _chunk_strides(dk_chunks, "dk")
    a.dv_stride, a.chunk_dv_bstride = _chunk_strides(dv_chunks, "dv")
    a.q_pos0 = int(q_pos0)
    a.causal = int(bool(causal))
    a.scale = float(scale)
    a.flags = ((ATTN_BWD_COMPUTE_DELTA if compute_delta else 0) | (ATTN_BWD_DQ_OVERWRITE if dq_overwrite else 0)
               | (ATTN_BWD_FINALIZE_DQ if finalize_dq else 0) | (ATTN_BWD_BALANCED if balanced else 0)
               | (ATTN_BWD_DETERMINISTIC if deterministic else 0))
    _check(load().attn_bwd_chunks(ctypes.byref(a), _stream(stream)))


def _packed3(t):
    """Element strides (batch, seq, head) of a packed [total, heads, dim] tensor; the batch stride is unused."""
    if t is None:
        return I64x3(0, 0, 0)
    assert t.dim() == 3 and t.stride(2) == 1
    return I64x3(0, t.stride(0), t.stride(1))


def _check_offsets(cu, name):
    assert cu.dtype == torch.int32 and cu.dim() == 1 and cu.is_contiguous() and cu.is_cuda, \
        f"{name} must be a contiguous int32 device tensor of batch + 1 offsets"


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
                    scale=0.0, accumulate=False, balanced=False, o_final=None, stream=None) -> None:
    """Packed variable-length batch: q, o [total_q, Hq, D], k, v [total_k, Hkv, D], lse fp32 [total_q, Hq]."""
    _check_offsets(cu_seqlens_q, "cu_seqlens_q")
    _check_offsets(cu_seqlens_k, "cu_seqlens_k")
    a = FwdArgs()
    a.struct_size = ctypes.sizeof(FwdArgs)
    a.dtype = _dtype_code(q)
    a.batch = cu_seqlens_q.numel() - 1
    _, a.heads_q, a.head_dim = q.shape
    a.heads_kv = k.shape[1]
    a.seqlen_q, a.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    a.q, a.q_stride = _ptr(q), _packed3(q)
    a.k, a.k_stride = _ptr(k), _packed3(k)
    a.v, a.v_stride = _ptr(v), _packed3(v)
    a.o, a.o_stride, a.o_dtype = _ptr(o), _packed3(o), _dtype_code(o)
    a.lse = _ptr(lse)
    a.o_final, a.o_final_stride = _ptr(o_final), _packed3(o_final)
    a.causal = int(bool(causal))
    a.scale = float(scale)
    a.flags = (ATTN_FWD_ACCUMULATE if accumulate else 0) | (ATTN_FWD_BALANCED if balanced else 0)
    a.cu_seqlens_q, a.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    _check(load().attn_fwd_partial(ctypes.byref(a), _stream(stream)))


def attn_bwd_varlen(q, k, v, o, dout, lse, workspace, dq_acc, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, *, dq=None, causal=False, scale=0.0, compute_delta=False, dq_overwrite=False,
                    finalize_dq=False, balanced=False, deterministic=False, stream=None) -> None:
    """Packed variable-length batch backward; layouts as attn_fwd_varlen, dq_acc fp32 [total_q, Hq, D]."""
    _check_offsets(cu_seqlens_q, "cu_seqlens_q")
    _check_offsets(cu_seqlens_k, "cu_seqlens_k")
    a = BwdArgs()
    a.struct_size = ctypes.sizeof(BwdArgs)
    a.dtype = _dtype_code(q)
    a.batch = cu_seqlens_q.numel() - 1
    _, a.heads_q, a.head_dim = q.shape
    a.heads_kv = k.shape[1]
    a.seqlen_q, a.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    a.q, a.q_stride = _ptr(q), _packed3(q)
    a.k, a.k_stride = _ptr(k), _packed3(k)
    a.v, a.v_stride = _ptr(v), _packed3(v)
    a.o, a.o_stride = _ptr(o), _packed3(o)
    a.dout, a.do_stride = _ptr(dout), _packed3(dout)
    a.lse, a.dq_acc = _ptr(lse), _ptr(dq_acc)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.dq, a.dq_stride = _ptr(dq), _packed3(dq)
    a.dk, a.dk_stride = _ptr(dk), _packed3(dk)
    a.dv, a.dv_stride = _ptr(dv), _packed3(dv)
    a.causal = int(bool(causal))
    a.scale = float(scale)
    a.flags = ((ATTN_BWD_COMPUTE_DELTA if compute_delta else 0) | (ATTN_BWD_DQ_OVERWRITE if dq_overwrite else 0)
               | (ATTN_BWD_FINALIZE_DQ if finalize_dq else 0) | (ATTN_BWD_BALANCED if balanced else 0)
               | (ATTN_BWD_DETERMINISTIC if deterministic else 0))
    a.cu_seqlens_q, a.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    _check(load().attn_bwd(ctypes.byref(a), _stream(stream)))


def _decode_args(q, k_cache, v_cache, o, lse, workspace, n_splits, seqlens, scale):
    a = DecodeArgs()
    a.struct_size = ctypes.sizeof(DecodeArgs)
    a.batch, a.heads_q, a.head_dim = q.shape
    a.heads_kv = k_cache.shape[2]
    a.cache_len = k_cache.shape[1]
    assert q.stride(2) == 1 and o.stride(2) == 1
    a.q, a.q_stride = _ptr(q), I64x2(q.stride(0), q.stride(1))
    a.k_cache, a.k_stride = _ptr(k_cache), _strides3(k_cache)
    a.v_cache, a.v_stride = _ptr(v_cache), _strides3(v_cache)
    a.seqlens = _ptr(seqlens)
    a.n_splits = int(n_splits)
    a.scale = float(scale)
    a.o, a.o_stride = _ptr(o), I64x2(o.stride(0), o.stride(1))
    a.lse = _ptr(lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a


def attn_decode_splitkv(q, k_cache, v_cache, o, lse, workspace, *, n_splits, seqlens=None, scale=0.0,
                        stream=None) -> None:
    """q [B,Hq,D] bf16, caches [B,L,Hkv,D] bf16 -> o [B,Hq,D] bf16, lse [B,Hq] fp32."""
    a = _decode_args(q, k_cache, v_cache, o, lse, workspace, n_splits, seqlens, scale)
    _check(load().attn_decode_splitkv(ctypes.byref(a), _stream(stream)))


def attn_decode_splitkv_noalloc(q, k_cache, v_cache, o, lse, *, n_splits, seqlens=None, scale=0.0,
                                stream=None) -> None:
    """As attn_decode_splitkv, with the split partials in the library's fixed per-device scratch (no workspace)."""
    a = _decode_args(q, k_cache, v_cache, o, lse, None, n_splits, seqlens, scale)
    _check(load().attn_decode_splitkv_noalloc(ctypes.byref(a), _stream(stream)))
