"""The C ABI on the host, without a GPU: the library loads, exports every symbol
include/attn.h declares, agrees with the ctypes binding on struct layouts, and
rejects every invalid argument before enqueueing anything.

Every call here fails validation or has nothing to do (no compute call is made):
pointers are fake, 16-byte aligned addresses that validation never dereferences.
"""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from exact_blockwise_attention_attn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
FAKE = 0x7F0000000000  # aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return B.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ATTN_API\s+[\w\s\*]+?\b(attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) == 14, names
    assert sorted(B.EXPORTED) == names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    # Internal kernels and launchers stay hidden.
    out = subprocess.run(["nm", "-D", "--defined-only", B.lib_path()], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert not any("launch_" in s for s in exported), "internal launchers are exported"


def test_struct_layouts_match_c():
    prog = r"""
#include <stdio.h>
#include <stddef.h>
#include "attn.h"
#define P(T, F) printf(#T "." #F " %zu\n", offsetof(T, F))
int main(void) {
  printf("fwd %zu\nmerge %zu\nbwd %zu\ndecode %zu\nchunks %zu\nbwdchunks %zu\n", sizeof(attn_fwd_args),
         sizeof(attn_merge_args), sizeof(attn_bwd_args), sizeof(attn_decode_args), sizeof(attn_fwd_chunks_args),
         sizeof(attn_bwd_chunks_args));
  P(attn_bwd_chunks_args, q); P(attn_bwd_chunks_args, dq_acc); P(attn_bwd_chunks_args, dq_stride);
  P(attn_bwd_chunks_args, k_chunks); P(attn_bwd_chunks_args, dv_chunks); P(attn_bwd_chunks_args, chunk_pos0);
  P(attn_bwd_chunks_args, dv_stride); P(attn_bwd_chunks_args, chunk_dv_bstride); P(attn_bwd_chunks_args, q_pos0);
  P(attn_bwd_chunks_args, flags);
  P(attn_fwd_chunks_args, k_chunks); P(attn_fwd_chunks_args, chunk_pos0); P(attn_fwd_chunks_args, v_stride);
  P(attn_fwd_chunks_args, o_final_stride); P(attn_fwd_chunks_args, q_pos0); P(attn_fwd_chunks_args, flags);
  P(attn_fwd_chunks_args, chunk_v_bstride); P(attn_fwd_chunks_args, o);
  P(attn_fwd_args, flags); P(attn_fwd_args, o_final_stride); P(attn_fwd_args, q_pos0);
  P(attn_fwd_args, cu_seqlens_q); P(attn_fwd_args, cu_seqlens_k);
  P(attn_bwd_args, cu_seqlens_q); P(attn_bwd_args, cu_seqlens_k);
  printf("tree %zu\n", sizeof(attn_decode_tree_args));
  P(attn_decode_tree_args, cache_len); P(attn_decode_tree_args, kv_start); P(attn_decode_tree_args, q_end);
  P(attn_decode_tree_args, scale); P(attn_decode_tree_args, o_stride); P(attn_decode_tree_args, workspace_bytes);
  P(attn_merge_args, mode); P(attn_merge_args, lse_out);
  P(attn_bwd_args, flags); P(attn_bwd_args, dv_stride); P(attn_bwd_args, dq_acc);
  P(attn_bwd_args, workspace); P(attn_bwd_args, workspace_bytes);
  P(attn_decode_args, workspace_bytes); P(attn_decode_args, n_splits); P(attn_decode_args, o_stride);
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "s.c"), os.path.join(d, "s")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(l.rsplit(" ", 1) for l in out.strip().splitlines())
    assert int(got["fwd"]) == ctypes.sizeof(B.FwdArgs)
    assert int(got["merge"]) == ctypes.sizeof(B.MergeArgs)
    assert int(got["bwd"]) == ctypes.sizeof(B.BwdArgs)
    assert int(got["decode"]) == ctypes.sizeof(B.DecodeArgs)
    assert int(got["chunks"]) == ctypes.sizeof(B.FwdChunksArgs)
    assert int(got["bwdchunks"]) == ctypes.sizeof(B.BwdChunksArgs)
    assert int(got["tree"]) == ctypes.sizeof(B.DecodeTreeArgs)
    cls = {"attn_fwd_args": B.FwdArgs, "attn_merge_args": B.MergeArgs, "attn_bwd_args": B.BwdArgs,
           "attn_decode_args": B.DecodeArgs, "attn_fwd_chunks_args": B.FwdChunksArgs,
           "attn_bwd_chunks_args": B.BwdChunksArgs, "attn_decode_tree_args": B.DecodeTreeArgs}
    for key, val in got.items():
        if "." in key:
            t, f = key.split(".")
            assert getattr(cls[t], f).offset == int(val), key


def test_header_constants_match_binding():
    """Every integer #define of include/attn.h that the binding names has the same value there."""
    text = open(HEADER).read()
    defs = {}
    for m in re.finditer(r"#define (ATTN_[A-Z0-9_]+) +(\(1u << (\d+)\)|(\d+))", text):
        defs[m.group(1)] = (1 << int(m.group(3))) if m.group(3) else int(m.group(4))
    checked = 0
    for name, val in defs.items():
        if hasattr(B, name):
            assert getattr(B, name) == val, name
            checked += 1
    assert "ATTN_BWD_DETERMINISTIC" in defs and checked >= 10, (checked, sorted(defs))


def test_helpers(lib):
    assert lib.attn_abi_version() == 10
    assert lib.attn_status_string(0) == b"ok"
    assert lib.attn_status_string(3) == b"workspace missing or too small"
    assert lib.attn_status_string(5) == b"non-finite output (ATTN_CHECK_FINITE)"
    assert lib.attn_status_string(99) == b"unknown status"
    # O partials [16, 32, 64, 128] fp32 + LSE [16, 32, 64] fp32, each rounded up to 256 bytes.
    # batch x heads_q x (n_splits + 1) rows of head_dim + 1 floats (the stream-K pieces fit in the extra row).
    assert lib.attn_decode_workspace_size(16, 32, 128, 64) == 16 * 32 * 65 * 128 * 4 + 16 * 32 * 65 * 4
    assert lib.attn_decode_workspace_size(1, 1, 96, 4) == 0
    assert lib.attn_decode_workspace_size(1, 1, 128, 0) == 0
    # Backward statistics: 2 floats per row, rows padded to 64, total rounded to 256 bytes.
    assert lib.attn_bwd_workspace_size(2, 32, 32768) == 2 * 32 * 2 * 32768 * 4
    assert lib.attn_bwd_workspace_size(1, 1, 1) == 512
    assert lib.attn_bwd_workspace_size(1, 3, 65) == 3 * 2 * 128 * 4
    assert lib.attn_bwd_workspace_size(1, 1, 0) == 0
    assert lib.attn_bwd_workspace_size(0, 1, 64) == 0
    assert lib.attn_bwd_workspace_size(1, 1, -1) == 0


def fwd_args(**kw):
    a = B.FwdArgs()
    a.struct_size = ctypes.sizeof(B.FwdArgs)
    a.dtype = B.ATTN_DTYPE_BF16
    a.batch, a.heads_q, a.heads_kv, a.seqlen_q, a.seqlen_k, a.head_dim = 1, 4, 2, 64, 64, 128
    for name in ("q", "k", "v", "o", "lse"):
        setattr(a, name, FAKE)
    st = B.I64x3(64 * 4 * 128, 4 * 128, 128)
    a.q_stride, a.o_stride = st, st
    a.k_stride = a.v_stride = B.I64x3(64 * 2 * 128, 2 * 128, 128)
    a.o_dtype = B.ATTN_DTYPE_F32
    a.o_stride = B.I64x3(64 * 4 * 128, 4 * 128, 128)
    for key, val in kw.items():
        setattr(a, key, val)
    return a


FWD_BAD = [
    (dict(struct_size=8), B.ATTN_ERR_INVALID_ARG, "struct_size"),
    (dict(head_dim=96), B.ATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(heads_kv=3), B.ATTN_ERR_INVALID_ARG, "multiple"),
    (dict(seqlen_q=-1), B.ATTN_ERR_INVALID_ARG, "sequence"),
    (dict(batch=0), B.ATTN_ERR_INVALID_ARG, "batch"),
    (dict(dtype=7), B.ATTN_ERR_UNSUPPORTED, "dtype"),
    (dict(q=None), B.ATTN_ERR_INVALID_ARG, "q is NULL"),
    (dict(k=FAKE + 8), B.ATTN_ERR_UNSUPPORTED, "aligned"),
    (dict(q_stride=B.I64x3(1, 4 * 128, 128)), B.ATTN_ERR_UNSUPPORTED, "alignment"),
    (dict(v_stride=B.I64x3(-256, 256, 128)), B.ATTN_ERR_INVALID_ARG, "negative"),
    (dict(lse=None), B.ATTN_ERR_INVALID_ARG, "lse"),
    (dict(scale=-1.0), B.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), B.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(flags=1 << 5), B.ATTN_ERR_INVALID_ARG, "flag"),
    (dict(flags=B.ATTN_FWD_ACCUMULATE, o_dtype=B.ATTN_DTYPE_BF16), B.ATTN_ERR_INVALID_ARG, "ACCUMULATE"),
    (dict(o_final=FAKE + 4), B.ATTN_ERR_UNSUPPORTED, "o_final"),
    (dict(k_stride=B.I64x3(0, (1 << 24) + 64, 128)), B.ATTN_ERR_UNSUPPORTED, "k sequence stride"),
    (dict(v_stride=B.I64x3(0, (1 << 24) + 64, 128)), B.ATTN_ERR_UNSUPPORTED, "v sequence stride"),
    # 1024 heads x 2^21 queries: 2^25 64-row units, but 2^24 workgroups of 256 threads = 2^32 work-items.
    (dict(heads_q=1024, heads_kv=1024, seqlen_q=1 << 21, seqlen_k=1,
          q_stride=B.I64x3(0, 1024 * 128, 128), o_stride=B.I64x3(0, 1024 * 128, 128),
          k_stride=B.I64x3(0, 1024 * 128, 128), v_stride=B.I64x3(0, 1024 * 128, 128)),
     B.ATTN_ERR_UNSUPPORTED, "work-items"),
]


@pytest.mark.parametrize("kw,code,msg", FWD_BAD, ids=[m for _, _, m in FWD_BAD])
def test_fwd_rejects(lib, kw, code, msg):
    a = fwd_args(**kw)
    assert lib.attn_fwd_partial(ctypes.byref(a), None) == code
    assert msg in lib.attn_last_error().decode()


def test_null_args_and_empty(lib):
    for fn in (lib.attn_fwd_partial, lib.attn_merge_lse, lib.attn_bwd, lib.attn_decode_splitkv):
        assert fn(None, None) == B.ATTN_ERR_INVALID_ARG
        assert lib.attn_last_error() == b"args is NULL"
    # No queries: nothing to do, no launch, success (and the error message is cleared).
    a = fwd_args(seqlen_q=0)
    assert lib.attn_fwd_partial(ctypes.byref(a), None) == B.ATTN_OK
    assert lib.attn_last_error() == b""


def merge_args(**kw):
    a = B.MergeArgs()
    a.struct_size = ctypes.sizeof(B.MergeArgs)
    a.n_parts, a.batch, a.seqlen, a.heads, a.head_dim = 4, 1, 16, 2, 64
    a.o_parts, a.lse_parts, a.o_out, a.lse_out = FAKE, FAKE, FAKE, FAKE
    a.o_part_stride, a.lse_part_stride = 16 * 2 * 64, 32
    a.o_stride = a.o_out_stride = B.I64x3(16 * 2 * 64, 2 * 64, 64)
    a.o_out_dtype = B.ATTN_DTYPE_F32
    for key, val in kw.items():
        setattr(a, key, val)
    return a


MERGE_BAD = [
    (dict(n_parts=0), B.ATTN_ERR_INVALID_ARG, "n_parts"),
    (dict(n_parts=2000), B.ATTN_ERR_INVALID_ARG, "n_parts"),
    (dict(mode=5), B.ATTN_ERR_INVALID_ARG, "mode"),
    (dict(head_dim=32), B.ATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(lse_out=None), B.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(o_part_stride=0), B.ATTN_ERR_INVALID_ARG, "part strides"),
    (dict(lse_part_stride=0), B.ATTN_ERR_INVALID_ARG, "part strides"),
    (dict(o_part_stride=-6), B.ATTN_ERR_UNSUPPORTED, "o_part_stride"),
    (dict(o_out_dtype=9), B.ATTN_ERR_UNSUPPORTED, "o_out_dtype"),
    # One thread per 4 features: 2^20 rows x 1024 heads x 32 threads = 2^35 work-items.
    (dict(n_parts=1, seqlen=1 << 20, heads=1024, head_dim=128, o_stride=B.I64x3(0, 1024 * 128, 128),
          o_out_stride=B.I64x3(0, 1024 * 128, 128)), B.ATTN_ERR_UNSUPPORTED, "work-items"),
]


@pytest.mark.parametrize("kw,code,msg", MERGE_BAD, ids=[m for _, _, m in MERGE_BAD])
def test_merge_rejects(lib, kw, code, msg):
    a = merge_args(**kw)
    assert lib.attn_merge_lse(ctypes.byref(a), None) == code
    assert msg in lib.attn_last_error().decode()


def bwd_args(**kw):
    a = B.BwdArgs()
    a.struct_size = ctypes.sizeof(B.BwdArgs)
    a.dtype = B.ATTN_DTYPE_BF16
    a.batch, a.heads_q, a.heads_kv, a.seqlen_q, a.seqlen_k, a.head_dim = 1, 2, 2, 32, 32, 64
    for name in ("q", "k", "v", "o", "dout", "lse", "workspace", "dq_acc", "dq", "dk", "dv"):
        setattr(a, name, FAKE)
    a.workspace_bytes = 2 * 2 * 64 * 4
    st = B.I64x3(32 * 2 * 64, 2 * 64, 64)
    for name in ("q_stride", "k_stride", "v_stride", "o_stride", "do_stride", "dq_stride", "dk_stride", "dv_stride"):
        setattr(a, name, st)
    for key, val in kw.items():
        setattr(a, key, val)
    return a


BWD_BAD = [
    (dict(flags=1 << 9), B.ATTN_ERR_INVALID_ARG, "flag"),
    (dict(dq_acc=None), B.ATTN_ERR_INVALID_ARG, "dq_acc"),
    # The DETERMINISTIC bit passes flag validation: the error is the next one checked.
    (dict(flags=B.ATTN_BWD_DETERMINISTIC, dq_acc=None), B.ATTN_ERR_INVALID_ARG, "dq_acc"),
    (dict(lse=FAKE + 4), B.ATTN_ERR_UNSUPPORTED, "aligned"),
    (dict(workspace=None), B.ATTN_ERR_WORKSPACE, "workspace of 1024 bytes"),
    (dict(workspace_bytes=1023), B.ATTN_ERR_WORKSPACE, "1023 given"),
    (dict(workspace=FAKE + 16), B.ATTN_ERR_WORKSPACE, "256-byte"),
    (dict(dk=None), B.ATTN_ERR_INVALID_ARG, "dk is NULL"),
    (dict(dq=None, flags=B.ATTN_BWD_FINALIZE_DQ), B.ATTN_ERR_INVALID_ARG, "dq is NULL"),
    (dict(o=None, flags=B.ATTN_BWD_COMPUTE_DELTA), B.ATTN_ERR_INVALID_ARG, "o is NULL"),
    (dict(head_dim=256), B.ATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(scale=float("inf")), B.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(k_stride=B.I64x3(0, (1 << 24) + 64, 64)), B.ATTN_ERR_UNSUPPORTED, "k sequence stride"),
    # dK/dV: 2 x 2^24 keys -> 2^17 128-key workgroups x 512 threads = 2^26 per head, x 64 heads = 2^32.
    (dict(heads_q=64, heads_kv=64, seqlen_q=64, seqlen_k=1 << 24, workspace_bytes=1 << 20,
          k_stride=B.I64x3(0, 64 * 64, 64), v_stride=B.I64x3(0, 64 * 64, 64), dk_stride=B.I64x3(0, 64 * 64, 64),
          dv_stride=B.I64x3(0, 64 * 64, 64)),
     B.ATTN_ERR_UNSUPPORTED, "work-items"),
]


@pytest.mark.parametrize("kw,code,msg", BWD_BAD, ids=[m for _, _, m in BWD_BAD])
def test_bwd_rejects(lib, kw, code, msg):
    a = bwd_args(**kw)
    assert lib.attn_bwd(ctypes.byref(a), None) == code
    assert msg in lib.attn_last_error().decode()


def chunks_args(n=2, lens=(64, 0), **kw):
    a = B.FwdChunksArgs()
    a.struct_size = ctypes.sizeof(B.FwdChunksArgs)
    a.dtype = B.ATTN_DTYPE_BF16
    a.batch, a.heads_q, a.heads_kv, a.seqlen_q, a.head_dim = 1, 2, 2, 32, 64
    a.q = a.o = a.lse = FAKE
    a.o_dtype = B.ATTN_DTYPE_F32
    st = B.I64x3(64 * 2 * 64, 2 * 64, 64)
    a.q_stride = a.o_stride = a.k_stride = a.v_stride = st
    a.n_chunks = n
    a._keep = ((ctypes.c_void_p * 2)(FAKE, FAKE), (ctypes.c_void_p * 2)(FAKE, FAKE),
               (ctypes.c_int32 * 2)(*lens), (ctypes.c_int64 * 2)(0, 64))
    a.k_chunks, a.v_chunks, a.chunk_len, a.chunk_pos0 = a._keep
    for key, val in kw.items():
        setattr(a, key, val)
    return a


CHUNKS_BAD = [
    (dict(n_chunks=65), B.ATTN_ERR_INVALID_ARG, "n_chunks"),
    (dict(n_chunks=-1), B.ATTN_ERR_INVALID_ARG, "n_chunks"),
    (dict(dtype=B.ATTN_DTYPE_F32), B.ATTN_ERR_UNSUPPORTED, "bf16 only"),
    (dict(flags=1 << 7), B.ATTN_ERR_INVALID_ARG, "flag"),
    (dict(flags=B.ATTN_FWD_ACCUMULATE, o_dtype=B.ATTN_DTYPE_BF16), B.ATTN_ERR_INVALID_ARG, "fp32 running"),
    (dict(k_chunks=None), B.ATTN_ERR_INVALID_ARG, "chunk arrays"),
    (dict(lse=None), B.ATTN_ERR_INVALID_ARG, "lse is NULL"),
    (dict(k_stride=B.I64x3(64 * 2 * 64, 2 * 64, 3)), B.ATTN_ERR_UNSUPPORTED, "k_chunks[0] stride"),
    (dict(head_dim=96), B.ATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(chunk_k_bstride=(ctypes.c_int64 * 2)(5, 5)), B.ATTN_ERR_UNSUPPORTED, "k_chunks[0] stride[0]"),
    (dict(v_stride=B.I64x3(0, (1 << 24) + 64, 64)), B.ATTN_ERR_UNSUPPORTED, "v_chunks sequence stride"),
]


@pytest.mark.parametrize("kw,code,msg", CHUNKS_BAD, ids=[m for _, _, m in CHUNKS_BAD])
def test_fwd_chunks_rejects(lib, kw, code, msg):
    a = chunks_args(**kw)
    assert lib.attn_fwd_chunks(ctypes.byref(a), None) == code
    assert msg in lib.attn_last_error().decode()


def test_fwd_chunks_rejects_negative_length(lib):
    a = chunks_args(lens=(64, -5))
    assert lib.attn_fwd_chunks(ctypes.byref(a), None) == B.ATTN_ERR_INVALID_ARG
    assert "chunk_len[1]" in lib.attn_last_error().decode()


def test_fwd_chunks_empty_query_is_noop(lib):
    # No query rows: nothing is launched and no pointer is dereferenced.
    a = chunks_args(seqlen_q=0, q=None, o=None, lse=None)
    assert lib.attn_fwd_chunks(ctypes.byref(a), None) == B.ATTN_OK


VARLEN_BAD = [
    (dict(cu_seqlens_k=None), B.ATTN_ERR_INVALID_ARG, "given together"),
    (dict(cu_seqlens_q=FAKE + 2), B.ATTN_ERR_UNSUPPORTED, "4-byte aligned"),
    (dict(q_pos0=5), B.ATTN_ERR_INVALID_ARG, "q_pos0 and k_pos0 must be 0"),
    (dict(dtype=B.ATTN_DTYPE_F32), B.ATTN_ERR_UNSUPPORTED, "bf16 only"),
]


@pytest.mark.parametrize("kw,code,msg", VARLEN_BAD, ids=[m for _, _, m in VARLEN_BAD])
def test_varlen_rejects(lib, kw, code, msg):
    kw = dict(kw)
    kw.setdefault("cu_seqlens_q", FAKE)
    kw.setdefault("cu_seqlens_k", FAKE + 256)
    a = bwd_args(**kw)
    assert lib.attn_bwd(ctypes.byref(a), None) == code
    assert msg in lib.attn_last_error().decode()
    f = B.FwdArgs()
    f.struct_size = ctypes.sizeof(B.FwdArgs)
    f.dtype = kw.get("dtype", B.ATTN_DTYPE_BF16)
    f.batch, f.heads_q, f.heads_kv, f.seqlen_q, f.seqlen_k, f.head_dim = 2, 2, 2, 32, 32, 64
    f.q = f.k = f.v = f.o = f.lse = FAKE
    f.o_dtype = B.ATTN_DTYPE_F32
    st = B.I64x3(0, 2 * 64, 64)
    f.q_stride = f.k_stride = f.v_stride = f.o_stride = st
    f.q_pos0 = kw.get("q_pos0", 0)
    f.cu_seqlens_q, f.cu_seqlens_k = kw["cu_seqlens_q"], kw["cu_seqlens_k"]
    assert lib.attn_fwd_partial(ctypes.byref(f), None) == code
    assert msg in lib.attn_last_error().decode()


def bwd_chunks_args(lens=(64, 0), **kw):
    a = B.BwdChunksArgs()
    a.struct_size = ctypes.sizeof(B.BwdChunksArgs)
    a.dtype = B.ATTN_DTYPE_BF16
    a.batch, a.heads_q, a.heads_kv, a.seqlen_q, a.head_dim = 1, 2, 2, 32, 64
    for name in ("q", "o", "dout", "lse", "workspace", "dq_acc", "dq"):
        setattr(a, name, FAKE)
    a.workspace_bytes = 2 * 2 * 64 * 4
    st = B.I64x3(64 * 2 * 64, 2 * 64, 64)
    for name in ("q_stride", "o_stride", "do_stride", "dq_stride", "k_stride", "v_stride", "dk_stride", "dv_stride"):
        setattr(a, name, st)
    n = len(lens)
    a.n_chunks = n
    ptrs = lambda: (ctypes.c_void_p * n)(*([FAKE] * n))  # noqa: E731
    a._keep = (ptrs(), ptrs(), ptrs(), ptrs(), (ctypes.c_int32 * n)(*lens), (ctypes.c_int64 * n)(*range(0, 64 * n, 64)))
    a.k_chunks, a.v_chunks, a.dk_chunks, a.dv_chunks, a.chunk_len, a.chunk_pos0 = a._keep
    for key, val in kw.items():
        setattr(a, key, val)
    return a


BWD_CHUNKS_BAD = [
    (dict(n_chunks=65), B.ATTN_ERR_INVALID_ARG, "n_chunks"),
    (dict(n_chunks=-1), B.ATTN_ERR_INVALID_ARG, "n_chunks"),
    (dict(dtype=B.ATTN_DTYPE_F32), B.ATTN_ERR_UNSUPPORTED, "bf16 only"),
    (dict(flags=1 << 9), B.ATTN_ERR_INVALID_ARG, "flag"),
    (dict(dq_acc=None), B.ATTN_ERR_INVALID_ARG, "dq_acc"),
    (dict(flags=B.ATTN_BWD_DETERMINISTIC, dq_acc=None), B.ATTN_ERR_INVALID_ARG, "dq_acc"),
    (dict(workspace_bytes=1023), B.ATTN_ERR_WORKSPACE, "1023 given"),
    (dict(workspace=FAKE + 16), B.ATTN_ERR_WORKSPACE, "256-byte"),
    (dict(dq=None, flags=B.ATTN_BWD_FINALIZE_DQ), B.ATTN_ERR_INVALID_ARG, "dq is NULL"),
    (dict(o=None, flags=B.ATTN_BWD_COMPUTE_DELTA), B.ATTN_ERR_INVALID_ARG, "o is NULL"),
    (dict(dv_chunks=None), B.ATTN_ERR_INVALID_ARG, "chunk arrays"),
    (dict(dk_stride=B.I64x3(64 * 2 * 64, 2 * 64, 3)), B.ATTN_ERR_UNSUPPORTED, "dk_chunks[0] stride"),
    (dict(chunk_dv_bstride=(ctypes.c_int64 * 2)(6, 6)), B.ATTN_ERR_UNSUPPORTED, "dv_chunks[0] stride[0]"),
    (dict(k_stride=B.I64x3(0, (1 << 24) + 64, 64)), B.ATTN_ERR_UNSUPPORTED, "k_chunks sequence stride"),
    (dict(head_dim=96), B.ATTN_ERR_UNSUPPORTED, "head_dim"),
]


@pytest.mark.parametrize("kw,code,msg", BWD_CHUNKS_BAD, ids=[m for _, _, m in BWD_CHUNKS_BAD])
def test_bwd_chunks_rejects(lib, kw, code, msg):
    a = bwd_chunks_args(**kw)
    assert lib.attn_bwd_chunks(ctypes.byref(a), None) == code
    assert msg in lib.attn_last_error().decode()


def test_bwd_chunks_rejects_negative_length_and_null_chunk(lib):
    a = bwd_chunks_args(lens=(64, -5))
    assert lib.attn_bwd_chunks(ctypes.byref(a), None) == B.ATTN_ERR_INVALID_ARG
    assert "chunk_len[1]" in lib.attn_last_error().decode()
    a = bwd_chunks_args(lens=(64, 64))
    a.dk_chunks[1] = None
    assert lib.attn_bwd_chunks(ctypes.byref(a), None) == B.ATTN_ERR_INVALID_ARG
    assert "dk_chunks[1] is NULL" in lib.attn_last_error().decode()


def test_bwd_chunks_nothing_to_do(lib):
    # No query rows and no chunk: nothing is launched and no pointer is dereferenced.
    a = bwd_chunks_args(lens=(), seqlen_q=0, q=None, o=None, dout=None, lse=None, dq_acc=None, workspace=None)
    assert lib.attn_bwd_chunks(ctypes.byref(a), None) == B.ATTN_OK


def tree_args(nodes=((0, 100, 0, 3), (100, 50, 1, 3)), **kw):
    """nodes: (kv_start, kv_len, q_begin, q_end) each."""
    a = B.DecodeTreeArgs()
    a.struct_size = ctypes.sizeof(B.DecodeTreeArgs)
    a.n_queries, a.heads_q, a.heads_kv, a.head_dim = 3, 8, 2, 128
    a.cache_len = 200
    a.q = a.k_cache = a.v_cache = a.o = a.lse = a.workspace = FAKE
    a.q_stride = a.o_stride = B.I64x2(8 * 128, 128)
    a.k_stride = a.v_stride = B.I64x2(2 * 128, 128)
    n = len(nodes)
    a.n_nodes = n
    a._keep = ((ctypes.c_int64 * max(n, 1))(*[x[0] for x in nodes]), (ctypes.c_int32 * max(n, 1))(*[x[1] for x in nodes]),
               (ctypes.c_int32 * max(n, 1))(*[x[2] for x in nodes]), (ctypes.c_int32 * max(n, 1))(*[x[3] for x in nodes]))
    a.kv_start, a.kv_len, a.q_begin, a.q_end = a._keep
    a.workspace_bytes = 1 << 20
    for key, val in kw.items():
        setattr(a, key, val)
    return a


TREE_BAD = [
    (dict(n_nodes=257), B.ATTN_ERR_INVALID_ARG, "n_nodes"),
    (dict(cache_len=120), B.ATTN_ERR_INVALID_ARG, "node 1: keys [100, 150) outside the cache of 120"),
    (dict(n_queries=2), B.ATTN_ERR_INVALID_ARG, "node 0: queries [0, 3) outside [0, 2)"),
    (dict(workspace_bytes=100), B.ATTN_ERR_WORKSPACE, "workspace of"),
    (dict(head_dim=80), B.ATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(lse=None), B.ATTN_ERR_INVALID_ARG, "lse is NULL"),
    (dict(kv_len=None), B.ATTN_ERR_INVALID_ARG, "node arrays"),
    (dict(k_stride=B.I64x2((1 << 24) + 64, 128)), B.ATTN_ERR_UNSUPPORTED, "k_cache sequence stride"),
]


@pytest.mark.parametrize("kw,code,msg", TREE_BAD, ids=[m for _, _, m in TREE_BAD])
def test_decode_tree_rejects(lib, kw, code, msg):
    a = tree_args(**kw)
    assert lib.attn_decode_tree(ctypes.byref(a), None) == code
    assert msg in lib.attn_last_error().decode()


def test_decode_tree_workspace_size(lib):
    # Two nodes of 100 and 50 keys (one segment each) over 3 and 2 queries: 5 entries x 8 heads x 128
    # fp32 partial rows, then their LSE, each part rounded up to 256 bytes.
    assert lib.attn_decode_tree_workspace_size(ctypes.byref(tree_args())) == 5 * 8 * 128 * 4 + 256
    # A node of 5000 keys is cut into segments of 2048 keys: 3 entries per query it covers.
    a = tree_args(nodes=((0, 5000, 0, 2),), cache_len=5000)
    assert lib.attn_decode_tree_workspace_size(ctypes.byref(a)) == 6 * 8 * 128 * 4 + 256
    # Invalid node lists give 0 and leave the last error alone.
    lib.attn_decode_tree(None, None)
    before = lib.attn_last_error()
    assert lib.attn_decode_tree_workspace_size(ctypes.byref(tree_args(cache_len=10))) == 0
    assert lib.attn_last_error() == before
    a = tree_args(workspace_bytes=lib.attn_decode_tree_workspace_size(ctypes.byref(tree_args())) - 1)
    assert lib.attn_decode_tree(ctypes.byref(a), None) == B.ATTN_ERR_WORKSPACE


def test_decode_tree_segments_fit_the_table(lib):
    # 200 nodes of 8192 keys would be 800 segments of 2048: the segment length doubles until the
    # segments fit the 256-entry table (here 8192 keys: one segment per node, 200 entries).
    nodes = tuple((0, 8192, 0, 1) for _ in range(200))
    a = tree_args(nodes=nodes, cache_len=8192, n_queries=1)
    assert lib.attn_decode_tree_workspace_size(ctypes.byref(a)) == 200 * 8 * 128 * 4 + 256 * ((200 * 8 * 4 + 255) // 256)


def decode_args(**kw):
    a = B.DecodeArgs()
    a.struct_size = ctypes.sizeof(B.DecodeArgs)
    a.batch, a.heads_q, a.heads_kv, a.head_dim, a.cache_len = 2, 8, 2, 128, 1000
    a.q, a.k_cache, a.v_cache, a.o, a.lse, a.workspace = FAKE, FAKE, FAKE, FAKE, FAKE, FAKE
    a.q_stride = a.o_stride = B.I64x2(8 * 128, 128)
    a.k_stride = a.v_stride = B.I64x3(1000 * 2 * 128, 2 * 128, 128)
    a.n_splits = 8
    a.workspace_bytes = 1 << 20
    for key, val in kw.items():
        setattr(a, key, val)
    return a


DECODE_BAD = [
    (dict(workspace_bytes=100), B.ATTN_ERR_WORKSPACE, "workspace"),
    (dict(workspace=None), B.ATTN_ERR_WORKSPACE, "workspace"),
    (dict(workspace=FAKE + 16), B.ATTN_ERR_WORKSPACE, "256-byte"),
    (dict(n_splits=0), B.ATTN_ERR_INVALID_ARG, "n_splits"),
    (dict(heads_kv=3), B.ATTN_ERR_INVALID_ARG, "multiple"),
    (dict(cache_len=-5), B.ATTN_ERR_INVALID_ARG, "cache_len"),
    (dict(seqlens=FAKE + 2), B.ATTN_ERR_UNSUPPORTED, "seqlens"),
    (dict(k_stride=B.I64x3(1000 * 2 * 128, 2 * 128 + 1, 128)), B.ATTN_ERR_UNSUPPORTED, "alignment"),
    (dict(lse=None), B.ATTN_ERR_INVALID_ARG, "lse"),
    # 2^14 sequences x 2 key/value heads x 1024 splits = 2^25 workgroups of 256 threads.
    (dict(batch=1 << 14, n_splits=1024, workspace_bytes=1 << 40), B.ATTN_ERR_UNSUPPORTED, "work-items"),
]


@pytest.mark.parametrize("kw,code,msg", DECODE_BAD, ids=[m for _, _, m in DECODE_BAD])
def test_decode_rejects(lib, kw, code, msg):
    a = decode_args(**kw)
    assert lib.attn_decode_splitkv(ctypes.byref(a), None) == code
    assert msg in lib.attn_last_error().decode()


def test_decode_noalloc_rejects(lib):
    # Same validation as the workspace form; the workspace fields are ignored.
    a = decode_args(n_splits=0, workspace=None, workspace_bytes=0)
    assert lib.attn_decode_splitkv_noalloc(ctypes.byref(a), None) == B.ATTN_ERR_INVALID_ARG
    assert "n_splits" in lib.attn_last_error().decode()
    # 16 x 32 heads x 128 splits x (128 + 1) x 4 bytes is just over the fixed 32 MiB scratch.
    need = lib.attn_decode_workspace_size(16, 32, 128, 128)
    assert need > 32 << 20
    a = decode_args(batch=16, heads_q=32, heads_kv=8, n_splits=128, workspace=None, workspace_bytes=0)
    assert lib.attn_decode_splitkv_noalloc(ctypes.byref(a), None) == B.ATTN_ERR_WORKSPACE
    msg = lib.attn_last_error().decode()
    assert "fixed scratch of 33554432 bytes" in msg and str(need) in msg


def test_last_error_is_thread_local(lib):
    import threading

    a = fwd_args(head_dim=96)
    assert lib.attn_fwd_partial(ctypes.byref(a), None) == B.ATTN_ERR_UNSUPPORTED
    seen = []
    t = threading.Thread(target=lambda: seen.append(lib.attn_last_error()))
    t.start()
    t.join()
    assert seen == [b""]
    assert b"head_dim" in lib.attn_last_error()


def test_debug_sync_keeps_host_validation(lib, monkeypatch):
    """With ATTN_DEBUG_SYNC set, invalid calls are still rejected on the host, before anything is
    enqueued or synchronised (the fake pointers are never touched)."""
    monkeypatch.setenv("ATTN_DEBUG_SYNC", "1")
    a = bwd_args(dq_acc=None)
    assert lib.attn_bwd(ctypes.byref(a), None) == B.ATTN_ERR_INVALID_ARG
    assert "dq_acc" in lib.attn_last_error().decode()


def test_library_override(monkeypatch):
    """ATTN_LIBRARY names the library the binding loads (the host-ASan build, say); unset, the in-tree one."""
    monkeypatch.delenv("ATTN_LIBRARY", raising=False)
    assert B.lib_path().endswith(os.path.join("exact_blockwise_attention_attn_amd", "libattn.so"))
    monkeypatch.setenv("ATTN_LIBRARY", "/some/other/libattn.so")
    assert B.lib_path() == "/some/other/libattn.so"


def test_log_only_on_enqueue(lib, monkeypatch, capfd):
    """ATTN_LOG logs calls that enqueue work; a call rejected on the host logs nothing."""
    monkeypatch.setenv("ATTN_LOG", "1")
    a = bwd_args(dq_acc=None)
    assert lib.attn_bwd(ctypes.byref(a), None) == B.ATTN_ERR_INVALID_ARG
    assert "[attn]" not in capfd.readouterr().err


def test_check_finite_keeps_host_validation(lib, monkeypatch):
    """With ATTN_CHECK_FINITE set, invalid calls are still rejected on the host before any scan (the fake
    pointers are never touched)."""
    monkeypatch.setenv("ATTN_CHECK_FINITE", "1")
    a = bwd_args(dq_acc=None)
    assert lib.attn_bwd(ctypes.byref(a), None) == B.ATTN_ERR_INVALID_ARG
    assert "dq_acc" in lib.attn_last_error().decode()
