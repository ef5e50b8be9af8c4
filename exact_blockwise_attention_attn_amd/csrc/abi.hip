// C ABI of libattn: argument validation on the host, then dispatch to the
// kernels.  Validation makes no HIP call, so a failing call enqueues nothing
// and touches no output, on any machine.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ATTN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// With the environment variable ATTN_LOG set (to anything but "0"), every
// compute call that enqueues work writes one line to stderr naming the call
// and its sizes.  Read on every call.
void log_call(const char* fmt, ...) {
  const char* v = getenv("ATTN_LOG");
  if (!v || !*v || strcmp(v, "0") == 0) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[attn] %s\n", buf);
}

bool env_on(const char* name) {
  const char* v = getenv(name);
  return v && *v && strcmp(v, "0") != 0;
}

// The outputs a compute call writes, for the non-finite scan (collected only
// while ATTN_CHECK_FINITE is set).  Each is up to four dimensions with element
// strides; an error message names dimensions first .. first + nd - 1 with
// `label`.  A packed variable-length tensor takes its row count (dimension 1)
// from cu[batch] on the device.
struct Outputs {
  bool on = env_on("ATTN_CHECK_FINITE");
  int n = 0;
  char name[attn::kMaxFiniteViews][24];
  const char* label[attn::kMaxFiniteViews];
  int first[attn::kMaxFiniteViews], nd[attn::kMaxFiniteViews];
  const int32_t* cu[attn::kMaxFiniteViews];
  int cu_batch[attn::kMaxFiniteViews];
  attn::FiniteView v[attn::kMaxFiniteViews];

  void add(const char* nm, const char* lab, int first_dim, int n_dims, const void* p, bool f32,
           const int64_t (&dims)[4], const int64_t (&st)[4], bool neg_inf_ok, const int32_t* cu_rows = nullptr,
           int batch = 0) {
    if (!on || n >= attn::kMaxFiniteViews || !p) return;
    snprintf(name[n], sizeof name[n], "%s", nm);
    label[n] = lab;
    first[n] = first_dim;
    nd[n] = n_dims;
    cu[n] = cu_rows;
    cu_batch[n] = batch;
    attn::FiniteView& f = v[n++];
    f.ptr = p;
    for (int k = 0; k < 4; ++k) f.n[k] = dims[k], f.st[k] = st[k];
    f.f32 = f32;
    f.allow_neg_inf = neg_inf_ok;
  }
  // A [batch, seq, heads, head_dim] tensor with three element strides; packed
  // (cu_rows != NULL): [rows, heads, head_dim], batch stride ignored.
  void bshd(const char* nm, const void* p, uint32_t dtype, int64_t b, int64_t sq, int64_t h, int64_t d,
            const int64_t* st, const int32_t* cu_rows = nullptr) {
    if (cu_rows)
      add(nm, "(row, head, dim)", 1, 3, p, dtype == ATTN_DTYPE_F32, {1, 0, h, d}, {0, st[1], st[2], 1}, false,
          cu_rows, (int)b);
    else
      add(nm, "(batch, seq, head, dim)", 0, 4, p, dtype == ATTN_DTYPE_F32, {b, sq, h, d}, {st[0], st[1], st[2], 1},
          false);
  }
  // LSE, contiguous [batch, heads, seq] fp32 (packed: [rows, heads]); -inf is allowed.
  void lse(const float* p, int64_t b, int64_t h, int64_t sq, const int32_t* cu_rows = nullptr) {
    if (cu_rows)
      add("lse", "(row, head)", 1, 2, p, true, {1, 0, h, 1}, {0, h, 1, 0}, true, cu_rows, (int)b);
    else
      add("lse", "(batch, head, seq)", 0, 3, p, true, {b, h, sq, 1}, {h * sq, sq, 1, 0}, true);
  }
  // A decode output o [rows, heads, head_dim] (strides o_st) and lse [rows, heads].
  void decode(const char* rows_name, const void* o, const int64_t* o_st, const float* l, int64_t rows, int64_t h,
              int64_t d) {
    const bool q = rows_name[0] == 'q';
    add("o", q ? "(query, head, dim)" : "(batch, head, dim)", 1, 3, o, false, {1, rows, h, d},
        {0, o_st[0], o_st[1], 1}, false);
    add("lse", q ? "(query, head)" : "(batch, head)", 1, 2, l, true, {1, rows, h, 1}, {0, h, 1, 0}, true);
  }
};

// Success of a compute call: its work is enqueued on `stream`.
//  - With the environment variable ATTN_DEBUG_SYNC set (to anything but "0"),
//    the call first waits for the stream, so a failure of its kernels is
//    reported here, by the call that caused it, instead of at the caller's
//    next synchronisation.
//  - With ATTN_CHECK_FINITE set (likewise), the call scans the outputs it wrote
//    after its kernels, waits, and returns ATTN_ERR_NONFINITE naming the first
//    NaN or infinity it finds (an LSE of -inf is a row with no visible key and
//    is allowed).  A running result read with ATTN_FWD_ACCUMULATE is scanned
//    as part of the output it becomes.
// Both are read on every call.
int enqueued(void* stream, const char* call, const Outputs* outs = nullptr) {
  hipStream_t s = (hipStream_t)stream;
  if (env_on("ATTN_DEBUG_SYNC")) {
    const hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s (ATTN_DEBUG_SYNC): HIP error %d (%s)", call, (int)e,
                                     hipGetErrorString(e));
  }
  if (outs && outs->on && outs->n > 0) {
    attn::FiniteView v[attn::kMaxFiniteViews];
    int64_t first[attn::kMaxFiniteViews];
    for (int i = 0; i < outs->n; ++i) {
      v[i] = outs->v[i];
      if (outs->cu[i]) {
        int32_t rows = 0;
        hipError_t e = hipMemcpyAsync(&rows, outs->cu[i] + outs->cu_batch[i], sizeof rows, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s (ATTN_CHECK_FINITE): HIP error %d (%s)", call, (int)e,
                                         hipGetErrorString(e));
        v[i].n[1] = rows > 0 ? rows : 0;
      }
    }
    const hipError_t e = attn::finite_scan(v, outs->n, s, first);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s (ATTN_CHECK_FINITE): HIP error %d (%s)", call, (int)e,
                                     hipGetErrorString(e));
    for (int i = 0; i < outs->n; ++i) {
      if (first[i] < 0) continue;
      int64_t idx[4], r = first[i];
      for (int k = 3; k >= 0; --k) idx[k] = r % v[i].n[k], r /= v[i].n[k];
      char at[96];
      int len = snprintf(at, sizeof at, "(");
      for (int k = 0; k < outs->nd[i]; ++k)
        len += snprintf(at + len, sizeof at - len, k ? ", %lld" : "%lld", (long long)idx[outs->first[i] + k]);
      snprintf(at + len, sizeof at - len, ")");
      return fail(ATTN_ERR_NONFINITE, "%s: non-finite value in %s at %s = %s", call, outs->name[i], outs->label[i], at);
    }
  }
  return ok();
}

size_t elem_size(uint32_t dtype) { return dtype == ATTN_DTYPE_F32 ? 4 : 2; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A [batch, seq, head, dim] view: pointer and strides must keep every row 16-byte aligned.
int check_view(const char* name, const void* p, const int64_t* st, int n_st, uint32_t dtype, bool needed) {
  if (!needed) return ATTN_OK;
  if (!p) return fail(ATTN_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(ATTN_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
  for (int i = 0; i < n_st; ++i) {
    if (st[i] < 0) return fail(ATTN_ERR_INVALID_ARG, "%s stride[%d] = %lld is negative", name, i, (long long)st[i]);
    if ((st[i] * (int64_t)elem_size(dtype)) % 16)
      return fail(ATTN_ERR_UNSUPPORTED, "%s stride[%d] = %lld breaks 16-byte row alignment", name, i,
                  (long long)st[i]);
  }
  return ATTN_OK;
}

// Key and value tiles are fetched as a wave-uniform row base plus a 32-bit
// per-lane offset spanning 64 rows, so a key/value sequence stride may not
// exceed 2^24 elements (a row stride of 32 MiB; [B, S, H, d] layouts have H * d).
constexpr int64_t kMaxSeqStride = int64_t{1} << 24;
int check_seq_stride(const char* name, int64_t ss, bool needed) {
  if (needed && ss > kMaxSeqStride)
    return fail(ATTN_ERR_UNSUPPORTED, "%s sequence stride %lld exceeds 2^24 elements", name, (long long)ss);
  return ATTN_OK;
}

// Every launch of a call must fit the 2^32 - 1 work-items a grid dimension
// allows; checked for all of a call's launches before the first is enqueued.
int check_items(int64_t items, const char* what) {
  if (items > (int64_t)0xffffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: problem too large for one launch (%lld work-items > 2^32 - 1)", what,
                (long long)items);
  return ATTN_OK;
}

int check_scale(float in, int head_dim, float* out) {
  if (in == 0.0f) {
    *out = 1.0f / sqrtf((float)head_dim);
    return ATTN_OK;
  }
  if (!isfinite(in) || in < 0.0f)
    return fail(ATTN_ERR_INVALID_ARG, "scale must be 0 (default) or finite and positive, got %g", (double)in);
  *out = in;
  return ATTN_OK;
}

int check_dims(int32_t batch, int32_t hq, int32_t hkv, int32_t sq, int32_t sk, int32_t d) {
  if (batch < 1 || hq < 1 || hkv < 1) return fail(ATTN_ERR_INVALID_ARG, "batch and head counts must be >= 1");
  if (sq < 0 || sk < 0) return fail(ATTN_ERR_INVALID_ARG, "sequence lengths must be >= 0");
  if (hq % hkv) return fail(ATTN_ERR_INVALID_ARG, "heads_q (%d) is not a multiple of heads_kv (%d)", hq, hkv);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", d);
  return ATTN_OK;
}

// Packed variable-length mode: both offset arrays or neither, 4-byte aligned,
// bf16, positions zero.
int check_varlen(const int32_t* cu_q, const int32_t* cu_k, uint32_t dtype, int64_t q_pos0, int64_t k_pos0,
                 bool* varlen) {
  *varlen = cu_q || cu_k;
  if (!*varlen) return ATTN_OK;
  if (!cu_q || !cu_k) return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be given together");
  if (((uintptr_t)cu_q | (uintptr_t)cu_k) & 3u) return fail(ATTN_ERR_UNSUPPORTED, "cu_seqlens are not 4-byte aligned");
  if (dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED, "variable-length batches are bf16 only");
  if (q_pos0 != 0 || k_pos0 != 0)
    return fail(ATTN_ERR_INVALID_ARG, "variable-length batches take their positions from the lengths: "
                                      "q_pos0 and k_pos0 must be 0");
  return ATTN_OK;
}

#define TRY(x)              \
  do {                      \
    int rc_ = (x);          \
    if (rc_) return rc_;    \
  } while (0)

attn::View view(const void* p, const int64_t* s) { return attn::View{p, s[0], s[1], s[2]}; }
attn::MView mview(void* p, const int64_t* s) { return attn::MView{p, s[0], s[1], s[2]}; }

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_last_error.c_str(); }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP error";
    case ATTN_ERR_NONFINITE: return "non-finite output (ATTN_CHECK_FINITE)";
    default: return "unknown status";
  }
}

int attn_fwd_partial(const attn_fwd_args* a, void* stream) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->struct_size < sizeof(attn_fwd_args))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %u < %zu", a->struct_size, sizeof(attn_fwd_args));
  if (a->dtype != ATTN_DTYPE_BF16 && a->dtype != ATTN_DTYPE_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %u is not supported", a->dtype);
  if (a->o_dtype != ATTN_DTYPE_BF16 && a->o_dtype != ATTN_DTYPE_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "o_dtype %u is not supported", a->o_dtype);
  if (a->flags & ~(ATTN_FWD_ACCUMULATE | ATTN_FWD_BALANCED))
    return fail(ATTN_ERR_INVALID_ARG, "unknown flag bits 0x%x", a->flags);
  const bool accumulate = a->flags & ATTN_FWD_ACCUMULATE;
  if (accumulate && a->o_dtype != ATTN_DTYPE_F32)
    return fail(ATTN_ERR_INVALID_ARG, "ATTN_FWD_ACCUMULATE needs an fp32 running output");
  TRY(check_dims(a->batch, a->heads_q, a->heads_kv, a->seqlen_q, a->seqlen_k, a->head_dim));
  float scale;
  TRY(check_scale(a->scale, a->head_dim, &scale));
  bool varlen;
  TRY(check_varlen(a->cu_seqlens_q, a->cu_seqlens_k, a->dtype, a->q_pos0, a->k_pos0, &varlen));
  const bool has_q = a->seqlen_q > 0, has_k = a->seqlen_k > 0;
  TRY(check_view("q", a->q, a->q_stride, 3, a->dtype, has_q));
  TRY(check_view("k", a->k, a->k_stride, 3, a->dtype, has_q && has_k));
  TRY(check_view("v", a->v, a->v_stride, 3, a->dtype, has_q && has_k));
  TRY(check_seq_stride("k", a->k_stride[1], has_q && has_k));
  TRY(check_seq_stride("v", a->v_stride[1], has_q && has_k));
  TRY(check_view("o", a->o, a->o_stride, 3, a->o_dtype, has_q));
  if (has_q && !a->lse) return fail(ATTN_ERR_INVALID_ARG, "lse is NULL");
  if (has_q && !aligned16(a->lse)) return fail(ATTN_ERR_UNSUPPORTED, "lse is not 16-byte aligned");
  if (a->o_final) TRY(check_view("o_final", a->o_final, a->o_final_stride, 3, ATTN_DTYPE_BF16, has_q));
  const int64_t units = (int64_t)a->batch * a->heads_q * ((a->seqlen_q + 63) / 64);
  if (units > 0x7fffffffLL) return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
  if (!has_q) return ok();

  attn::FwdParams p{};
  p.q = view(a->q, a->q_stride);
  p.k = view(a->k, a->k_stride);
  p.v = view(a->v, a->v_stride);
  p.o = mview(a->o, a->o_stride);
  p.o_final = mview(a->o_final, a->o_final_stride);
  p.lse = a->lse;
  p.lse_sb = varlen ? 0 : (int64_t)a->heads_q * a->seqlen_q;
  p.lse_sh = varlen ? 1 : a->seqlen_q;
  p.lse_ss = varlen ? a->heads_q : 1;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.B = a->batch;
  p.Hq = a->heads_q;
  p.Hkv = a->heads_kv;
  p.Sq = a->seqlen_q;
  p.Sk = a->seqlen_k;
  p.group = a->heads_q / a->heads_kv;
  p.delta = a->q_pos0 - a->k_pos0;
  p.causal = a->causal != 0;
  p.o_f32 = a->o_dtype == ATTN_DTYPE_F32;
  p.accumulate = accumulate;
  p.balanced = (a->flags & ATTN_FWD_BALANCED) != 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;

  // A chunk that no query sees leaves a running result unchanged (per sequence
  // in a variable-length batch, where the kernel decides).
  const bool invisible = !varlen && (a->seqlen_k == 0 || (p.causal && p.delta + (a->seqlen_q - 1) < 0));
  if (invisible && accumulate && !a->o_final) return ok();

  TRY(check_items(a->dtype == ATTN_DTYPE_BF16 ? attn::items_fwd_bf16(p) : attn::items_fwd_f32(p),
                  "attn_fwd_partial"));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = a->dtype == ATTN_DTYPE_BF16 ? attn::launch_fwd_bf16(p, a->head_dim, s)
                                             : attn::launch_fwd_f32(p, a->head_dim, s);
  if (e != hipSuccess) return hip_fail(e, "attn_fwd_partial launch");
  log_call("attn_fwd_partial dtype=%u batch=%d heads_q=%d heads_kv=%d seqlen_q=%d seqlen_k=%d head_dim=%d causal=%d "
           "flags=0x%x varlen=%d stream=%p", a->dtype, a->batch, a->heads_q, a->heads_kv, a->seqlen_q, a->seqlen_k,
           a->head_dim, a->causal, a->flags, a->cu_seqlens_q != nullptr, stream);
  Outputs outs;
  const int32_t* cu_q = varlen ? a->cu_seqlens_q : nullptr;
  outs.bshd("o", a->o, a->o_dtype, a->batch, a->seqlen_q, a->heads_q, a->head_dim, a->o_stride, cu_q);
  outs.lse(a->lse, a->batch, a->heads_q, a->seqlen_q, cu_q);
  outs.bshd("o_final", a->o_final, ATTN_DTYPE_BF16, a->batch, a->seqlen_q, a->heads_q, a->head_dim,
            a->o_final_stride, cu_q);
  return enqueued(stream, "attn_fwd_partial", &outs);
}

int attn_fwd_chunks(const attn_fwd_chunks_args* a, void* stream) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->struct_size < sizeof(attn_fwd_chunks_args))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %u < %zu", a->struct_size, sizeof(attn_fwd_chunks_args));
  if (a->dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED, "dtype %u is not supported (bf16 only)", a->dtype);
  if (a->o_dtype != ATTN_DTYPE_BF16 && a->o_dtype != ATTN_DTYPE_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "o_dtype %u is not supported", a->o_dtype);
  if (a->flags & ~(ATTN_FWD_ACCUMULATE | ATTN_FWD_BALANCED))
    return fail(ATTN_ERR_INVALID_ARG, "unknown flag bits 0x%x", a->flags);
  const bool accumulate = a->flags & ATTN_FWD_ACCUMULATE;
  if (accumulate && a->o_dtype != ATTN_DTYPE_F32)
    return fail(ATTN_ERR_INVALID_ARG, "ATTN_FWD_ACCUMULATE needs an fp32 running output");
  if (a->n_chunks < 0 || a->n_chunks > ATTN_MAX_CHUNKS)
    return fail(ATTN_ERR_INVALID_ARG, "n_chunks must be in [0, %d]", ATTN_MAX_CHUNKS);
  TRY(check_dims(a->batch, a->heads_q, a->heads_kv, a->seqlen_q, 0, a->head_dim));
  float scale;
  TRY(check_scale(a->scale, a->head_dim, &scale));
  const bool has_q = a->seqlen_q > 0;
  TRY(check_view("q", a->q, a->q_stride, 3, a->dtype, has_q));
  TRY(check_view("o", a->o, a->o_stride, 3, a->o_dtype, has_q));
  if (has_q && !a->lse) return fail(ATTN_ERR_INVALID_ARG, "lse is NULL");
  if (has_q && !aligned16(a->lse)) return fail(ATTN_ERR_UNSUPPORTED, "lse is not 16-byte aligned");
  if (a->o_final) TRY(check_view("o_final", a->o_final, a->o_final_stride, 3, ATTN_DTYPE_BF16, has_q));
  if (a->n_chunks > 0 && (!a->k_chunks || !a->v_chunks || !a->chunk_len || !a->chunk_pos0))
    return fail(ATTN_ERR_INVALID_ARG, "chunk arrays must not be NULL");
  TRY(check_seq_stride("k_chunks", a->k_stride[1], has_q && a->n_chunks > 0));
  TRY(check_seq_stride("v_chunks", a->v_stride[1], has_q && a->n_chunks > 0));
  attn::ChunkTable ct{};
  ct.q_pos0 = a->q_pos0;
  for (int c = 0; c < a->n_chunks; ++c) {
    if (a->chunk_len[c] < 0) return fail(ATTN_ERR_INVALID_ARG, "chunk_len[%d] is negative", c);
    if (a->chunk_len[c] == 0) continue;
    const int64_t ks[3] = {a->chunk_k_bstride ? a->chunk_k_bstride[c] : a->k_stride[0], a->k_stride[1],
                           a->k_stride[2]};
    const int64_t vs[3] = {a->chunk_v_bstride ? a->chunk_v_bstride[c] : a->v_stride[0], a->v_stride[1],
                           a->v_stride[2]};
    char name[32];
    snprintf(name, sizeof name, "k_chunks[%d]", c);
    TRY(check_view(name, a->k_chunks[c], ks, 3, a->dtype, has_q));
    snprintf(name, sizeof name, "v_chunks[%d]", c);
    TRY(check_view(name, a->v_chunks[c], vs, 3, a->dtype, has_q));
    ct.k[ct.n] = a->k_chunks[c];
    ct.v[ct.n] = a->v_chunks[c];
    ct.kb[ct.n] = ks[0];
    ct.vb[ct.n] = vs[0];
    ct.len[ct.n] = a->chunk_len[c];
    ct.pos0[ct.n] = a->chunk_pos0[c];
    ++ct.n;
  }
  const int64_t units = (int64_t)a->batch * a->heads_q * ((a->seqlen_q + 63) / 64);
  if (units > 0x7fffffffLL) return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
  if (!has_q) return ok();
  // No chunk with keys: a running result is left as it is.
  if (ct.n == 0 && accumulate && !a->o_final) return ok();

  attn::FwdParams p{};
  p.q = view(a->q, a->q_stride);
  p.k = view(nullptr, a->k_stride);
  p.v = view(nullptr, a->v_stride);
  p.o = mview(a->o, a->o_stride);
  p.o_final = mview(a->o_final, a->o_final_stride);
  p.lse = a->lse;
  p.lse_sb = (int64_t)a->heads_q * a->seqlen_q;
  p.lse_sh = a->seqlen_q;
  p.lse_ss = 1;
  p.B = a->batch;
  p.Hq = a->heads_q;
  p.Hkv = a->heads_kv;
  p.Sq = a->seqlen_q;
  p.group = a->heads_q / a->heads_kv;
  p.causal = a->causal != 0;
  p.o_f32 = a->o_dtype == ATTN_DTYPE_F32;
  p.accumulate = accumulate;
  p.balanced = (a->flags & ATTN_FWD_BALANCED) != 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  TRY(check_items(attn::items_fwd_bf16(p), "attn_fwd_chunks"));
  hipError_t e = attn::launch_fwd_chunks_bf16(p, ct, a->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_fwd_chunks launch");
  log_call("attn_fwd_chunks batch=%d heads_q=%d heads_kv=%d seqlen_q=%d head_dim=%d n_chunks=%d causal=%d flags=0x%x "
           "stream=%p", a->batch, a->heads_q, a->heads_kv, a->seqlen_q, a->head_dim, a->n_chunks, a->causal, a->flags,
           stream);
  Outputs outs;
  outs.bshd("o", a->o, a->o_dtype, a->batch, a->seqlen_q, a->heads_q, a->head_dim, a->o_stride);
  outs.lse(a->lse, a->batch, a->heads_q, a->seqlen_q);
  outs.bshd("o_final", a->o_final, ATTN_DTYPE_BF16, a->batch, a->seqlen_q, a->heads_q, a->head_dim,
            a->o_final_stride);
  return enqueued(stream, "attn_fwd_chunks", &outs);
}

int attn_merge_lse(const attn_merge_args* a, void* stream) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->struct_size < sizeof(attn_merge_args))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %u < %zu", a->struct_size, sizeof(attn_merge_args));
  if (a->n_parts < 1 || a->n_parts > 1024) return fail(ATTN_ERR_INVALID_ARG, "n_parts must be in [1, 1024]");
  if (a->mode != ATTN_MERGE_SEQUENTIAL && a->mode != ATTN_MERGE_TREE)
    return fail(ATTN_ERR_INVALID_ARG, "unknown merge mode %u", a->mode);
  if (a->o_out_dtype != ATTN_DTYPE_BF16 && a->o_out_dtype != ATTN_DTYPE_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "o_out_dtype %u is not supported", a->o_out_dtype);
  if (a->batch < 1 || a->heads < 1 || a->seqlen < 0)
    return fail(ATTN_ERR_INVALID_ARG, "batch and heads must be >= 1, seqlen >= 0");
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", a->head_dim);
  const bool any = a->seqlen > 0;
  TRY(check_view("o_parts", a->o_parts, a->o_stride, 3, ATTN_DTYPE_F32, any));
  TRY(check_view("o_out", a->o_out, a->o_out_stride, 3, a->o_out_dtype, any));
  if (any && (!a->lse_parts || !a->lse_out)) return fail(ATTN_ERR_INVALID_ARG, "lse_parts or lse_out is NULL");
  if (any && (!aligned16(a->lse_parts) || !aligned16(a->lse_out)))
    return fail(ATTN_ERR_UNSUPPORTED, "lse_parts or lse_out is not 16-byte aligned");
  if (a->n_parts > 1 && (a->o_part_stride == 0 || a->lse_part_stride == 0))
    return fail(ATTN_ERR_INVALID_ARG, "part strides must be nonzero");
  if ((a->o_part_stride * 4) % 16) return fail(ATTN_ERR_UNSUPPORTED, "o_part_stride breaks 16-byte alignment");
  if (!any) return ok();
  attn::MergeParams p{};
  p.o_parts = a->o_parts;
  p.o_part_stride = a->o_part_stride;
  p.o_sb = a->o_stride[0];
  p.o_ss = a->o_stride[1];
  p.o_sh = a->o_stride[2];
  p.lse_parts = a->lse_parts;
  p.lse_part_stride = a->lse_part_stride;
  p.out = mview(a->o_out, a->o_out_stride);
  p.out_f32 = a->o_out_dtype == ATTN_DTYPE_F32;
  p.lse_out = a->lse_out;
  p.n_parts = a->n_parts;
  p.B = a->batch;
  p.S = a->seqlen;
  p.H = a->heads;
  p.tree = a->mode == ATTN_MERGE_TREE;
  TRY(check_items(attn::items_merge(p, a->head_dim), "attn_merge_lse"));
  hipError_t e = attn::launch_merge(p, a->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_merge_lse launch");
  log_call("attn_merge_lse n_parts=%d batch=%d seqlen=%d heads=%d head_dim=%d mode=%u stream=%p", a->n_parts, a->batch,
           a->seqlen, a->heads, a->head_dim, a->mode, stream);
  Outputs outs;
  outs.bshd("o_out", a->o_out, a->o_out_dtype, a->batch, a->seqlen, a->heads, a->head_dim, a->o_out_stride);
  outs.lse(a->lse_out, a->batch, a->heads, a->seqlen);
  return enqueued(stream, "attn_merge_lse", &outs);
}

int attn_bwd(const attn_bwd_args* a, void* stream) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->struct_size < sizeof(attn_bwd_args))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %u < %zu", a->struct_size, sizeof(attn_bwd_args));
  if (a->dtype != ATTN_DTYPE_BF16 && a->dtype != ATTN_DTYPE_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %u is not supported", a->dtype);
  const uint32_t known = ATTN_BWD_COMPUTE_DELTA | ATTN_BWD_DQ_OVERWRITE | ATTN_BWD_FINALIZE_DQ | ATTN_BWD_BALANCED |
                         ATTN_BWD_DETERMINISTIC;
  if (a->flags & ~known) return fail(ATTN_ERR_INVALID_ARG, "unknown flag bits 0x%x", a->flags);
  TRY(check_dims(a->batch, a->heads_q, a->heads_kv, a->seqlen_q, a->seqlen_k, a->head_dim));
  float scale;
  TRY(check_scale(a->scale, a->head_dim, &scale));
  bool varlen;
  TRY(check_varlen(a->cu_seqlens_q, a->cu_seqlens_k, a->dtype, a->q_pos0, a->k_pos0, &varlen));
  const bool has_q = a->seqlen_q > 0, has_k = a->seqlen_k > 0;
  const bool finalize = a->flags & ATTN_BWD_FINALIZE_DQ;
  TRY(check_view("q", a->q, a->q_stride, 3, a->dtype, has_q));
  TRY(check_view("k", a->k, a->k_stride, 3, a->dtype, has_k));
  TRY(check_view("v", a->v, a->v_stride, 3, a->dtype, has_k));
  TRY(check_seq_stride("k", a->k_stride[1], has_q && has_k));
  TRY(check_seq_stride("v", a->v_stride[1], has_q && has_k));
  TRY(check_view("o", a->o, a->o_stride, 3, a->dtype, has_q && (a->flags & ATTN_BWD_COMPUTE_DELTA)));
  TRY(check_view("dout", a->dout, a->do_stride, 3, a->dtype, has_q));
  TRY(check_view("dk", a->dk, a->dk_stride, 3, a->dtype, has_k));
  TRY(check_view("dv", a->dv, a->dv_stride, 3, a->dtype, has_k));
  TRY(check_view("dq", a->dq, a->dq_stride, 3, a->dtype, has_q && finalize));
  if (has_q && (!a->lse || !a->dq_acc)) return fail(ATTN_ERR_INVALID_ARG, "lse and dq_acc must not be NULL");
  if (has_q && (!aligned16(a->lse) || !aligned16(a->dq_acc)))
    return fail(ATTN_ERR_UNSUPPORTED, "lse and dq_acc must be 16-byte aligned");
  if (has_q) {
    const size_t need = attn_bwd_workspace_size(a->batch, a->heads_q, a->seqlen_q);
    if (!a->workspace || a->workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if ((uintptr_t)a->workspace & 255u) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const int64_t units = (int64_t)a->batch * a->heads_q * ((a->seqlen_q + 63) / 64) +
                        (int64_t)a->batch * a->heads_kv * ((a->seqlen_k + 63) / 64);
  if (units > 0x7fffffffLL) return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");

  attn::BwdParams p{};
  p.q = view(a->q, a->q_stride);
  p.k = view(a->k, a->k_stride);
  p.v = view(a->v, a->v_stride);
  p.o = view(a->o, a->o_stride);
  p.dout = view(a->dout, a->do_stride);
  p.dq = mview(a->dq, a->dq_stride);
  p.dk = mview(a->dk, a->dk_stride);
  p.dv = mview(a->dv, a->dv_stride);
  p.lse = a->lse;
  p.lse_sb = varlen ? 0 : (int64_t)a->heads_q * a->seqlen_q;
  p.lse_sh = varlen ? 1 : a->seqlen_q;
  p.lse_ss = varlen ? a->heads_q : 1;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.stats = (float*)a->workspace;
  p.Sq_pad = (a->seqlen_q + 63) / 64 * 64;
  p.dq_acc = a->dq_acc;
  p.B = a->batch;
  p.Hq = a->heads_q;
  p.Hkv = a->heads_kv;
  p.Sq = a->seqlen_q;
  p.Sk = a->seqlen_k;
  p.group = a->heads_q / a->heads_kv;
  p.delta_pos = a->q_pos0 - a->k_pos0;
  p.causal = a->causal != 0;
  p.dq_overwrite = (a->flags & ATTN_BWD_DQ_OVERWRITE) != 0;
  p.finalize_dq = finalize;
  p.balanced = (a->flags & ATTN_BWD_BALANCED) != 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;

  const int D = a->head_dim;
  const int bf16 = a->dtype == ATTN_DTYPE_BF16;
  TRY(check_items(attn::items_bwd_prepare(p, D), "attn_bwd"));
  TRY(check_items(bf16 ? attn::items_bwd_bf16(p) : attn::items_bwd_f32(p), "attn_bwd"));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (has_q && (a->flags & ATTN_BWD_COMPUTE_DELTA)) {
    e = attn::launch_bwd_prepare(p, D, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd prepare launch");
  }
  // dQ needs a pass unless this chunk is invisible and dq_acc is left as it is.
  const bool invisible = !varlen && (!has_k || (p.causal && p.delta_pos + (a->seqlen_q - 1) < 0));
  const int run_dq = has_q && (!invisible || p.dq_overwrite || finalize);
  e = bf16 ? attn::launch_bwd_bf16(p, D, run_dq, s) : attn::launch_bwd_f32(p, D, run_dq, s);
  if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
  log_call("attn_bwd dtype=%u batch=%d heads_q=%d heads_kv=%d seqlen_q=%d seqlen_k=%d head_dim=%d causal=%d flags=0x%x "
           "varlen=%d stream=%p", a->dtype, a->batch, a->heads_q, a->heads_kv, a->seqlen_q, a->seqlen_k, a->head_dim,
           a->causal, a->flags, a->cu_seqlens_q != nullptr, stream);
  Outputs outs;
  const int32_t* cu_q = varlen ? a->cu_seqlens_q : nullptr;
  const int32_t* cu_k = varlen ? a->cu_seqlens_k : nullptr;
  if (has_q) {
    const int64_t acc_st[3] = {(int64_t)a->seqlen_q * a->heads_q * D, (int64_t)a->heads_q * D, D};
    outs.bshd("dq_acc", a->dq_acc, ATTN_DTYPE_F32, a->batch, a->seqlen_q, a->heads_q, D, acc_st, cu_q);
    if (finalize) outs.bshd("dq", a->dq, a->dtype, a->batch, a->seqlen_q, a->heads_q, D, a->dq_stride, cu_q);
  }
  outs.bshd("dk", a->dk, a->dtype, a->batch, a->seqlen_k, a->heads_kv, D, a->dk_stride, cu_k);
  outs.bshd("dv", a->dv, a->dtype, a->batch, a->seqlen_k, a->heads_kv, D, a->dv_stride, cu_k);
  return enqueued(stream, "attn_bwd", &outs);
}

int attn_bwd_chunks(const attn_bwd_chunks_args* a, void* stream) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->struct_size < sizeof(attn_bwd_chunks_args))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %u < %zu", a->struct_size, sizeof(attn_bwd_chunks_args));
  if (a->dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED, "dtype %u is not supported (bf16 only)", a->dtype);
  const uint32_t known = ATTN_BWD_COMPUTE_DELTA | ATTN_BWD_DQ_OVERWRITE | ATTN_BWD_FINALIZE_DQ | ATTN_BWD_BALANCED |
                         ATTN_BWD_DETERMINISTIC;
  if (a->flags & ~known) return fail(ATTN_ERR_INVALID_ARG, "unknown flag bits 0x%x", a->flags);
  if (a->n_chunks < 0 || a->n_chunks > ATTN_MAX_CHUNKS)
    return fail(ATTN_ERR_INVALID_ARG, "n_chunks must be in [0, %d]", ATTN_MAX_CHUNKS);
  TRY(check_dims(a->batch, a->heads_q, a->heads_kv, a->seqlen_q, 0, a->head_dim));
  float scale;
  TRY(check_scale(a->scale, a->head_dim, &scale));
  const bool has_q = a->seqlen_q > 0;
  const bool finalize = a->flags & ATTN_BWD_FINALIZE_DQ;
  TRY(check_view("q", a->q, a->q_stride, 3, a->dtype, has_q));
  TRY(check_view("o", a->o, a->o_stride, 3, a->dtype, has_q && (a->flags & ATTN_BWD_COMPUTE_DELTA)));
  TRY(check_view("dout", a->dout, a->do_stride, 3, a->dtype, has_q));
  TRY(check_view("dq", a->dq, a->dq_stride, 3, a->dtype, has_q && finalize));
  if (has_q && (!a->lse || !a->dq_acc)) return fail(ATTN_ERR_INVALID_ARG, "lse and dq_acc must not be NULL");
  if (has_q && (!aligned16(a->lse) || !aligned16(a->dq_acc)))
    return fail(ATTN_ERR_UNSUPPORTED, "lse and dq_acc must be 16-byte aligned");
  if (has_q) {
    const size_t need = attn_bwd_workspace_size(a->batch, a->heads_q, a->seqlen_q);
    if (!a->workspace || a->workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if ((uintptr_t)a->workspace & 255u) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if (a->n_chunks > 0 && (!a->k_chunks || !a->v_chunks || !a->dk_chunks || !a->dv_chunks || !a->chunk_len ||
                          !a->chunk_pos0))
    return fail(ATTN_ERR_INVALID_ARG, "chunk arrays must not be NULL");
  TRY(check_seq_stride("k_chunks", a->k_stride[1], a->seqlen_q > 0 && a->n_chunks > 0));
  TRY(check_seq_stride("v_chunks", a->v_stride[1], a->seqlen_q > 0 && a->n_chunks > 0));
  attn::BwdChunkTable ct{};
  ct.kv.q_pos0 = a->q_pos0;
  int64_t key_tiles = 0;
  for (int c = 0; c < a->n_chunks; ++c) {
    if (a->chunk_len[c] < 0) return fail(ATTN_ERR_INVALID_ARG, "chunk_len[%d] is negative", c);
    if (a->chunk_len[c] == 0) continue;
    auto bs = [&](const int64_t* arr, const int64_t* st) { return arr ? arr[c] : st[0]; };
    const int64_t ks[3] = {bs(a->chunk_k_bstride, a->k_stride), a->k_stride[1], a->k_stride[2]};
    const int64_t vs[3] = {bs(a->chunk_v_bstride, a->v_stride), a->v_stride[1], a->v_stride[2]};
    const int64_t dks[3] = {bs(a->chunk_dk_bstride, a->dk_stride), a->dk_stride[1], a->dk_stride[2]};
    const int64_t dvs[3] = {bs(a->chunk_dv_bstride, a->dv_stride), a->dv_stride[1], a->dv_stride[2]};
    char name[32];
    snprintf(name, sizeof name, "k_chunks[%d]", c);
    TRY(check_view(name, a->k_chunks[c], ks, 3, a->dtype, true));
    snprintf(name, sizeof name, "v_chunks[%d]", c);
    TRY(check_view(name, a->v_chunks[c], vs, 3, a->dtype, true));
    snprintf(name, sizeof name, "dk_chunks[%d]", c);
    TRY(check_view(name, a->dk_chunks[c], dks, 3, a->dtype, true));
    snprintf(name, sizeof name, "dv_chunks[%d]", c);
    TRY(check_view(name, a->dv_chunks[c], dvs, 3, a->dtype, true));
    ct.kv.k[ct.kv.n] = a->k_chunks[c];
    ct.kv.v[ct.kv.n] = a->v_chunks[c];
    ct.kv.kb[ct.kv.n] = ks[0];
    ct.kv.vb[ct.kv.n] = vs[0];
    ct.kv.len[ct.kv.n] = a->chunk_len[c];
    ct.kv.pos0[ct.kv.n] = a->chunk_pos0[c];
    ct.dk[ct.kv.n] = a->dk_chunks[c];
    ct.dv[ct.kv.n] = a->dv_chunks[c];
    ct.dkb[ct.kv.n] = dks[0];
    ct.dvb[ct.kv.n] = dvs[0];
    ++ct.kv.n;
    key_tiles += (a->chunk_len[c] + 63) / 64;
  }
  const int64_t units = (int64_t)a->batch * a->heads_q * ((a->seqlen_q + 63) / 64) +
                        (int64_t)a->batch * a->heads_kv * key_tiles;
  if (units > 0x7fffffffLL) return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");

  attn::BwdParams p{};
  p.q = view(a->q, a->q_stride);
  p.k = view(nullptr, a->k_stride);
  p.v = view(nullptr, a->v_stride);
  p.o = view(a->o, a->o_stride);
  p.dout = view(a->dout, a->do_stride);
  p.dq = mview(a->dq, a->dq_stride);
  p.dk = mview(nullptr, a->dk_stride);
  p.dv = mview(nullptr, a->dv_stride);
  p.lse = a->lse;
  p.lse_sb = (int64_t)a->heads_q * a->seqlen_q;
  p.lse_sh = a->seqlen_q;
  p.lse_ss = 1;
  p.stats = (float*)a->workspace;
  p.Sq_pad = (a->seqlen_q + 63) / 64 * 64;
  p.dq_acc = a->dq_acc;
  p.B = a->batch;
  p.Hq = a->heads_q;
  p.Hkv = a->heads_kv;
  p.Sq = a->seqlen_q;
  p.group = a->heads_q / a->heads_kv;
  p.causal = a->causal != 0;
  p.dq_overwrite = (a->flags & ATTN_BWD_DQ_OVERWRITE) != 0;
  p.finalize_dq = finalize;
  p.balanced = (a->flags & ATTN_BWD_BALANCED) != 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;

  TRY(check_items(attn::items_bwd_prepare(p, a->head_dim), "attn_bwd_chunks"));
  TRY(check_items(attn::items_bwd_chunks_bf16(p, ct), "attn_bwd_chunks"));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (has_q && (a->flags & ATTN_BWD_COMPUTE_DELTA)) {
    e = attn::launch_bwd_prepare(p, a->head_dim, 1, s);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd_chunks prepare launch");
  }
  // Without queries the dK/dV kernel writes zeros for every chunk and no dQ pass runs.
  e = attn::launch_bwd_chunks_bf16(p, ct, a->head_dim, s);
  if (e != hipSuccess) return hip_fail(e, "attn_bwd_chunks launch");
  log_call("attn_bwd_chunks batch=%d heads_q=%d heads_kv=%d seqlen_q=%d head_dim=%d n_chunks=%d causal=%d flags=0x%x "
           "stream=%p", a->batch, a->heads_q, a->heads_kv, a->seqlen_q, a->head_dim, a->n_chunks, a->causal, a->flags,
           stream);
  Outputs outs;
  const int D = a->head_dim;
  if (has_q) {
    const int64_t acc_st[3] = {(int64_t)a->seqlen_q * a->heads_q * D, (int64_t)a->heads_q * D, D};
    outs.bshd("dq_acc", a->dq_acc, ATTN_DTYPE_F32, a->batch, a->seqlen_q, a->heads_q, D, acc_st);
    if (finalize) outs.bshd("dq", a->dq, a->dtype, a->batch, a->seqlen_q, a->heads_q, D, a->dq_stride);
  }
  for (int c = 0; c < ct.kv.n; ++c) {
    const int64_t dks[3] = {ct.dkb[c], a->dk_stride[1], a->dk_stride[2]};
    const int64_t dvs[3] = {ct.dvb[c], a->dv_stride[1], a->dv_stride[2]};
    char name[24];
    snprintf(name, sizeof name, "dk (chunk entry %d)", c);
    outs.bshd(name, ct.dk[c], a->dtype, a->batch, ct.kv.len[c], a->heads_kv, D, dks);
    snprintf(name, sizeof name, "dv (chunk entry %d)", c);
    outs.bshd(name, ct.dv[c], a->dtype, a->batch, ct.kv.len[c], a->heads_kv, D, dvs);
  }
  return enqueued(stream, "attn_bwd_chunks", &outs);
}

}  // extern "C"

namespace {

// Nodes of a decode tree are cut into segments of at most `seg` keys (each a
// table entry with the node's query range), so a long shared prefix is
// streamed by many workgroups.  seg starts at kTreeSeg and doubles until the
// segments fit the table.  Returns false (with the error set) on invalid nodes.
constexpr int64_t kTreeSeg = 2048;
bool tree_table(const attn_decode_tree_args* a, attn::TreeTable* tt, int64_t* entries, int* code) {
  *tt = attn::TreeTable{};
  *entries = 0;
  if (a->n_nodes < 0 || a->n_nodes > ATTN_MAX_TREE_NODES) {
    *code = fail(ATTN_ERR_INVALID_ARG, "n_nodes must be in [0, %d]", ATTN_MAX_TREE_NODES);
    return false;
  }
  if (a->n_nodes > 0 && (!a->kv_start || !a->kv_len || !a->q_begin || !a->q_end)) {
    *code = fail(ATTN_ERR_INVALID_ARG, "node arrays must not be NULL");
    return false;
  }
  for (int n = 0; n < a->n_nodes; ++n) {
    if (a->kv_len[n] < 0 || a->kv_start[n] < 0 || a->kv_start[n] + a->kv_len[n] > a->cache_len) {
      *code = fail(ATTN_ERR_INVALID_ARG, "node %d: keys [%lld, %lld) outside the cache of %lld", n,
                   (long long)a->kv_start[n], (long long)a->kv_start[n] + a->kv_len[n], (long long)a->cache_len);
      return false;
    }
    if (a->q_begin[n] < 0 || a->q_end[n] < a->q_begin[n] || a->q_end[n] > a->n_queries) {
      *code = fail(ATTN_ERR_INVALID_ARG, "node %d: queries [%d, %d) outside [0, %d)", n, a->q_begin[n], a->q_end[n],
                   a->n_queries);
      return false;
    }
  }
  int64_t seg = kTreeSeg;
  for (;;) {
    int64_t pieces = 0;
    for (int n = 0; n < a->n_nodes; ++n) pieces += std::max<int64_t>(1, (a->kv_len[n] + seg - 1) / seg);
    if (pieces <= attn::kMaxTreeNodes) break;
    seg *= 2;
  }
  for (int n = 0; n < a->n_nodes; ++n) {
    const int64_t len = a->kv_len[n];
    const int64_t np = std::max<int64_t>(1, (len + seg - 1) / seg);
    for (int64_t j = 0; j < np; ++j) {
      const int e = tt->n++;
      tt->kv_start[e] = a->kv_start[n] + j * seg;
      tt->kv_len[e] = (int)std::min(seg, len - j * seg);
      tt->q_begin[e] = a->q_begin[n];
      tt->q_end[e] = a->q_end[n];
      tt->e0[e] = (int)*entries;
      *entries += a->q_end[n] - a->q_begin[n];
    }
  }
  if (*entries > 0x7fffffffLL / std::max(1, a->heads_q)) {
    *code = fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    return false;
  }
  return true;
}

size_t tree_workspace_bytes(int64_t entries, int heads_q, int head_dim) {
  const size_t rows = (size_t)entries * heads_q;
  return ((rows * head_dim * 4 + 255) & ~(size_t)255) + ((rows * 4 + 255) & ~(size_t)255);
}

}  // namespace

extern "C" {

size_t attn_decode_tree_workspace_size(const attn_decode_tree_args* a) {
  if (!a || a->struct_size < sizeof(attn_decode_tree_args) || a->heads_q < 1 ||
      (a->head_dim != 64 && a->head_dim != 128))
    return 0;
  attn::TreeTable tt;
  int64_t entries;
  int code;
  const std::string saved = g_last_error;
  const bool okay = tree_table(a, &tt, &entries, &code);
  g_last_error = saved;  // a size query leaves the last error as it was
  return okay ? tree_workspace_bytes(entries, a->heads_q, a->head_dim) : 0;
}

int attn_decode_tree(const attn_decode_tree_args* a, void* stream) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->struct_size < sizeof(attn_decode_tree_args))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %u < %zu", a->struct_size, sizeof(attn_decode_tree_args));
  if (a->n_queries < 0) return fail(ATTN_ERR_INVALID_ARG, "n_queries must be >= 0");
  TRY(check_dims(1, a->heads_q, a->heads_kv, 1, 0, a->head_dim));
  if (a->cache_len < 0) return fail(ATTN_ERR_INVALID_ARG, "cache_len must be >= 0");
  float scale;
  TRY(check_scale(a->scale, a->head_dim, &scale));
  attn::TreeTable tt;
  int64_t entries;
  int code;
  if (!tree_table(a, &tt, &entries, &code)) return code;
  if (a->n_queries == 0) return ok();
  TRY(check_view("q", a->q, a->q_stride, 2, ATTN_DTYPE_BF16, true));
  TRY(check_view("k_cache", a->k_cache, a->k_stride, 2, ATTN_DTYPE_BF16, a->cache_len > 0));
  TRY(check_view("v_cache", a->v_cache, a->v_stride, 2, ATTN_DTYPE_BF16, a->cache_len > 0));
  TRY(check_seq_stride("k_cache", a->k_stride[0], a->cache_len > 0));
  TRY(check_seq_stride("v_cache", a->v_stride[0], a->cache_len > 0));
  TRY(check_view("o", a->o, a->o_stride, 2, ATTN_DTYPE_BF16, true));
  if (!a->lse) return fail(ATTN_ERR_INVALID_ARG, "lse is NULL");
  if (!aligned16(a->lse)) return fail(ATTN_ERR_UNSUPPORTED, "lse is not 16-byte aligned");
  const size_t need = tree_workspace_bytes(entries, a->heads_q, a->head_dim);
  if (need > 0 && (!a->workspace || a->workspace_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                a->workspace ? a->workspace_bytes : (size_t)0);
  if (need > 0 && ((uintptr_t)a->workspace & 255u))
    return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  // The per-segment pass is the forward over (the node's queries) x (the segment's
  // keys), non-causal, writing fp32 partials [entries, heads_q, head_dim] and their
  // LSE [entries, heads_q].
  const size_t rows = (size_t)entries * a->heads_q;
  attn::FwdParams p{};
  p.q = attn::View{a->q, 0, a->q_stride[0], a->q_stride[1]};
  p.k = attn::View{a->k_cache, 0, a->k_stride[0], a->k_stride[1]};
  p.v = attn::View{a->v_cache, 0, a->v_stride[0], a->v_stride[1]};
  p.o = attn::MView{a->workspace, 0, (int64_t)a->heads_q * a->head_dim, a->head_dim};
  p.o_final = attn::MView{nullptr, 0, 0, 0};
  p.lse = (float*)((char*)a->workspace + ((rows * a->head_dim * 4 + 255) & ~(size_t)255));
  p.lse_sb = 0;
  p.lse_sh = 1;
  p.lse_ss = a->heads_q;
  p.B = 1;
  p.Hq = a->heads_q;
  p.Hkv = a->heads_kv;
  p.group = a->heads_q / a->heads_kv;
  p.causal = 0;
  p.o_f32 = 1;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  TRY(check_items(attn::items_tree_decode(p, tt, a->n_queries, a->head_dim), "attn_decode_tree"));
  hipError_t e = attn::launch_tree_decode(p, tt, a->n_queries, a->o, a->o_stride[0], a->o_stride[1], a->lse,
                                          a->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_decode_tree launch");
  log_call("attn_decode_tree n_queries=%d heads_q=%d heads_kv=%d head_dim=%d n_nodes=%d segments=%d stream=%p",
           a->n_queries, a->heads_q, a->heads_kv, a->head_dim, a->n_nodes, tt.n, stream);
  Outputs outs;
  outs.decode("query", a->o, a->o_stride, a->lse, a->n_queries, a->heads_q, a->head_dim);
  return enqueued(stream, "attn_decode_tree", &outs);
}

size_t attn_bwd_workspace_size(int32_t batch, int32_t heads_q, int32_t seqlen_q) {
  if (batch < 1 || heads_q < 1 || seqlen_q < 0) return 0;
  const size_t sq_pad = ((size_t)seqlen_q + 63) / 64 * 64;
  return ((size_t)batch * heads_q * 2 * sq_pad * sizeof(float) + 255) & ~(size_t)255;
}

size_t attn_decode_workspace_size(int32_t batch, int32_t heads_q, int32_t head_dim, int32_t n_splits) {
  if (batch < 1 || heads_q < 1 || n_splits < 1 || n_splits > 1024 || (head_dim != 64 && head_dim != 128)) return 0;
  const size_t rows = (size_t)batch * heads_q * (n_splits + 1);
  const size_t o_bytes = (rows * head_dim * 4 + 255) & ~(size_t)255;
  return o_bytes + ((rows * 4 + 255) & ~(size_t)255);
}

// Split-KV decode with the partials in the caller's workspace, or (noalloc) in
// the library's fixed per-device scratch.
static int decode_splitkv(const attn_decode_args* a, void* stream, bool noalloc) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->struct_size < sizeof(attn_decode_args))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %u < %zu", a->struct_size, sizeof(attn_decode_args));
  TRY(check_dims(a->batch, a->heads_q, a->heads_kv, 1, 0, a->head_dim));
  if (a->cache_len < 0) return fail(ATTN_ERR_INVALID_ARG, "cache_len must be >= 0");
  if (a->n_splits < 1 || a->n_splits > 1024) return fail(ATTN_ERR_INVALID_ARG, "n_splits must be in [1, 1024]");
  float scale;
  TRY(check_scale(a->scale, a->head_dim, &scale));
  TRY(check_view("q", a->q, a->q_stride, 2, ATTN_DTYPE_BF16, true));
  TRY(check_view("k_cache", a->k_cache, a->k_stride, 3, ATTN_DTYPE_BF16, a->cache_len > 0));
  TRY(check_view("v_cache", a->v_cache, a->v_stride, 3, ATTN_DTYPE_BF16, a->cache_len > 0));
  TRY(check_view("o", a->o, a->o_stride, 2, ATTN_DTYPE_BF16, true));
  if (!a->lse) return fail(ATTN_ERR_INVALID_ARG, "lse is NULL");
  if (a->seqlens && ((uintptr_t)a->seqlens & 3u)) return fail(ATTN_ERR_UNSUPPORTED, "seqlens is misaligned");
  const size_t need = attn_decode_workspace_size(a->batch, a->heads_q, a->head_dim, a->n_splits);
  if (noalloc) {
    if (need > attn::kNoAllocScratchBytes)
      return fail(ATTN_ERR_WORKSPACE,
                  "attn_decode_splitkv_noalloc: the split partials need %zu bytes, more than its fixed scratch of "
                  "%zu bytes (batch x heads_q x n_splits x (head_dim + 1) x 4 bytes, each part 256-byte aligned)",
                  need, attn::kNoAllocScratchBytes);
  } else {
    if (!a->workspace || a->workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if ((uintptr_t)a->workspace & 255u) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const int group = a->heads_q / a->heads_kv;
  const int64_t grid = (int64_t)a->batch * a->heads_kv * ((group + 3) / 4) * a->n_splits;
  if (grid > 0x7fffffffLL || (int64_t)a->batch * a->heads_q > 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");

  attn::DecodeParams p{};
  p.q = (const uint16_t*)a->q;
  p.q_sb = a->q_stride[0];
  p.q_sh = a->q_stride[1];
  p.k = (const uint16_t*)a->k_cache;
  p.k_sb = a->k_stride[0];
  p.k_sl = a->k_stride[1];
  p.k_sh = a->k_stride[2];
  p.v = (const uint16_t*)a->v_cache;
  p.v_sb = a->v_stride[0];
  p.v_sl = a->v_stride[1];
  p.v_sh = a->v_stride[2];
  p.seqlens = a->seqlens;
  p.L = a->cache_len;
  p.B = a->batch;
  p.Hq = a->heads_q;
  p.Hkv = a->heads_kv;
  p.group = group;
  p.n_splits = a->n_splits;
  p.split_len = (a->cache_len + a->n_splits - 1) / a->n_splits;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.o = (uint16_t*)a->o;
  p.o_sb = a->o_stride[0];
  p.o_sh = a->o_stride[1];
  p.lse = a->lse;
  TRY(check_items(attn::items_decode(p), noalloc ? "attn_decode_splitkv_noalloc" : "attn_decode_splitkv"));
  // Validation is complete; the scratch lookup is the first HIP call.
  void* ws = a->workspace;
  if (noalloc) {
    hipError_t e = attn::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "attn_decode_splitkv_noalloc scratch lookup");
  }
  // Stream-K (equal keys per work unit) when the lengths differ and the merge
  // tree can hold every piece of a sequence; fixed splits otherwise.
  p.streamk = a->seqlens && a->batch <= 1024 && (int64_t)a->batch * a->n_splits <= 1024;
  p.n_pieces = (int64_t)a->batch * (a->n_splits + 1);
  const size_t rows = (size_t)a->batch * a->heads_q * (a->n_splits + 1);
  p.part_o = (float*)ws;
  p.part_lse = (float*)((char*)ws + ((rows * a->head_dim * 4 + 255) & ~(size_t)255));
  hipError_t e = attn::launch_decode(p, a->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, noalloc ? "attn_decode_splitkv_noalloc launch" : "attn_decode_splitkv launch");
  log_call("%s batch=%d heads_q=%d heads_kv=%d head_dim=%d cache_len=%lld n_splits=%d seqlens=%d streamk=%d stream=%p",
           noalloc ? "attn_decode_splitkv_noalloc" : "attn_decode_splitkv", a->batch, a->heads_q, a->heads_kv,
           a->head_dim, (long long)a->cache_len, a->n_splits, a->seqlens != nullptr, p.streamk, stream);
  Outputs outs;
  outs.decode("batch", a->o, a->o_stride, a->lse, a->batch, a->heads_q, a->head_dim);
  return enqueued(stream, noalloc ? "attn_decode_splitkv_noalloc" : "attn_decode_splitkv", &outs);
}

int attn_decode_splitkv(const attn_decode_args* a, void* stream) { return decode_splitkv(a, stream, false); }

int attn_decode_splitkv_noalloc(const attn_decode_args* a, void* stream) { return decode_splitkv(a, stream, true); }

}  // extern "C"
