/*
 * attn.h - C ABI of libattn: exact blockwise softmax attention on one device's
 * sequence shard, for AMD Instinct MI355X (gfx950).
 *
 * Four operations, each computing exactly (up to floating-point rounding) the
 * plain softmax attention result that the source pages' blockwise methods reach:
 *
 *   attn_fwd_partial     attention of a query shard over one chunk of keys,
 *                        producing a partial output O and a row log-sum-exp
 *                        (BurstAttention, "local attention computation"; the
 *                        per-chunk step of ring-style attention).
 *   attn_merge_lse       log-sum-exp weighted merge of partial (O, LSE) pairs
 *                        over disjoint key sets, sequential or as a binary tree
 *                        (BurstAttention, "global aggregation"; Tree Attention,
 *                        reduction over the sequence axis).
 *   attn_bwd             gradients dQ, dK, dV for one key chunk from the saved
 *                        final O and LSE, with no re-run of the forward
 *                        (DistFlashAttn digest, rematerialisation-aware
 *                        gradient checkpointing).
 *   attn_decode_splitkv  single-token decode over a long KV cache split into
 *                        chunks whose partials are reduced by a binary tree
 *                        (Lean Attention and Tree Attention abstracts).
 *
 * Definitions (one batch b, query head h):
 *   query i sits at global position p_i = q_pos0 + i, key j at r_j = k_pos0 + j;
 *   with causal != 0, key j is visible to query i iff r_j <= p_i.
 *   s_ij = scale * q_i . k_j, LSE_i = ln sum_{visible j} exp(s_ij) (natural log),
 *   O_i = sum_{visible j} exp(s_ij - LSE_i) v_j.
 *   A row with no visible key has O_i = 0 and LSE_i = -inf (the merge identity).
 *   NaN propagates as in these formulas: a NaN score that a row sees makes the
 *   row's O and LSE NaN, and a key a row does not see never enters its softmax.
 *   (A non-finite value row that the causal mask hides but that shares a
 *   64-key tile with keys the row sees reaches the row's O through 0 * NaN.)
 *
 * Conventions shared by every entry point:
 *   - Tensors of shape [batch, seq, heads, head_dim] are given by a base pointer
 *     and three element strides (batch, seq, head); the head_dim stride is 1.
 *     LSE vectors are contiguous fp32 [batch, heads, seq].
 *   - All pointers are device pointers unless stated otherwise, 16-byte
 *     aligned, and element strides must keep every row start 16-byte aligned.
 *     Strides are never negative.  The sequence stride of keys and values (and
 *     of the decode-tree caches) is at most 2^24 elements: tiles of 64 rows are
 *     addressed as one row base plus a 32-bit offset per lane; a larger stride
 *     returns ATTN_ERR_UNSUPPORTED.
 *     The caller owns every buffer; the library never allocates, frees or
 *     retains a pointer past the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Success means the work is enqueued on `stream`; nothing synchronises.
 *     Device-side faults surface at the caller's next synchronisation.  For
 *     debugging, the environment variable ATTN_DEBUG_SYNC (set, and not "0";
 *     read on every call) makes each compute call wait for `stream` before it
 *     returns, so that a failure of its kernels is returned as ATTN_ERR_HIP by
 *     the call itself.  ATTN_CHECK_FINITE (set, and not "0"; read on every
 *     call) makes each compute call scan the outputs it wrote (o, lse, o_final,
 *     dq_acc, dq, dk, dv) after its kernels, wait for `stream`, and return
 *     ATTN_ERR_NONFINITE if one holds a NaN or an infinity, naming the tensor
 *     and the index of the first such element in attn_last_error().  An LSE of
 *     -inf (a row with no visible key) is not an error.  NaN inputs propagate
 *     to the outputs that depend on them (see the definitions above), so this
 *     also reports non-finite inputs where they are read.  The scan shares one
 *     small device buffer per device; checked calls are serialised within the
 *     process.  Both variables make calls wait for `stream`, so neither may be
 *     set while `stream` is being captured into a graph.  ATTN_LOG (set, and
 *     not "0") writes one line to stderr per enqueued call, naming the call and
 *     its sizes.
 *   - Every argument is checked on the host before anything is enqueued; on
 *     error the call returns a nonzero status, enqueues nothing, leaves every
 *     output untouched and records a message for attn_last_error().  This
 *     includes the size of every kernel launch the call would make: a problem
 *     that needs more than 2^32 - 1 work-items in one launch returns
 *     ATTN_ERR_UNSUPPORTED before the first launch.
 *   - Argument structs start with struct_size = sizeof(the struct).
 *   - head_dim must be 64 or 128.  Scale 0 means 1/sqrt(head_dim); otherwise it
 *     must be finite and positive.
 *   - The library keeps no mutable global state apart from two fixed device
 *     buffers (the scratch of attn_decode_splitkv_noalloc and the result
 *     buffer of the ATTN_CHECK_FINITE scan); calls are thread-safe, except
 *     that attn_decode_splitkv_noalloc calls overlapping on one device race.
 *   - Scratch memory is caller-provided (a workspace argument sized by
 *     attn_*_workspace_size), apart from the two fixed buffers above; the
 *     library never allocates.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#define ATTN_ABI_VERSION 10

/* Status codes. */
#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARG 1 /* null pointer, bad size, bad stride, bad scale, bad flag */
#define ATTN_ERR_UNSUPPORTED 2 /* valid request outside what is built (head_dim, dtype, alignment) */
#define ATTN_ERR_WORKSPACE 3   /* workspace missing or too small */
#define ATTN_ERR_HIP 4         /* a HIP launch failed; attn_last_error() holds the HIP message */
#define ATTN_ERR_NONFINITE 5   /* ATTN_CHECK_FINITE found a NaN or infinity in an output */

/* Element types. */
#define ATTN_DTYPE_F32 0
#define ATTN_DTYPE_BF16 1

/* attn_fwd_partial flags. */
#define ATTN_FWD_ACCUMULATE (1u << 0) /* (o, lse) hold a running fp32 result over earlier key
                                         chunks; replace it by merge(running, this chunk) */
#define ATTN_FWD_BALANCED (1u << 1)   /* causal work order pairing early and late query tiles */

/*
 * attn_fwd_partial: exact attention of q over the keys of one chunk.
 *
 * q [batch, seqlen_q, heads_q, head_dim], k and v [batch, seqlen_k, heads_kv, head_dim],
 * all of element type `dtype`; query head h reads key/value head
 * h / (heads_q / heads_kv) (heads_q must be a multiple of heads_kv).
 * Writes o [batch, seqlen_q, heads_q, head_dim] of type o_dtype and
 * lse [batch, heads_q, seqlen_q] fp32.  With ATTN_FWD_ACCUMULATE, o must be fp32
 * and (o, lse) are read as the running result before being replaced by the
 * merged one; a chunk that no query can see then changes nothing.  If o_final is
 * not NULL, the (merged) output is also written there as bf16.
 * Aliasing: o, lse and o_final must not overlap q, k, v or each other.
 *
 * Packed variable-length batches (cu_seqlens_q and cu_seqlens_k not NULL; the
 * variable-length form of the pages' per-device shards): `batch` sequences
 * are packed along the sequence axis.  cu_seqlens_q and cu_seqlens_k are
 * device int32 arrays of batch + 1 non-decreasing offsets starting at 0;
 * sequence b's queries are rows cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1 of q
 * and o, its keys rows cu_seqlens_k[b] .. cu_seqlens_k[b + 1] - 1 of k and v,
 * and the batch strides are ignored.  seqlen_q and seqlen_k must be at least
 * the longest query and key lengths (they size the launch; longer sequences
 * are cut to them).  Sequence b's query i sits at position
 * i + len_k(b) - len_q(b) and key j at position j (the queries are the last
 * len_q(b) positions of the sequence), so q_pos0 and k_pos0 must be 0.  lse is
 * then [total queries, heads_q] fp32.  dtype must be ATTN_DTYPE_BF16.  The
 * offsets are read on the device; offsets outside the tensors are the
 * caller's error and are not detected.
 */
typedef struct attn_fwd_args {
  uint32_t struct_size;
  uint32_t dtype; /* ATTN_DTYPE_BF16 or ATTN_DTYPE_F32: type of q, k, v */
  int32_t batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim;
  const void* q;
  int64_t q_stride[3];
  const void* k;
  int64_t k_stride[3];
  const void* v;
  int64_t v_stride[3];
  void* o;
  int64_t o_stride[3];
  uint32_t o_dtype; /* ATTN_DTYPE_F32 or ATTN_DTYPE_BF16 (the latter only without ACCUMULATE) */
  float* lse;       /* [batch, heads_q, seqlen_q] */
  void* o_final;    /* optional bf16 copy of the output, NULL to skip */
  int64_t o_final_stride[3];
  int64_t q_pos0, k_pos0; /* global positions of query 0 and key 0 */
  int32_t causal;
  float scale;
  uint32_t flags; /* ATTN_FWD_* */
  const int32_t* cu_seqlens_q; /* packed variable-length batches: device [batch + 1], or NULL */
  const int32_t* cu_seqlens_k; /* device [batch + 1], or NULL */
} attn_fwd_args;

ATTN_API int attn_fwd_partial(const attn_fwd_args* args, void* stream);

#define ATTN_MAX_CHUNKS 64

/*
 * attn_fwd_chunks: the forward of a query shard over a sequence of key/value
 * chunks in one call -- the aggregation of local results of the BurstAttention
 * and ring-attention pages, with the running (O, LSE) of each query kept on
 * chip across the chunks instead of being merged through memory chunk by
 * chunk.  The result equals attn_fwd_partial over the union of the chunks'
 * keys (key j of chunk c sits at global position chunk_pos0[c] + j), which is
 * also what chained attn_fwd_partial(ACCUMULATE) calls over the chunks give.
 *
 * Chunk c is a key tensor k_chunks[c] and a value tensor v_chunks[c], both
 * [batch, chunk_len[c], heads_kv, head_dim] bf16.  Their sequence and head
 * element strides are the shared k_stride[1..2] / v_stride[1..2]; the batch
 * stride is chunk_k_bstride[c] / chunk_v_bstride[c], or k_stride[0] /
 * v_stride[0] for every chunk when those arrays are NULL (so separately
 * allocated chunks of different lengths can be passed).  k_chunks, v_chunks,
 * chunk_len, chunk_pos0 and the batch-stride arrays are HOST arrays of
 * n_chunks entries (read during the call; the device pointers they hold must
 * stay valid until the stream work finishes).  A
 * chunk of length 0 is skipped.  dtype must be ATTN_DTYPE_BF16.  o, lse,
 * o_final, ACCUMULATE and BALANCED behave as in attn_fwd_partial; a query that
 * sees no key of any chunk gets O = 0, LSE = -inf (or, with ACCUMULATE, keeps
 * its running result).
 */
typedef struct attn_fwd_chunks_args {
  uint32_t struct_size;
  uint32_t dtype; /* ATTN_DTYPE_BF16 */
  int32_t batch, heads_q, heads_kv, seqlen_q, head_dim;
  int32_t n_chunks; /* 0 .. ATTN_MAX_CHUNKS */
  const void* q;
  int64_t q_stride[3];
  const void* const* k_chunks;  /* host array of n_chunks device pointers */
  const void* const* v_chunks;  /* host array of n_chunks device pointers */
  const int32_t* chunk_len;     /* host array: keys in each chunk (>= 0) */
  const int64_t* chunk_pos0;    /* host array: global position of each chunk's key 0 */
  int64_t k_stride[3];
  int64_t v_stride[3];
  const int64_t* chunk_k_bstride; /* host array or NULL: batch stride of each key chunk */
  const int64_t* chunk_v_bstride; /* host array or NULL: batch stride of each value chunk */
  void* o;
  int64_t o_stride[3];
  uint32_t o_dtype; /* ATTN_DTYPE_F32 or ATTN_DTYPE_BF16 (the latter only without ACCUMULATE) */
  float* lse;       /* [batch, heads_q, seqlen_q] */
  void* o_final;    /* optional bf16 copy of the output, NULL to skip */
  int64_t o_final_stride[3];
  int64_t q_pos0;
  int32_t causal;
  float scale;
  uint32_t flags; /* ATTN_FWD_ACCUMULATE, ATTN_FWD_BALANCED */
} attn_fwd_chunks_args;

ATTN_API int attn_fwd_chunks(const attn_fwd_chunks_args* args, void* stream);

/* attn_merge_lse modes. */
#define ATTN_MERGE_SEQUENTIAL 0 /* fold parts 0, 1, ..., n-1 in order */
#define ATTN_MERGE_TREE 1       /* binary tree: adjacent pairs per level, odd part carried */

/*
 * attn_merge_lse: merge n partial results over disjoint key sets.
 *
 * Part c is O_c [batch, seqlen, heads, head_dim] fp32 at o_parts + c * o_part_stride
 * (element strides o_stride) and LSE_c [batch, heads, seqlen] fp32 at
 * lse_parts + c * lse_part_stride.  With m = max_c LSE_c:
 * LSE = m + ln sum_c exp(LSE_c - m) and O = sum_c exp(LSE_c - LSE) O_c; parts
 * with LSE_c = -inf contribute nothing and an all -inf row gives O = 0, LSE = -inf;
 * a NaN LSE_c makes the row's O and LSE NaN.
 * The part strides are element offsets between consecutive parts (nonzero
 * when n_parts > 1) and may be negative, so two partials in separate buffers A
 * and B (same strides, both 16-byte aligned) are merged as a pair with
 * o_parts = A and o_part_stride = B - A in fp32 elements (likewise for the
 * LSE); this is the two-pointer form of the merge.
 * o_out may be fp32 or bf16; it may alias part 0 exactly (same pointer and
 * strides, fp32), and lse_out may alias part 0's LSE.  No other overlap.
 */
typedef struct attn_merge_args {
  uint32_t struct_size;
  int32_t n_parts; /* >= 1 */
  int32_t batch, seqlen, heads, head_dim;
  const float* o_parts;
  int64_t o_part_stride;
  int64_t o_stride[3];
  const float* lse_parts;
  int64_t lse_part_stride;
  void* o_out;
  int64_t o_out_stride[3];
  uint32_t o_out_dtype;
  float* lse_out;
  uint32_t mode; /* ATTN_MERGE_* */
} attn_merge_args;

ATTN_API int attn_merge_lse(const attn_merge_args* args, void* stream);

/* attn_bwd flags. */
#define ATTN_BWD_COMPUTE_DELTA (1u << 0) /* fill the workspace from o, dout and lse first; else reuse it */
#define ATTN_BWD_DQ_OVERWRITE (1u << 1)  /* dq_acc = this chunk's dQ instead of dq_acc += it */
#define ATTN_BWD_FINALIZE_DQ (1u << 2)   /* after accumulating, write dq = dq_acc in `dtype` */
#define ATTN_BWD_BALANCED (1u << 3)      /* causal work order pairing early and late key tiles */
/* Ask for results that do not depend on scheduling (no floating-point atomics).  Every backward
 * call of this library is deterministic, so the flag is accepted and changes nothing. */
#define ATTN_BWD_DETERMINISTIC (1u << 4)

/*
 * attn_bwd: gradients of sum(dO * O) for one chunk of keys.
 *
 * q, o, dout [batch, seqlen_q, heads_q, head_dim]; k, v [batch, seqlen_k, heads_kv,
 * head_dim]; all of element type `dtype`.  o and lse are the FINAL (merged over
 * every chunk) forward output and row LSE.  With P_ij = exp(s_ij - LSE_i) on
 * visible pairs, delta_i = sum dO_i * O_i and dS_ij = P_ij (dO_i . v_j - delta_i):
 *   dv_j = sum_i P_ij dO_i,   dk_j = scale sum_i dS_ij q_i   (written, this chunk's keys)
 *   dq_i += scale sum_j dS_ij k_j                           (accumulated in dq_acc)
 * With grouped heads, dk/dv of a key/value head sum over the query heads that
 * share it.  dq_acc is fp32 [batch, seqlen_q, heads_q, head_dim] contiguous.
 * The workspace (device memory of at least attn_bwd_workspace_size(...) bytes,
 * 256-byte aligned) holds the per-row statistics: for each (b, h) in row-major
 * order, Sq_pad = round_up(seqlen_q, 64) floats of LSE * log2(e) (+inf for rows
 * with LSE = -inf and for padding rows) followed by Sq_pad floats of -delta (0 on
 * padding rows; in a packed variable-length batch b is the sequence, and rows
 * past its length are padding).  ATTN_BWD_COMPUTE_DELTA fills it; later calls for other key
 * chunks of the same o, dout and lse may reuse it without the flag.  A row with
 * LSE = -inf must have no visible key; it contributes nothing.  A chunk no query
 * sees writes dk = dv = 0 and adds nothing to dq.  Results do not depend on
 * scheduling: no floating-point atomics are used.  dq, dk, dv are written in
 * `dtype`.
 *
 * Packed variable-length batches (cu_seqlens_q and cu_seqlens_k not NULL) are
 * laid out and positioned as for attn_fwd_partial: q, o, dout, dq rows and k,
 * v, dk, dv rows are packed per sequence, lse is [total queries, heads_q],
 * dq_acc is [total queries, heads_q, head_dim] fp32 contiguous, seqlen_q and
 * seqlen_k are the longest lengths, and q_pos0 = k_pos0 = 0.  bf16 only.
 */
typedef struct attn_bwd_args {
  uint32_t struct_size;
  uint32_t dtype;
  int32_t batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim;
  const void* q;
  int64_t q_stride[3];
  const void* k;
  int64_t k_stride[3];
  const void* v;
  int64_t v_stride[3];
  const void* o;
  int64_t o_stride[3];
  const void* dout;
  int64_t do_stride[3];
  const float* lse;
  void* workspace;
  size_t workspace_bytes;
  float* dq_acc;
  void* dq; /* used with ATTN_BWD_FINALIZE_DQ, else may be NULL */
  int64_t dq_stride[3];
  void* dk;
  int64_t dk_stride[3];
  void* dv;
  int64_t dv_stride[3];
  int64_t q_pos0, k_pos0;
  int32_t causal;
  float scale;
  uint32_t flags; /* ATTN_BWD_* */
  const int32_t* cu_seqlens_q; /* packed variable-length batches: device [batch + 1], or NULL */
  const int32_t* cu_seqlens_k; /* device [batch + 1], or NULL */
} attn_bwd_args;

ATTN_API int attn_bwd(const attn_bwd_args* args, void* stream);

/*
 * attn_bwd_chunks: the backward of a query shard over a sequence of key/value
 * chunks in one call -- the per-chunk backward of the BurstAttention and
 * ring-attention pages (each chunk's dK/dV from the global LSE and delta, dQ
 * summed over the chunks), with dQ kept on chip across the chunks instead of
 * passing through dq_acc once per chunk.  The result equals attn_bwd over the
 * union of the chunks' keys (key j of chunk c at global position
 * chunk_pos0[c] + j), which is also what chained attn_bwd calls over the chunks
 * give:
 *   dk_chunks[c], dv_chunks[c]  chunk c's key and value gradients (written; a
 *                               chunk no query sees gets zeros),
 *   dq_acc                      the sum of every chunk's dQ contribution,
 *                               written once (added to its contents without
 *                               ATTN_BWD_DQ_OVERWRITE),
 *   dq                          dq_acc in bf16 with ATTN_BWD_FINALIZE_DQ.
 * Chunks are given as in attn_fwd_chunks: k_chunks[c] and v_chunks[c] are
 * [batch, chunk_len[c], heads_kv, head_dim] bf16 with the shared sequence and
 * head strides k_stride[1..2] / v_stride[1..2] and batch stride
 * chunk_k_bstride[c] / chunk_v_bstride[c] (k_stride[0] / v_stride[0] when the
 * array is NULL); dk_chunks[c] and dv_chunks[c] likewise with dk_stride /
 * dv_stride and chunk_dk_bstride / chunk_dv_bstride.  All chunk arrays are HOST
 * arrays of n_chunks entries, read during the call (the device pointers they
 * hold must stay valid until the stream work finishes); a chunk of length 0 is
 * skipped.  q, o, dout, lse, workspace, dq_acc, dq, causal, scale and the flags
 * mean what they mean for attn_bwd; dtype must be ATTN_DTYPE_BF16.  Launches:
 * the statistics pass (with ATTN_BWD_COMPUTE_DELTA), one dK/dV kernel over the
 * key tiles of all chunks, one dQ kernel over all chunks.  No floating-point
 * atomics are used.
 */
typedef struct attn_bwd_chunks_args {
  uint32_t struct_size;
  uint32_t dtype; /* ATTN_DTYPE_BF16 */
  int32_t batch, heads_q, heads_kv, seqlen_q, head_dim;
  int32_t n_chunks; /* 0 .. ATTN_MAX_CHUNKS */
  const void* q;
  int64_t q_stride[3];
  const void* o;
  int64_t o_stride[3];
  const void* dout;
  int64_t do_stride[3];
  const float* lse;
  void* workspace;
  size_t workspace_bytes;
  float* dq_acc;
  void* dq; /* used with ATTN_BWD_FINALIZE_DQ, else may be NULL */
  int64_t dq_stride[3];
  const void* const* k_chunks;  /* host array of n_chunks device pointers */
  const void* const* v_chunks;  /* host array of n_chunks device pointers */
  void* const* dk_chunks;       /* host array of n_chunks device pointers */
  void* const* dv_chunks;       /* host array of n_chunks device pointers */
  const int32_t* chunk_len;     /* host array: keys in each chunk (>= 0) */
  const int64_t* chunk_pos0;    /* host array: global position of each chunk's key 0 */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t dk_stride[3];
  int64_t dv_stride[3];
  const int64_t* chunk_k_bstride;  /* host arrays or NULL: per-chunk batch strides */
  const int64_t* chunk_v_bstride;
  const int64_t* chunk_dk_bstride;
  const int64_t* chunk_dv_bstride;
  int64_t q_pos0;
  int32_t causal;
  float scale;
  uint32_t flags; /* ATTN_BWD_* */
} attn_bwd_chunks_args;

ATTN_API int attn_bwd_chunks(const attn_bwd_chunks_args* args, void* stream);

/*
 * attn_decode_splitkv: one query token per sequence over a KV cache.
 *
 * q [batch, heads_q, head_dim] bf16 (element strides q_stride = {batch, head});
 * k_cache, v_cache [batch, cache_len, heads_kv, head_dim] bf16; query head h reads
 * key/value head h / (heads_q / heads_kv).  The query attends every cached key
 * 0 .. len_b - 1 with len_b = seqlens[b] (device int32 [batch], each in
 * [0, cache_len]) or cache_len when seqlens is NULL; no causal mask applies.
 * Without seqlens, the keys are cut into n_splits contiguous splits of
 * ceil(cache_len / n_splits) keys; each split yields a partial (O, LSE) in the
 * workspace and the partials of each (b, h) are reduced by a binary tree of
 * adjacent pairs (an odd node is carried up a level): the tree is built over the
 * split LSEs, and O is the sum of the split partials weighted by their weights
 * in the tree's root, which is the tree's result up to the order of the
 * additions.
 * With seqlens (sequences of different lengths) and batch * n_splits <= 1024,
 * the work is cut into equal-key units instead (stream-K, as in the Lean
 * Attention abstract): the keys of all sequences in order form one range per
 * key/value head, cut into units of the same length (about 4096 keys, the
 * number of units rounded to whole rounds of the workgroups the device holds,
 * at most batch * n_splits).  A unit that crosses the end of a sequence yields
 * one partial per sequence it touches, and each (b, h) reduces its partials, in
 * key order, by the same adjacent-pair tree.  Larger batch * n_splits keep the
 * fixed splits.  Either way the result is the exact attention up to rounding.
 * Writes o [batch, heads_q, head_dim] bf16 (strides o_stride = {batch, head}) and
 * lse [batch, heads_q] fp32.  The workspace (device memory of at least
 * attn_decode_workspace_size(...) bytes, 256-byte aligned) is overwritten.
 */
typedef struct attn_decode_args {
  uint32_t struct_size;
  int32_t batch, heads_q, heads_kv, head_dim;
  int64_t cache_len;
  const void* q;
  int64_t q_stride[2];
  const void* k_cache;
  int64_t k_stride[3];
  const void* v_cache;
  int64_t v_stride[3];
  const int32_t* seqlens; /* optional */
  int32_t n_splits;       /* 1 .. 1024, power of two not required */
  float scale;
  void* o;
  int64_t o_stride[2];
  float* lse;
  void* workspace;
  size_t workspace_bytes;
} attn_decode_args;

ATTN_API int attn_decode_splitkv(const attn_decode_args* args, void* stream);

/*
 * attn_decode_splitkv_noalloc: attn_decode_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, same kernels and the same
 * results, except that `workspace` and `workspace_bytes` are ignored: the split
 * partials go to a fixed scratch array of 32 MiB inside the library, one per
 * device, which each device holds until the process ends.  The call makes no
 * allocation of any kind.
 *
 * Limit: attn_decode_workspace_size(batch, heads_q, head_dim, n_splits) must
 * not exceed 32 MiB (33554432 bytes), else ATTN_ERR_WORKSPACE.  For example,
 * batch 16 x heads_q 32 x 64 splits at head_dim 128 needs 16.1 MiB.
 *
 * The scratch of a device is looked up on the first call with that device
 * current (the device of `stream` must be current).  Every call on one device
 * shares that device's scratch, which keeps whatever the last call wrote; the
 * kernels write every partial before reading it, so nothing needs clearing.
 * Calls that overlap on one device (different streams, or host threads without
 * ordering between their streams) race on the scratch and may return wrong
 * results; calls on one stream are ordered and safe.
 */
ATTN_API int attn_decode_splitkv_noalloc(const attn_decode_args* args, void* stream);

/* Most nodes a decode tree may have (attn_decode_tree below). */
#define ATTN_MAX_TREE_NODES 256

/*
 * attn_decode_tree: one decode query per leaf of a prefix tree whose nodes own
 * segments of a packed KV cache (tree-structured decoding: DeFT, under the
 * Tree Attention page's related papers).  Queries are numbered so that the
 * queries below any node are contiguous (leaves in depth-first order): node n
 * owns keys kv_start[n] .. kv_start[n] + kv_len[n] - 1 of the cache and is on
 * the path of queries q_begin[n] .. q_end[n] - 1.  Query i attends, with no
 * mask, every key of every node whose query range holds i; query head h reads
 * key/value head h / (heads_q / heads_kv).  Each node's keys are read once per
 * key/value head for all of its queries and all query heads of the group; the
 * per-node partial results of a query are then combined by one LSE-weighted
 * sum (the same result as merging them in node order, up to rounding).  A
 * query that no node covers gets O = 0, LSE = -inf.
 *
 * q [n_queries, heads_q, head_dim] bf16 (strides q_stride = {query, head});
 * k_cache, v_cache [cache_len, heads_kv, head_dim] bf16 (strides {token, head});
 * o [n_queries, heads_q, head_dim] bf16 (strides o_stride); lse [n_queries, heads_q]
 * fp32 contiguous.  kv_start, kv_len, q_begin and q_end are HOST arrays of
 * n_nodes entries (0 <= n_nodes <= ATTN_MAX_TREE_NODES).  The workspace (device
 * memory of at least attn_decode_tree_workspace_size(args) bytes, 256-byte
 * aligned) receives the per-node partials and is overwritten.  Nodes with many
 * keys are processed as segments of up to 2048 keys (more when the segments of
 * all nodes would not fit ATTN_MAX_TREE_NODES table entries), each merged like
 * a node of its own.
 */
typedef struct attn_decode_tree_args {
  uint32_t struct_size;
  int32_t n_queries, heads_q, heads_kv, head_dim;
  int32_t n_nodes;
  int64_t cache_len;
  const void* q;
  int64_t q_stride[2];
  const void* k_cache;
  int64_t k_stride[2];
  const void* v_cache;
  int64_t v_stride[2];
  const int64_t* kv_start; /* host arrays of n_nodes entries */
  const int32_t* kv_len;
  const int32_t* q_begin;
  const int32_t* q_end;
  float scale;
  void* o;
  int64_t o_stride[2];
  float* lse;
  void* workspace;
  size_t workspace_bytes;
} attn_decode_tree_args;

ATTN_API int attn_decode_tree(const attn_decode_tree_args* args, void* stream);

/* Workspace bytes attn_decode_tree needs for these arguments (the node arrays, heads_q and
 * head_dim are read); 0 if they are invalid. */
ATTN_API size_t attn_decode_tree_workspace_size(const attn_decode_tree_args* args);

/* Bytes of workspace attn_bwd needs for these sizes (0 on invalid sizes). */
ATTN_API size_t attn_bwd_workspace_size(int32_t batch, int32_t heads_q, int32_t seqlen_q);

/* Bytes of workspace attn_decode_splitkv needs for these sizes (0 on invalid sizes):
 * batch * heads_q * (n_splits + 1) partial rows of head_dim + 1 floats. */
ATTN_API size_t attn_decode_workspace_size(int32_t batch, int32_t heads_q, int32_t head_dim, int32_t n_splits);

/* Static description of a status code. */
ATTN_API const char* attn_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
ATTN_API const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the built library. */
ATTN_API int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
