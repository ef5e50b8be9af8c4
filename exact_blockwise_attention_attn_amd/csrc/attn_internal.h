// Internal parameter blocks passed by value to the kernels, and the host-side
// launchers each kernel file exports to the ABI layer.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// One [batch, seq, head, dim] tensor view: base pointer plus element strides.
struct View {
  const void* ptr;
  int64_t sb, ss, sh;
};

struct MView {
  void* ptr;
  int64_t sb, ss, sh;
};

struct FwdParams {
  View q, k, v;
  MView o;
  MView o_final;  // ptr == nullptr to skip
  float* lse;
  int64_t lse_sb, lse_sh, lse_ss;  // element strides of lse over (batch, head, query)
  // Packed variable-length batches: sequence b's queries are rows cu_q[b] ..
  // cu_q[b + 1] - 1 of q and o, its keys rows cu_k[b] .. cu_k[b + 1] - 1 of k
  // and v (device arrays; nullptr for the dense layout).  Sq and Sk are then
  // the longest lengths, and each sequence's queries sit at the end of its keys.
  const int* cu_q;
  const int* cu_k;
  int B, Hq, Hkv, Sq, Sk;
  int group;        // Hq / Hkv
  int64_t delta;    // q_pos0 - k_pos0: key j is visible to query i iff j <= delta + i (causal)
  int causal;
  int o_f32;        // o is fp32 (else bf16)
  int accumulate;   // merge into the running (o, lse)
  int balanced;     // each workgroup takes query tiles t and n-1-t
  float scale;      // softmax scale (natural units)
  float scale_log2; // scale * log2(e)
  int n_qtiles;     // query tiles per (b, h)
  int n_units;      // work units per (b, h) (n_qtiles, or ceil(n_qtiles / 2) when balanced)
};

// Key/value chunks of a fused multi-chunk forward: chunk c has len[c] keys at
// global positions pos0[c] .. pos0[c] + len[c] - 1, in tensors at k[c] and v[c]
// with batch strides kb[c], vb[c] and the sequence and head strides of
// FwdParams::k and FwdParams::v.
constexpr int kMaxChunks = 64;
struct ChunkTable {
  const void* k[kMaxChunks];
  const void* v[kMaxChunks];
  int64_t kb[kMaxChunks], vb[kMaxChunks];
  int64_t pos0[kMaxChunks];
  int len[kMaxChunks];
  int n;
  int64_t q_pos0;
};

struct MergeParams {
  const float* o_parts;
  int64_t o_part_stride, o_sb, o_ss, o_sh;
  const float* lse_parts;
  int64_t lse_part_stride;
  MView out;
  int out_f32;
  float* lse_out;
  int n_parts, B, S, H;
  int tree;
};

struct BwdParams {
  View q, k, v, o, dout;
  MView dq, dk, dv;
  const float* lse;
  int64_t lse_sb, lse_sh, lse_ss;  // element strides of lse over (batch, head, query)
  // Packed variable-length batches, as in FwdParams; dq_acc is then
  // [total queries, Hq, D] and the statistics of sequence b start at
  // b * Hq * 2 * Sq_pad with Sq_pad from the longest sequence.
  const int* cu_q;
  const int* cu_k;
  // Per-row statistics workspace: for each (b, h), Sq_pad floats of LSE*log2(e)
  // (+inf on rows that see no key and on padding rows) followed by Sq_pad
  // floats of -delta (0 on padding rows).  Sq_pad = Sq rounded up to 64.
  float* stats;
  int Sq_pad;
  float* dq_acc;  // contiguous [B, Sq, Hq, D]
  int B, Hq, Hkv, Sq, Sk;
  int group;
  int64_t delta_pos;  // q_pos0 - k_pos0
  int causal;
  int dq_overwrite;
  int finalize_dq;
  int balanced;
  float scale, scale_log2;
  int n_qtiles, n_ktiles, n_units_k;  // filled in by the launchers
};

// Key/value chunks of a fused multi-chunk backward: the forward's chunk table
// (keys, values, positions, lengths) plus each chunk's dK and dV outputs, with
// batch strides dkb[c], dvb[c] and the sequence and head strides of
// BwdParams::dk and BwdParams::dv.  unit0[c] is the first dK/dV work unit of
// chunk c (a prefix sum over the chunks); n_units is the total.
struct BwdChunkTable {
  ChunkTable kv;
  void* dk[kMaxChunks];
  void* dv[kMaxChunks];
  int64_t dkb[kMaxChunks], dvb[kMaxChunks];
  int unit0[kMaxChunks + 1];
  int n_units;
};

// Tree-structured decode: node n holds keys kv_start[n] .. + kv_len[n] - 1 of
// the packed cache and is attended by queries q_begin[n] .. q_end[n] - 1; its
// partial results go to workspace entries e0[n] .. e0[n] + (q_end - q_begin) - 1.
constexpr int kMaxTreeNodes = 256;
struct TreeTable {
  int64_t kv_start[kMaxTreeNodes];
  int kv_len[kMaxTreeNodes];
  int q_begin[kMaxTreeNodes], q_end[kMaxTreeNodes];
  int e0[kMaxTreeNodes];
  // Row tiles of the per-segment pass before segment i (filled by the launcher):
  // segment i owns tiles u0[i] .. u0[i + 1] - 1, one per 128 rows it holds.
  int u0[kMaxTreeNodes + 1];
  int n;
};

struct DecodeParams {
  const uint16_t* q;
  int64_t q_sb, q_sh;
  const uint16_t* k;
  int64_t k_sb, k_sl, k_sh;
  const uint16_t* v;
  int64_t v_sb, v_sl, v_sh;
  const int32_t* seqlens;
  int64_t L;
  int B, Hq, Hkv, group;
  int n_splits;
  int64_t split_len;
  float scale, scale_log2;
  float* part_o;    // fixed splits: [B, Hq, n_splits, D]; stream-K: [Hq, n_pieces, D]
  float* part_lse;  // fixed splits: [B, Hq, n_splits]; stream-K: [Hq, n_pieces]
  // Equal-key work units over sequences of different lengths (seqlens given,
  // B <= 1024 and B * n_splits <= 1024); n_pieces = B * (n_splits + 1) rows
  // of partials per query head, more than the U + B - 1 pieces there can be.
  int streamk;
  int64_t n_pieces;
  int sk_granule;  // stream-K units per (key/value head, head slice) in one round of resident workgroups
  uint16_t* o;
  int64_t o_sb, o_sh;
  float* lse;
};

// Launchers (return the launch status).  D is the head dimension.
// Largest number of work-items (workgroups x threads per workgroup) any one
// launch of the matching launcher would use, from the launcher's own grid
// formulas; a launch is limited to 2^32 - 1 work-items per grid dimension, and
// the host checks every launch of a call before enqueueing the first.
int64_t items_fwd_bf16(const FwdParams& p);
int64_t items_fwd_f32(const FwdParams& p);
int64_t items_merge(const MergeParams& p, int D);
int64_t items_bwd_prepare(const BwdParams& p, int D);
int64_t items_bwd_bf16(const BwdParams& p);
int64_t items_bwd_chunks_bf16(const BwdParams& p, const BwdChunkTable& ct);
int64_t items_bwd_f32(const BwdParams& p);
int64_t items_decode(const DecodeParams& p);
int64_t items_tree_decode(const FwdParams& p, const TreeTable& tt, int n_q, int D);

hipError_t launch_fwd_bf16(const FwdParams& p, int D, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int D, hipStream_t s);
// Fused forward over a chunk table (bf16): one launch, the running (O, LSE) of
// each query stays in registers across chunks.
hipError_t launch_fwd_chunks_bf16(const FwdParams& p, const ChunkTable& c, int D, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, int D, hipStream_t s);
// Backward: fill the statistics workspace (delta = rowsum(dO * O), rescaled
// LSE); then dK/dV (key-outer) and, when run_dq, dQ (query-outer, accumulated
// into dq_acc).  Both kernels write every row they own even when no pair is
// visible.
hipError_t launch_bwd_prepare(const BwdParams& p, int D, int is_bf16, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdParams& p, int D, int run_dq, hipStream_t s);
// dK/dV of every chunk of the table and dQ over all of them, in two launches.
// p supplies everything but the key/value tensors and their outputs; p.Sk and
// p.delta_pos are ignored.  The table's unit0 and n_units are filled in here.
hipError_t launch_bwd_chunks_bf16(const BwdParams& p, const BwdChunkTable& ct, int D, hipStream_t s);
hipError_t launch_bwd_f32(const BwdParams& p, int D, int run_dq, hipStream_t s);
// Decode: split partials into the workspace, then the per-(b, h) tree merge.
hipError_t launch_decode(const DecodeParams& p, int D, hipStream_t s);

// Fixed scratch of attn_decode_splitkv_noalloc (the split partials), one per
// device; noalloc_scratch gives its device address on the current device
// (looked up once per device).  It allocates nothing.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
hipError_t noalloc_scratch(void** ptr);
// Tree decode: p describes the queries (q, Hq, Hkv, group, scale), the packed
// cache (k, v with their token and head strides), the fp32 partials (o as
// [entries, Hq, D], lse as [entries, Hq]) and is the forward parameter block
// of the per-node pass; the merge writes out_o [n_q, Hq, D] bf16 and out_lse.
hipError_t launch_tree_decode(const FwdParams& p, const TreeTable& t, int n_q, void* out_o, int64_t out_o_sq,
                              int64_t out_o_sh, float* out_lse, int D, hipStream_t s);

// Debug scan of a call's outputs for non-finite values.  A view is up to four
// dimensions n[0..3] with element strides st[0..3] (unused dimensions have
// n = 1); the flat index of an element is row-major over n.
struct FiniteView {
  const void* ptr;
  int64_t n[4];
  int64_t st[4];
  int f32;            // element type fp32 (else bf16)
  int allow_neg_inf;  // -inf is a legitimate value (the LSE of a row with no visible key)
};
constexpr int kMaxFiniteViews = 2 * kMaxChunks + 4;
// Scans the views on s and waits for s; first[i] is the flat index of view i's
// first NaN or infinity (-inf excepted where allowed), or -1 if it has none.
// Calls are serialised within the process (they share one device buffer).
hipError_t finite_scan(const FiniteView* v, int n, hipStream_t s, int64_t* first);

}  // namespace attn
