// Forward partial attention for bf16 inputs on gfx950 (CDNA4), bf16 MFMA with
// fp32 accumulation.
//
// Computes, for one chunk of keys, the exact softmax attention of a query
// shard: the local attention step of the BurstAttention page and the per-step
// blockwise computation of ring-style attention, as a partial (O, LSE).
//
// Layout of the work:
//   * each wavefront owns 32 queries of one (batch, head); a workgroup of 8
//     wavefronts (256 queries, one per CU) in the dense and chunk-table
//     kernels, of 4 (128 queries, two per CU) in the variable-length and tree
//     kernels;
//   * key and value tiles of 64 rows go straight from HBM to LDS
//     (global_load_lds, no register staging), double buffered: the next tile
//     streams in while the current one is used.  Chunks are swizzled so both
//     the row reads and the transposing reads are free of bank conflicts;
//   * scores are formed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA:
//     the accumulator puts one query per lane (column) and 16 of its keys in
//     the lane's registers, so row max and row sum are in-lane reductions plus
//     one exchange between the two half-waves (v_permlane32_swap);
//   * O^T += V^T P^T takes P^T straight from the registers; the V^T operand is
//     read from the row-major value tile with the transposing LDS read
//     (ds_read_b64_tr_b16), keys landing in the same slot order as P^T;
//   * the output accumulator is rescaled only when a row's running maximum
//     grows by more than 2^8 in exp2 units (the stale maximum is an equally
//     valid stabiliser, so the result is unchanged);
//   * causal tiles are classified per workgroup: tiles no query sees are never
//     visited, tiles every query sees skip the mask, the rest are masked per
//     element.
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"
#include "tile_lds.h"

namespace attn {
namespace {

// A wavefront owns 32 query rows.  The dense and chunk-table kernels run 8
// wavefronts (256 rows share each key/value tile in LDS, half the tile loads
// per query of 4 wavefronts); the variable-length and tree kernels run 4 (128
// rows), since their short sequences and small nodes would leave larger tiles
// mostly empty.
constexpr int NW_DENSE = 8, NW_SHORT = 4;
constexpr int BM = 32 * NW_SHORT;  // query rows per workgroup, variable-length and tree kernels
constexpr int NT = 64 * NW_SHORT;  // threads per workgroup, variable-length and tree kernels
constexpr int BM_D = 32 * NW_DENSE;  // the same, dense and chunk-table kernels
constexpr int NT_D = 64 * NW_DENSE;
constexpr int BN = 64;  // keys per tile
#ifndef SB_AHEAD_PV
#define SB_AHEAD_PV 3
#endif
#ifndef SB_AHEAD
#define SB_AHEAD 4
#endif
constexpr float kRescaleSlack = 8.0f;  // exp2 units a row max may grow before O is rescaled

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct RowState {
  float m;  // running maximum of the raw scores used as the stabiliser
  float l;  // this lane's partial row sum
};

// One 64-key tile: scores, online softmax, O^T update.
template <int D>
__device__ __forceinline__ void tile_step(const u16* ks, const u16* vs, const bf16x8* qf, f32x16* oacc,
                                          RowState& st, int key0, bool need_mask, int64_t lim64, float sl2,
                                          const RowFrag<D>& rf, const TrFrag<D>& tf, int lane) {
  constexpr int NS = D / 16, NDB = D / 32;
  const int lr = lane & 31, lg = lane >> 5;

  f32x16 sacc[2] = {f32x16{}, f32x16{}};
  {
    // Operand j = 2s + kb2.  Keep AH reads in flight ahead of the MFMA that
    // uses them: the hard scheduling boundaries hold each read in its slot.
    constexpr int NJ = 2 * NS, AH = SB_AHEAD;
    bf16x8 kf[NJ];
#pragma unroll
    for (int j = 0; j < AH; ++j) kf[j] = rf.get(ks, j & 1, j >> 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + AH < NJ) kf[j + AH] = rf.get(ks, (j + AH) & 1, (j + AH) >> 1);
      sacc[j & 1] = mfma32(kf[j], qf[j >> 1], sacc[j & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (need_mask) {
    const int lim = (int)max<int64_t>(-1, min<int64_t>(lim64 - key0, BN));
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kl = kb2 * 32 + (i >> 2) * 8 + lg * 4 + (i & 3);
        if (kl > lim) sacc[kb2][i] = neg_inf();
      }
  }
  float mt = sacc[0][0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sacc[0][i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[1][i]);
  mt = half_max(mt);
  // Rescale only when some row of the wavefront outgrows its stabiliser.
  const bool grow = (mt - st.m) * sl2 > kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float m_new = grow ? mt : st.m;
    const float alpha = grow ? exp2_fast((st.m - m_new) * sl2) : 1.f;  // 0 when st.m = -inf
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    st.m = m_new;
  }
  const float m_use = (st.m == neg_inf()) ? 0.f : st.m;
  const float nbias = -m_use * sl2;
  float rs = 0.f;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = exp2_fast(fmaf(sacc[kb2][i], sl2, nbias));
      sacc[kb2][i] = e;
      rs += e;
    }
  st.l += rs;

  // O^T += V^T P^T over four 16-key slabs; V^T comes from the transposing read.
  bf16x8 pb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int kb2 = ks >> 1, o = (ks & 1) * 8;
    pb[ks] = cvt_bf16x8(sacc[kb2][o + 0], sacc[kb2][o + 1], sacc[kb2][o + 2], sacc[kb2][o + 3],
                        sacc[kb2][o + 4], sacc[kb2][o + 5], sacc[kb2][o + 6], sacc[kb2][o + 7]);
  }
  {
    // Operand j = NDB ks + db, read AH fragments ahead as for the scores.
    constexpr int NJ = 4 * NDB, AH = SB_AHEAD_PV;
    bf16x8 vf[NJ];
#pragma unroll
    for (int j = 0; j < AH; ++j) vf[j] = tf.get(vs, j / NDB, j % NDB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + AH < NJ) vf[j + AH] = tf.get(vs, (j + AH) / NDB, (j + AH) % NDB);
      oacc[j % NDB] = mfma32(vf[j], pb[j / NDB], oacc[j % NDB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Epilogue: normalise, optionally merge into the running result, store.
template <int D>
__device__ __forceinline__ void fwd_store(const FwdParams& p, const f32x16* oacc, const RowState& st, int qi,
                                          bool qok, int b, int h, int lg) {
  constexpr int NDB = D / 32;
  const float l_tot = half_sum(st.l);
  if (!qok) return;
  // Only an exactly zero sum is a row with no visible key; a NaN score keeps
  // the sum NaN and so reaches the row's O and LSE.
  const bool empty = l_tot == 0.f;
  const float lse_this = empty ? neg_inf() : fmaf(st.m, p.scale, logf(l_tot));
  const float inv = empty ? 0.f : 1.0f / l_tot;
  float* lse_ptr = p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)qi * p.lse_ss;
  float w_old = 0.f, w_new = 1.f, L = lse_this;
  if (p.accumulate) merge_weights(*lse_ptr, lse_this, w_old, w_new, L);
  w_new *= inv;
  const int64_t orow = (int64_t)b * p.o.sb + (int64_t)qi * p.o.ss + (int64_t)h * p.o.sh;
  const int64_t frow = (int64_t)b * p.o_final.sb + (int64_t)qi * p.o_final.ss + (int64_t)h * p.o_final.sh;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = db * 32 + j * 8 + lg * 4;
      f32x4 v = {oacc[db][4 * j] * w_new, oacc[db][4 * j + 1] * w_new, oacc[db][4 * j + 2] * w_new,
                 oacc[db][4 * j + 3] * w_new};
      if (p.o_f32) {
        f32x4* dst = (f32x4*)((float*)p.o.ptr + orow + d);
        if (p.accumulate && w_old != 0.f) v += w_old * (*dst);
        *dst = v;
      } else {
        *(u32x2*)((u16*)p.o.ptr + orow + d) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
      if (p.o_final.ptr)
        *(u32x2*)((u16*)p.o_final.ptr + frow + d) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
  if (lg == 0) *lse_ptr = L;
}

// One tile of 128 rows against keys [0, Sk).  Normally row i is query i of head
// h.  With PACK (non-causal only) the rows are the queries of a whole GQA group:
// row r is query r / group of head h + r % group, so the group's heads share
// every key and value tile, and p.Sq counts rows (queries x group).
template <int D, int NW, bool PACK = false>
__device__ __forceinline__ void fwd_tile(const FwdParams& p, u16* k0s, u16* v0s, u16* k1s, u16* v1s, int qt, int b,
                                         int h, const u16* qb, const u16* kb, const u16* vb) {
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int lr = lane & 31, lg = lane >> 5;

  const int q0 = qt * 32 * NW;
  const int qi = q0 + wave * 32 + lr;
  const bool qok = qi < p.Sq;
  int q_row = qi, h_row = h;  // query and head of this lane's row
  if constexpr (PACK) {
    q_row = qi / p.group;
    h_row = h + (qi - q_row * p.group);
  }

  // Keys [0, kv_end) are visible to some query of this tile; keys [0, full_end)
  // to all of them.  Causal visibility: key j is visible to query i iff j <= delta + i.
  const int q_last = min(q0 + 32 * NW, p.Sq) - 1;
  int kv_end = p.Sk, full_end = p.Sk;
  int64_t lim64 = (int64_t)p.Sk - 1;
  if (!PACK && p.causal) {
    kv_end = (int)max<int64_t>(0, min<int64_t>(p.delta + q_last + 1, p.Sk));
    full_end = (int)max<int64_t>(0, min<int64_t>(p.delta + q0 + 1, p.Sk));
    lim64 = min<int64_t>(p.delta + qi, lim64);
  }
  const int n_tiles = (kv_end + BN - 1) / BN;
  TileSrc<D, NW> ksrc, vsrc;
  ksrc.init(p.k.ss, wave, lane);
  vsrc.init(p.v.ss, wave, lane);
  auto issue = [&](u16* ks, u16* vs, int key0) {
    ksrc.issue(ks, kb, p.k.ss, key0, p.Sk, wave, lane);
    vsrc.issue(vs, vb, p.v.ss, key0, p.Sk, wave, lane);
  };
  if (n_tiles > 0) issue(k0s, v0s, 0);

  bf16x8 qf[NS];
  {
    const u16* qrow = qb + (int64_t)q_row * p.q.ss + (int64_t)(h_row - h) * p.q.sh + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = qok ? as_bf16x8(*(const u32x4*)(qrow + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  RowState st{neg_inf(), 0.f};
  const float sl2 = p.scale_log2;
  RowFrag<D> rf;
  TrFrag<D> tf;
  rf.init(lane);
  tf.init(lane);

  // With PACK, a wavefront whose rows all lie past the end only helps with the
  // loads and barriers (a node with few queries fills part of a tile).
  const bool live = !PACK || q0 + wave * 32 < p.Sq;
  for (int t = 0; t < n_tiles; t += 2) {
    wait_loads();
    __syncthreads();
    if (t + 1 < n_tiles) issue(k1s, v1s, (t + 1) * BN);
    if (live)
      tile_step<D>(k0s, v0s, qf, oacc, st, t * BN, t * BN + BN > full_end, lim64, sl2, rf, tf, lane);
    if (t + 1 >= n_tiles) break;
    wait_loads();
    __syncthreads();
    if (t + 2 < n_tiles) issue(k0s, v0s, (t + 2) * BN);
    if (live)
      tile_step<D>(k1s, v1s, qf, oacc, st, (t + 1) * BN, (t + 1) * BN + BN > full_end, lim64, sl2, rf, tf, lane);
  }
  __syncthreads();  // the next call of this function reuses the buffers

  fwd_store<D>(p, oacc, st, q_row, qok, b, h_row, lg);
}

template <int D>
__global__ __launch_bounds__(NT_D) void fwd_bf16_kernel(FwdParams p) {
  // Two separate LDS objects per buffer so the compiler can tell the tile being
  // read from the tile being filled.
  __shared__ __attribute__((aligned(16))) u16 k0s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v0s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 k1s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v1s[SwTile<D>::SIZE];
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_units;
  const int bh = lin / p.n_units;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int hk = h / p.group;
  const u16* qb = (const u16*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
  const u16* kb = (const u16*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const u16* vb = (const u16*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;
  if (p.balanced) {
    // Pair an early and a late query tile so every workgroup carries the same causal work.
    const int t0 = unit, t1 = p.n_qtiles - 1 - unit;
    fwd_tile<D, NW_DENSE>(p, k0s, v0s, k1s, v1s, t1, b, h, qb, kb, vb);
    if (t0 != t1) fwd_tile<D, NW_DENSE>(p, k0s, v0s, k1s, v1s, t0, b, h, qb, kb, vb);
  } else {
    // Causal: heaviest tiles first, so the light ones fill the tail.
    const int qt = p.causal ? p.n_qtiles - 1 - unit : unit;
    fwd_tile<D, NW_DENSE>(p, k0s, v0s, k1s, v1s, qt, b, h, qb, kb, vb);
  }
}

// Packed variable-length batches: workgroup (sequence b, head h, unit) runs the
// same tiles with every pointer moved to the sequence's first row, that
// sequence's lengths, and its queries aligned to the end of its keys (query i
// sees keys j <= i + Sk_b - Sq_b).  Lengths are clamped to the declared longest
// ones; units past a sequence's tiles exit at once.
template <int D>
__global__ __launch_bounds__(NT, 2) void fwd_varlen_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) u16 k0s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v0s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 k1s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v1s[SwTile<D>::SIZE];
  const SeqHeadUnit w = varlen_order(blockIdx.x, p.Hq, p.n_units);
  const int unit = w.unit, h = w.h, b = w.b;
  const int hk = h / p.group;
  const int q_beg = p.cu_q[b], k_beg = p.cu_k[b];
  FwdParams s = p;
  s.Sq = min(max(p.cu_q[b + 1] - q_beg, 0), p.Sq);
  s.Sk = min(max(p.cu_k[b + 1] - k_beg, 0), p.Sk);
  s.delta = (int64_t)s.Sk - s.Sq;
  s.n_qtiles = (s.Sq + BM - 1) / BM;
  const int64_t o_el = p.o_f32 ? 4 : 2;
  s.o.ptr = (char*)p.o.ptr + (int64_t)q_beg * p.o.ss * o_el;
  if (p.o_final.ptr) s.o_final.ptr = (u16*)p.o_final.ptr + (int64_t)q_beg * p.o_final.ss;
  s.lse = p.lse + (int64_t)q_beg * p.lse_ss;
  const u16* qb = (const u16*)p.q.ptr + (int64_t)q_beg * p.q.ss + (int64_t)h * p.q.sh;
  const u16* kb = (const u16*)p.k.ptr + (int64_t)k_beg * p.k.ss + (int64_t)hk * p.k.sh;
  const u16* vb = (const u16*)p.v.ptr + (int64_t)k_beg * p.v.ss + (int64_t)hk * p.v.sh;
  if (p.balanced) {
    const int t0 = unit, t1 = s.n_qtiles - 1 - unit;
    if (t1 < t0) return;
    fwd_tile<D, NW_SHORT>(s, k0s, v0s, k1s, v1s, t1, 0, h, qb, kb, vb);
    if (t0 != t1) fwd_tile<D, NW_SHORT>(s, k0s, v0s, k1s, v1s, t0, 0, h, qb, kb, vb);
  } else {
    if (unit >= s.n_qtiles) return;
    const int qt = p.causal ? s.n_qtiles - 1 - unit : unit;
    fwd_tile<D, NW_SHORT>(s, k0s, v0s, k1s, v1s, qt, 0, h, qb, kb, vb);
  }
}

// ------------------------------------------------------ tree decode -------
//
// Tree-structured decoding (DeFT under the Tree Attention page's related
// papers): the queries below a node of a prefix tree share that node's keys.
// Pass 1 reads each node's keys once per key/value head for all of its queries
// and all query heads of the GQA group (workgroup = node, key/value head, tile
// of 128 rows of (query, head in group)), through the same tile code as the
// forward, and writes a partial (O, LSE) per (node, query, head).  Pass 2
// merges each query's partials in node order.

//
// The grid holds only tiles that have rows: (segment, row tile) pairs are
// numbered through the prefix u0, in segment order, so the long tiles of the
// nodes near the root are dispatched first and no workgroup exits empty.  (A
// grid padded to the largest node's tile count interleaves empty workgroups
// with live ones; the dispatcher then spreads the live ones unevenly over the
// shader engines, and leaf tiles waited for the root's to finish instead of
// taking the CUs' free slots.)  Key/value heads go round the XCDs.
template <int D>
__global__ __launch_bounds__(NT, 2) void tree_fwd_kernel(FwdParams p, TreeTable tt) {
  __shared__ __attribute__((aligned(16))) u16 k0s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v0s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 k1s[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v1s[SwTile<D>::SIZE];
  constexpr int kXcd = 8;
  const int bid = blockIdx.x;
  int hk, idx;
  if (p.Hkv % kXcd == 0) {
    const int hpx = p.Hkv / kXcd, s_ = bid / kXcd;
    hk = (s_ % hpx) * kXcd + bid % kXcd;
    idx = s_ / hpx;
  } else {
    hk = bid % p.Hkv;
    idx = bid / p.Hkv;
  }
  int n = 0, hi = tt.n - 1;  // the segment holding tile idx: the last n with u0[n] <= idx
  while (n < hi) {
    const int mid = (n + hi + 1) >> 1;
    if (tt.u0[mid] <= idx) n = mid;
    else hi = mid - 1;
  }
  const int unit = idx - tt.u0[n];
  const int h0 = hk * p.group;
  FwdParams s = p;
  s.Sq = (tt.q_end[n] - tt.q_begin[n]) * p.group;  // rows: (query, head in group)
  s.Sk = tt.kv_len[n];
  s.n_qtiles = (s.Sq + BM - 1) / BM;
  s.o.ptr = (float*)p.o.ptr + (int64_t)tt.e0[n] * p.o.ss;
  s.lse = p.lse + (int64_t)tt.e0[n] * p.lse_ss;
  const u16* qb = (const u16*)p.q.ptr + (int64_t)tt.q_begin[n] * p.q.ss + (int64_t)h0 * p.q.sh;
  const u16* kb = (const u16*)p.k.ptr + tt.kv_start[n] * p.k.ss + (int64_t)hk * p.k.sh;
  const u16* vb = (const u16*)p.v.ptr + tt.kv_start[n] * p.v.ss + (int64_t)hk * p.v.sh;
  fwd_tile<D, NW_SHORT, true>(s, k0s, v0s, k1s, v1s, unit, 0, h0, qb, kb, vb);
}

// One workgroup per (query, head), one thread per feature.  The first
// wavefront lists the query's partials in node order (an ordered compaction of
// the nodes whose range holds the query), then the partials are combined in
// one LSE-weighted sum stabilised by their largest LSE: every load of the sum
// is independent of the others, unlike a chain of pairwise merges, and the
// result is the same up to rounding (the merge is associative).
template <int D>
__global__ __launch_bounds__(D) void tree_merge_kernel(const float* po, const float* pl, int Hq, TreeTable tt,
                                                       u16* out_o, int64_t o_sq, int64_t o_sh, float* out_lse) {
  __shared__ int ent[kMaxTreeNodes];  // partial rows of this query, in node order
  __shared__ float lv[kMaxTreeNodes];  // their LSE
  __shared__ int n_ent;
  const int i = blockIdx.x / Hq, h = blockIdx.x % Hq, t = threadIdx.x;
  if (t < 64) {
    int k = 0;
    for (int n0 = 0; n0 < tt.n; n0 += 64) {
      const int n = n0 + t;
      const int nc = min(n, tt.n - 1);
      const int qb = tt.q_begin[nc], qe = tt.q_end[nc], e = tt.e0[nc] + (i - qb);
      const bool hit = (n < tt.n) & (i >= qb) & (i < qe);
      const unsigned long long m = __ballot(hit);
      if (hit) ent[k + __popcll(m & ((1ull << t) - 1ull))] = e;
      k += __popcll(m);
    }
    if (t == 0) n_ent = k;
  }
  __syncthreads();
  const int K = n_ent;
  for (int k = t; k < K; k += D) lv[k] = pl[(int64_t)ent[k] * Hq + h];
  __syncthreads();
  float M = neg_inf();
  for (int k = 0; k < K; ++k) M = fmaxf(M, lv[k]);
  // An empty partial (LSE -inf) has weight 0 even when every partial is
  // empty; a NaN LSE gives NaN weights, so it reaches O and the LSE.
  float S = 0.f, O = 0.f;
#pragma unroll 8
  for (int k = 0; k < K; ++k) {
    const float w = (lv[k] == neg_inf()) ? 0.f : expf(lv[k] - M);
    S += w;
    O = fmaf(w, po[((int64_t)ent[k] * Hq + h) * D + t], O);
  }
  const bool empty = S == 0.f;
  out_o[(int64_t)i * o_sq + (int64_t)h * o_sh + t] = f32_to_bf16(empty ? 0.f : O / S);
  if (t == 0) out_lse[(int64_t)i * Hq + h] = empty ? neg_inf() : M + logf(S);
}

// ------------------------------------------------------ fused chunk table --
//
// The same tile step over the keys of several chunks, in chunk order, in one
// launch: the online softmax state and O^T stay in registers from the first
// chunk to the last, and the result is written once.  Each chunk's causal
// visibility is classified from its own global position; chunks or tiles no
// query of the tile sees are skipped.  The next tile (possibly the first of a
// later chunk) streams into the other LDS buffer while the current one is
// used; the loads are untracked by the compiler and waited for explicitly.

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier for LDS data only; the tile prefetch stays in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D, int NW>
__device__ __forceinline__ void fwd_chunk_tile(const FwdParams& p, const ChunkTable& ct, u16* k_s, u16* v_s, int qt,
                                               int b, int h, int hk, const u16* qb) {
  constexpr int NS = D / 16, NDB = D / 32, SZ = SwTile<D>::SIZE;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int lr = lane & 31, lg = lane >> 5;
  const int q0 = qt * 32 * NW;
  const int qi = q0 + wave * 32 + lr;
  const bool qok = qi < p.Sq;
  const int q_last = min(q0 + 32 * NW, p.Sq) - 1;

  // Keys [0, kv_end) of chunk c are visible to some query of this tile, keys
  // [0, full_end) to all of them.
  auto chunk_range = [&](int c, int& kv_end, int& full_end) {
    const int len = ct.len[c];
    kv_end = full_end = len;
    if (p.causal) {
      const int64_t dl = ct.q_pos0 - ct.pos0[c];
      kv_end = (int)max<int64_t>(0, min<int64_t>(dl + q_last + 1, len));
      full_end = (int)max<int64_t>(0, min<int64_t>(dl + q0 + 1, len));
    }
  };
  auto n_tiles_of = [&](int c) {
    int e, f;
    chunk_range(c, e, f);
    return (e + BN - 1) / BN;
  };
  auto first_from = [&](int c) {
    while (c < ct.n && n_tiles_of(c) == 0) ++c;
    return c;
  };

  bf16x8 qf[NS];
  {
    const u16* qrow = qb + (int64_t)qi * p.q.ss + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = qok ? as_bf16x8(*(const u32x4*)(qrow + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  wait_vm<0>();  // the query rows are complete before any tile load is in flight
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  RowState st{neg_inf(), 0.f};
  const float sl2 = p.scale_log2;
  RowFrag<D> rf;
  TrFrag<D> tf;
  rf.init(lane);
  tf.init(lane);

  TileSrc<D, NW> ksrc, vsrc;
  ksrc.init(p.k.ss, wave, lane);
  vsrc.init(p.v.ss, wave, lane);
  // What the steps need of a chunk, read from the table once per chunk (the
  // table lives in kernel-argument memory: a read per step would put a scalar
  // load's latency into every step).
  struct Chunk {
    const u16* kb;
    const u16* vb;
    int len, kv_end, full_end;
    int64_t lim64;  // this lane's last visible key of the chunk
  };
  auto chunk_of = [&](int cc) {
    Chunk k;
    k.kb = (const u16*)ct.k[cc] + (int64_t)b * ct.kb[cc] + (int64_t)hk * p.k.sh;
    k.vb = (const u16*)ct.v[cc] + (int64_t)b * ct.vb[cc] + (int64_t)hk * p.v.sh;
    k.len = ct.len[cc];
    chunk_range(cc, k.kv_end, k.full_end);
    k.lim64 = (int64_t)k.len - 1;
    if (p.causal) k.lim64 = min<int64_t>(ct.q_pos0 - ct.pos0[cc] + qi, k.lim64);
    return k;
  };
  auto issue = [&](const Chunk& k, int tile, int slot) {
    ksrc.issue(k_s + slot * SZ, k.kb, p.k.ss, tile * BN, k.len, wave, lane);
    vsrc.issue(v_s + slot * SZ, k.vb, p.v.ss, tile * BN, k.len, wave, lane);
  };

  int c = first_from(0), t = 0;
  Chunk cur{};
  if (c < ct.n) {
    cur = chunk_of(c);
    issue(cur, 0, 0);
    wait_vm<0>();
    lds_barrier();
  }
  // One step per tile; the loop is unrolled over the two LDS slots so that each
  // step's slot is a compile-time constant folded into its LDS read offsets.
  auto step = [&](auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    // Next tile in sequence: the rest of this chunk, then the next chunk with visible keys.
    int nc = c, nt = t + 1;
    Chunk nxt = cur;
    if (nt * BN >= cur.kv_end) {
      nc = first_from(c + 1);
      nt = 0;
      if (nc < ct.n) nxt = chunk_of(nc);
    }
    if (nc < ct.n) issue(nxt, nt, SLOT ^ 1);
    tile_step<D>(k_s + SLOT * SZ, v_s + SLOT * SZ, qf, oacc, st, t * BN, t * BN + BN > cur.full_end, cur.lim64, sl2,
                 rf, tf, lane);
    wait_vm<0>();  // the next tile, the only load in flight
    lds_barrier();
    c = nc;
    t = nt;
    cur = nxt;
  };
  while (c < ct.n) {
    step(std::integral_constant<int, 0>{});
    if (c >= ct.n) break;
    step(std::integral_constant<int, 1>{});
  }
  fwd_store<D>(p, oacc, st, qi, qok, b, h, lg);
}

template <int D>
__global__ __launch_bounds__(NT_D) void fwd_chunks_kernel(FwdParams p, ChunkTable ct) {
  __shared__ __attribute__((aligned(16))) u16 k_s[2 * SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v_s[2 * SwTile<D>::SIZE];
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_units;
  const int bh = lin / p.n_units;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int hk = h / p.group;
  const u16* qb = (const u16*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
  // Balanced: pair a late and an early query tile; otherwise causal grids run
  // the heaviest tiles first.
  const int last = p.n_qtiles - 1 - unit;
  const int n = (p.balanced && last != unit) ? 2 : 1;
  for (int k = 0; k < n; ++k) {
    const int qt = p.balanced ? (k == 0 ? last : unit) : (p.causal ? last : unit);
    fwd_chunk_tile<D, NW_DENSE>(p, ct, k_s, v_s, qt, b, h, hk, qb);
  }
}

}  // namespace

int64_t items_fwd_bf16(const FwdParams& p) {
  const int bm = p.cu_q ? BM : BM_D, nt = p.cu_q ? NT : NT_D;
  const int64_t n_qtiles = (p.Sq + bm - 1) / bm;
  const int64_t n_units = p.balanced ? (n_qtiles + 1) / 2 : n_qtiles;
  return (int64_t)p.B * p.Hq * n_units * nt;
}

// Row tiles of the tree pass over all segments; with u0, fills the prefix.
static int64_t tree_tiles(const TreeTable& tt, int group, int* u0) {
  int64_t t = 0;
  for (int i = 0; i < tt.n; ++i) {
    if (u0) u0[i] = (int)t;
    t += ((int64_t)(tt.q_end[i] - tt.q_begin[i]) * group + BM - 1) / BM;
  }
  if (u0) u0[tt.n] = (int)t;
  return t;
}

int64_t items_tree_decode(const FwdParams& p, const TreeTable& tt, int n_q, int D) {
  return std::max<int64_t>(tree_tiles(tt, p.group, nullptr) * p.Hkv * NT, (int64_t)n_q * p.Hq * D);
}

hipError_t launch_fwd_chunks_bf16(const FwdParams& p0, const ChunkTable& ct, int D, hipStream_t s) {
  FwdParams p = p0;
  p.n_qtiles = (p.Sq + BM_D - 1) / BM_D;
  p.n_units = p.balanced ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
  const int64_t grid = (int64_t)p.B * p.Hq * p.n_units;
  if (grid == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(fwd_chunks_kernel<128>, dim3((unsigned)grid), dim3(NT_D), 0, s, p, ct);
  else
    hipLaunchKernelGGL(fwd_chunks_kernel<64>, dim3((unsigned)grid), dim3(NT_D), 0, s, p, ct);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdParams& p0, int D, hipStream_t s) {
  FwdParams p = p0;
  const int bm = p.cu_q ? BM : BM_D;
  p.n_qtiles = (p.Sq + bm - 1) / bm;
  p.n_units = p.balanced ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
  const int64_t grid = (int64_t)p.B * p.Hq * p.n_units;
  if (grid == 0) return hipSuccess;
  if (p.cu_q) {
    if (D == 128)
      hipLaunchKernelGGL(fwd_varlen_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    else
      hipLaunchKernelGGL(fwd_varlen_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    return hipGetLastError();
  }
  if (D == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((unsigned)grid), dim3(NT_D), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((unsigned)grid), dim3(NT_D), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_tree_decode(const FwdParams& p0, const TreeTable& tt, int n_q, void* out_o, int64_t out_o_sq,
                              int64_t out_o_sh, float* out_lse, int D, hipStream_t s) {
  FwdParams p = p0;
  TreeTable t = tt;
  const int64_t grid = tree_tiles(t, p.group, t.u0) * p.Hkv;
  if (grid > 0) {
    if (D == 128)
      hipLaunchKernelGGL(tree_fwd_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p, t);
    else
      hipLaunchKernelGGL(tree_fwd_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p, t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t gm = (int64_t)n_q * p.Hq;
  if (gm == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(tree_merge_kernel<128>, dim3((unsigned)gm), dim3(128), 0, s, (const float*)p.o.ptr, p.lse,
                       p.Hq, tt, (u16*)out_o, out_o_sq, out_o_sh, out_lse);
  else
    hipLaunchKernelGGL(tree_merge_kernel<64>, dim3((unsigned)gm), dim3(64), 0, s, (const float*)p.o.ptr, p.lse, p.Hq,
                       tt, (u16*)out_o, out_o_sq, out_o_sh, out_lse);
  return hipGetLastError();
}

}  // namespace attn
