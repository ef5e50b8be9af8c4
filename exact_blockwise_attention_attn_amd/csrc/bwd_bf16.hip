// Backward of exact attention for bf16 inputs on gfx950, from the saved final
// output O and row LSE: no re-run of the forward (DistFlashAttn digest,
// rematerialisation-aware gradient checkpointing).  bf16 MFMA with fp32
// accumulation everywhere.
//
// Two kernels, each owning its outputs, so no floating-point atomics are used
// and results do not depend on scheduling:
//
//   dK/dV kernel (key-outer).  A workgroup owns 128 keys of one key/value head
//   and walks the query tiles of every query head that reads that key/value
//   head.  Scores are formed as S = Q K^T, which puts one key per lane with the
//   tile's queries in the lane's registers; P and dS then feed dV^T += dO^T P
//   and dK^T += Q^T dS straight from registers.  Each group of 32 keys is
//   served by a pair of wavefronts, one producing P and dV, the other dS and dK
//   (see below).  Query and dO tiles stream from HBM into LDS (global_load_lds,
//   double buffered); the transposed operands Q^T, dO^T are read from the same
//   row-major tiles with ds_read_b64_tr_b16.
//
//   dQ kernel (query-outer).  A workgroup owns 128 queries (32 per wavefront,
//   Q and dO in registers) and walks the key tiles.  Scores are formed
//   transposed, S^T = K Q^T, one query per lane, so the row statistics (LSE,
//   delta) are per-lane scalars and dS^T feeds dQ^T += K^T dS^T straight from
//   registers; K^T is read from the row-major key tile with the transposing
//   LDS read.  dQ is added into an fp32 accumulator that persists across key
//   chunks and is cast once at the end.
//
// The dQ pass recomputes S and dP (7 contractions in all instead of 5); that
// is the price of determinism without atomics.
#include "attn_device.h"
#include "attn_internal.h"
#include "tile_lds.h"

namespace attn {
namespace {

constexpr int NT = 256;
constexpr int KBN = 128;  // keys per dK/dV workgroup
constexpr int KBM = 64;   // queries per tile in the dK/dV kernel
constexpr int QBM = 128;  // queries per dQ workgroup
constexpr int QBN = 64;   // keys per tile in the dQ kernel

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of this wavefront are in
// flight (LDS and export counters left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for data exchanged through LDS by ordinary LDS stores.  A
// fenced barrier (__syncthreads, or any release fence, since global_load_lds
// writes LDS) makes every wavefront wait for all of its loads in flight, which
// would drain the prefetches of later tiles at every barrier.  Here each
// wavefront waits only for its own LDS stores; global_load_lds tiles are
// waited for explicitly (wait_vm) before the barrier that publishes them.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 slab8(const f32x16& a, int o) {
  return cvt_bf16x8(a[o], a[o + 1], a[o + 2], a[o + 3], a[o + 4], a[o + 5], a[o + 6], a[o + 7]);
}

// ---------------------------------------------------------------- dK / dV --
//
// Eight wavefronts in four pairs; pair w%4 owns keys j0 + 32*(w%4) .. +31.
// The "P" wavefront (w < 4) holds K as its register operand and accumulates
// dV: it forms S = Q K^T, P = exp(S - LSE) (masked), hands P to its partner
// through LDS and then runs dV^T += dO^T P.  The "dS" wavefront (w >= 4) holds
// V and accumulates dK: it forms dP = dO V^T, reads P, dS = P (dP - delta) and
// runs dK^T += Q^T dS.  Both halves carry 32 MFMAs per query tile, and each
// wavefront keeps one operand and one accumulator instead of two of each, so
// two wavefronts fit per SIMD.

constexpr int DKV_NT = 512;
constexpr int DKV_STAGES = 3;  // query tiles in flight: the one in use and two being fetched

// One pipeline stage: a query tile, a dO tile and their 64 rows of statistics.
// Each stage is its own LDS object and every access names its stage at compile
// time, so the compiler can see that reading one stage never overlaps the
// global_load_lds writes still filling another.
template <int D>
struct DkvStage {
  u16* q;
  u16* dO;
  float* st;  // [0, 64): LSE in log2 units, [64, 128): delta, [128, 256): unused
};

template <int D>
struct DkvCtx {
  const BwdParams& p;
  DkvStage<D> s0, s1, s2;
  u32x4 (*pex)[4][64];  // [4 pairs] P in bf16, in accumulator (lane) order
  RowFrag<D> rf;
  TrFrag<D> tf;
  int wave, lane, lr, lg, pair;
};

template <int D, int ST>
__device__ __forceinline__ const DkvStage<D>& stage(const DkvCtx<D>& c) {
  if constexpr (ST == 0) return c.s0;
  else if constexpr (ST == 1) return c.s1;
  else return c.s2;
}

// Fetch query tile tq of one head into stage ST: Q and dO rows, and (wave 0)
// the 64 statistics of each kind in one 1 KB run.  The loads are untracked by
// the compiler; dkdv_step waits for them before the barrier that publishes
// the stage, and the last step of every head waits for all of them.
template <int D, int ST>
__device__ __forceinline__ void dkdv_issue(const DkvCtx<D>& c, const u16* qb, const u16* dob, const float* stb,
                                           int tq) {
  const DkvStage<D>& s = stage<D, ST>(c);
  if (c.wave == 0) {
    const int part = (c.lane >> 4) & 1;  // lanes 0-15 LSE, 16-31 delta; 32-63 repeat them
    const float* src = stb + part * c.p.Sq_pad + tq * KBM + 4 * (c.lane & 15);
    dma16_untracked(src, (lds_void*)s.st);
  }
  issue_swtile<D, 8, true>(s.q, qb, c.p.q.ss, tq * KBM, c.p.Sq, c.wave, c.lane);
  issue_swtile<D, 8, true>(s.dO, dob, c.p.dout.ss, tq * KBM, c.p.Sq, c.wave, c.lane);
}

// One query tile of the dK/dV kernel from stage ST, for the P wavefront (PW)
// or the dS wavefront.  The role is a compile-time constant so that every LDS
// read names its tile directly: the compiler can then tell these reads apart
// from the global_load_lds writes still filling the other stages and does not
// wait for those.
template <int D, int ST, bool PW>
__device__ __forceinline__ void dkdv_compute(const DkvCtx<D>& c, const bf16x8* kv, f32x16* acc, int i0, bool need_mask,
                                             int64_t key_lim, float sl2) {
  constexpr int NS = D / 16, NDB = D / 32;
  const DkvStage<D>& s = stage<D, ST>(c);
  const int lg = c.lg, lane = c.lane;
  // S = Q K^T (P wavefront) or dP = dO V^T (dS wavefront): lane = key,
  // registers = two 32-query blocks.
  const u16* rows = PW ? s.q : s.dO;
  f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int si = 0; si < NS; ++si) {
#pragma unroll
    for (int qb2 = 0; qb2 < 2; ++qb2) sc[qb2] = mfma32(c.rf.get(rows, qb2, si), kv[si], sc[qb2]);
  }
  bf16x8 opnd[4];  // B operands of the second contraction, one per 16-query slab
  if constexpr (PW) {
#pragma unroll
    for (int qb2 = 0; qb2 < 2; ++qb2) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 l4 = *(const f32x4*)(s.st + qb2 * 32 + g4 * 8 + lg * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[qb2][g4 * 4 + e] = exp2_fast(fmaf(sc[qb2][g4 * 4 + e], sl2, -l4[e]));
      }
    }
    if (need_mask) {
      // Causal mask: query i0 + q is hidden from this lane's key when
      // q < key_lim - i0.  The sign of q - (key_lim - i0) selects it as a bit
      // mask, which keeps the 32 decisions in vector registers.
      const int rel = (int)max<int64_t>(-1, min<int64_t>(key_lim - i0, KBM));
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qo = qb2 * 32 + (i >> 2) * 8 + lg * 4 + (i & 3);
          const unsigned keep = ~(unsigned)((qo - rel) >> 31);
          sc[qb2][i] = __uint_as_float(__float_as_uint(sc[qb2][i]) & keep);
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      opnd[ks] = slab8(sc[ks >> 1], (ks & 1) * 8);
      c.pex[c.pair][ks][lane] = __builtin_bit_cast(u32x4, opnd[ks]);
    }
  }
  lds_barrier();
  if constexpr (!PW) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, c.pex[c.pair][ks][lane]);
      const int qb2 = ks >> 1, o = (ks & 1) * 8;
      // Slab ks holds queries 16*ks + 8*(e/4) + 4*lg + e%4: two groups of 4 consecutive deltas.
      const f32x4 d0 = *(const f32x4*)(s.st + KBM + ks * 16 + lg * 4);
      const f32x4 d1 = *(const f32x4*)(s.st + KBM + ks * 16 + 8 + lg * 4);
      float ds[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ds[e] = (float)pb[e] * (sc[qb2][o + e] - (e < 4 ? d0[e] : d1[e - 4]));
      opnd[ks] = cvt_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
    }
  }
  // dV^T += dO^T P (P wavefront) or dK^T += Q^T dS (dS wavefront).
  const u16* tsrc = PW ? s.dO : s.q;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = mfma32(c.tf.get(tsrc, ks, db), opnd[ks], acc[db]);
  }
}

// Vector-memory operations one query tile adds per wavefront (wave 0 issues one more).
template <int D>
constexpr int dkdv_loads_per_tile() {
  return 2 * ((SwTile<D>::RUNS + 7) / 8);
}

// Pipeline step for tile t in stage ST: wait for it, release the stage that
// tile t + 2 will use, fetch tile t + 2, compute tile t.  Every wavefront of
// either role passes the same two barriers per step.
template <int D, int ST, bool PW>
__device__ __forceinline__ void dkdv_step(const DkvCtx<D>& c, const bf16x8* kv, f32x16* acc, const u16* qb,
                                          const u16* dob, const float* stb, int t, int n_qt, int i_full,
                                          int64_t key_lim, float sl2) {
  if (t + 1 < n_qt) wait_vm<dkdv_loads_per_tile<D>()>();  // only tile t + 1 may remain in flight
  else wait_vm<0>();
  lds_barrier();
  if (t + 2 < n_qt) dkdv_issue<D, (ST + 2) % 3>(c, qb, dob, stb, t + 2);
  dkdv_compute<D, ST, PW>(c, kv, acc, t * KBM, c.p.causal && t * KBM < i_full, key_lim, sl2);
}

template <int D, bool PW>
__device__ __forceinline__ void dkdv_tile(const DkvCtx<D>& c, int kt, int b, int hk) {
  constexpr int NS = D / 16, NDB = D / 32;
  const BwdParams& p = c.p;
  const int j0 = kt * KBN;
  const int kj = j0 + c.pair * 32 + c.lr;  // this lane's key
  const bool kok = kj < p.Sk;

  // Register operand: K rows for the P wavefront, V rows for the dS wavefront.
  bf16x8 kv[NS];
  {
    const View& src = PW ? p.k : p.v;
    const u16* base = (const u16*)src.ptr + (int64_t)b * src.sb + (int64_t)hk * src.sh + (int64_t)kj * src.ss;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kv[s] = kok ? as_bf16x8(*(const u32x4*)(base + c.lg * 8 + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  // Complete these loads here: left to the compiler, the wait for them sits at
  // their first use inside the loop, where it would also drain every tile
  // prefetch in flight on each pass.
  wait_vm<0>();
  f32x16 acc[NDB];  // dV^T (P wavefront) or dK^T (dS wavefront)
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // Query i sees key j iff j <= delta + i (causal).  Queries before i_start see
  // no key of this tile; from i_full on every query sees every key of it.
  // Query rows past the end carry LSE = +inf in the statistics, so their P is 0.
  const int j_last = min(j0 + KBN, p.Sk) - 1;
  int i_start = 0, i_full = 0;
  if (p.causal) {
    i_start = (int)min<int64_t>(p.Sq, max<int64_t>(0, (int64_t)j0 - p.delta_pos));
    i_full = (int)min<int64_t>(p.Sq, max<int64_t>(0, (int64_t)j_last - p.delta_pos));
  }
  const int t_start = i_start / KBM;
  const int n_qt = (p.Sq + KBM - 1) / KBM;
  const int64_t key_lim = (int64_t)kj - p.delta_pos;  // query index must be >= this (causal)
  const float sl2 = p.scale_log2;

  for (int hh = 0; hh < p.group; ++hh) {
    const int h = hk * p.group + hh;
    const u16* qb = (const u16*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
    const u16* dob = (const u16*)p.dout.ptr + (int64_t)b * p.dout.sb + (int64_t)h * p.dout.sh;
    const float* stb = p.stats + ((int64_t)b * p.Hq + h) * 2 * p.Sq_pad;
    if (t_start < n_qt) dkdv_issue<D, 0>(c, qb, dob, stb, t_start);
    if (t_start + 1 < n_qt) dkdv_issue<D, 1>(c, qb, dob, stb, t_start + 1);
    for (int t = t_start; t < n_qt; t += 3) {
      dkdv_step<D, 0, PW>(c, kv, acc, qb, dob, stb, t, n_qt, i_full, key_lim, sl2);
      if (t + 1 >= n_qt) break;
      dkdv_step<D, 1, PW>(c, kv, acc, qb, dob, stb, t + 1, n_qt, i_full, key_lim, sl2);
      if (t + 2 >= n_qt) break;
      dkdv_step<D, 2, PW>(c, kv, acc, qb, dob, stb, t + 2, n_qt, i_full, key_lim, sl2);
    }
    lds_barrier();  // stages are reused by the next head / tile
  }

  if (!kok) return;
  const float f = PW ? 1.0f : p.scale;
  const MView& dst = PW ? p.dv : p.dk;
  u16* out = (u16*)dst.ptr + (int64_t)b * dst.sb + (int64_t)kj * dst.ss + (int64_t)hk * dst.sh;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = db * 32 + j * 8 + c.lg * 4;
      const f32x16& A = acc[db];
      *(u32x2*)(out + d) = u32x2{pack_bf16x2(A[4 * j] * f, A[4 * j + 1] * f), pack_bf16x2(A[4 * j + 2] * f, A[4 * j + 3] * f)};
    }
  }
}

// A work unit is one key tile, or with the balanced order the pair of key
// tiles (u, n - 1 - u), whose causal work adds up to about the same for every u.
// Early keys are seen by the most queries, so they come first.
template <int D, bool PW>
__device__ __forceinline__ void dkdv_unit(const DkvCtx<D>& c, int unit, int b, int hk) {
  const BwdParams& p = c.p;
  const int last = p.n_ktiles - 1 - unit;
  const int n = (p.balanced && last != unit) ? 2 : 1;
  for (int k = 0; k < n; ++k) dkdv_tile<D, PW>(c, k == 0 ? unit : last, b, hk);
}

template <int D>
__global__ __launch_bounds__(DKV_NT) void dkdv_bf16_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) u16 q0[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 q1[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 q2[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 d0[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 d1[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 d2[SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) float st0[256];
  __shared__ __attribute__((aligned(16))) float st1[256];
  __shared__ __attribute__((aligned(16))) float st2[256];
  __shared__ __attribute__((aligned(16))) u32x4 pex_s[4][4][64];
  // The wavefront index is uniform across the wavefront; say so, so that the
  // role branch below is a scalar branch.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  DkvCtx<D> c{p, {q0, d0, st0}, {q1, d1, st1}, {q2, d2, st2}, pex_s, {}, {}, wave, lane, lane & 31, lane >> 5, wave & 3};
  c.rf.init(lane);
  c.tf.init(lane);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_units_k;
  const int bh = lin / p.n_units_k;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  if (wave < 4) dkdv_unit<D, true>(c, unit, b, hk);
  else dkdv_unit<D, false>(c, unit, b, hk);
}

// --------------------------------------------------------------------- dQ --
//
// Eight wavefronts in four pairs; pair w%4 owns queries q0 + 32*(w%4) .. +31.
// Key/value tiles of 64 rows stream through a 3-stage LDS ring and are
// consumed in 32-key steps.  At step k:
//   * the "S" wavefront (w < 4) holds Q in registers, forms S^T = K Q^T for the
//     keys of step k (one query per lane), P = exp(S - LSE) with the mask, and
//     hands P to its partner through LDS;
//   * the "dP" wavefront (w >= 4) holds dO and the whole dQ^T accumulator,
//     forms dP^T = V dO^T for step k, and for step k - 1 (one step behind, so
//     that P is already published) reads P, forms dS = P (dP - delta) and runs
//     dQ^T += K^T dS^T.
// The S wavefront carries the exponentials, the dP wavefront two thirds of the
// contractions; a pair shares one SIMD, whose matrix core they keep busy in
// turn.  One LDS-only barrier per step publishes P and, every other step, the
// next key/value tile.

constexpr int DQ_NT = 512;

template <int D>
constexpr int dq_loads_per_tile() {
  return 2 * (SwTile<D>::RUNS / 8);
}

template <int D, bool SW>
__device__ __forceinline__ void dq_role(const BwdParams& p, u16* k_s, u16* v_s, u32x4 (*pex)[2][2][64], int wave,
                                        int lane, int b, int h, int q0) {
  constexpr int NS = D / 16, NDB = D / 32, SZ = SwTile<D>::SIZE, L = dq_loads_per_tile<D>();
  const int lr = lane & 31, lg = lane >> 5, pair = wave & 3;
  const int hk = h / p.group;
  const int qi = q0 + pair * 32 + lr;
  const bool qok = qi < p.Sq;
  const u16* kb = (const u16*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const u16* vb = (const u16*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;
  const int q_last = min(q0 + QBM, p.Sq) - 1;
  int kv_end = p.Sk, full_end = p.Sk;
  int64_t lim64 = (int64_t)p.Sk - 1;  // last key this lane's query sees
  if (p.causal) {
    kv_end = (int)max<int64_t>(0, min<int64_t>(p.delta_pos + q_last + 1, p.Sk));
    full_end = (int)max<int64_t>(0, min<int64_t>(p.delta_pos + q0 + 1, p.Sk));
    lim64 = min<int64_t>(p.delta_pos + qi, lim64);
  }
  const int n = (kv_end + QBN - 1) / QBN;

  // Register operand (Q rows or dO rows of this lane's query) and statistic.
  bf16x8 op[NS];
  {
    const View& src = SW ? p.q : p.dout;
    const u16* row = (const u16*)src.ptr + (int64_t)b * src.sb + (int64_t)h * src.sh + (int64_t)qi * src.ss + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      op[s] = qok ? as_bf16x8(*(const u32x4*)(row + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  // Statistics rows exist up to Sq_pad >= Sq; rows past Sq hold LSE = +inf, delta = 0.
  const float* stb = p.stats + ((int64_t)b * p.Hq + h) * 2 * p.Sq_pad;
  const float stat = SW ? (qi < p.Sq_pad ? stb[qi] : pos_inf()) : (qi < p.Sq_pad ? stb[p.Sq_pad + qi] : 0.f);
  const float sl2 = p.scale_log2;
  RowFrag<D> rf;
  rf.init(lane);
  TrFrag<D> tf;
  if constexpr (!SW) tf.init(lane);
  // Complete these loads here: left to the compiler, the wait for them sits at
  // their first use inside the loop, where it would also drain every tile
  // prefetch in flight on each pass.
  wait_vm<0>();

  f32x16 acc[SW ? 1 : NDB];  // dQ^T (dP wavefront)
#pragma unroll
  for (int db = 0; db < (SW ? 1 : NDB); ++db) acc[db] = f32x16{};
  f32x16 dp_prev = f32x16{};

  auto issue = [&](int tile) {
    const int slot = tile % 3;
    issue_swtile<D, 8, true>(k_s + slot * SZ, kb, p.k.ss, tile * QBN, p.Sk, wave, lane);
    issue_swtile<D, 8, true>(v_s + slot * SZ, vb, p.v.ss, tile * QBN, p.Sk, wave, lane);
  };

  if (n > 0) {
    issue(0);
    if (n > 1) issue(1);
    if (n > 1) wait_vm<L>();
    else wait_vm<0>();
    lds_barrier();
  }
  const int steps = n > 0 ? 2 * n + 1 : 0;
  for (int k = 0; k < steps; ++k) {
    const int T = k >> 1, hf = k & 1;
    // Tile T + 2 takes the slot of tile T - 1, whose last reader (the dP
    // wavefront, one step behind) finished before the previous barrier.
    if (hf == 1 && T + 2 < n) issue(T + 2);
    f32x16 sc = f32x16{};
    if (k < 2 * n) {
      const u16* rows = (SW ? k_s : v_s) + (T % 3) * SZ;
#pragma unroll
      for (int s = 0; s < NS; ++s) sc = mfma32(rf.get(rows, hf, s), op[s], sc);
      if constexpr (SW) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = exp2_fast(fmaf(sc[i], sl2, -stat));
        if (32 * k + 32 > full_end) {
          // Key of register i: 32k + 8(i/4) + 4lg + i%4; hidden when it exceeds
          // lim64.  The sign of the difference gives a bit mask.
          const int rel = (int)max<int64_t>(-1, min<int64_t>(lim64 - 32 * k, 32)) - 4 * lg;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const unsigned keep = ~(unsigned)((rel - (8 * (i >> 2) + (i & 3))) >> 31);
            sc[i] = __uint_as_float(__float_as_uint(sc[i]) & keep);
          }
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) pex[pair][k & 1][hs][lane] = __builtin_bit_cast(u32x4, slab8(sc, hs * 8));
      }
    }
    if constexpr (!SW) {
      if (k >= 1) {
        const int kp = k - 1;
        const u16* kt = k_s + ((kp >> 1) % 3) * SZ;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pex[pair][kp & 1][hs][lane]);
          float ds[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) ds[e] = (float)pb[e] * (dp_prev[hs * 8 + e] - stat);
          const bf16x8 sb = cvt_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[db] = mfma32(tf.get(kt, (kp & 1) * 2 + hs, db), sb, acc[db]);
        }
      }
      dp_prev = sc;
    }
    // The next tile must be resident before the barrier that ends its
    // predecessor's second step.
    if (hf == 1 && k < 2 * n) {
      if (T + 2 < n) wait_vm<L>();
      else wait_vm<0>();
    }
    lds_barrier();
  }

  if constexpr (!SW) {
    if (!qok) return;
    float* accp = p.dq_acc + (((int64_t)b * p.Sq + qi) * p.Hq + h) * D;
    u16* dqp = p.finalize_dq ? (u16*)p.dq.ptr + (int64_t)b * p.dq.sb + (int64_t)qi * p.dq.ss + (int64_t)h * p.dq.sh
                             : nullptr;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + j * 8 + lg * 4;
        f32x4 v = {acc[db][4 * j] * p.scale, acc[db][4 * j + 1] * p.scale, acc[db][4 * j + 2] * p.scale,
                   acc[db][4 * j + 3] * p.scale};
        if (!p.dq_overwrite) v += *(const f32x4*)(accp + d);
        *(f32x4*)(accp + d) = v;
        if (dqp) *(u32x2*)(dqp + d) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(DQ_NT) void dq_bf16_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) u16 k_s[3 * SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v_s[3 * SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u32x4 pex_s[4][2][2][64];  // [pair][step parity][slab][lane]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_qtiles;
  const int bh = lin / p.n_qtiles;
  const int h = bh % p.Hq, b = bh / p.Hq;
  // Causal: late query tiles see the most keys; start with them.
  const int qt = p.causal ? p.n_qtiles - 1 - unit : unit;
  if (wave < 4) dq_role<D, true>(p, k_s, v_s, pex_s, wave, lane, b, h, qt * QBM);
  else dq_role<D, false>(p, k_s, v_s, pex_s, wave, lane, b, h, qt * QBM);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p0, int D, int run_dq, hipStream_t s) {
  BwdParams p = p0;
  p.n_ktiles = (p.Sk + KBN - 1) / KBN;
  p.n_units_k = p.balanced ? (p.n_ktiles + 1) / 2 : p.n_ktiles;
  p.n_qtiles = (p.Sq + QBM - 1) / QBM;
  const int64_t gk = (int64_t)p.B * p.Hkv * p.n_units_k;
  if (gk > 0) {
    if (D == 128)
      hipLaunchKernelGGL(dkdv_bf16_kernel<128>, dim3((unsigned)gk), dim3(DKV_NT), 0, s, p);
    else
      hipLaunchKernelGGL(dkdv_bf16_kernel<64>, dim3((unsigned)gk), dim3(DKV_NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t gq = (int64_t)p.B * p.Hq * p.n_qtiles;
  if (run_dq && gq > 0) {
    if (D == 128)
      hipLaunchKernelGGL(dq_bf16_kernel<128>, dim3((unsigned)gq), dim3(DQ_NT), 0, s, p);
    else
      hipLaunchKernelGGL(dq_bf16_kernel<64>, dim3((unsigned)gq), dim3(DQ_NT), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace attn
