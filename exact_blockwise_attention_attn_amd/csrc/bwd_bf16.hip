// Backward of exact attention for bf16 inputs on gfx950, from the saved final
// output O and row LSE: no re-run of the forward (DistFlashAttn digest,
// rematerialisation-aware gradient checkpointing).  bf16 MFMA with fp32
// accumulation everywhere.
//
// Two kernels, each owning its outputs, so no floating-point atomics are used
// and results do not depend on scheduling:
//
//   dK/dV kernel (key-outer).  A workgroup owns 128 keys of one key/value head
//   (32 per wavefront, K and V held in registers as MFMA operands) and walks
//   the query tiles of every query head that reads that key/value head.  Scores
//   are formed as S = Q K^T, which puts one key per lane with the tile's
//   queries in the lane's registers; P and dS then feed dV^T += dO^T P and
//   dK^T += Q^T dS straight from registers.  Query and dO tiles stream from HBM
//   into LDS (global_load_lds, double buffered); the transposed operands Q^T,
//   dO^T are read from the same row-major tiles with ds_read_b64_tr_b16.
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

namespace attn {
namespace {

constexpr int NT = 256;
constexpr int KBN = 128;  // keys per dK/dV workgroup
constexpr int KBM = 64;   // queries per tile in the dK/dV kernel
constexpr int QBM = 128;  // queries per dQ workgroup
constexpr int QBN = 64;   // keys per tile in the dQ kernel
constexpr int TR = 64;    // rows of a streamed tile

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef i16x4 __attribute__((address_space(3))) lds_i16x4;
typedef void __attribute__((address_space(3))) lds_void;

// A streamed 64-row tile in LDS: rows padded by 16 bytes so the 8 rows an MFMA
// operand read touches per LDS cycle start on distinct 16-byte bank groups.
template <int D>
struct Tile {
  static constexpr int LD = D + 8;
  static constexpr int RUNS = (TR * LD * 2 + 1023) / 1024;  // 1 KB global_load_lds runs
  static constexpr int SIZE = RUNS * 512;                   // elements
};

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Issue the copy of rows [row0, row0 + 64) of a [rows, D] view into a padded
// LDS tile.  Wave w issues runs w, w+4, ...; lane l fills the l-th 16-byte slot
// of a run.  Pad slots get a copy of the row's first chunk and are never read;
// rows past the end load a valid row (their results are masked or dropped).
template <int D>
__device__ __forceinline__ void issue_tile(u16* lds, const u16* g, int64_t ss, int row0, int nrows, int wave,
                                           int lane) {
  using T = Tile<D>;
#pragma unroll
  for (int run = wave; run < T::RUNS; run += 4) {
    const int e = run * 512 + lane * 8;
    const int r = e / T::LD;
    int col = e - r * T::LD;
    if (col >= D) col = 0;
    const int row = min(row0 + r, nrows - 1);
    __builtin_amdgcn_global_load_lds((const void*)(g + (int64_t)row * ss + col), (lds_void*)(lds + run * 512), 16, 0,
                                     0);
  }
}

__device__ __forceinline__ bf16x8 slab8(const f32x16& a, int o) {
  return cvt_bf16x8(a[o], a[o + 1], a[o + 2], a[o + 3], a[o + 4], a[o + 5], a[o + 6], a[o + 7]);
}

// Transposed operand for a 32x32x16 MFMA from a row-major padded tile: lane
// (16q + s) gets feature (dcol + 16*(q%2) + s) of rows slab + 4*(q/2) + {0..3}
// and slab + 8 + 4*(q/2) + {0..3}, which is the k-slot order of an operand that
// comes straight out of an MFMA accumulator.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const u16* t, int slab_row, int dcol, int lane) {
  const int q16 = lane >> 4, s16 = lane & 15;
  const int r = slab_row + (q16 >> 1) * 4 + (s16 >> 2);
  const int c = dcol + (q16 & 1) * 16 + 4 * (s16 & 3);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + r * Tile<D>::LD + c));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + (r + 8) * Tile<D>::LD + c));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// LSE in log2 units; a row that sees no key gets +inf so that its P is 0.
__device__ __forceinline__ float lse_log2(float lse) { return (lse == neg_inf()) ? pos_inf() : lse * kLog2e; }

// ---------------------------------------------------------------- dK / dV --

template <int D>
__device__ __forceinline__ void dkdv_step(const u16* qs, const u16* dos, const float* l2s, const float* dls,
                                          const bf16x8* kf, const bf16x8* vf, f32x16* dk, f32x16* dv, int i0,
                                          bool need_mask, int64_t key_lim, float sl2, int lane) {
  constexpr int NS = D / 16, NDB = D / 32, LD = Tile<D>::LD;
  const int lr = lane & 31, lg = lane >> 5;
  // S = Q K^T and dP = dO V^T: lane = key, registers = 32-query blocks.
  f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const bf16x8 aq = as_bf16x8(*(const u32x4*)(qs + (qb * 32 + lr) * LD + s * 16 + lg * 8));
      sacc[qb] = mfma32(aq, kf[s], sacc[qb]);
      const bf16x8 ad = as_bf16x8(*(const u32x4*)(dos + (qb * 32 + lr) * LD + s * 16 + lg * 8));
      pacc[qb] = mfma32(ad, vf[s], pacc[qb]);
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int qo = qb * 32 + g4 * 8 + lg * 4;
      const f32x4 l4 = *(const f32x4*)(l2s + qo);
      const f32x4 d4 = *(const f32x4*)(dls + qo);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = g4 * 4 + e;
        float pv = exp2_fast(fmaf(sacc[qb][i], sl2, -l4[e]));
        if (need_mask && (int64_t)(i0 + qo + e) < key_lim) pv = 0.f;
        sacc[qb][i] = pv;
        pacc[qb][i] = pv * (pacc[qb][i] - d4[e]);
      }
    }
  }
  // dV^T += dO^T P, dK^T += Q^T dS over four 16-query slabs.
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 pb = slab8(sacc[ks >> 1], (ks & 1) * 8);
    const bf16x8 sb = slab8(pacc[ks >> 1], (ks & 1) * 8);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dv[db] = mfma32(tr_operand<D>(dos, ks * 16, db * 32, lane), pb, dv[db]);
      dk[db] = mfma32(tr_operand<D>(qs, ks * 16, db * 32, lane), sb, dk[db]);
    }
  }
}

template <int D>
struct DkvSmem {
  u16 q[2][Tile<D>::SIZE];
  u16 dO[2][Tile<D>::SIZE];
  float lse2[2][KBM];
  float dlt[2][KBM];
};

template <int D>
__device__ __forceinline__ void dkdv_tile(const BwdParams& p, DkvSmem<D>& sm, int kt, int b, int hk) {
  constexpr int NS = D / 16, NDB = D / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int j0 = kt * KBN;
  const int kj = j0 + wave * 32 + lr;  // this lane's key
  const bool kok = kj < p.Sk;

  const u16* kb = (const u16*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const u16* vb = (const u16*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;
  bf16x8 kf[NS], vf[NS];
  {
    const u16* kr = kb + (int64_t)kj * p.k.ss + lg * 8;
    const u16* vr = vb + (int64_t)kj * p.v.ss + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = kok ? as_bf16x8(*(const u32x4*)(kr + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      vf[s] = kok ? as_bf16x8(*(const u32x4*)(vr + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // Query i sees key j iff j <= delta + i (causal).  Queries before i_start see
  // no key of this tile; from i_full on every query sees every key of it.
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
    const float* lseb = p.lse + ((int64_t)b * p.Hq + h) * p.Sq;
    const float* dltb = p.delta + ((int64_t)b * p.Hq + h) * p.Sq;
    // Row statistics of the next tile go through registers (one value per thread).
    float nl = 0.f, nd = 0.f;
    auto fetch_stats = [&](int tq) {
      const int i = tq * KBM + tid;
      if (tid < KBM) {
        nl = (i < p.Sq) ? lse_log2(lseb[i]) : pos_inf();
        nd = (i < p.Sq) ? dltb[i] : 0.f;
      }
    };
    auto store_stats = [&](int buf) {
      if (tid < KBM) {
        sm.lse2[buf][tid] = nl;
        sm.dlt[buf][tid] = nd;
      }
    };
    if (t_start < n_qt) {
      issue_tile<D>(sm.q[0], qb, p.q.ss, t_start * KBM, p.Sq, wave, lane);
      issue_tile<D>(sm.dO[0], dob, p.dout.ss, t_start * KBM, p.Sq, wave, lane);
      fetch_stats(t_start);
      store_stats(0);
    }
    int buf = 0;
    for (int t = t_start; t < n_qt; ++t) {
      wait_loads();
      __syncthreads();
      if (t + 1 < n_qt) {
        issue_tile<D>(sm.q[buf ^ 1], qb, p.q.ss, (t + 1) * KBM, p.Sq, wave, lane);
        issue_tile<D>(sm.dO[buf ^ 1], dob, p.dout.ss, (t + 1) * KBM, p.Sq, wave, lane);
        fetch_stats(t + 1);
      }
      const int i0 = t * KBM;
      dkdv_step<D>(sm.q[buf], sm.dO[buf], sm.lse2[buf], sm.dlt[buf], kf, vf, dk, dv, i0,
                   p.causal && i0 < i_full, key_lim, sl2, lane);
      if (t + 1 < n_qt) store_stats(buf ^ 1);
      buf ^= 1;
    }
    __syncthreads();  // buffers are reused by the next head / tile
  }

  if (!kok) return;
  u16* dkp = (u16*)p.dk.ptr + (int64_t)b * p.dk.sb + (int64_t)kj * p.dk.ss + (int64_t)hk * p.dk.sh;
  u16* dvp = (u16*)p.dv.ptr + (int64_t)b * p.dv.sb + (int64_t)kj * p.dv.ss + (int64_t)hk * p.dv.sh;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = db * 32 + j * 8 + lg * 4;
      const f32x16& K = dk[db];
      const f32x16& V = dv[db];
      *(u32x2*)(dkp + d) = u32x2{pack_bf16x2(K[4 * j] * p.scale, K[4 * j + 1] * p.scale),
                                 pack_bf16x2(K[4 * j + 2] * p.scale, K[4 * j + 3] * p.scale)};
      *(u32x2*)(dvp + d) = u32x2{pack_bf16x2(V[4 * j], V[4 * j + 1]), pack_bf16x2(V[4 * j + 2], V[4 * j + 3])};
    }
  }
}

template <int D>
__global__ __launch_bounds__(NT) void dkdv_bf16_kernel(BwdParams p) {
  __shared__ DkvSmem<D> sm;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_units_k;
  const int bh = lin / p.n_units_k;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  if (p.balanced) {
    const int t0 = unit, t1 = p.n_ktiles - 1 - unit;
    dkdv_tile<D>(p, sm, t0, b, hk);
    if (t1 != t0) dkdv_tile<D>(p, sm, t1, b, hk);
  } else {
    // Causal: early keys are seen by the most queries; start with them.
    dkdv_tile<D>(p, sm, unit, b, hk);
  }
}

// --------------------------------------------------------------------- dQ --

template <int D>
__device__ __forceinline__ void dq_step(const u16* ks, const u16* vs, const bf16x8* qf, const bf16x8* dof,
                                        f32x16* acc, float lse2, float dlt, int key0, bool need_mask, int64_t lim64,
                                        float sl2, int lane) {
  constexpr int NS = D / 16, NDB = D / 32, LD = Tile<D>::LD;
  const int lr = lane & 31, lg = lane >> 5;
  const int lim = (int)max<int64_t>(-1, min<int64_t>(lim64 - key0, QBN));
  // Two 32-key halves keep only one score block live at a time.
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    // S^T = K Q^T and dP^T = V dO^T: lane = query, registers = 32 keys.
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 ak = as_bf16x8(*(const u32x4*)(ks + (kb2 * 32 + lr) * LD + s * 16 + lg * 8));
      sacc = mfma32(ak, qf[s], sacc);
      const bf16x8 av = as_bf16x8(*(const u32x4*)(vs + (kb2 * 32 + lr) * LD + s * 16 + lg * 8));
      pacc = mfma32(av, dof[s], pacc);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float pv = exp2_fast(fmaf(sacc[i], sl2, -lse2));
      if (need_mask && kb2 * 32 + (i >> 2) * 8 + lg * 4 + (i & 3) > lim) pv = 0.f;
      pacc[i] = pv * (pacc[i] - dlt);
    }
    // dQ^T += K^T dS^T over the two 16-key slabs of this half.
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const bf16x8 sb = slab8(pacc, hs * 8);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma32(tr_operand<D>(ks, kb2 * 32 + hs * 16, db * 32, lane), sb, acc[db]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(NT) void dq_bf16_kernel(BwdParams p) {
  constexpr int NS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) u16 k0s[Tile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v0s[Tile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 k1s[Tile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 v1s[Tile<D>::SIZE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_qtiles;
  const int bh = lin / p.n_qtiles;
  const int h = bh % p.Hq, b = bh / p.Hq, hk = h / p.group;
  const int qt = p.causal ? p.n_qtiles - 1 - unit : unit;
  const int q0 = qt * QBM;
  const int qi = q0 + wave * 32 + lr;
  const bool qok = qi < p.Sq;

  const u16* kb = (const u16*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const u16* vb = (const u16*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;
  const int q_last = min(q0 + QBM, p.Sq) - 1;
  int kv_end = p.Sk, full_end = p.Sk;
  int64_t lim64 = (int64_t)p.Sk - 1;
  if (p.causal) {
    kv_end = (int)max<int64_t>(0, min<int64_t>(p.delta_pos + q_last + 1, p.Sk));
    full_end = (int)max<int64_t>(0, min<int64_t>(p.delta_pos + q0 + 1, p.Sk));
    lim64 = min<int64_t>(p.delta_pos + qi, lim64);
  }
  const int n_tiles = (kv_end + QBN - 1) / QBN;
  if (n_tiles > 0) {
    issue_tile<D>(k0s, kb, p.k.ss, 0, p.Sk, wave, lane);
    issue_tile<D>(v0s, vb, p.v.ss, 0, p.Sk, wave, lane);
  }

  bf16x8 qf[NS], dof[NS];
  {
    const u16* qrow = (const u16*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh + (int64_t)qi * p.q.ss + lg * 8;
    const u16* drow =
        (const u16*)p.dout.ptr + (int64_t)b * p.dout.sb + (int64_t)h * p.dout.sh + (int64_t)qi * p.dout.ss + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = qok ? as_bf16x8(*(const u32x4*)(qrow + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      dof[s] = qok ? as_bf16x8(*(const u32x4*)(drow + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }
  const int64_t srow = ((int64_t)b * p.Hq + h) * p.Sq + qi;
  const float lse2 = qok ? lse_log2(p.lse[srow]) : pos_inf();
  const float dlt = qok ? p.delta[srow] : 0.f;
  const float sl2 = p.scale_log2;

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  for (int t = 0; t < n_tiles; t += 2) {
    wait_loads();
    __syncthreads();
    if (t + 1 < n_tiles) {
      issue_tile<D>(k1s, kb, p.k.ss, (t + 1) * QBN, p.Sk, wave, lane);
      issue_tile<D>(v1s, vb, p.v.ss, (t + 1) * QBN, p.Sk, wave, lane);
    }
    dq_step<D>(k0s, v0s, qf, dof, acc, lse2, dlt, t * QBN, t * QBN + QBN > full_end, lim64, sl2, lane);
    if (t + 1 >= n_tiles) break;
    wait_loads();
    __syncthreads();
    if (t + 2 < n_tiles) {
      issue_tile<D>(k0s, kb, p.k.ss, (t + 2) * QBN, p.Sk, wave, lane);
      issue_tile<D>(v0s, vb, p.v.ss, (t + 2) * QBN, p.Sk, wave, lane);
    }
    dq_step<D>(k1s, v1s, qf, dof, acc, lse2, dlt, (t + 1) * QBN, (t + 1) * QBN + QBN > full_end, lim64, sl2, lane);
  }

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

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p0, int D, int run_dq, hipStream_t s) {
  BwdParams p = p0;
  p.n_ktiles = (p.Sk + KBN - 1) / KBN;
  p.n_units_k = p.balanced ? (p.n_ktiles + 1) / 2 : p.n_ktiles;
  p.n_qtiles = (p.Sq + QBM - 1) / QBM;
  const int64_t gk = (int64_t)p.B * p.Hkv * p.n_units_k;
  if (gk > 0) {
    if (D == 128)
      hipLaunchKernelGGL(dkdv_bf16_kernel<128>, dim3((unsigned)gk), dim3(NT), 0, s, p);
    else
      hipLaunchKernelGGL(dkdv_bf16_kernel<64>, dim3((unsigned)gk), dim3(NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t gq = (int64_t)p.B * p.Hq * p.n_qtiles;
  if (run_dq && gq > 0) {
    if (D == 128)
      hipLaunchKernelGGL(dq_bf16_kernel<128>, dim3((unsigned)gq), dim3(NT), 0, s, p);
    else
      hipLaunchKernelGGL(dq_bf16_kernel<64>, dim3((unsigned)gq), dim3(NT), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace attn
