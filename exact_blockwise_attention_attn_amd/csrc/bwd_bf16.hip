// Backward of exact attention for bf16 inputs on gfx950, from the saved final
// output O and row LSE: no re-run of the forward (DistFlashAttn digest,
// rematerialisation-aware gradient checkpointing).  bf16 MFMA with fp32
// accumulation everywhere.
//
// Two kernels, each owning its outputs, so no floating-point atomics are used
// and results do not depend on scheduling:
//
//   dK/dV kernel (key-outer).  A workgroup owns 128 keys of one key/value head
//   (32 per wavefront, held in registers as MFMA operands) and walks the query
//   tiles of every query head that reads that key/value head.  Scores are
//   formed as S = Q K^T, which puts one key per lane with the tile's queries in
//   the lane's registers; P and dS then feed dV^T += dO^T P and
//   dK^T += Q^T dS straight from registers.  Q and dO are staged in LDS both
//   row-major (for S and dP) and transposed in slot order (for dK, dV).
//
//   dQ kernel (query-outer).  A workgroup owns 128 queries (32 per wavefront,
//   Q and dO in registers) and walks the key tiles.  Scores are formed
//   transposed, S^T = K Q^T, one query per lane, so the row statistics (LSE,
//   delta) are per-lane scalars and dS^T feeds dQ^T += K^T dS^T straight from
//   registers.  dQ is added into an fp32 accumulator that persists across key
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

__device__ __forceinline__ u32x4 load16(const u16* ptr, bool ok) {
  if (ok) return *(const u32x4*)ptr;
  return u32x4{0u, 0u, 0u, 0u};
}

// 4 consecutive rows x 8 features per thread (16 row groups x D/8 feature groups).
template <int D>
struct Rows4 {
  u32x4 r[4];
};

template <int D>
__device__ __forceinline__ void load_rows4(Rows4<D>& x, const u16* base, int64_t ss, int row0, int nrows, int tid) {
  const int rg = tid & 15, fg = tid >> 4;
  if (fg < D / 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = row0 + rg * 4 + j;
      x.r[j] = load16(base + (int64_t)row * ss + fg * 8, row < nrows);
    }
  }
}

// Row-major store of a 64-row tile: rows rg*4+j, features fg*8..+7.
template <int D, int LD>
__device__ __forceinline__ void store_rows4(u16 (*t)[LD], const Rows4<D>& x, int tid) {
  const int rg = tid & 15, fg = tid >> 4;
  if (fg < D / 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4*)&t[rg * 4 + j][fg * 8] = x.r[j];
  }
}

// Transposed store: one LDS row per feature, the 4 rows in slot order.
template <int D, int LD>
__device__ __forceinline__ void store_rows4_t(u16 (*t)[LD], const Rows4<D>& x, int tid) {
  const int rg = tid & 15, fg = tid >> 4;
  if (fg < D / 8) {
    const int pos = slot_pos(rg * 4);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t w0 = x.r[0][w], w1 = x.r[1][w], w2 = x.r[2][w], w3 = x.r[3][w];
      *(u32x2*)&t[fg * 8 + 2 * w][pos] = u32x2{(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
      *(u32x2*)&t[fg * 8 + 2 * w + 1][pos] = u32x2{(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
    }
  }
}

__device__ __forceinline__ bf16x8 slab8(const f32x16& a, int o) {
  return cvt_bf16x8(a[o], a[o + 1], a[o + 2], a[o + 3], a[o + 4], a[o + 5], a[o + 6], a[o + 7]);
}

// LSE in log2 units; a row that sees no key gets +inf so that its P is 0.
__device__ __forceinline__ float lse_log2(float lse) { return (lse == neg_inf()) ? pos_inf() : lse * kLog2e; }

// ---------------------------------------------------------------- dK / dV --

template <int D>
struct alignas(16) DkvTile {
  u16 q[KBM][D + 8];
  u16 dO[KBM][D + 8];
  u16 qt[D][KBM + 8];
  u16 dOt[D][KBM + 8];
  float lse2[KBM];
  float dlt[KBM];
};

template <int D>
__device__ __forceinline__ void dkdv_tile(const BwdParams& p, DkvTile<D>& sm, int kt, int b, int hk) {
  constexpr int NS = D / 16, NDB = D / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int j0 = kt * KBN;
  const int kj = j0 + wave * 32 + lr;  // this lane's key
  const bool kok = kj < p.Sk;

  const u16* kb = (const u16*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const u16* vb = (const u16*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;
  bf16x8 kf[NS], vf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = as_bf16x8(load16(kb + (int64_t)kj * p.k.ss + s * 16 + lg * 8, kok));
    vf[s] = as_bf16x8(load16(vb + (int64_t)kj * p.v.ss + s * 16 + lg * 8, kok));
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

  for (int hh = 0; hh < p.group; ++hh) {
    const int h = hk * p.group + hh;
    const u16* qb = (const u16*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
    const u16* dob = (const u16*)p.dout.ptr + (int64_t)b * p.dout.sb + (int64_t)h * p.dout.sh;
    const float* lseb = p.lse + ((int64_t)b * p.Hq + h) * p.Sq;
    const float* dltb = p.delta + ((int64_t)b * p.Hq + h) * p.Sq;

    Rows4<D> rq, rdo;
    if (t_start < n_qt) {
      load_rows4<D>(rq, qb, p.q.ss, t_start * KBM, p.Sq, tid);
      load_rows4<D>(rdo, dob, p.dout.ss, t_start * KBM, p.Sq, tid);
    }
    for (int t = t_start; t < n_qt; ++t) {
      const int i0 = t * KBM;
      __syncthreads();
      store_rows4<D, D + 8>(sm.q, rq, tid);
      store_rows4_t<D, KBM + 8>(sm.qt, rq, tid);
      store_rows4<D, D + 8>(sm.dO, rdo, tid);
      store_rows4_t<D, KBM + 8>(sm.dOt, rdo, tid);
      if (tid < KBM) {
        const int i = i0 + tid;
        sm.lse2[tid] = (i < p.Sq) ? lse_log2(lseb[i]) : pos_inf();
        sm.dlt[tid] = (i < p.Sq) ? dltb[i] : 0.f;
      }
      __syncthreads();
      if (t + 1 < n_qt) {
        load_rows4<D>(rq, qb, p.q.ss, i0 + KBM, p.Sq, tid);
        load_rows4<D>(rdo, dob, p.dout.ss, i0 + KBM, p.Sq, tid);
      }

      // S = Q K^T and dP = dO V^T: lane = key, registers = 32-query blocks.
      f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int qb2 = 0; qb2 < 2; ++qb2) {
          const bf16x8 aq = as_bf16x8(*(const u32x4*)&sm.q[qb2 * 32 + lr][s * 16 + lg * 8]);
          sacc[qb2] = mfma32(aq, kf[s], sacc[qb2]);
          const bf16x8 ad = as_bf16x8(*(const u32x4*)&sm.dO[qb2 * 32 + lr][s * 16 + lg * 8]);
          pacc[qb2] = mfma32(ad, vf[s], pacc[qb2]);
        }
      }
      const bool need_mask = p.causal && i0 < i_full;
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qo = qb2 * 32 + g4 * 8 + lg * 4;
          const f32x4 l4 = *(const f32x4*)&sm.lse2[qo];
          const f32x4 d4 = *(const f32x4*)&sm.dlt[qo];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = g4 * 4 + e;
            float pv = exp2_fast(fmaf(sacc[qb2][i], p.scale_log2, -l4[e]));
            if (need_mask && (int64_t)(i0 + qo + e) < key_lim) pv = 0.f;
            sacc[qb2][i] = pv;
            pacc[qb2][i] = pv * (pacc[qb2][i] - d4[e]);
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
          const bf16x8 ad = as_bf16x8(*(const u32x4*)&sm.dOt[db * 32 + lr][ks * 16 + lg * 8]);
          dv[db] = mfma32(ad, pb, dv[db]);
          const bf16x8 aq = as_bf16x8(*(const u32x4*)&sm.qt[db * 32 + lr][ks * 16 + lg * 8]);
          dk[db] = mfma32(aq, sb, dk[db]);
        }
      }
    }
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
  __shared__ DkvTile<D> sm;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_units_k;
  const int bh = lin / p.n_units_k;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  if (p.balanced) {
    const int t0 = unit, t1 = p.n_ktiles - 1 - unit;
    dkdv_tile<D>(p, sm, t0, b, hk);
    if (t1 != t0) {
      __syncthreads();
      dkdv_tile<D>(p, sm, t1, b, hk);
    }
  } else {
    // Causal: early keys are seen by the most queries; start with them.
    dkdv_tile<D>(p, sm, unit, b, hk);
  }
}

// --------------------------------------------------------------------- dQ --

template <int D>
struct alignas(16) DqTile {
  u16 k[QBN][D + 8];
  u16 v[QBN][D + 8];
  u16 kt[D][QBN + 8];
};

template <int D>
__global__ __launch_bounds__(NT) void dq_bf16_kernel(BwdParams p) {
  constexpr int NS = D / 16, NDB = D / 32;
  __shared__ DqTile<D> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_qtiles;
  const int bh = lin / p.n_qtiles;
  const int h = bh % p.Hq, b = bh / p.Hq, hk = h / p.group;
  const int qt = p.causal ? p.n_qtiles - 1 - unit : unit;
  const int q0 = qt * QBM;
  const int qi = q0 + wave * 32 + lr;
  const bool qok = qi < p.Sq;

  const u16* qb = (const u16*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
  const u16* dob = (const u16*)p.dout.ptr + (int64_t)b * p.dout.sb + (int64_t)h * p.dout.sh;
  const u16* kb = (const u16*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const u16* vb = (const u16*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;
  bf16x8 qf[NS], dof[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = as_bf16x8(load16(qb + (int64_t)qi * p.q.ss + s * 16 + lg * 8, qok));
    dof[s] = as_bf16x8(load16(dob + (int64_t)qi * p.dout.ss + s * 16 + lg * 8, qok));
  }
  const int64_t srow = ((int64_t)b * p.Hq + h) * p.Sq + qi;
  const float lse2 = qok ? lse_log2(p.lse[srow]) : pos_inf();
  const float dlt = qok ? p.delta[srow] : 0.f;

  const int q_last = min(q0 + QBM, p.Sq) - 1;
  int kv_end = p.Sk, full_end = p.Sk;
  int64_t lim64 = (int64_t)p.Sk - 1;
  if (p.causal) {
    kv_end = (int)max<int64_t>(0, min<int64_t>(p.delta_pos + q_last + 1, p.Sk));
    full_end = (int)max<int64_t>(0, min<int64_t>(p.delta_pos + q0 + 1, p.Sk));
    lim64 = min<int64_t>(p.delta_pos + qi, lim64);
  }
  const int n_tiles = (kv_end + QBN - 1) / QBN;

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  Rows4<D> rk, rv;
  if (n_tiles > 0) {
    load_rows4<D>(rk, kb, p.k.ss, 0, p.Sk, tid);
    load_rows4<D>(rv, vb, p.v.ss, 0, p.Sk, tid);
  }
  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * QBN;
    __syncthreads();
    store_rows4<D, D + 8>(sm.k, rk, tid);
    store_rows4_t<D, QBN + 8>(sm.kt, rk, tid);
    store_rows4<D, D + 8>(sm.v, rv, tid);
    __syncthreads();
    if (t + 1 < n_tiles) {
      load_rows4<D>(rk, kb, p.k.ss, key0 + QBN, p.Sk, tid);
      load_rows4<D>(rv, vb, p.v.ss, key0 + QBN, p.Sk, tid);
    }
    // S^T = K Q^T and dP^T = V dO^T: lane = query, registers = 32-key blocks.
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 ak = as_bf16x8(*(const u32x4*)&sm.k[kb2 * 32 + lr][s * 16 + lg * 8]);
        sacc[kb2] = mfma32(ak, qf[s], sacc[kb2]);
        const bf16x8 av = as_bf16x8(*(const u32x4*)&sm.v[kb2 * 32 + lr][s * 16 + lg * 8]);
        pacc[kb2] = mfma32(av, dof[s], pacc[kb2]);
      }
    }
    const bool need_mask = key0 + QBN > full_end;
    const int lim = (int)max<int64_t>(-1, min<int64_t>(lim64 - key0, QBN));
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = exp2_fast(fmaf(sacc[kb2][i], p.scale_log2, -lse2));
        if (need_mask && kb2 * 32 + (i >> 2) * 8 + lg * 4 + (i & 3) > lim) pv = 0.f;
        pacc[kb2][i] = pv * (pacc[kb2][i] - dlt);
      }
    }
    // dQ^T += K^T dS^T over four 16-key slabs.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 sb = slab8(pacc[ks >> 1], (ks & 1) * 8);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)&sm.kt[db * 32 + lr][ks * 16 + lg * 8]);
        acc[db] = mfma32(a, sb, acc[db]);
      }
    }
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
