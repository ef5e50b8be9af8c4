// Forward partial attention for bf16 inputs on gfx950 (CDNA4), bf16 MFMA with
// fp32 accumulation.
//
// Computes, for one chunk of keys, the exact softmax attention of a query
// shard: the local attention step of the BurstAttention page and the per-step
// blockwise computation of ring-style attention, as a partial (O, LSE).
//
// Layout of the work:
//   * one workgroup = 4 wavefronts = 128 queries of one (batch, head); each
//     wavefront owns 32 queries;
//   * keys stream through LDS in tiles of 64 (double buffered, the next tile is
//     fetched into registers while the current one is used);
//   * scores are formed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA:
//     the accumulator puts one query per lane (column) and 16 of its keys in
//     the lane's registers, so row max and row sum are in-lane reductions plus
//     one exchange with the other half of the wavefront;
//   * O^T += V^T P^T uses P^T straight from the registers (no LDS round trip);
//     V is stored transposed in LDS with keys in the matching slot order;
//   * causal tiles are classified per workgroup: tiles no query sees are never
//     visited, tiles every query sees skip the mask, the rest are masked per
//     element.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int BM = 128;  // queries per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int NT = 256;  // threads per workgroup

template <int D>
struct alignas(16) FwdTile {
  u16 k[BN][D + 8];   // keys row-major; the pad puts 8 consecutive rows on distinct banks
  u16 vt[D][BN + 8];  // values transposed: one row per feature, keys in slot order
};

template <int D>
struct KVRegs {
  static constexpr int KCH = D / 8;            // 16-byte chunks per key row
  static constexpr int KPASS = BN * KCH / NT;  // chunks of the key tile per thread
  u32x4 k[KPASS];
  u32x4 v[4];  // 4 consecutive keys x 8 features, for the transposed store
};

__device__ __forceinline__ u32x4 load16(const u16* ptr, bool ok) {
  if (ok) return *(const u32x4*)ptr;
  return u32x4{0u, 0u, 0u, 0u};
}

template <int D>
__device__ __forceinline__ void load_kv(KVRegs<D>& r, const u16* kb, const u16* vb, int64_t k_ss, int64_t v_ss,
                                        int key0, int Sk, int tid) {
  constexpr int KCH = KVRegs<D>::KCH;
  constexpr int RPP = NT / KCH;
#pragma unroll
  for (int p = 0; p < KVRegs<D>::KPASS; ++p) {
    const int row = tid / KCH + p * RPP;
    const int key = key0 + row;
    r.k[p] = load16(kb + (int64_t)key * k_ss + (tid % KCH) * 8, key < Sk);
  }
  const int kg = tid & 15, dg = tid >> 4;
  if (dg < KCH) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = key0 + kg * 4 + j;
      r.v[j] = load16(vb + (int64_t)key * v_ss + dg * 8, key < Sk);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_kv(FwdTile<D>& t, const KVRegs<D>& r, int tid) {
  constexpr int KCH = KVRegs<D>::KCH;
  constexpr int RPP = NT / KCH;
#pragma unroll
  for (int p = 0; p < KVRegs<D>::KPASS; ++p) {
    const int row = tid / KCH + p * RPP;
    *(u32x4*)&t.k[row][(tid % KCH) * 8] = r.k[p];
  }
  const int kg = tid & 15, dg = tid >> 4;
  if (dg < KCH) {
    const int pos = slot_pos(kg * 4);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t w0 = r.v[0][w], w1 = r.v[1][w], w2 = r.v[2][w], w3 = r.v[3][w];
      const u32x2 even = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
      const u32x2 odd = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
      *(u32x2*)&t.vt[dg * 8 + 2 * w][pos] = even;
      *(u32x2*)&t.vt[dg * 8 + 2 * w + 1][pos] = odd;
    }
  }
}

template <int D>
__device__ __forceinline__ void fwd_tile(const FwdParams& p, FwdTile<D>* sm, int qt, int b, int h, const u16* qb,
                                         const u16* kb, const u16* vb) {
  constexpr int NS = D / 16;   // 16-feature slabs of the score contraction
  constexpr int NDB = D / 32;  // 32-feature blocks of the output
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;

  const int q0 = qt * BM;
  const int qi = q0 + wave * 32 + lr;
  const bool qok = qi < p.Sq;

  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s] = as_bf16x8(load16(qb + (int64_t)qi * p.q.ss + s * 16 + lg * 8, qok));

  // Keys [0, kv_end) are visible to some query of this tile; keys [0, full_end)
  // to all of them.  Causal visibility: key j is visible to query i iff j <= delta + i.
  const int q_last = min(q0 + BM, p.Sq) - 1;
  int kv_end = p.Sk, full_end = p.Sk;
  int64_t lim64 = (int64_t)p.Sk - 1;
  if (p.causal) {
    kv_end = (int)max<int64_t>(0, min<int64_t>(p.delta + q_last + 1, p.Sk));
    full_end = (int)max<int64_t>(0, min<int64_t>(p.delta + q0 + 1, p.Sk));
    lim64 = min<int64_t>(p.delta + qi, lim64);
  }
  const int n_tiles = (kv_end + BN - 1) / BN;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = neg_inf(), l_run = 0.f;

  KVRegs<D> regs;
  if (n_tiles > 0) {
    load_kv<D>(regs, kb, vb, p.k.ss, p.v.ss, 0, p.Sk, tid);
    store_kv<D>(sm[0], regs, tid);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    const int key0 = t * BN;
    if (t + 1 < n_tiles) load_kv<D>(regs, kb, vb, p.k.ss, p.v.ss, key0 + BN, p.Sk, tid);

    // S^T = K Q^T for 64 keys (two 32-key blocks) x this wave's 32 queries.
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)&sm[cur].k[kb2 * 32 + lr][s * 16 + lg * 8]);
        sacc[kb2] = mfma32(a, qf[s], sacc[kb2]);
      }
    }
    if (key0 + BN > full_end) {
      const int lim = (int)max<int64_t>(-1, min<int64_t>(lim64 - key0, BN));
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = kb2 * 32 + (i >> 2) * 8 + lg * 4 + (i & 3);
          if (kl > lim) sacc[kb2][i] = neg_inf();
        }
    }

    // Online softmax on raw scores; the scale is folded into the exponent.
    float mt = neg_inf();
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb2][i]);
    mt = fmaxf(mt, other_half(mt));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = exp2_fast((m_run - m_use) * p.scale_log2);
    const float nbias = -m_use * p.scale_log2;
    float rs = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = exp2_fast(fmaf(sacc[kb2][i], p.scale_log2, nbias));
        sacc[kb2][i] = e;
        rs += e;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T += V^T P^T over four 16-key slabs.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb2 = ks >> 1, o = (ks & 1) * 8;
      const bf16x8 pb = cvt_bf16x8(sacc[kb2][o + 0], sacc[kb2][o + 1], sacc[kb2][o + 2], sacc[kb2][o + 3],
                                   sacc[kb2][o + 4], sacc[kb2][o + 5], sacc[kb2][o + 6], sacc[kb2][o + 7]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)&sm[cur].vt[db * 32 + lr][ks * 16 + lg * 8]);
        oacc[db] = mfma32(a, pb, oacc[db]);
      }
    }

    if (t + 1 < n_tiles) store_kv<D>(sm[cur ^ 1], regs, tid);
    __syncthreads();
  }

  // Epilogue: normalise, optionally merge into the running result, store.
  const float l_tot = l_run + other_half(l_run);
  if (!qok) return;
  const float lse_this = (m_run == neg_inf()) ? neg_inf() : fmaf(m_run, p.scale, logf(l_tot));
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  float* lse_ptr = p.lse + ((int64_t)b * p.Hq + h) * p.Sq + qi;
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

template <int D>
__global__ __launch_bounds__(NT) void fwd_bf16_kernel(FwdParams p) {
  __shared__ FwdTile<D> sm[2];
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
    fwd_tile<D>(p, sm, t1, b, h, qb, kb, vb);
    if (t0 != t1) {
      __syncthreads();
      fwd_tile<D>(p, sm, t0, b, h, qb, kb, vb);
    }
  } else {
    // Causal: heaviest tiles first, so the light ones fill the tail.
    const int qt = p.causal ? p.n_qtiles - 1 - unit : unit;
    fwd_tile<D>(p, sm, qt, b, h, qb, kb, vb);
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p0, int D, hipStream_t s) {
  FwdParams p = p0;
  p.n_qtiles = (p.Sq + BM - 1) / BM;
  p.n_units = p.balanced ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
  const int64_t grid = (int64_t)p.B * p.Hq * p.n_units;
  if (grid == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
