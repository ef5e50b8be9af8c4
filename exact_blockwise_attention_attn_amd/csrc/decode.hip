// Split-KV decode with grouped heads, then a binary-tree merge of the split
// partials (Lean Attention and Tree Attention abstracts: the softmax reduction
// is associative, so a long KV sequence can be cut into chunks whose partial
// results are reduced as a tree).
//
// Split kernel: one workgroup per (batch, key/value head, group slice of up to
// 4 query heads, split).  The cache is read exactly once per key/value head, so
// the 4 query heads of a GQA group share every byte.  Per 64-key block a
// wavefront
//   * loads K with one key per lane (16 keys x 4 lane groups of features) and
//     forms the scores with the 16x16x32 bf16 MFMA, the 4 queries replicated
//     over the 16 rows so every lane receives all 4 scores of its key;
//   * applies the online softmax per 64-key block (max over 16 lanes);
//   * passes P through a small per-wavefront LDS buffer to the layout in which
//     V is loaded (16 lanes cover one 256-byte key row, fully coalesced) and
//     accumulates O on the vector ALUs.
// The four wavefronts' partials are merged in LDS and written to the workspace.
//
// Tree kernel: one workgroup per (batch, query head), one thread per feature;
// a binary-carry stack realises the adjacent-pair tree over the splits.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int NT = 256;
constexpr int NW = 4;    // wavefronts
constexpr int KB = 64;   // keys per wavefront block
constexpr int QPW = 4;   // query heads per workgroup
constexpr int kMaxLevels = 11;

template <int D>
struct DecodeSmem {
  f32x4 p[NW][KB];         // P exchange, 4 queries per key
  float m[NW][QPW], l[NW][QPW];
  float o[NW][QPW][D];
};

template <int D>
__global__ __launch_bounds__(NT) void decode_split_kernel(DecodeParams prm, int n_qblk) {
  constexpr int FPL = D / 4;   // K features per lane group
  constexpr int NKK = FPL / 8; // MFMA k-steps over the features
  constexpr int FPV = D / 16;  // V features per lane
  __shared__ DecodeSmem<D> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;

  int lin = blockIdx.x;
  const int sp = lin % prm.n_splits;
  lin /= prm.n_splits;
  const int qblk = lin % n_qblk;
  lin /= n_qblk;
  const int hk = lin % prm.Hkv;
  const int b = lin / prm.Hkv;
  const int h0 = hk * prm.group + qblk * QPW;
  const int nq = min(QPW, prm.group - qblk * QPW);

  int64_t Lb = prm.L;
  if (prm.seqlens) Lb = min<int64_t>(max<int64_t>(prm.seqlens[b], 0), prm.L);
  const int64_t k_begin = (int64_t)sp * prm.split_len;
  const int64_t k_end = min<int64_t>(k_begin + prm.split_len, Lb);
  const int64_t n_keys = max<int64_t>(0, k_end - k_begin);
  const int n_blocks = (int)((n_keys + KB - 1) / KB);
  const int n_iter = (n_blocks + NW - 1) / NW;

  // A operand: row r of the 16x32 tile is query r % 4 (zero when outside the group slice).
  bf16x8 qa[NKK];
  {
    const int qq = l16 & 3;
    const bool ok = qq < nq;
    const u16* qp = prm.q + (int64_t)b * prm.q_sb + (int64_t)(h0 + qq) * prm.q_sh + g * FPL;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qa[kk] = ok ? as_bf16x8(*(const u32x4*)(qp + kk * 8)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  const u16* kbase = prm.k + (int64_t)b * prm.k_sb + (int64_t)hk * prm.k_sh;
  const u16* vbase = prm.v + (int64_t)b * prm.v_sb + (int64_t)hk * prm.v_sh;

  float m[QPW], lsum[QPW], acc[QPW][FPV];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    m[i] = neg_inf();
    lsum[i] = 0.f;
#pragma unroll
    for (int e = 0; e < FPV; ++e) acc[i][e] = 0.f;
  }

  for (int it = 0; it < n_iter; ++it) {
    const int64_t kb0 = k_begin + (int64_t)(it * NW + wave) * KB;
    // Scores for 4 sub-blocks of 16 keys.
    f32x4 sv[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t key = kb0 + nb * 16 + l16;
      const bool ok = key < k_end;
      const u16* kp = kbase + key * prm.k_sl + g * FPL;
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 kr = ok ? *(const u32x4*)(kp + kk * 8) : u32x4{0u, 0u, 0u, 0u};
        c = mfma16(qa[kk], as_bf16x8(kr), c);
      }
      if (!ok) c = f32x4{neg_inf(), neg_inf(), neg_inf(), neg_inf()};
      sv[nb] = c;
    }
    // V for this lane: keys kb0 + 4*jj + g, features l16*FPV ..
    u32x4 vr[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int64_t key = kb0 + 4 * jj + g;
      const bool ok = key < k_end;
      const u16* vp = vbase + key * prm.v_sl + l16 * FPV;
      if (FPV == 8) {
        vr[jj] = ok ? *(const u32x4*)vp : u32x4{0u, 0u, 0u, 0u};
      } else {
        const u32x2 t = ok ? *(const u32x2*)vp : u32x2{0u, 0u};
        vr[jj] = u32x4{t[0], t[1], 0u, 0u};
      }
    }
    // Online softmax per query over the block (max across the 16 key lanes).
    float pv[4][QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      float mt = fmaxf(fmaxf(sv[0][i], sv[1][i]), fmaxf(sv[2][i], sv[3][i]));
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
      const float m_new = fmaxf(m[i], mt);
      const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = exp2_fast((m[i] - m_use) * prm.scale_log2);
      const float nbias = -m_use * prm.scale_log2;
      float rs = 0.f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        pv[nb][i] = exp2_fast(fmaf(sv[nb][i], prm.scale_log2, nbias));
        rs += pv[nb][i];
      }
      lsum[i] = lsum[i] * alpha + rs;
      m[i] = m_new;
#pragma unroll
      for (int e = 0; e < FPV; ++e) acc[i][e] *= alpha;
    }
    if (g == 0) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) sm.p[wave][nb * 16 + l16] = f32x4{pv[nb][0], pv[nb][1], pv[nb][2], pv[nb][3]};
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const f32x4 p4 = sm.p[wave][4 * jj + g];
      float vf[FPV];
#pragma unroll
      for (int w = 0; w < FPV / 2; ++w) {
        vf[2 * w] = bf16_lo(vr[jj][w]);
        vf[2 * w + 1] = bf16_hi(vr[jj][w]);
      }
#pragma unroll
      for (int i = 0; i < QPW; ++i)
#pragma unroll
        for (int e = 0; e < FPV; ++e) acc[i][e] = fmaf(p4[i], vf[e], acc[i][e]);
    }
    __syncthreads();
  }

  // Reduce within the wavefront: lsum over the 16 key lanes, acc over the 4 lane groups.
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) lsum[i] += __shfl_xor(lsum[i], off, 64);
#pragma unroll
    for (int e = 0; e < FPV; ++e) {
      acc[i][e] += __shfl_xor(acc[i][e], 16, 64);
      acc[i][e] += __shfl_xor(acc[i][e], 32, 64);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      sm.m[wave][i] = m[i];
      sm.l[wave][i] = lsum[i];
    }
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < QPW; ++i)
#pragma unroll
      for (int e = 0; e < FPV; ++e) sm.o[wave][i][l16 * FPV + e] = acc[i][e];
  }
  __syncthreads();

  // Merge the four wavefronts and write this split's partial.
  for (int x = tid; x < nq * D; x += NT) {
    const int i = x / D, d = x % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][i]);
    float tot = 0.f, o = 0.f;
    if (M != neg_inf()) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2_fast((sm.m[w][i] - M) * prm.scale_log2);
        tot = fmaf(f, sm.l[w][i], tot);
        o = fmaf(f, sm.o[w][i][d], o);
      }
    }
    const int h = h0 + i;
    const int64_t prow = ((int64_t)b * prm.Hq + h) * prm.n_splits + sp;
    prm.part_o[prow * D + d] = (tot > 0.f) ? o / tot : 0.f;
    if (d == 0) prm.part_lse[prow] = (M == neg_inf()) ? neg_inf() : fmaf(M, prm.scale, logf(tot));
  }
}

__device__ __forceinline__ void merge_scalar(float& La, float& Oa, float Lb, float Ob) {
  float wa, wb, L;
  merge_weights(La, Lb, wa, wb, L);
  float r = 0.f;
  if (wa != 0.f) r += wa * Oa;
  if (wb != 0.f) r += wb * Ob;
  Oa = r;
  La = L;
}

template <int D>
__global__ __launch_bounds__(D) void decode_tree_kernel(DecodeParams prm) {
  const int d = threadIdx.x;
  const int h = blockIdx.x % prm.Hq, b = blockIdx.x / prm.Hq;
  const int64_t base = ((int64_t)b * prm.Hq + h) * prm.n_splits;
  float sl[kMaxLevels], so[kMaxLevels];
  unsigned pending = 0;
  for (int i = 0; i < prm.n_splits; ++i) {
    float xl = prm.part_lse[base + i];
    float xo = prm.part_o[(base + i) * D + d];
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k) {
      if (pending & (1u << k)) {
        merge_scalar(sl[k], so[k], xl, xo);
        xl = sl[k];
        xo = so[k];
        pending &= ~(1u << k);
      } else {
        sl[k] = xl;
        so[k] = xo;
        pending |= 1u << k;
        break;
      }
    }
  }
  float L = neg_inf(), O = 0.f;
  bool have = false;
#pragma unroll
  for (int k = 0; k < kMaxLevels; ++k) {
    if (pending & (1u << k)) {
      if (!have) {
        L = sl[k];
        O = so[k];
        have = true;
      } else {
        float l2 = sl[k], o2 = so[k];
        merge_scalar(l2, o2, L, O);
        L = l2;
        O = o2;
      }
    }
  }
  prm.o[(int64_t)b * prm.o_sb + (int64_t)h * prm.o_sh + d] = f32_to_bf16(O);
  if (d == 0) prm.lse[(int64_t)b * prm.Hq + h] = L;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int D, hipStream_t s) {
  const int n_qblk = (p.group + QPW - 1) / QPW;
  const int64_t grid = (int64_t)p.B * p.Hkv * n_qblk * p.n_splits;
  if (grid == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(decode_split_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p, n_qblk);
  else
    hipLaunchKernelGGL(decode_split_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p, n_qblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 tg((unsigned)((int64_t)p.B * p.Hq));
  if (D == 128)
    hipLaunchKernelGGL(decode_tree_kernel<128>, tg, dim3(128), 0, s, p);
  else
    hipLaunchKernelGGL(decode_tree_kernel<64>, tg, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
