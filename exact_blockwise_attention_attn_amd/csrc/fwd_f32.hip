// Forward partial attention for fp32 inputs: fp32 end to end on the vector ALUs.
//
// The fp32 path serves small problems that must not lose precision to a bf16
// cast.  Sixteen threads own one query row, each with D/16 features of the
// query and the accumulator in registers; the dot products are summed across
// the row's lanes.  Key and value tiles of 32 rows are staged in LDS.
// The online softmax is applied once per tile.  Same semantics, flags and
// epilogue as the bf16 kernel.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int TPR = 16;         // threads per query row
constexpr int BM = 16;          // queries per workgroup
constexpr int NT = TPR * BM;    // threads per workgroup
constexpr int TK = 32;          // keys per tile

// Sum over the 16 lanes of this thread's row group (TPR = 16 lanes, one DPP row).
__device__ __forceinline__ float row_sum(float x) { return sum16(x); }

template <int D>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(FwdParams p) {
  constexpr int F = D / TPR;  // features per thread
  __shared__ __attribute__((aligned(16))) float ks[TK][D];
  __shared__ __attribute__((aligned(16))) float vs[TK][D];
  const int tid = threadIdx.x, r = tid / TPR, c = tid % TPR, f0 = c * F;
  const int unit = blockIdx.x % p.n_units;
  const int bh = blockIdx.x / p.n_units;
  const int h = bh % p.Hq, b = bh / p.Hq, hk = h / p.group;
  const float* qb = (const float*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
  const float* kb = (const float*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const float* vb = (const float*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;

  const int qt = p.causal ? p.n_qtiles - 1 - unit : unit;
  const int q0 = qt * BM;
  const int qi = q0 + r;
  const bool qok = qi < p.Sq;

  float q[F], acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    q[f] = qok ? qb[(int64_t)qi * p.q.ss + f0 + f] : 0.f;
    acc[f] = 0.f;
  }
  const int q_last = min(q0 + BM, p.Sq) - 1;
  int kv_end = p.Sk;
  int64_t lim = (int64_t)p.Sk - 1;
  if (p.causal) {
    kv_end = (int)max<int64_t>(0, min<int64_t>(p.delta + q_last + 1, p.Sk));
    lim = min<int64_t>(p.delta + qi, lim);
  }
  // Every lane of a row holds the row's running maximum and sum.
  float m_run = neg_inf(), l_run = 0.f;
  for (int key0 = 0; key0 < kv_end; key0 += TK) {
    __syncthreads();
    for (int e = tid; e < TK * D; e += NT) {
      const int rr = e / D, cc = e % D;
      const int key = key0 + rr;
      const bool ok = key < p.Sk;
      ks[rr][cc] = ok ? kb[(int64_t)key * p.k.ss + cc] : 0.f;
      vs[rr][cc] = ok ? vb[(int64_t)key * p.v.ss + cc] : 0.f;
    }
    __syncthreads();
    float s[TK];
    float mt = neg_inf();
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int f = 0; f < F; ++f) dot = fmaf(q[f], ks[j][f0 + f], dot);
      dot = row_sum(dot);
      s[j] = (key0 + j <= lim) ? dot * p.scale : neg_inf();
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float pj = expf(s[j] - m_use);
      l_run += pj;
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = fmaf(pj, vs[j][f0 + f], acc[f]);
    }
    m_run = m_new;
  }
  if (!qok) return;
  const float lse_this = (m_run == neg_inf()) ? neg_inf() : m_run + logf(l_run);
  const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
  float* lse_ptr = p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)qi * p.lse_ss;
  // The row's 16 lanes are in one wavefront: all read the running LSE before lane 0 writes it.
  float w_old = 0.f, w_new = 1.f, L = lse_this;
  if (p.accumulate) merge_weights(*lse_ptr, lse_this, w_old, w_new, L);
  w_new *= inv;
  const int64_t orow = (int64_t)b * p.o.sb + (int64_t)qi * p.o.ss + (int64_t)h * p.o.sh + f0;
  const int64_t frow = (int64_t)b * p.o_final.sb + (int64_t)qi * p.o_final.ss + (int64_t)h * p.o_final.sh + f0;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    float v = acc[f] * w_new;
    if (p.o_f32) {
      float* dst = (float*)p.o.ptr + orow + f;
      if (p.accumulate && w_old != 0.f) v = fmaf(w_old, *dst, v);
      *dst = v;
    } else {
      ((u16*)p.o.ptr)[orow + f] = f32_to_bf16(v);
    }
    if (p.o_final.ptr) ((u16*)p.o_final.ptr)[frow + f] = f32_to_bf16(v);
  }
  if (c == 0) *lse_ptr = L;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p0, int D, hipStream_t s) {
  FwdParams p = p0;
  p.n_qtiles = (p.Sq + BM - 1) / BM;
  p.n_units = p.n_qtiles;
  const int64_t grid = (int64_t)p.B * p.Hq * p.n_units;
  if (grid == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
