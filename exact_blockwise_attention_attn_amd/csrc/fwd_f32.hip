// Forward partial attention for fp32 inputs: fp32 end to end on the vector ALUs.
//
// The fp32 path serves small problems that must not lose precision to a bf16
// cast.  One thread owns one query row (query and accumulator in registers);
// key and value tiles of 32 rows are staged in LDS and read as broadcasts.
// The online softmax is applied once per tile.  Same semantics, flags and
// epilogue as the bf16 kernel.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int BM = 64;  // queries per workgroup (one per thread)
constexpr int TK = 32;  // keys per tile

template <int D>
__global__ __launch_bounds__(BM) void fwd_f32_kernel(FwdParams p) {
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x % p.n_units;
  const int bh = blockIdx.x / p.n_units;
  const int h = bh % p.Hq, b = bh / p.Hq, hk = h / p.group;
  const float* qb = (const float*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
  const float* kb = (const float*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const float* vb = (const float*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;

  const int qt = p.causal ? p.n_qtiles - 1 - unit : unit;
  const int q0 = qt * BM;
  const int qi = q0 + tid;
  const bool qok = qi < p.Sq;

  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qok ? qb[(int64_t)qi * p.q.ss + d] : 0.f;
    acc[d] = 0.f;
  }
  const int q_last = min(q0 + BM, p.Sq) - 1;
  int kv_end = p.Sk;
  int64_t lim = (int64_t)p.Sk - 1;
  if (p.causal) {
    kv_end = (int)max<int64_t>(0, min<int64_t>(p.delta + q_last + 1, p.Sk));
    lim = min<int64_t>(p.delta + qi, lim);
  }
  float m_run = neg_inf(), l_run = 0.f;
  for (int key0 = 0; key0 < kv_end; key0 += TK) {
    __syncthreads();
    for (int e = tid; e < TK * D; e += BM) {
      const int r = e / D, c = e % D;
      const int key = key0 + r;
      const bool ok = key < p.Sk;
      ks[r][c] = ok ? kb[(int64_t)key * p.k.ss + c] : 0.f;
      vs[r][c] = ok ? vb[(int64_t)key * p.v.ss + c] : 0.f;
    }
    __syncthreads();
    float s[TK];
    float mt = neg_inf();
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(q[d], ks[j][d], dot);
      s[j] = (key0 + j <= lim) ? dot * p.scale : neg_inf();
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float pj = expf(s[j] - m_use);
      l_run += pj;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(pj, vs[j][d], acc[d]);
    }
    m_run = m_new;
  }
  if (!qok) return;
  const float lse_this = (m_run == neg_inf()) ? neg_inf() : m_run + logf(l_run);
  const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
  float* lse_ptr = p.lse + ((int64_t)b * p.Hq + h) * p.Sq + qi;
  float w_old = 0.f, w_new = 1.f, L = lse_this;
  if (p.accumulate) merge_weights(*lse_ptr, lse_this, w_old, w_new, L);
  w_new *= inv;
  const int64_t orow = (int64_t)b * p.o.sb + (int64_t)qi * p.o.ss + (int64_t)h * p.o.sh;
  const int64_t frow = (int64_t)b * p.o_final.sb + (int64_t)qi * p.o_final.ss + (int64_t)h * p.o_final.sh;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    float v = acc[d] * w_new;
    if (p.o_f32) {
      float* dst = (float*)p.o.ptr + orow + d;
      if (p.accumulate && w_old != 0.f) v = fmaf(w_old, *dst, v);
      *dst = v;
    } else {
      ((u16*)p.o.ptr)[orow + d] = f32_to_bf16(v);
    }
    if (p.o_final.ptr) ((u16*)p.o_final.ptr)[frow + d] = f32_to_bf16(v);
  }
  *lse_ptr = L;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p0, int D, hipStream_t s) {
  FwdParams p = p0;
  p.n_qtiles = (p.Sq + BM - 1) / BM;
  p.n_units = p.n_qtiles;
  const int64_t grid = (int64_t)p.B * p.Hq * p.n_units;
  if (grid == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(BM), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(BM), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
