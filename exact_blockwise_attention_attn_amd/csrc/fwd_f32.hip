// Forward partial attention for fp32 inputs: fp32 end to end on the vector ALUs.
//
// The fp32 path serves small problems that must not lose precision to a bf16
// cast.  Sixteen threads own one query row, each with D/16 features of the
// query and the accumulator in registers; the dot products are summed across
// the row's lanes.  Key and value tiles of 32 rows are staged in LDS.
// The online softmax is applied once per tile.  Same semantics, flags and
// epilogue as the bf16 kernel.
//
// Small problems give few workgroups, so a workgroup splits its keys over
// KSPL groups of threads: group g takes key tiles g, g + KSPL, ..., keeps its
// own running (max, sum, O), and the groups' results are merged in LDS in a
// fixed order at the end (deterministic; no atomics).
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int TPR = 16;         // threads per query row
constexpr int BM = 16;          // queries per workgroup
constexpr int KSPL = 2;         // groups splitting the keys
constexpr int GT = TPR * BM;    // threads per group
constexpr int NT = GT * KSPL;   // threads per workgroup
constexpr int TK = 32;          // keys per tile

// Sum over the 16 lanes of this thread's row group (TPR = 16 lanes, one DPP row).
__device__ __forceinline__ float row_sum(float x) { return sum16(x); }

template <int D>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(FwdParams p) {
  constexpr int F = D / TPR;  // features per thread
  __shared__ __attribute__((aligned(16))) float ks[KSPL][TK][D];
  __shared__ __attribute__((aligned(16))) float vs[KSPL][TK][D];
  __shared__ float m_s[KSPL][BM], l_s[KSPL][BM];
  const int tid = threadIdx.x, g = tid / GT, lt = tid % GT, r = lt / TPR, c = lt % TPR, f0 = c * F;
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
  // Every lane of a row holds the row's running maximum and sum (of its group's keys).
  float m_run = neg_inf(), l_run = 0.f;
  const int n_iter = ((kv_end + TK - 1) / TK + KSPL - 1) / KSPL;  // the same count for every group
  for (int it = 0; it < n_iter; ++it) {
    const int key0 = (it * KSPL + g) * TK;
    __syncthreads();
    for (int e = lt; e < TK * D; e += GT) {
      const int rr = e / D, cc = e % D;
      const int key = key0 + rr;
      const bool ok = key < p.Sk;
      ks[g][rr][cc] = ok ? kb[(int64_t)key * p.k.ss + cc] : 0.f;
      vs[g][rr][cc] = ok ? vb[(int64_t)key * p.v.ss + cc] : 0.f;
    }
    __syncthreads();
    float s[TK];
    float mt = neg_inf();
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int f = 0; f < F; ++f) dot = fmaf(q[f], ks[g][j][f0 + f], dot);
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
      for (int f = 0; f < F; ++f) acc[f] = fmaf(pj, vs[g][j][f0 + f], acc[f]);
    }
    m_run = m_new;
  }
  // Merge the groups' partial results (group order), then the epilogue in group 0.
  __syncthreads();
  float* accs = &ks[0][0][0];  // [KSPL][BM][D]
  if (c == 0) {
    m_s[g][r] = m_run;
    l_s[g][r] = l_run;
  }
#pragma unroll
  for (int f = 0; f < F; ++f) accs[(g * BM + r) * D + f0 + f] = acc[f];
  __syncthreads();
  if (g != 0) return;
  float M = neg_inf();
#pragma unroll
  for (int k = 0; k < KSPL; ++k) M = fmaxf(M, m_s[k][r]);
  l_run = 0.f;
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = 0.f;
#pragma unroll
  for (int k = 0; k < KSPL; ++k) {
    // Weight 0 for a group whose stabiliser is still -inf (it saw no key, or
    // only NaN scores: its NaN sum then survives 0 * NaN).
    const float w = (m_s[k][r] == neg_inf()) ? 0.f : expf(m_s[k][r] - M);
    l_run = fmaf(w, l_s[k][r], l_run);
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = fmaf(w, accs[(k * BM + r) * D + f0 + f], acc[f]);
  }
  m_run = M;
  if (!qok) return;
  // Only an exactly zero sum is a row with no visible key; NaN stays NaN.
  const bool empty = l_run == 0.f;
  const float lse_this = empty ? neg_inf() : m_run + logf(l_run);
  const float inv = empty ? 0.f : 1.0f / l_run;
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

int64_t items_fwd_f32(const FwdParams& p) { return (int64_t)p.B * p.Hq * ((p.Sq + BM - 1) / BM) * NT; }

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
