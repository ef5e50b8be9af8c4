// Backward helpers shared by both dtypes (the per-row statistics: delta =
// rowsum(dO * O) and the rescaled LSE) and the fp32 backward kernels (vector
// ALUs, fp32 end to end).
//
// fp32 dQ kernel: 16 threads per query row; key/value tiles staged in LDS.
// fp32 dK/dV kernel: 16 threads per key row; query tiles (q, dO, LSE, delta)
// staged in LDS, looping over every query head that reads the key/value head.
// Both recompute P = exp(s - LSE) from the saved LSE; neither re-runs the forward.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

// ---------------------------------------------------------------- prepare --
// Fills the statistics workspace: for row i of (b, h), LSE_i * log2(e) (+inf
// when LSE_i = -inf, i.e. the row sees no key) and -delta_i with delta_i =
// sum_t dO_it O_it, plus padding rows up to a multiple of 64 (LSE +inf, delta 0)
// so that the kernels can fetch whole 64-row tiles of statistics.  The negated
// delta lets the bf16 dK/dV kernel start its dP accumulator at -delta, so the
// matrix cores form dP - delta.

template <int D, bool BF16>
__global__ __launch_bounds__(256) void prepare_kernel(BwdParams p) {
  constexpr int TPR = D / 8;  // threads per row, 8 features each
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / TPR;  // over (b, h, padded i), i fastest
  const int c = (int)(gid % TPR);
  const int64_t rows = (int64_t)p.B * p.Hq * p.Sq_pad;
  const bool ok = row < rows;
  int i = 0, h = 0, b = 0, sq = 0;
  int64_t bh = 0, r0 = 0;  // r0: first row of the sequence (packed variable-length batches)
  float acc = 0.f;
  if (ok) {
    i = (int)(row % p.Sq_pad);
    bh = row / p.Sq_pad;
    h = (int)(bh % p.Hq);
    b = (int)(bh / p.Hq);
    sq = p.Sq;
    if (p.cu_q) {
      r0 = p.cu_q[b];
      sq = min(max(p.cu_q[b + 1] - p.cu_q[b], 0), p.Sq);  // never past the declared longest length
      b = 0;
    }
    if (i < sq) {
      const int64_t oo = (int64_t)b * p.o.sb + (r0 + i) * p.o.ss + (int64_t)h * p.o.sh + c * 8;
      const int64_t od = (int64_t)b * p.dout.sb + (r0 + i) * p.dout.ss + (int64_t)h * p.dout.sh + c * 8;
      if (BF16) {
        const u32x4 a = *(const u32x4*)((const u16*)p.o.ptr + oo);
        const u32x4 g = *(const u32x4*)((const u16*)p.dout.ptr + od);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc = fmaf(bf16_lo(a[w]), bf16_lo(g[w]), acc);
          acc = fmaf(bf16_hi(a[w]), bf16_hi(g[w]), acc);
        }
      } else {
        const float* a = (const float*)p.o.ptr + oo;
        const float* g = (const float*)p.dout.ptr + od;
#pragma unroll
        for (int w = 0; w < 8; ++w) acc = fmaf(a[w], g[w], acc);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (ok && c == 0) {
    float* base = p.stats + bh * 2 * p.Sq_pad;
    float l2 = pos_inf();
    if (i < sq) {
      const float lse = p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (r0 + i) * p.lse_ss];
      l2 = (lse == neg_inf()) ? pos_inf() : lse * kLog2e;
    }
    base[i] = l2;
    base[p.Sq_pad + i] = (i < sq) ? -acc : 0.f;
  }
}

// ------------------------------------------------------------- fp32 dQ ----
//
// Both fp32 kernels give each row (a query for dQ, a key for dK/dV) 16
// threads: thread c of a row holds features c*F .. c*F+F-1 (F = D/16) of the
// row's operands and accumulators, the two dot products of a pair are summed
// over the row's 16 lanes, and each thread updates its own features.  Tiles of
// the other side's rows are staged in LDS and read by all rows.

// Small problems give few workgroups, so each workgroup also splits the
// dimension it walks over groups of threads (keys for dQ, queries for dK/dV);
// the groups' partial sums are added in LDS in a fixed order at the end
// (deterministic; no atomics).
constexpr int TPR = 16;                 // threads per row
constexpr int FROWS = 16;               // query rows per dQ workgroup
constexpr int QSPL = 2;                 // dQ: groups splitting the keys
constexpr int FTK = 32;                 // dQ: key rows per staged tile
constexpr int QGT = TPR * FROWS;        // dQ: threads per group
constexpr int QNT = QGT * QSPL;         // dQ: threads per workgroup
constexpr int KROWS = 8;                // key rows per dK/dV workgroup
constexpr int KSPL = 8;                 // dK/dV: groups splitting the queries
constexpr int KTK = 16;                 // dK/dV: query rows per staged tile
constexpr int KGT = TPR * KROWS;        // dK/dV: threads per group
constexpr int KNT = KGT * KSPL;         // dK/dV: threads per workgroup

// Sum over the 16 lanes of this thread's row group (TPR = 16 lanes, one DPP row).
__device__ __forceinline__ float row_sum(float x) { return sum16(x); }

template <int D>
__global__ __launch_bounds__(QNT) void dq_f32_kernel(BwdParams p) {
  constexpr int F = D / TPR;
  __shared__ __attribute__((aligned(16))) float ks[QSPL][FTK][D];
  __shared__ __attribute__((aligned(16))) float vs[QSPL][FTK][D];
  const int tid = threadIdx.x, g = tid / QGT, lt = tid % QGT, r = lt / TPR, c = lt % TPR, f0 = c * F;
  const int qt = blockIdx.x % p.n_qtiles;
  const int bh = blockIdx.x / p.n_qtiles;
  const int h = bh % p.Hq, b = bh / p.Hq, hk = h / p.group;
  const int qi = qt * FROWS + r;
  const bool qok = qi < p.Sq;
  const float* qb = (const float*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
  const float* dob = (const float*)p.dout.ptr + (int64_t)b * p.dout.sb + (int64_t)h * p.dout.sh;
  const float* kb = (const float*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const float* vb = (const float*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;
  float q[F], dO[F], dq[F];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    q[f] = qok ? qb[(int64_t)qi * p.q.ss + f0 + f] : 0.f;
    dO[f] = qok ? dob[(int64_t)qi * p.dout.ss + f0 + f] : 0.f;
    dq[f] = 0.f;
  }
  const float lse = qok ? p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)qi * p.lse_ss] : neg_inf();
  const float dlt = qok ? -p.stats[((int64_t)b * p.Hq + h) * 2 * p.Sq_pad + p.Sq_pad + qi] : 0.f;
  const bool live = lse != neg_inf();
  const int q_last = min(qt * FROWS + FROWS, p.Sq) - 1;
  int kv_end = p.Sk;
  int64_t lim = (int64_t)p.Sk - 1;  // last key this row sees
  if (p.causal) {
    kv_end = (int)max<int64_t>(0, min<int64_t>(p.delta_pos + q_last + 1, p.Sk));
    lim = min<int64_t>(p.delta_pos + qi, lim);
  }
  // Group g takes key tiles g, g + QSPL, ...; every group runs the same count.
  const int n_iter = ((kv_end + FTK - 1) / FTK + QSPL - 1) / QSPL;
  for (int it = 0; it < n_iter; ++it) {
    const int key0 = (it * QSPL + g) * FTK;
    __syncthreads();
    for (int e = lt; e < FTK * D; e += QGT) {
      const int rr = e / D, cc = e % D;
      const int key = key0 + rr;
      const bool ok = key < p.Sk;
      ks[g][rr][cc] = ok ? kb[(int64_t)key * p.k.ss + cc] : 0.f;
      vs[g][rr][cc] = ok ? vb[(int64_t)key * p.v.ss + cc] : 0.f;
    }
    __syncthreads();
    // Every lane runs every step (the row sums exchange data across lanes);
    // pairs a row does not see get P = 0.
#pragma unroll 16
    for (int j = 0; j < FTK; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int f = 0; f < F; ++f) {
        s = fmaf(q[f], ks[g][j][f0 + f], s);
        dp = fmaf(dO[f], vs[g][j][f0 + f], dp);
      }
      s = row_sum(s);
      dp = row_sum(dp);
      const bool vis = live && key0 + j <= lim;
      const float pj = vis ? expf(s * p.scale - lse) : 0.f;
      const float ds = pj * (dp - dlt);
#pragma unroll
      for (int f = 0; f < F; ++f) dq[f] = fmaf(ds, ks[g][j][f0 + f], dq[f]);
    }
  }
  // Add the groups' partials in group order.
  __syncthreads();
  float* red = &ks[0][0][0];  // [QSPL][FROWS][D]
#pragma unroll
  for (int f = 0; f < F; ++f) red[(g * FROWS + r) * D + f0 + f] = dq[f];
  __syncthreads();
  if (g != 0 || !qok) return;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    float t = red[r * D + f0 + f];
#pragma unroll
    for (int k = 1; k < QSPL; ++k) t += red[(k * FROWS + r) * D + f0 + f];
    dq[f] = t;
  }
  float* accp = p.dq_acc + (((int64_t)b * p.Sq + qi) * p.Hq + h) * D + f0;
  float* dqp = p.finalize_dq
                   ? (float*)p.dq.ptr + (int64_t)b * p.dq.sb + (int64_t)qi * p.dq.ss + (int64_t)h * p.dq.sh + f0
                   : nullptr;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    float v = dq[f] * p.scale;
    if (!p.dq_overwrite) v += accp[f];
    accp[f] = v;
    if (dqp) dqp[f] = v;
  }
}

// ---------------------------------------------------------- fp32 dK/dV ----

template <int D>
__global__ __launch_bounds__(KNT) void dkdv_f32_kernel(BwdParams p) {
  constexpr int F = D / TPR;
  __shared__ __attribute__((aligned(16))) float qs[KSPL][KTK][D];
  __shared__ __attribute__((aligned(16))) float dos[KSPL][KTK][D];
  __shared__ float ls[KSPL][KTK];
  __shared__ float ds_[KSPL][KTK];
  const int tid = threadIdx.x, g = tid / KGT, lt = tid % KGT, r = lt / TPR, c = lt % TPR, f0 = c * F;
  const int kt = blockIdx.x % p.n_ktiles;
  const int bh = blockIdx.x / p.n_ktiles;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  const int kj = kt * KROWS + r;
  const bool kok = kj < p.Sk;
  const float* kb = (const float*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh;
  const float* vb = (const float*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh;
  float k[F], v[F], dk[F], dv[F];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    k[f] = kok ? kb[(int64_t)kj * p.k.ss + f0 + f] : 0.f;
    v[f] = kok ? vb[(int64_t)kj * p.v.ss + f0 + f] : 0.f;
    dk[f] = 0.f;
    dv[f] = 0.f;
  }
  const int64_t need = (int64_t)kj - p.delta_pos;  // causal: query index must be >= need
  int i_start = 0;
  if (p.causal) i_start = (int)min<int64_t>(p.Sq, max<int64_t>(0, (int64_t)kt * KROWS - p.delta_pos));
  i_start = (i_start / KTK) * KTK;
  // Group g takes query tiles g, g + KSPL, ... from i_start; every group runs the same count.
  const int n_iter = ((p.Sq - i_start + KTK - 1) / KTK + KSPL - 1) / KSPL;
  for (int hh = 0; hh < p.group; ++hh) {
    const int h = hk * p.group + hh;
    const float* qb = (const float*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
    const float* dob = (const float*)p.dout.ptr + (int64_t)b * p.dout.sb + (int64_t)h * p.dout.sh;
    const float* lseb = p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh;
    const float* dltb = p.stats + ((int64_t)b * p.Hq + h) * 2 * p.Sq_pad + p.Sq_pad;
    for (int it = 0; it < n_iter; ++it) {
      const int i0 = i_start + (it * KSPL + g) * KTK;
      __syncthreads();
      for (int e = lt; e < KTK * D; e += KGT) {
        const int rr = e / D, cc = e % D;
        const int i = i0 + rr;
        const bool ok = i < p.Sq;
        qs[g][rr][cc] = ok ? qb[(int64_t)i * p.q.ss + cc] : 0.f;
        dos[g][rr][cc] = ok ? dob[(int64_t)i * p.dout.ss + cc] : 0.f;
      }
      if (lt < KTK) {
        const int i = i0 + lt;
        ls[g][lt] = (i < p.Sq) ? lseb[(int64_t)i * p.lse_ss] : neg_inf();
        ds_[g][lt] = (i < p.Sq) ? -dltb[i] : 0.f;
      }
      __syncthreads();
#pragma unroll 2
      for (int rr = 0; rr < KTK; ++rr) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int f = 0; f < F; ++f) {
          s = fmaf(k[f], qs[g][rr][f0 + f], s);
          dp = fmaf(v[f], dos[g][rr][f0 + f], dp);
        }
        s = row_sum(s);
        dp = row_sum(dp);
        const float lse = ls[g][rr];
        const bool vis = kok && lse != neg_inf() && !(p.causal && (int64_t)(i0 + rr) < need);
        const float pj = vis ? expf(s * p.scale - lse) : 0.f;
        const float ds = pj * (dp - ds_[g][rr]);
#pragma unroll
        for (int f = 0; f < F; ++f) {
          dv[f] = fmaf(pj, dos[g][rr][f0 + f], dv[f]);
          dk[f] = fmaf(ds, qs[g][rr][f0 + f], dk[f]);
        }
      }
    }
  }
  // Add the groups' partials in group order.
  __syncthreads();
  float* redk = &qs[0][0][0];   // [KSPL][KROWS][D]
  float* redv = &dos[0][0][0];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    redk[(g * KROWS + r) * D + f0 + f] = dk[f];
    redv[(g * KROWS + r) * D + f0 + f] = dv[f];
  }
  __syncthreads();
  if (g != 0 || !kok) return;
  float* dkp = (float*)p.dk.ptr + (int64_t)b * p.dk.sb + (int64_t)kj * p.dk.ss + (int64_t)hk * p.dk.sh + f0;
  float* dvp = (float*)p.dv.ptr + (int64_t)b * p.dv.sb + (int64_t)kj * p.dv.ss + (int64_t)hk * p.dv.sh + f0;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    float tk = redk[r * D + f0 + f], tv = redv[r * D + f0 + f];
#pragma unroll
    for (int k2 = 1; k2 < KSPL; ++k2) {
      tk += redk[(k2 * KROWS + r) * D + f0 + f];
      tv += redv[(k2 * KROWS + r) * D + f0 + f];
    }
    dkp[f] = tk * p.scale;
    dvp[f] = tv;
  }
}

}  // namespace

int64_t items_bwd_prepare(const BwdParams& p, int D) {
  const int64_t threads = (int64_t)p.B * p.Hq * p.Sq_pad * (D / 8);
  return (threads + 255) / 256 * 256;
}

int64_t items_bwd_f32(const BwdParams& p) {
  const int64_t gk = (int64_t)p.B * p.Hkv * ((p.Sk + KROWS - 1) / KROWS);
  const int64_t gq = (int64_t)p.B * p.Hq * ((p.Sq + FROWS - 1) / FROWS);
  return std::max(gk * KNT, gq * QNT);
}

hipError_t launch_bwd_prepare(const BwdParams& p, int D, int is_bf16, hipStream_t s) {
  const int64_t threads = (int64_t)p.B * p.Hq * p.Sq_pad * (D / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (D == 128) {
    if (is_bf16) hipLaunchKernelGGL((prepare_kernel<128, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prepare_kernel<128, false>), grid, dim3(256), 0, s, p);
  } else {
    if (is_bf16) hipLaunchKernelGGL((prepare_kernel<64, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prepare_kernel<64, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const BwdParams& p0, int D, int run_dq, hipStream_t s) {
  BwdParams p = p0;
  p.n_ktiles = (p.Sk + KROWS - 1) / KROWS;
  p.n_qtiles = (p.Sq + FROWS - 1) / FROWS;
  const int64_t gk = (int64_t)p.B * p.Hkv * p.n_ktiles;
  if (gk > 0) {
    if (D == 128) hipLaunchKernelGGL(dkdv_f32_kernel<128>, dim3((unsigned)gk), dim3(KNT), 0, s, p);
    else hipLaunchKernelGGL(dkdv_f32_kernel<64>, dim3((unsigned)gk), dim3(KNT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t gq = (int64_t)p.B * p.Hq * p.n_qtiles;
  if (run_dq && gq > 0) {
    if (D == 128) hipLaunchKernelGGL(dq_f32_kernel<128>, dim3((unsigned)gq), dim3(QNT), 0, s, p);
    else hipLaunchKernelGGL(dq_f32_kernel<64>, dim3((unsigned)gq), dim3(QNT), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace attn
