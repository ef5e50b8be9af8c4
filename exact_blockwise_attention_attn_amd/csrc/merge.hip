// Log-sum-exp weighted merge of partial (O, LSE) results over disjoint key sets:
// the aggregation of local results into the global one (BurstAttention page)
// and the reduction over sequence chunks (Tree Attention page).
//
// One thread merges a 4-feature slice of one row across all parts, so the
// work is a pure streaming pass (HBM-bound).  The tree mode reproduces the
// level-by-level adjacent-pair tree with a binary-carry stack: pushing part i
// merges equal-sized subtrees as they complete, and the leftover subtrees are
// merged from the right at the end, which yields exactly the tree in which
// each level pairs (2i, 2i+1) and carries an odd element upward.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int NT = 256;
constexpr int kMaxLevels = 11;  // up to 1024 parts

__device__ __forceinline__ void merge2(float& La, f32x4& Oa, float Lb, f32x4 Ob) {
  float wa, wb, L;
  merge_weights(La, Lb, wa, wb, L);
  f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wa != 0.f) r += wa * Oa;
  if (wb != 0.f) r += wb * Ob;
  Oa = r;
  La = L;
}

template <int D>
__global__ __launch_bounds__(NT) void merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t row = gid / TPR;
  const int c = (int)(gid % TPR);
  const int64_t rows = (int64_t)p.B * p.S * p.H;
  if (row >= rows) return;
  const int h = (int)(row % p.H);
  const int64_t r2 = row / p.H;
  const int s = (int)(r2 % p.S);
  const int b = (int)(r2 / p.S);
  const float* op = p.o_parts + (int64_t)b * p.o_sb + (int64_t)s * p.o_ss + (int64_t)h * p.o_sh + c * 4;
  const float* lp = p.lse_parts + ((int64_t)b * p.H + h) * p.S + s;

  float L = neg_inf();
  f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
  // The parts are read U at a time, all loads issued before the batch is
  // folded in part order (the arithmetic is that of one part at a time): with
  // one load in flight per fold the pass was latency-bound (4.75 TB/s on 17
  // parts of 64 MiB; 5.0 batched, 5.15 with the sequential mode's batches
  // double-buffered).  Indices past the last part re-read it and are not
  // folded.
  constexpr int U = 8;
  float xl[U];
  f32x4 xo[U];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(i0 + u, p.n_parts - 1);
      xl[u] = lp[(int64_t)i * p.lse_part_stride];
      xo[u] = *(const f32x4*)(op + (int64_t)i * p.o_part_stride);
    }
  };
  if (!p.tree) {
    // Double-buffered: the next batch's loads are issued before this one is folded.
    load_batch(0);
    for (int i0 = 0; i0 < p.n_parts; i0 += U) {
      float cl[U];
      f32x4 co[U];
#pragma unroll
      for (int u = 0; u < U; ++u) cl[u] = xl[u], co[u] = xo[u];
      if (i0 + U < p.n_parts) load_batch(i0 + U);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u < p.n_parts) merge2(L, O, cl[u], co[u]);
    }
  } else {
    float sl[kMaxLevels];
    f32x4 so[kMaxLevels];
    unsigned pending = 0;
    for (int i0 = 0; i0 < p.n_parts; i0 += U) {
      load_batch(i0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i0 + u >= p.n_parts) break;
        float cl = xl[u];
        f32x4 co = xo[u];
        // Carry the new subtree up the stack until it finds a free level.  A
        // flag instead of a break keeps every stack index a compile-time
        // constant, so the stack lives in registers.
        bool carry = true;
#pragma unroll
        for (int k = 0; k < kMaxLevels; ++k) {
          if (carry) {
            if (pending & (1u << k)) {
              merge2(sl[k], so[k], cl, co);  // left = earlier subtree
              cl = sl[k];
              co = so[k];
              pending &= ~(1u << k);
            } else {
              sl[k] = cl;
              so[k] = co;
              pending |= 1u << k;
              carry = false;
            }
          }
        }
      }
    }
    bool have = false;
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k) {
      if (pending & (1u << k)) {
        if (!have) {
          L = sl[k];
          O = so[k];
          have = true;
        } else {
          float l2 = sl[k];
          f32x4 o2 = so[k];
          merge2(l2, o2, L, O);  // earlier (larger) subtree on the left
          L = l2;
          O = o2;
        }
      }
    }
  }
  const int64_t orow = (int64_t)b * p.out.sb + (int64_t)s * p.out.ss + (int64_t)h * p.out.sh + c * 4;
  if (p.out_f32) {
    *(f32x4*)((float*)p.out.ptr + orow) = O;
  } else {
    *(u32x2*)((u16*)p.out.ptr + orow) = u32x2{pack_bf16x2(O[0], O[1]), pack_bf16x2(O[2], O[3])};
  }
  if (c == 0) p.lse_out[((int64_t)b * p.H + h) * p.S + s] = L;
}

}  // namespace

int64_t items_merge(const MergeParams& p, int D) {
  const int64_t threads = (int64_t)p.B * p.S * p.H * (D / 4);
  return (threads + NT - 1) / NT * NT;
}

hipError_t launch_merge(const MergeParams& p, int D, hipStream_t s) {
  const int64_t threads = (int64_t)p.B * p.S * p.H * (D / 4);
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + NT - 1) / NT;
  if (D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
