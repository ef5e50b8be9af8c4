// Split-KV decode with grouped heads, then a binary-tree merge of the split
// partials (Lean Attention and Tree Attention abstracts: the softmax reduction
// is associative, so a long KV sequence can be cut into chunks whose partial
// results are reduced as a tree).
//
// Split kernel: one workgroup per (batch, key/value head, group slice of up to
// 4 query heads, split).  The cache is read exactly once per key/value head, so
// the 4 query heads of a GQA group share every byte.  The split's keys come in
// tiles of 16; wavefront w takes tiles w, w + 4, w + 8, ... and runs on its own
// (no barrier until the final merge), loading K and V straight into registers
// with four tiles in flight, so that a CU keeps about 256 KB of loads
// outstanding, enough to cover HBM latency under full load.  Per tile:
//   * scores with the 16x16x32 bf16 MFMA, the 4 queries replicated over the 16
//     rows so every lane receives the 4 scores of its key (lane group g holds
//     features 8 (4 kk + g) .. +7 of k-step kk, loaded as 64-byte row pieces);
//   * online softmax per tile (max over the 16 key lanes);
//   * P goes through a small per-wavefront LDS buffer to the layout in which V
//     was loaded (16 lanes cover one key row) and O accumulates on the vector
//     ALUs.
// The four wavefronts' partials are merged in LDS and written to the workspace.
//
// Tree kernel: one workgroup per (batch, query head); the adjacent-pair tree
// over the split LSEs is built level by level in LDS and fixes each split's
// weight in the root (see decode_tree_kernel).
#include <mutex>
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int NT = 256;
constexpr int NW = 4;      // wavefronts
constexpr int KW = 16;     // keys per tile
constexpr int DEPTH = 4;   // tiles in flight per wavefront
constexpr int QPW = 4;     // query heads per workgroup

// Cache bytes are read exactly once per call.  V rows are read whole (16 lanes
// x 16 B cover a 256-byte row) with the non-temporal hint, so they stream past
// the caches.  K rows are read 64 bytes per instruction (the operand layout of
// the score MFMA), two instructions per 128-byte line; with the streaming hint
// on K as well, a call fetched 9% more bytes than the cache holds (lines
// fetched twice) and ran slower, so K loads stay ordinary.
template <class T>
__device__ __forceinline__ T stream_load(const T* p) {
  return __builtin_nontemporal_load(p);
}

template <int D>
struct KvTile {
  using VT = typename std::conditional<D == 128, u32x4, u32x2>::type;
  u32x4 k[D / 32];  // K: this lane's key, features 8 (4 kk + g) ..
  VT v[4];          // V: keys 4 j + g, features (D / 16) l16 ..
};

// One partial: keys [k_begin, k_begin + n_keys) of sequence b for the query
// heads h0 .. h0 + nq - 1 (one group slice of key/value head hk), written to
// row row(q) of the partials for query q of the slice.  Every thread of the
// workgroup calls it with the same arguments; it ends with the partial written.
template <int D, class Row>
__device__ __forceinline__ void split_piece(const DecodeParams& prm, int b, int hk, int h0, int nq, int64_t k_begin,
                                            int n_keys, Row row) {
  constexpr int NKK = D / 32;  // MFMA k-steps over the features
  constexpr int FPV = D / 16;  // V features per lane
  __shared__ __attribute__((aligned(16))) f32x4 pex[NW][KW];  // P of 4 queries per key
  __shared__ float m_s[NW][QPW], l_s[NW][QPW];
  __shared__ __attribute__((aligned(16))) float o_s[NW][QPW][D];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int n_tiles = (n_keys + KW - 1) / KW;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + NW - 1) / NW : 0;

  // A operand: row r of the 16x32 tile is query r % 4 (zero outside the group slice).
  bf16x8 qa[NKK];
  {
    const int qq = l16 & 3;
    const bool ok = qq < nq;
    const u16* qp = prm.q + (int64_t)b * prm.q_sb + (int64_t)(h0 + qq) * prm.q_sh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qa[kk] = ok ? as_bf16x8(*(const u32x4*)(qp + (4 * kk + g) * 8)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  const u16* kbase = prm.k + (int64_t)b * prm.k_sb + (int64_t)hk * prm.k_sh + k_begin * prm.k_sl;
  const u16* vbase = prm.v + (int64_t)b * prm.v_sb + (int64_t)hk * prm.v_sh + k_begin * prm.v_sl;

  // Load this wavefront's i-th tile.  Indices past its last tile load the last
  // tile again (cache hits, never used), so every pass issues the same loads.
  auto load = [&](int i, KvTile<D>& t) {
    const int key0 = (wave + NW * min(i, max(my_tiles - 1, 0))) * KW;
    const int kkey = min(key0 + l16, n_keys - 1);
    const u16* kp = kbase + (int64_t)kkey * prm.k_sl;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) t.k[kk] = *(const u32x4*)(kp + (4 * kk + g) * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vkey = min(key0 + 4 * j + g, n_keys - 1);
      t.v[j] = stream_load((const typename KvTile<D>::VT*)(vbase + (int64_t)vkey * prm.v_sl + FPV * l16));
    }
  };

  float m[QPW], lsum[QPW], acc[QPW][FPV];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    m[i] = neg_inf();
    lsum[i] = 0.f;
#pragma unroll
    for (int e = 0; e < FPV; ++e) acc[i][e] = 0.f;
  }

  auto compute = [&](int i, const KvTile<D>& t) {
    const int key0 = (wave + NW * i) * KW;
    f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) c = mfma16(qa[kk], as_bf16x8(t.k[kk]), c);
    if (key0 + l16 >= n_keys) c = f32x4{neg_inf(), neg_inf(), neg_inf(), neg_inf()};
    // Online softmax per query over the 16 keys.
    float pv[QPW];
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
      float mt = c[q];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
      const float m_new = fmaxf(m[q], mt);
      const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = exp2_fast((m[q] - m_use) * prm.scale_log2);
      pv[q] = exp2_fast(fmaf(c[q], prm.scale_log2, -m_use * prm.scale_log2));
      lsum[q] = lsum[q] * alpha + pv[q];
      m[q] = m_new;
#pragma unroll
      for (int e = 0; e < FPV; ++e) acc[q][e] *= alpha;
    }
    // Hand P to the V layout within the wavefront (LDS operations of one
    // wavefront complete in order; the wait makes the stores visible).
    if (g == 0) pex[wave][l16] = f32x4{pv[0], pv[1], pv[2], pv[3]};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 p4 = pex[wave][4 * j + g];
      float vf[FPV];
#pragma unroll
      for (int x = 0; x < FPV / 2; ++x) {
        vf[2 * x] = bf16_lo(t.v[j][x]);
        vf[2 * x + 1] = bf16_hi(t.v[j][x]);
      }
#pragma unroll
      for (int q = 0; q < QPW; ++q)
#pragma unroll
        for (int e = 0; e < FPV; ++e) acc[q][e] = fmaf(p4[q], vf[e], acc[q][e]);
    }
    // The next tile's P store must not overtake these reads (in-order LDS).
    asm volatile("" ::: "memory");
  };

  if (my_tiles > 0) {
    KvTile<D> buf[DEPTH];
#pragma unroll
    for (int r = 0; r < DEPTH; ++r) load(r, buf[r]);
    for (int i = 0; i < my_tiles; i += DEPTH) {
#pragma unroll
      for (int r = 0; r < DEPTH; ++r) {
        if (i + r < my_tiles) {
          compute(i + r, buf[r]);
          load(i + r + DEPTH, buf[r]);
        }
      }
    }
  }

  // Reduce within the wavefront: lsum over the 16 key lanes (every lane group
  // holds the same values), acc over the 4 lane groups (disjoint keys).
#pragma unroll
  for (int q = 0; q < QPW; ++q) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) lsum[q] += __shfl_xor(lsum[q], off, 64);
#pragma unroll
    for (int e = 0; e < FPV; ++e) {
      acc[q][e] += __shfl_xor(acc[q][e], 16, 64);
      acc[q][e] += __shfl_xor(acc[q][e], 32, 64);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
      m_s[wave][q] = m[q];
      l_s[wave][q] = lsum[q];
    }
  }
  if (g == 0) {
#pragma unroll
    for (int q = 0; q < QPW; ++q)
#pragma unroll
      for (int e = 0; e < FPV; ++e) o_s[wave][q][l16 * FPV + e] = acc[q][e];
  }
  __syncthreads();

  // Merge the four wavefronts and write this split's partial.
  for (int x = tid; x < nq * D; x += NT) {
    const int q = x / D, d = x % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, m_s[w][q]);
    // Weight 0 for a wavefront whose stabiliser is still -inf; only an exactly
    // zero sum is an empty split, so a NaN score reaches the partial.
    float tot = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = (m_s[w][q] == neg_inf()) ? 0.f : exp2_fast((m_s[w][q] - M) * prm.scale_log2);
      tot = fmaf(f, l_s[w][q], tot);
      o = fmaf(f, o_s[w][q][d], o);
    }
    const bool empty = tot == 0.f;
    const int64_t prow = row(q);
    prm.part_o[prow * D + d] = empty ? 0.f : o / tot;
    if (d == 0) prm.part_lse[prow] = empty ? neg_inf() : fmaf(M, prm.scale, logf(tot));
  }
  // The next piece of the workgroup reuses the LDS buffers.
  __syncthreads();
}

// Fixed splits: workgroup (b, hk, slice, split sp) takes keys
// [sp * split_len, (sp + 1) * split_len) of sequence b.
template <int D>
__global__ __launch_bounds__(NT, 2) void decode_split_kernel(DecodeParams prm, int n_qblk) {
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
  const int n_keys = (int)max<int64_t>(0, min<int64_t>(k_begin + prm.split_len, Lb) - k_begin);
  split_piece<D>(prm, b, hk, h0, nq, k_begin, n_keys,
                 [&](int q) { return ((int64_t)b * prm.Hq + h0 + q) * prm.n_splits + sp; });
}

// Equal-key work units (stream-K) for sequences of different lengths.  The
// keys of all sequences, in sequence order, form one range of T keys per
// key/value head; work unit u takes keys [u c, (u + 1) c) of it, so every unit
// reads the same number of keys whatever the lengths and no short or empty
// units trail the grid.  The number of units, Ue <= U = B * n_splits (the
// grid), is made from T: about kUnitKeys keys per unit, rounded up to a whole
// number of rounds of the workgroups the device holds at once (sk_granule units
// per (key/value head, head slice)); c = ceil(T / Ue), and units past the last
// exit at once.  A unit whose range crosses the end of a sequence writes one partial
// ("piece") per sequence it touches.  Pieces are numbered in key order: a new
// piece starts at every unit start and at every sequence start that falls
// strictly inside a unit, so the piece holding key x is
//   piece(x) = floor(x / c) + cnt[b(x)],
// with b(x) the sequence of x and cnt[b] the number of sequence starts
// pref[b'] (1 <= b' <= b, pref[b'] > pref[b' - 1]) that are not multiples of
// c.  A sequence's pieces are then consecutive, and the tree kernel merges them
// in key order.  There are fewer than U + B pieces, stored at row
// h * n_pieces + piece for query head h.
constexpr int kMaxStreamB = 1024;  // sequences a stream-K call may have
// Keys per work unit aimed at.  On the uneven 16 x 8K.k-token benchmark cache
// (A/B in alternating processes on one MI355X): 1536 keys 0.799 ms, 2048
// 0.790, 3072 0.767, 4096 0.754, 6144 0.760; fixed 2048-key splits 0.857 ms.
constexpr int64_t kUnitKeys = 4096;

struct StreamK {
  int64_t c;  // keys per work unit
  int64_t T;  // total keys
};

__device__ __forceinline__ int64_t streamk_unit_keys(const DecodeParams& prm, int64_t T) {
  const int64_t U = (int64_t)prm.B * prm.n_splits, g = prm.sk_granule;
  int64_t ue = ((T + kUnitKeys - 1) / kUnitKeys + g - 1) / g * g;
  ue = min<int64_t>(max<int64_t>(ue, 1), U);
  return max<int64_t>(1, (T + ue - 1) / ue);
}

// Prefix sums of the clamped lengths (pref[0 .. B]) and the boundary counts
// cnt[0 .. B - 1] in LDS.  Every thread of the workgroup calls it; it ends
// with a barrier after which both arrays are complete.
// With first_unit >= 0 (a split workgroup's unit), a unit past the last
// returns before the boundary counts are made (its caller exits).
__device__ __forceinline__ StreamK streamk_tables(const DecodeParams& prm, int64_t* pref, int* cnt,
                                                  int64_t first_unit = -1) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = prm.B;
  if (tid < 64) {
    int64_t carry = 0;
    for (int base = 0; base < B; base += 64) {
      const int i = base + lane;
      int64_t x = i < B ? min<int64_t>(max<int64_t>(prm.seqlens[i], 0), prm.L) : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (i < B) pref[i + 1] = carry + x;
      carry += __shfl(x, 63, 64);
    }
    if (lane == 0) pref[0] = 0;
  }
  __syncthreads();
  StreamK sk;
  sk.T = pref[B];
  sk.c = streamk_unit_keys(prm, sk.T);
  if (first_unit >= 0 && first_unit * sk.c >= sk.T) return sk;  // a unit past the last: nothing to do
  if (tid < 64) {
    int carry = 0;
    for (int base = 0; base < B; base += 64) {
      const int i = base + lane;
      int f = 0;
      if (i >= 1 && i < B) f = (pref[i] > pref[i - 1] && pref[i] % sk.c != 0) ? 1 : 0;
      int x = f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (i < B) cnt[i] = carry + x;
      carry += __shfl(x, 63, 64);
    }
  }
  __syncthreads();
  return sk;
}

// The sequence holding key x of the concatenated range (pref[b] <= x < pref[b + 1]).
__device__ __forceinline__ int seq_of(const int64_t* pref, int B, int64_t x) {
  int lo = 0, hi = B - 1;  // the last b with pref[b] <= x
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int D>
__global__ __launch_bounds__(NT, 2) void decode_streamk_kernel(DecodeParams prm, int n_qblk) {
  __shared__ int64_t pref[kMaxStreamB + 1];
  __shared__ int cnt[kMaxStreamB];
  const int64_t U = (int64_t)prm.B * prm.n_splits;
  int lin = blockIdx.x;
  const int64_t u = lin % U;
  lin /= (int)U;
  const int qblk = lin % n_qblk;
  const int hk = lin / n_qblk;
  const int h0 = hk * prm.group + qblk * QPW;
  const int nq = min(QPW, prm.group - qblk * QPW);
  const StreamK sk = streamk_tables(prm, pref, cnt, u);
  const int64_t s = u * sk.c, e = min(s + sk.c, sk.T);
  if (s >= e) return;
  int b = seq_of(pref, prm.B, s);
  for (int64_t x = s; x < e;) {
    while (pref[b + 1] <= x) ++b;  // skip sequences that end at x (empty ones included)
    const int64_t seg_end = min(e, pref[b + 1]);
    const int64_t piece = x / sk.c + cnt[b];
    split_piece<D>(prm, b, hk, h0, nq, x - pref[b], (int)(seg_end - x),
                   [&](int q) { return (int64_t)(h0 + q) * prm.n_pieces + piece; });
    x = seg_end;
  }
}

// Tree kernel: one workgroup per (batch, query head).  The adjacent-pair tree
// is built over the split LSEs level by level in LDS: at each level node k of
// the next level merges nodes 2k and 2k+1 (an odd last node is carried up
// unchanged), and each node keeps the weight e^{L_node - L_parent} it gets in
// its parent.  A split's weight in the root is the product of the weights on
// its path, so the root's O is the sum of the split partials with those
// weights: the same tree, with the O additions done in one pass whose loads
// are all independent (a chain of pairwise merges in registers would wait on
// each load in turn).  Rows whose splits are all empty get O = 0, LSE = -inf.
constexpr int TREE_NT = 512;
constexpr int kMaxNodes = 2 * 1024 + 16;  // nodes of all levels for up to 1025 partials

template <int D>
__global__ __launch_bounds__(TREE_NT) void decode_tree_kernel(DecodeParams prm) {
  constexpr int NC = TREE_NT / D;  // groups of D threads, one thread per feature
  __shared__ float lv[kMaxNodes];  // node LSEs, level 0 (the splits) first
  __shared__ float wv[kMaxNodes];  // weight of each node in its parent
  __shared__ float wl[kMaxNodes / 2];  // weight of each split in the root
  __shared__ float red[NC][D];
  const int tid = threadIdx.x, d = tid % D, c = tid / D;
  const int h = blockIdx.x % prm.Hq, b = blockIdx.x / prm.Hq;
  int n = prm.n_splits;
  int64_t base = ((int64_t)b * prm.Hq + h) * n;
  if (prm.streamk) {
    // Sequence b's pieces: ids piece(pref[b]) .. piece(pref[b + 1] - 1), all
    // in one run (none for an empty sequence).
    __shared__ int64_t pref[kMaxStreamB + 1];
    __shared__ int cnt[kMaxStreamB];
    const StreamK sk = streamk_tables(prm, pref, cnt);
    const int64_t lo = pref[b], hi = pref[b + 1];
    n = hi > lo ? (int)((hi - 1) / sk.c - lo / sk.c + 1) : 0;
    base = (int64_t)h * prm.n_pieces + (hi > lo ? lo / sk.c + cnt[b] : 0);
  }
  for (int i = tid; i < n; i += TREE_NT) lv[i] = prm.part_lse[base + i];
  if (n == 0 && tid == 0) lv[0] = neg_inf();  // a sequence with no keys: O = 0, LSE = -inf
  __syncthreads();
  int off = 0, m = n;  // this level's nodes are lv[off .. off + m)
  while (m > 1) {
    const int mp = (m + 1) / 2;
    for (int k = tid; k < mp; k += TREE_NT) {
      if (2 * k + 1 < m) {
        float wa, wb, L;
        merge_weights(lv[off + 2 * k], lv[off + 2 * k + 1], wa, wb, L);
        wv[off + 2 * k] = wa;
        wv[off + 2 * k + 1] = wb;
        lv[off + m + k] = L;
      } else {
        wv[off + 2 * k] = 1.f;
        lv[off + m + k] = lv[off + 2 * k];
      }
    }
    __syncthreads();
    off += m;
    m = mp;
  }
  const float L_root = lv[off];
  for (int i = tid; i < n; i += TREE_NT) {
    float w = 1.f;
    for (int j = i, o = 0, mm = n; mm > 1; o += mm, j >>= 1, mm = (mm + 1) / 2) w *= wv[o + j];
    wl[i] = w;
  }
  __syncthreads();
  // Sixteen loads in flight per thread; an empty split's partial is 0 with
  // weight 0, so no branch is needed.
  constexpr int U = 16;
  const float* po = prm.part_o + base * D + d;
  float acc = 0.f;
  int i = c;
  for (; i + (U - 1) * NC < n; i += U * NC) {
    float v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = po[(int64_t)(i + k * NC) * D];
#pragma unroll
    for (int k = 0; k < U; ++k) acc = fmaf(wl[i + k * NC], v[k], acc);
  }
  for (; i < n; i += NC) acc = fmaf(wl[i], po[(int64_t)i * D], acc);
  red[c][d] = acc;
  __syncthreads();
  if (c != 0) return;
#pragma unroll
  for (int k = 1; k < NC; ++k) acc += red[k][d];
  prm.o[(int64_t)b * prm.o_sb + (int64_t)h * prm.o_sh + d] = f32_to_bf16(L_root == neg_inf() ? 0.f : acc);
  if (d == 0) prm.lse[(int64_t)b * prm.Hq + h] = L_root;
}

}  // namespace

// Scratch of the allocation-free decode entry point: the split partials live
// here instead of in a caller's workspace.  One copy per device, held until the
// process ends.  Host code must not pass the array's name to a kernel (on the
// host it is a stand-in, not a device address): its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cus[kMaxDevices];
hipError_t g_cu_err[kMaxDevices];

// Compute units of the current device (queried once per device).
hipError_t device_cus(int* cus) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_cu_once[dev], [dev] {
    g_cu_err[dev] = hipDeviceGetAttribute(&g_cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
  });
  *cus = g_cus[dev];
  return g_cu_err[dev];
}

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int64_t items_decode(const DecodeParams& p) {
  const int64_t n_qblk = (p.group + QPW - 1) / QPW;
  return std::max((int64_t)p.B * p.Hkv * n_qblk * p.n_splits * NT, (int64_t)p.B * p.Hq * TREE_NT);
}

hipError_t launch_decode(const DecodeParams& p0, int D, hipStream_t s) {
  DecodeParams p = p0;
  const int n_qblk = (p.group + QPW - 1) / QPW;
  if (p.streamk) {
    // Stream-K units per (key/value head, head slice) in one round of the
    // workgroups resident at once (two per CU).
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    p.sk_granule = max(1, 2 * cus / max(1, p.Hkv * n_qblk));
  }
  const int64_t grid = (int64_t)p.B * p.Hkv * n_qblk * p.n_splits;  // the same count in both modes
  if (grid == 0) return hipSuccess;
  if (p.streamk) {
    if (D == 128)
      hipLaunchKernelGGL(decode_streamk_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p, n_qblk);
    else
      hipLaunchKernelGGL(decode_streamk_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p, n_qblk);
  } else {
    if (D == 128)
      hipLaunchKernelGGL(decode_split_kernel<128>, dim3((unsigned)grid), dim3(NT), 0, s, p, n_qblk);
    else
      hipLaunchKernelGGL(decode_split_kernel<64>, dim3((unsigned)grid), dim3(NT), 0, s, p, n_qblk);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 tg((unsigned)((int64_t)p.B * p.Hq));
  if (D == 128)
    hipLaunchKernelGGL(decode_tree_kernel<128>, tg, dim3(TREE_NT), 0, s, p);
  else
    hipLaunchKernelGGL(decode_tree_kernel<64>, tg, dim3(TREE_NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
