// Backward of exact attention for bf16 inputs on gfx950, from the saved final
// output O and row LSE: no re-run of the forward (DistFlashAttn digest,
// rematerialisation-aware gradient checkpointing).  bf16 MFMA with fp32
// accumulation everywhere.
//
// Two kernels, each owning its outputs, so no floating-point atomics are used
// and results do not depend on scheduling:
//
//   dK/dV kernel (key-outer).  A workgroup owns 128 keys of one key/value head
//   and walks the query tiles of every query head that reads that key/value
//   head.  Scores are formed as S = Q K^T, which puts one key per lane with the
//   tile's queries in the lane's registers; P and dS then feed dV^T += dO^T P
//   and dK^T += Q^T dS straight from registers.  Each group of 32 keys is
//   served by a pair of wavefronts, one producing P and dV, the other dS and dK
//   (see below).  Query and dO tiles stream from HBM into LDS (global_load_lds,
//   a 3-stage ring); the transposed operands Q^T, dO^T are read from the same
//   row-major tiles with ds_read_b64_tr_b16.
//
//   dQ kernel (query-outer).  A workgroup owns 128 queries (32 per wavefront
//   pair, Q and dO in registers) and walks the key tiles; the two wavefronts
//   of a pair split each tile's keys.  Scores are formed transposed,
//   S^T = K Q^T, one query per lane, so the row statistics (LSE, delta) are
//   per-lane scalars and dS^T feeds dQ^T += K^T dS^T straight from registers;
//   K^T is read from the row-major key tile with the transposing LDS read.  dQ
//   is added into an fp32 accumulator that persists across key chunks and is
//   cast once at the end.
//
// The dQ pass recomputes S and dP (7 contractions in all instead of 5); that
// is the price of determinism without atomics.
//
// Around each block of matrix products a wavefront raises its issue priority
// (s_setprio), so that while one wavefront of a SIMD has products ready the
// matrix core is fed first and its partner's vector work fills the gaps.
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"
#include "tile_lds.h"

namespace attn {
namespace {

#ifndef KV_AHEAD
#define KV_AHEAD 4
#endif
#ifndef KV_AHEAD_T
#define KV_AHEAD_T 2
#endif
#ifndef DQ_AHEAD
#define DQ_AHEAD 4
#endif
#ifndef DQ_AHEAD_T
#define DQ_AHEAD_T 3
#endif
constexpr int NT = 256;
constexpr int KBN = 128;  // keys per dK/dV workgroup
constexpr int KBM = 64;   // queries per tile in the dK/dV kernel
constexpr int QBM = 128;  // queries per dQ workgroup
constexpr int QBN = 64;   // keys per tile in the dQ kernel

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of this wavefront are in
// flight (LDS and export counters left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for data exchanged through LDS by ordinary LDS stores.  A
// fenced barrier (__syncthreads, or any release fence, since global_load_lds
// writes LDS) makes every wavefront wait for all of its loads in flight, which
// would drain the prefetches of later tiles at every barrier.  Here each
// wavefront waits only for its own LDS stores; global_load_lds tiles are
// waited for explicitly (wait_vm) before the barrier that publishes them.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 slab8(const f32x16& a, int o) {
  return cvt_bf16x8(a[o], a[o + 1], a[o + 2], a[o + 3], a[o + 4], a[o + 5], a[o + 6], a[o + 7]);
}

// ---------------------------------------------------------------- dK / dV --
//
// Eight wavefronts in four pairs; pair w%4 owns keys j0 + 32*(w%4) .. +31.
// Query tiles of 64 rows (Q, dO and their statistics) stream through a
// 3-stage LDS ring, one tile per step.  At step t:
//   * the "P" wavefront (w < 4) holds K in registers and accumulates dV: it
//     forms S = Q K^T for tile t (one key per lane), P = exp(S - LSE) with the
//     mask, hands P to its partner through LDS and runs dV^T += dO^T P;
//   * the "dS" wavefront (w >= 4) holds V and accumulates dK: it forms
//     dP - delta = dO V^T - delta for tile t (its accumulator starts at the
//     stored -delta), and for tile t - 1 (one step behind, so that P is
//     already published) reads P, forms dS = P (dP - delta) and runs
//     dK^T += Q^T dS.
// Both carry 32 contractions per tile; the exponentials of one overlap the
// contractions of the other on their shared SIMD.  One LDS-only barrier per
// step publishes P and the next tile.

constexpr int DKV_NT = 512;

template <int D, bool PW>
__device__ __forceinline__ void dkdv_tile(const BwdParams& p, u16* q_s, u16* d_s, float (*st_s)[256],
                                          u32x4 (*pex)[2][4][64], RowFrag<D>& rf, TrFrag<D>& tf,
                                          int wave, int lane, int kt, int b, int hk) {
  constexpr int NS = D / 16, NDB = D / 32, SZ = SwTile<D>::SIZE;
  // Per-lane values of a tile are derived here from an opaque copy of the
  // lane index, so they are not computed once for both tiles of a unit and
  // kept live across the first.
  asm volatile("" : "+v"(lane));
  const int lg = lane >> 5, pair = wave & 3;
  const int j0 = kt * KBN;
  const int kj = j0 + pair * 32 + (lane & 31);  // this lane's key
  const bool kok = kj < p.Sk;

  // Register operand: K rows for the P wavefront, V rows for the dS wavefront.
  bf16x8 kv[NS];
  {
    const View& src = PW ? p.k : p.v;
    const u16* base = (const u16*)src.ptr + (int64_t)b * src.sb + (int64_t)hk * src.sh + (int64_t)kj * src.ss;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kv[s] = kok ? as_bf16x8(*(const u32x4*)(base + lg * 8 + s * 16)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  // Complete these loads here: left to the compiler, the wait for them sits at
  // their first use inside the loop, where it would also drain every tile
  // prefetch in flight on each pass.
  wait_vm<0>();
  f32x16 acc[NDB];  // dV^T (P wavefront) or dK^T (dS wavefront)
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // Query i sees key j iff j <= delta + i (causal).  Queries before i_start see
  // no key of this tile; from i_full on every query sees every key of it.
  // Query rows past the end carry LSE = +inf in the statistics, so their P is 0.
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
  // Query tiles before t_mask hold queries that some key of this tile hides
  // from (i < i_full); only those steps apply the causal mask.
  const int t_mask = p.causal ? min(n_qt, (i_full + KBM - 1) / KBM) : 0;

  for (int hh = 0; hh < p.group; ++hh) {
    const int h = hk * p.group + hh;
    const u16* qb = (const u16*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh;
    const u16* dob = (const u16*)p.dout.ptr + (int64_t)b * p.dout.sb + (int64_t)h * p.dout.sh;
    const float* stb = p.stats + ((int64_t)b * p.Hq + h) * 2 * p.Sq_pad;
    // Step t works on ring slot (t - t_start) % 3 and exchange buffer
    // (t - t_start) % 2.  Fetch query tile tq into ring slot `slot`: Q and dO
    // rows, and (wave 0) the 64 statistics of each kind in one 1 KB run.  The
    // loads are untracked by the compiler and waited for before the barrier
    // that publishes the slot.
    auto issue = [&](int tq, int slot) {
      if (wave == 0) {
        const int part = (lane >> 4) & 1;  // lanes 0-15 LSE, 16-31 delta; 32-63 repeat them
        dma16_untracked(stb + part * p.Sq_pad + tq * KBM + 4 * (lane & 15), (lds_void*)st_s[slot]);
      }
      issue_swtile<D, 8, true>(q_s + slot * SZ, qb, p.q.ss, tq * KBM, p.Sq, wave, lane);
      issue_swtile<D, 8, true>(d_s + slot * SZ, dob, p.dout.ss, tq * KBM, p.Sq, wave, lane);
    };
    if (t_start >= n_qt) continue;
    issue(t_start, 0);
    wait_vm<0>();
    lds_barrier();
    f32x16 dpa[2] = {f32x16{}, f32x16{}}, dpb[2] = {f32x16{}, f32x16{}};
    // slot_c: the ring slot, an int or a compile-time constant (which folds
    // into the LDS reads' immediate offsets); par_c: the exchange buffer and
    // the dP registers' roles, always a compile-time constant.
    auto step = [&](int t, auto slot_c, auto par_c, auto masked_c) {
      const int slot = slot_c;
      constexpr int par = decltype(par_c)::value;
      rf.refresh();
      tf.refresh();
      f32x16* const dp_in = par ? dpb : dpa;   // dP - delta of tile t - 1
      f32x16* const dp_out = par ? dpa : dpb;  // dP - delta of tile t
      // Tile t + 1 takes the slot of tile t - 2, last read (by the dS
      // wavefront) before the previous barrier.
      if (t + 1 < n_qt) issue(t + 1, slot == 2 ? 0 : slot + 1);
      f32x16 sc[2] = {f32x16{}, f32x16{}};
      if (t < n_qt) {
        // S = Q K^T (P wavefront) or dP - delta = dO V^T - delta (dS
        // wavefront, accumulating onto the stored -delta): lane = key,
        // registers = two 32-query blocks.
        const int tile_o = slot * SZ * 2;  // byte offset of the slot in either ring
        if constexpr (!PW) {
          const float* nd = st_s[slot] + KBM;
#pragma unroll
          for (int qb2 = 0; qb2 < 2; ++qb2) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x4 n4 = *(const f32x4*)(nd + qb2 * 32 + g4 * 8 + lg * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) sc[qb2][g4 * 4 + e] = n4[e];
            }
          }
        }
        __builtin_amdgcn_s_setprio(1);
        {
          // Operand j = 2 si + qb2, read AH ahead of the MFMA that uses it;
          // the hard scheduling boundaries hold each read in its slot.
          constexpr int NJ = 2 * NS, AH = KV_AHEAD;
          bf16x8 f[NJ];
#pragma unroll
          for (int j = 0; j < AH; ++j) f[j] = rf.get_at(tile_o, j & 1, j >> 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            if (j + AH < NJ) f[j + AH] = rf.get_at(tile_o, (j + AH) & 1, (j + AH) >> 1);
            sc[j & 1] = mfma32(f[j], kv[j >> 1], sc[j & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        if constexpr (!PW) {
          dp_out[0] = sc[0];
          dp_out[1] = sc[1];
        }
        if constexpr (PW) {
          const float* st = st_s[slot];
#pragma unroll
          for (int qb2 = 0; qb2 < 2; ++qb2) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x4 l4 = *(const f32x4*)(st + qb2 * 32 + g4 * 8 + lg * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) sc[qb2][g4 * 4 + e] = exp2_fast(fmaf(sc[qb2][g4 * 4 + e], sl2, -l4[e]));
            }
          }
          if constexpr (decltype(masked_c)::value) {
            const int i0 = t * KBM;
            // Causal mask: query i0 + q is hidden from this lane's key when
            // q < key_lim - i0.  The sign of q - (key_lim - i0) selects it as a
            // bit mask, which keeps the 32 decisions in vector registers.
            const int64_t rel64 = key_lim - i0;
            const int rel = rel64 < -1 ? -1 : (rel64 > KBM ? KBM : (int)rel64);
#pragma unroll
            for (int qb2 = 0; qb2 < 2; ++qb2) {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int qo = qb2 * 32 + (i >> 2) * 8 + lg * 4 + (i & 3);
                const unsigned keep = ~(unsigned)((qo - rel) >> 31);
                sc[qb2][i] = __uint_as_float(__float_as_uint(sc[qb2][i]) & keep);
              }
            }
          }
          // P in bf16, one B operand per 16-query slab: published for the
          // partner and used right away for dV^T += dO^T P.
          bf16x8 pb[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            pb[ks] = slab8(sc[ks >> 1], (ks & 1) * 8);
            pex[pair][par][ks][lane] = __builtin_bit_cast(u32x4, pb[ks]);
          }
          __builtin_amdgcn_s_setprio(1);
          {
            constexpr int NJ = 4 * NDB, AH = KV_AHEAD_T;
            bf16x8 f[NJ];
#pragma unroll
            for (int j = 0; j < AH; ++j) f[j] = tf.get_at(tile_o, j / NDB, j % NDB);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              if (j + AH < NJ) f[j + AH] = tf.get_at(tile_o, (j + AH) / NDB, (j + AH) % NDB);
              acc[j % NDB] = mfma32(f[j], pb[j / NDB], acc[j % NDB]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          __builtin_amdgcn_s_setprio(0);
        }
      }
      if constexpr (!PW) {
        if (t > t_start) {
          // dS for tile t - 1 from the published P and last step's dP - delta,
          // then dK^T += Q^T dS.
          const int sp = slot == 0 ? 2 : slot - 1;
          const int prev_o = sp * SZ * 2;
          bf16x8 sbs[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pex[pair][par ^ 1][ks][lane]);
            const int qb2 = ks >> 1, o = (ks & 1) * 8;
            float ds[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ds[e] = (float)pb[e] * dp_in[qb2][o + e];
            sbs[ks] = cvt_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
          }
          __builtin_amdgcn_s_setprio(1);
          {
            constexpr int NJ = 4 * NDB, AH = KV_AHEAD_T;
            bf16x8 f[NJ];
#pragma unroll
            for (int j = 0; j < AH; ++j) f[j] = tf.get_at(prev_o, j / NDB, j % NDB);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              if (j + AH < NJ) f[j + AH] = tf.get_at(prev_o, (j + AH) / NDB, (j + AH) % NDB);
              acc[j % NDB] = mfma32(f[j], sbs[j / NDB], acc[j % NDB]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          __builtin_amdgcn_s_setprio(0);
        }
      }
      wait_vm<0>();  // tile t + 1, the only load in flight, is needed next step
      lds_barrier();
    };
    // The masked steps come first, in pairs (runtime ring slot), and run on
    // until the step count is a multiple of six (masking a tile that needs
    // none keeps every entry).  The unmasked steps then run six at a time,
    // so every ring slot and exchange buffer is a compile-time constant.
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    int t = t_start;
    for (; t <= n_qt && (t < t_mask || (t - t_start) % 6 != 0); t += 2) {
      const int s0 = (t - t_start) % 3;
      step(t, s0, P0{}, std::true_type{});
      if (t + 1 <= n_qt) step(t + 1, s0 == 2 ? 0 : s0 + 1, P1{}, std::true_type{});
    }
    for (; t <= n_qt; t += 6) {
      step(t, S0{}, P0{}, std::false_type{});
      if (t + 1 > n_qt) break;
      step(t + 1, S1{}, P1{}, std::false_type{});
      if (t + 2 > n_qt) break;
      step(t + 2, S2{}, P0{}, std::false_type{});
      if (t + 3 > n_qt) break;
      step(t + 3, S0{}, P1{}, std::false_type{});
      if (t + 4 > n_qt) break;
      step(t + 4, S1{}, P0{}, std::false_type{});
      if (t + 5 > n_qt) break;
      step(t + 5, S2{}, P1{}, std::false_type{});
    }
  }

  if (!kok) return;
  const float f = PW ? 1.0f : p.scale;
  const MView& dst = PW ? p.dv : p.dk;
  u16* out = (u16*)dst.ptr + (int64_t)b * dst.sb + (int64_t)kj * dst.ss + (int64_t)hk * dst.sh;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = db * 32 + j * 8 + lg * 4;
      const f32x16& A = acc[db];
      *(u32x2*)(out + d) = u32x2{pack_bf16x2(A[4 * j] * f, A[4 * j + 1] * f), pack_bf16x2(A[4 * j + 2] * f, A[4 * j + 3] * f)};
    }
  }
}

// A work unit is one key tile, or with the balanced order the pair of key
// tiles (u, n - 1 - u), whose causal work adds up to about the same for every u.
// Early keys are seen by the most queries, so they come first.
template <int D, bool PW>
__device__ __forceinline__ void dkdv_unit(const BwdParams& p, u16* q_s, u16* d_s, float (*st_s)[256],
                                          u32x4 (*pex)[2][4][64], int wave, int unit, int b, int hk) {
  // The two roles run in one kernel behind a wave-uniform branch, and the
  // compiler places the second role's code after the first's.  The lane index
  // comes from an opaque copy of the thread index made inside each role, so
  // no per-lane value of the second role is computed ahead of the branch,
  // where it would stay live through the first role.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  RowFrag<D> rf;
  TrFrag<D> tf;
  rf.init(lane);
  tf.init(lane);
  // The P wavefront reads Q rows and dO transposed, the dS wavefront dO rows
  // and Q transposed.
  rf.rebase(PW ? q_s : d_s);
  tf.rebase(PW ? d_s : q_s);
  const int last = p.n_ktiles - 1 - unit;
  const int n = (p.balanced && last != unit) ? 2 : 1;
  for (int k = 0; k < n; ++k) dkdv_tile<D, PW>(p, q_s, d_s, st_s, pex, rf, tf, wave, lane, k == 0 ? unit : last, b, hk);
}

template <int D>
__global__ __launch_bounds__(DKV_NT) void dkdv_bf16_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) u16 q_s[3 * SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 d_s[3 * SwTile<D>::SIZE];
  // [slot] [0, 64): LSE in log2 units, [64, 128): -delta, [128, 256): unused
  __shared__ __attribute__((aligned(16))) float st_s[3][256];
  __shared__ __attribute__((aligned(16))) u32x4 pex_s[4][2][4][64];  // [pair][step parity][slab][lane]
  // The wavefront index is uniform across the wavefront; say so, so that the
  // role branch below is a scalar branch.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_units_k;
  const int bh = lin / p.n_units_k;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  if (wave < 4) dkdv_unit<D, true>(p, q_s, d_s, st_s, pex_s, wave, unit, b, hk);
  else dkdv_unit<D, false>(p, q_s, d_s, st_s, pex_s, wave, unit, b, hk);
}

// The same over the chunks of a table: work unit u of the whole grid belongs
// to the chunk c with unit0[c] <= u < unit0[c + 1], and runs with that chunk's
// key/value tensors, dK/dV outputs, length and position.
template <int D>
__global__ __launch_bounds__(DKV_NT) void dkdv_chunks_kernel(BwdParams p, BwdChunkTable ct) {
  __shared__ __attribute__((aligned(16))) u16 q_s[3 * SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 d_s[3 * SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) float st_s[3][256];
  __shared__ __attribute__((aligned(16))) u32x4 pex_s[4][2][4][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int gunit = lin % ct.n_units;
  const int bh = lin / ct.n_units;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  int c = 0;
  while (c + 1 < ct.kv.n && ct.unit0[c + 1] <= gunit) ++c;
  BwdParams pc = p;
  pc.k.ptr = ct.kv.k[c];
  pc.k.sb = ct.kv.kb[c];
  pc.v.ptr = ct.kv.v[c];
  pc.v.sb = ct.kv.vb[c];
  pc.dk.ptr = ct.dk[c];
  pc.dk.sb = ct.dkb[c];
  pc.dv.ptr = ct.dv[c];
  pc.dv.sb = ct.dvb[c];
  pc.Sk = ct.kv.len[c];
  pc.delta_pos = ct.kv.q_pos0 - ct.kv.pos0[c];
  pc.n_ktiles = (pc.Sk + KBN - 1) / KBN;
  const int unit = gunit - ct.unit0[c];
  if (wave < 4) dkdv_unit<D, true>(pc, q_s, d_s, st_s, pex_s, wave, unit, b, hk);
  else dkdv_unit<D, false>(pc, q_s, d_s, st_s, pex_s, wave, unit, b, hk);
}

// --------------------------------------------------------------------- dQ --
//
// Eight wavefronts in four pairs; pair w%4 owns queries q0 + 32*(w%4) .. +31
// and holds their Q and dO rows in registers.  Key/value tiles of 64 rows
// stream through a 3-stage LDS ring; wavefront w takes keys 32*(w/4) .. +31 of
// every tile and runs the whole chain for them on its own: S^T = K Q^T and
// dP^T = V dO^T (one query per lane), P = exp(S - LSE) with the mask,
// dS = P (dP - delta), dQ^T += K^T dS^T.  The two wavefronts of a pair share
// no data until the end, where their dQ^T partials are added through LDS.

constexpr int DQ_NT = 512;
constexpr int DQ_STAGES = 3;

// The keys of a dQ pass come in segments (one tensor, or the chunks of a
// table); seg(c, b, hk) gives segment c's key and value rows for (b, hk), its
// length and the offset of the query positions from its key positions.
struct KeySeg {
  const u16* kb;
  const u16* vb;
  int Sk;
  int64_t delta_pos;
};

// Lane index within the wavefront, from the count of lanes below this one
// (two vector instructions).  Volatile, so the compiler recomputes it where it
// is written instead of hoisting it and keeping a register live meanwhile.
__device__ __forceinline__ int lane_id() {
  int r;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
  return r;
}

// x clamped to [0, n], for wave-uniform x.  Written as compares and selects:
// as a 64-bit min/max the compiler forms it with double-precision vector
// operations, whose operands then sit in vector registers.
__device__ __forceinline__ int clamp_len(int64_t x, int n) { return x <= 0 ? 0 : (x >= n ? n : (int)x); }

template <int D, class Seg>
__device__ __forceinline__ void dq_body(const BwdParams& p, int b, int h, int unit, int n_seg, Seg seg) {
  constexpr int NS = D / 16, NDB = D / 32, SZ = SwTile<D>::SIZE;
  constexpr int NLD = 2 * (SwTile<D>::RUNS / 8);  // loads per tile per wavefront
  // Key ring, then value ring; after the loop the start holds the partial dQ^T
  // exchange (4 pairs x NDB x 16 x 64 floats, at most 64 KB <= the rings' size).
  __shared__ __attribute__((aligned(16))) u16 tiles[2 * DQ_STAGES * SZ];
  static_assert(4 * NDB * 16 * 64 * 4 <= 2 * DQ_STAGES * SZ * 2, "exchange must fit in the rings");
  u16* const k_s = tiles;
  u16* const v_s = tiles + DQ_STAGES * SZ;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int lr = lane & 31, lg = lane >> 5, pair = wave & 3, kh = wave >> 2;
  const int hk = h / p.group;
  // Causal: late query tiles see the most keys; start with them.
  const int qt = p.causal ? p.n_qtiles - 1 - unit : unit;
  const int q0 = qt * QBM;
  const int qi = q0 + pair * 32 + lr;
  const bool qok = qi < p.Sq;
  const int q_last = min(q0 + QBM, p.Sq) - 1;

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
  // Statistics rows exist up to Sq_pad >= Sq; rows past Sq hold LSE = +inf, delta = 0.
  // The workspace holds -delta.
  const float* stb = p.stats + ((int64_t)b * p.Hq + h) * 2 * p.Sq_pad;
  const float lse2 = qi < p.Sq_pad ? stb[qi] : pos_inf();
  const float ndlt = qi < p.Sq_pad ? stb[p.Sq_pad + qi] : 0.f;
  const float sl2 = p.scale_log2;
  RowFrag<D> rf;
  TrFrag<D> tf;
  rf.init(lane);
  tf.init(lane);
  // Complete these loads here: left to the compiler, the wait for them sits at
  // their first use inside the loop and drains the tile prefetches there.
  wait_vm<0>();

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  TileSrc<D, 8> ksrc, vsrc;
  ksrc.init(p.k.ss, wave, lane);
  vsrc.init(p.v.ss, wave, lane);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  static_assert(DQ_STAGES == 3, "the loop below is unrolled over three ring slots");

  // dQ accumulates in registers over every segment.  A segment's last step
  // waits for all its loads and ends with a barrier, so the next segment may
  // refill the ring from slot 0.
  for (int c = 0; c < n_seg; ++c) {
    const KeySeg sg = seg(c, b, hk);
    int kv_end = sg.Sk, full_end = sg.Sk;
    int64_t lim64 = (int64_t)sg.Sk - 1;  // last key of the segment this lane's query sees
    if (p.causal) {
      kv_end = clamp_len(sg.delta_pos + q_last + 1, sg.Sk);
      full_end = clamp_len(sg.delta_pos + q0 + 1, sg.Sk);
      // The query index is recomputed here from the lane index rather than
      // kept live across all segments.
      const int qi_s = q0 + pair * 32 + (lane_id() & 31);
      lim64 = min<int64_t>(sg.delta_pos + qi_s, lim64);
    }
    const int n = (kv_end + QBN - 1) / QBN;
    auto issue = [&](int tile, int slot) {
      ksrc.issue(k_s + slot * SZ, sg.kb, p.k.ss, tile * QBN, sg.Sk, wave, lane);
      vsrc.issue(v_s + slot * SZ, sg.vb, p.v.ss, tile * QBN, sg.Sk, wave, lane);
    };
    if (n > 0) {
      issue(0, 0);
      if (n > 1) {
        issue(1, 1);
        wait_vm<NLD>();
      } else {
        wait_vm<0>();
      }
      lds_barrier();
    }
    // One step per key tile.  The ring slot is a compile-time constant so that
    // it folds into the LDS reads' immediate offsets; only tiles that reach past
    // full_end (the last key every query of the tile sees) apply the mask.
    auto step = [&](int t, auto slot_c, auto masked_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      // Tile t + 2 takes the slot of tile t - 1, which every wavefront finished
      // before the previous barrier.
      if (t + 2 < n) issue(t + 2, (SLOT + 2) % DQ_STAGES);
      const u16* kt = k_s + SLOT * SZ;
      const u16* vt = v_s + SLOT * SZ;
      f32x16 sc = f32x16{}, dp = f32x16{};
      __builtin_amdgcn_s_setprio(1);
      {
        // Operand j: key rows (even j) or value rows (odd j) of slab j/2, read
        // AH ahead of the MFMA that uses them; the hard scheduling boundaries
        // hold each read in its slot.
        constexpr int NJ = 2 * NS, AH = decltype(masked_c)::value ? 2 : DQ_AHEAD;
        bf16x8 f[NJ];
#pragma unroll
        for (int j = 0; j < AH; ++j) f[j] = rf.get((j & 1) ? vt : kt, kh, j >> 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (j + AH < NJ) f[j + AH] = rf.get(((j + AH) & 1) ? vt : kt, kh, (j + AH) >> 1);
          if (j & 1) dp = mfma32(f[j], dof[j >> 1], dp);
          else sc = mfma32(f[j], qf[j >> 1], sc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = exp2_fast(fmaf(sc[i], sl2, -lse2));
      if constexpr (decltype(masked_c)::value) {
        // Key of register i: key0 + 8(i/4) + 4lg + i%4; hidden when it exceeds
        // lim64.  The sign of the difference gives a bit mask.
        const int key0 = QBN * t + 32 * kh;
        const int rel = (int)max<int64_t>(-1, min<int64_t>(lim64 - key0, 32)) - 4 * lg;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const unsigned keep = ~(unsigned)((rel - (8 * (i >> 2) + (i & 3))) >> 31);
          sc[i] = __uint_as_float(__float_as_uint(sc[i]) & keep);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = sc[i] * (dp[i] + ndlt);
      const bf16x8 sb[2] = {slab8(sc, 0), slab8(sc, 8)};
      __builtin_amdgcn_s_setprio(1);
      {
        constexpr int NJ = 2 * NDB, AH = decltype(masked_c)::value ? 2 : DQ_AHEAD_T;
        bf16x8 f[NJ];
#pragma unroll
        for (int j = 0; j < AH; ++j) f[j] = tf.get(kt, kh * 2 + j / NDB, j % NDB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (j + AH < NJ) f[j + AH] = tf.get(kt, kh * 2 + (j + AH) / NDB, (j + AH) % NDB);
          acc[j % NDB] = mfma32(f[j], sb[j / NDB], acc[j % NDB]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // Tile t + 1 must have landed before the barrier that starts its step.
      if (t + 2 < n) wait_vm<NLD>();
      else wait_vm<0>();
      lds_barrier();
    };
    // Whole tiles at or below full_end need no mask.
    const int n_full = min(n, full_end / QBN);
    int t = 0;
    for (; t + 3 <= n_full; t += 3) {
      step(t, I0{}, std::false_type{});
      step(t + 1, I1{}, std::false_type{});
      step(t + 2, I2{}, std::false_type{});
    }
    // The last few tiles (at most two unmasked ones, then the masked ones).
    for (; t < n; ++t) {
      const int slot = t % DQ_STAGES;
      if (slot == 0) step(t, I0{}, std::true_type{});
      else if (slot == 1) step(t, I1{}, std::true_type{});
      else step(t, I2{}, std::true_type{});
    }
  }

  // Add the pair's two partials: the key-half-1 wavefront hands its dQ^T to
  // its partner through LDS (the tile ring is free now).  The lane index is
  // recomputed here rather than kept live across the loop.
  const int lane_e = lane_id();
  float* red = (float*)tiles + pair * (NDB * 16 * 64) + lane_e * 4;
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *(f32x4*)(red + (db * 16 + i) * 64) = f32x4{acc[db][i], acc[db][i + 1], acc[db][i + 2], acc[db][i + 3]};
  }
  lds_barrier();
  const int qi_e = q0 + pair * 32 + (lane_e & 31);
  if (kh == 1 || qi_e >= p.Sq) return;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const f32x4 o = *(const f32x4*)(red + (db * 16 + i) * 64);
      acc[db][i] += o[0];
      acc[db][i + 1] += o[1];
      acc[db][i + 2] += o[2];
      acc[db][i + 3] += o[3];
    }
  float* accp = p.dq_acc + (((int64_t)b * p.Sq + qi_e) * p.Hq + h) * D;
  u16* dqp = p.finalize_dq ? (u16*)p.dq.ptr + (int64_t)b * p.dq.sb + (int64_t)qi_e * p.dq.ss + (int64_t)h * p.dq.sh
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

template <int D>
__global__ __launch_bounds__(DQ_NT) void dq_bf16_kernel(BwdParams p) {
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_qtiles;
  const int bh = lin / p.n_qtiles;
  dq_body<D>(p, bh / p.Hq, bh % p.Hq, unit, 1, [&](int, int b, int hk) {
    return KeySeg{(const u16*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)hk * p.k.sh,
                  (const u16*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)hk * p.v.sh, p.Sk, p.delta_pos};
  });
}

template <int D>
__global__ __launch_bounds__(DQ_NT) void dq_chunks_kernel(BwdParams p, BwdChunkTable ct) {
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = lin % p.n_qtiles;
  const int bh = lin / p.n_qtiles;
  dq_body<D>(p, bh / p.Hq, bh % p.Hq, unit, ct.kv.n, [&](int c, int b, int hk) {
    return KeySeg{(const u16*)ct.kv.k[c] + (int64_t)b * ct.kv.kb[c] + (int64_t)hk * p.k.sh,
                  (const u16*)ct.kv.v[c] + (int64_t)b * ct.kv.vb[c] + (int64_t)hk * p.v.sh, ct.kv.len[c],
                  ct.kv.q_pos0 - ct.kv.pos0[c]};
  });
}

// Packed variable-length batches: the workgroup's sequence b is read from the
// offsets, every pointer is moved to the sequence's first row, and the tile
// code runs with that sequence's lengths (clamped to the declared longest ones)
// and its queries aligned to the end of its keys.  Units past the sequence's
// tiles exit at once, before any barrier.
__device__ __forceinline__ BwdParams varlen_seq(const BwdParams& p, int b, int D) {
  const int q_beg = p.cu_q[b], k_beg = p.cu_k[b];
  BwdParams s = p;
  s.Sq = min(max(p.cu_q[b + 1] - q_beg, 0), p.Sq);
  s.Sk = min(max(p.cu_k[b + 1] - k_beg, 0), p.Sk);
  s.delta_pos = (int64_t)s.Sk - s.Sq;
  s.q.ptr = (const u16*)p.q.ptr + (int64_t)q_beg * p.q.ss;
  s.dout.ptr = (const u16*)p.dout.ptr + (int64_t)q_beg * p.dout.ss;
  s.k.ptr = (const u16*)p.k.ptr + (int64_t)k_beg * p.k.ss;
  s.v.ptr = (const u16*)p.v.ptr + (int64_t)k_beg * p.v.ss;
  s.dk.ptr = (u16*)p.dk.ptr + (int64_t)k_beg * p.dk.ss;
  s.dv.ptr = (u16*)p.dv.ptr + (int64_t)k_beg * p.dv.ss;
  if (p.dq.ptr) s.dq.ptr = (u16*)p.dq.ptr + (int64_t)q_beg * p.dq.ss;
  s.dq_acc = p.dq_acc + (int64_t)q_beg * p.Hq * D;
  s.stats = p.stats + (int64_t)b * p.Hq * 2 * p.Sq_pad;
  return s;
}

template <int D>
__global__ __launch_bounds__(DKV_NT) void dkdv_varlen_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) u16 q_s[3 * SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) u16 d_s[3 * SwTile<D>::SIZE];
  __shared__ __attribute__((aligned(16))) float st_s[3][256];
  __shared__ __attribute__((aligned(16))) u32x4 pex_s[4][2][4][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const SeqHeadUnit w = varlen_order(blockIdx.x, p.Hkv, p.n_units_k);
  const int unit = w.unit, hk = w.h, b = w.b;
  BwdParams s = varlen_seq(p, b, D);
  s.n_ktiles = (s.Sk + KBN - 1) / KBN;
  if (unit >= (p.balanced ? (s.n_ktiles + 1) / 2 : s.n_ktiles)) return;
  if (wave < 4) dkdv_unit<D, true>(s, q_s, d_s, st_s, pex_s, wave, unit, 0, hk);
  else dkdv_unit<D, false>(s, q_s, d_s, st_s, pex_s, wave, unit, 0, hk);
}

template <int D>
__global__ __launch_bounds__(DQ_NT) void dq_varlen_kernel(BwdParams p) {
  const SeqHeadUnit w = varlen_order(blockIdx.x, p.Hq, p.n_qtiles);
  const int unit = w.unit, h = w.h, b = w.b;
  BwdParams s = varlen_seq(p, b, D);
  s.n_qtiles = (s.Sq + QBM - 1) / QBM;
  if (unit >= s.n_qtiles) return;
  dq_body<D>(s, 0, h, unit, 1, [&](int, int, int hk) {
    return KeySeg{(const u16*)s.k.ptr + (int64_t)hk * s.k.sh, (const u16*)s.v.ptr + (int64_t)hk * s.v.sh, s.Sk,
                  s.delta_pos};
  });
}

}  // namespace

int64_t items_bwd_bf16(const BwdParams& p) {
  const int64_t n_ktiles = (p.Sk + KBN - 1) / KBN;
  const int64_t gk = (int64_t)p.B * p.Hkv * (p.balanced ? (n_ktiles + 1) / 2 : n_ktiles);
  const int64_t gq = (int64_t)p.B * p.Hq * ((p.Sq + QBM - 1) / QBM);
  return std::max(gk * DKV_NT, gq * DQ_NT);
}

int64_t items_bwd_chunks_bf16(const BwdParams& p, const BwdChunkTable& ct) {
  int64_t units = 0;
  for (int c = 0; c < ct.kv.n; ++c) {
    const int64_t nk = (ct.kv.len[c] + KBN - 1) / KBN;
    units += p.balanced ? (nk + 1) / 2 : nk;
  }
  const int64_t gq = (int64_t)p.B * p.Hq * ((p.Sq + QBM - 1) / QBM);
  return std::max((int64_t)p.B * p.Hkv * units * DKV_NT, gq * DQ_NT);
}

hipError_t launch_bwd_bf16(const BwdParams& p0, int D, int run_dq, hipStream_t s) {
  BwdParams p = p0;
  p.n_ktiles = (p.Sk + KBN - 1) / KBN;
  p.n_units_k = p.balanced ? (p.n_ktiles + 1) / 2 : p.n_ktiles;
  p.n_qtiles = (p.Sq + QBM - 1) / QBM;
  const int64_t gk = (int64_t)p.B * p.Hkv * p.n_units_k;
  const bool vl = p.cu_q != nullptr;
  if (gk > 0) {
    if (D == 128)
      hipLaunchKernelGGL(vl ? dkdv_varlen_kernel<128> : dkdv_bf16_kernel<128>, dim3((unsigned)gk), dim3(DKV_NT), 0,
                         s, p);
    else
      hipLaunchKernelGGL(vl ? dkdv_varlen_kernel<64> : dkdv_bf16_kernel<64>, dim3((unsigned)gk), dim3(DKV_NT), 0, s,
                         p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t gq = (int64_t)p.B * p.Hq * p.n_qtiles;
  if (run_dq && gq > 0) {
    if (D == 128)
      hipLaunchKernelGGL(vl ? dq_varlen_kernel<128> : dq_bf16_kernel<128>, dim3((unsigned)gq), dim3(DQ_NT), 0, s, p);
    else
      hipLaunchKernelGGL(vl ? dq_varlen_kernel<64> : dq_bf16_kernel<64>, dim3((unsigned)gq), dim3(DQ_NT), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_bwd_chunks_bf16(const BwdParams& p0, const BwdChunkTable& ct0, int D, hipStream_t s) {
  BwdParams p = p0;
  BwdChunkTable ct = ct0;
  int units = 0;
  for (int c = 0; c < ct.kv.n; ++c) {
    ct.unit0[c] = units;
    const int nk = (ct.kv.len[c] + KBN - 1) / KBN;
    units += p.balanced ? (nk + 1) / 2 : nk;
  }
  ct.unit0[ct.kv.n] = units;
  ct.n_units = units;
  p.n_qtiles = (p.Sq + QBM - 1) / QBM;
  const int64_t gk = (int64_t)p.B * p.Hkv * units;
  if (gk > 0) {
    if (D == 128)
      hipLaunchKernelGGL(dkdv_chunks_kernel<128>, dim3((unsigned)gk), dim3(DKV_NT), 0, s, p, ct);
    else
      hipLaunchKernelGGL(dkdv_chunks_kernel<64>, dim3((unsigned)gk), dim3(DKV_NT), 0, s, p, ct);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t gq = (int64_t)p.B * p.Hq * p.n_qtiles;
  if (gq > 0) {
    if (D == 128)
      hipLaunchKernelGGL(dq_chunks_kernel<128>, dim3((unsigned)gq), dim3(DQ_NT), 0, s, p, ct);
    else
      hipLaunchKernelGGL(dq_chunks_kernel<64>, dim3((unsigned)gq), dim3(DQ_NT), 0, s, p, ct);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace attn
