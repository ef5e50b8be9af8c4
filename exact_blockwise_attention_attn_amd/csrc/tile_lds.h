// 64-row bf16 tiles in LDS, shared by the forward and backward kernels.
//
// A tile holds 64 rows of D elements with no padding (D*2 bytes per row).  The
// 16-byte chunk c of row r sits at chunk position c ^ swz(r).  The swizzle is
// chosen so that both ways a tile is read are free of LDS bank conflicts on
// gfx950 (64 banks of 4 bytes):
//   * row reads (ds_read_b128, an MFMA operand with 8 consecutive elements of
//     one row per lane): the 16 lanes served per cycle read 16 consecutive
//     rows at the same logical chunk and land on 16 distinct chunk slots;
//   * transposing reads (ds_read_b64_tr_b16): the 32 lanes served per cycle
//     read 4 consecutive rows x 64 bytes and land on 16 distinct slots.
// Tiles are filled straight from HBM with global_load_lds: each 1 KB run of 64
// lanes writes 64 consecutive 16-byte slots, and lane l loads the logical chunk
// that belongs in slot l.
#pragma once

#include "attn_device.h"

namespace attn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef i16x4 __attribute__((address_space(3))) lds_i16x4;
typedef void __attribute__((address_space(3))) lds_void;
typedef u32x4 __attribute__((address_space(3))) lds_u32x4;

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const lds_void*)p;
}

template <int D>
struct SwTile {
  static constexpr int ROWS = 64;
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int SIZE = ROWS * D;          // elements
  static constexpr int RUNS = ROWS * CH / 64;    // 1 KB global_load_lds runs per tile
};

__device__ __forceinline__ int rev3(int x) { return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1); }

// Chunk swizzle of row r.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return rev3((r >> 1) & 7);
}

// Element offset of logical element e of row r.
template <int D>
__device__ __forceinline__ int sw_off(int r, int e) {
  return r * D + (((e >> 3) ^ swz<D>(r)) << 3) + (e & 7);
}

// Copy 16 bytes per lane from global memory into LDS: lane l writes bytes
// [16 l, 16 l + 16) after lds_base.  This is global_load_lds issued as inline
// assembly, so the compiler does not see the load and inserts no waits for it
// (its own tracking of LDS-bound loads gives up at loop headers and waits for
// every load in flight, which would drain a deep prefetch).  The caller must
// wait for the load itself (s_waitcnt vmcnt) before any wavefront reads the
// destination, and before the wavefront exits.  M0 holds the LDS base; the
// s_nop covers the wait state between writing M0 and the LDS-bound load.
// The LDS address is passed as base + offset, each wave-uniform, so that a
// constant base need not stay live in a scalar register of its own.
__device__ __forceinline__ void dma16_untracked(const void* src, lds_void* lds_base, unsigned off = 0) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"((unsigned)(size_t)lds_base), "s"(off)
               : "memory", "m0", "scc");
}

// Issue the copy of rows [row0, row0 + 64) of a [rows, D] bf16 view into a
// tile, spread over NW wavefronts (wave w issues runs w, w + NW, ...).  Rows
// past the end load a valid row (their results are masked or dropped), so LDS
// never holds uninitialised values.
//
// Each wavefront issues exactly RUNS / NW loads (a compile-time count), so code
// that waits for a given number of loads in flight can rely on it, and so can
// the compiler's own wait insertion.
// With UNTRACKED the loads are issued with dma16_untracked (see there).
template <int D, int NW, bool UNTRACKED = false>
__device__ __forceinline__ void issue_swtile(u16* lds, const u16* g, int64_t ss, int row0, int nrows, int wave,
                                             int lane) {
  using T = SwTile<D>;
  static_assert(T::RUNS % NW == 0, "runs must split evenly over the wavefronts");
#pragma unroll
  for (int i = 0; i < T::RUNS / NW; ++i) {
    const int run = wave + i * NW;
    const int slot = run * 64 + lane;
    const int r = slot / T::CH;
    const int c = (slot % T::CH) ^ swz<D>(r);
    const int row = min(row0 + r, nrows - 1);
    const void* src = g + (int64_t)row * ss + c * 8;
    if constexpr (UNTRACKED) dma16_untracked(src, (lds_void*)(lds + i * NW * 512), (unsigned)wave * 1024u);
    else __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + run * 512), 16, 0, 0);
  }
}

// As dma16_untracked, with the source given as a wave-uniform base (held in
// scalar registers) plus a per-lane 32-bit byte offset: the load adds them
// itself, so issuing it takes no vector arithmetic.
__device__ __forceinline__ void dma16_untracked_s(const void* sbase, unsigned voff, lds_void* lds_base,
                                                  unsigned off = 0) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"((unsigned)(size_t)lds_base), "s"(off)
               : "memory", "m0", "scc");
}

// Per-lane byte offset of the 64-row tile copy (the pattern issue_swtile
// follows), computed once, so that each later load is a wave-uniform base plus
// this lane's offset.  A wavefront's i-th load covers the rows of its first
// load plus 64 * NW * i / CH, a multiple of 16, and the chunk swizzle depends
// only on the row modulo 16, so every load of the wavefront shares one lane
// offset and the row step goes into the scalar base.  A tile that runs past
// the last row clamps each lane's row to it and recomputes the offset on the
// spot (no per-lane pointers stay live).  The offset is 32-bit, so the row
// stride ss must lie in [0, 2^24] elements (64 rows then span under 2 GiB);
// the host rejects larger key/value sequence strides.
template <int D, int NW>
struct TileSrc {
  static constexpr int N = SwTile<D>::RUNS / NW;             // loads per wavefront per tile
  static constexpr int ROW_STEP = NW * 64 / SwTile<D>::CH;  // rows between a wavefront's loads
  static_assert(ROW_STEP % 16 == 0, "the swizzle must repeat between a wavefront's loads");
  unsigned off;
  __device__ __forceinline__ void init(int64_t ss, int wave, int lane) {
    using T = SwTile<D>;
    const int slot = wave * 64 + lane;
    const int r = slot / T::CH;
    off = (unsigned)(((int64_t)r * ss + ((slot % T::CH) ^ swz<D>(r)) * 8) * 2);
  }
  // Copy rows [row0, row0 + 64) of g (row stride ss) into lds, untracked; rows
  // at or past nrows load row nrows - 1 (row0 < nrows).
  __device__ __forceinline__ void issue(u16* lds, const u16* g, int64_t ss, int row0, int nrows, int wave,
                                        int lane) const {
    using T = SwTile<D>;
    const u16* base = g + (int64_t)row0 * ss;
    if (row0 + 64 <= nrows) {
#pragma unroll
      for (int i = 0; i < N; ++i)
        dma16_untracked_s(base + (int64_t)(i * ROW_STEP) * ss, off, (lds_void*)(lds + i * NW * 512),
                          (unsigned)wave * 1024u);
    } else {
      const int last = nrows - 1 - row0;  // last valid row of the tile, >= 0
      const int slot = wave * 64 + lane;
      const int r0 = slot / T::CH;
      const int cpos = ((slot % T::CH) ^ swz<D>(r0)) * 8;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int r = min(r0 + i * ROW_STEP, last);
        dma16_untracked_s(base, (unsigned)(r * (int)ss + cpos) * 2u, (lds_void*)(lds + i * NW * 512),
                          (unsigned)wave * 1024u);
      }
    }
  }
};

// Per-lane byte offsets of the row-read operand fragments: row (32*blk + lane%32),
// logical chunk 2*s + lane/32, for s = 0 .. D/16-1.  The block of 32 rows adds
// 64*D bytes (an immediate), since the swizzle repeats every 16 rows.  Byte
// offsets let a tile base that is a compile-time constant fold into the LDS
// read's immediate offset with no vector instruction.
template <int D>
struct RowFrag {
  int off[D / 16];
  __device__ __forceinline__ void init(int lane) {
    const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) off[s] = 2 * sw_off<D>(lr, (2 * s + lg) * 8);
  }
  __device__ __forceinline__ bf16x8 get(const u16* t, int blk, int s) const {
    return as_bf16x8(*(const u32x4*)((const char*)t + blk * 64 * D + off[s]));
  }
  // Based form: rebase(t) adds the LDS address of tensor t to the offsets
  // once; get_at(o, ...) then reads the tile o bytes past t.  A constant o
  // below 64 KB becomes the LDS read's immediate offset even where the
  // tensor itself sits above the 64 KB an immediate can reach.
  __device__ __forceinline__ void rebase(const u16* t) {
    const unsigned a = lds_addr(t);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) off[s] += (int)a;
  }
  __device__ __forceinline__ bf16x8 get_at(int o, int blk, int s) const {
    return as_bf16x8(*(const lds_u32x4*)(uintptr_t)(unsigned)(o + blk * 64 * D + off[s]));
  }
  // Make the offsets opaque to the compiler at this point (no instruction):
  // addresses derived from them after it cannot be hoisted above it, where each
  // (tile base, fragment) pair would otherwise hold a register of its own.
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) asm volatile("" : "+v"(off[s]));
  }
};

// Per-lane offsets of transposed operand fragments.  For a 16-row slab of a tile
// and a 32-feature block db, lane (16q + s) reads 4 features of row
// slab + 8h + 4*(q/2) + s/4 at feature 32*db + 16*(q%2) + 4*(s%4); the
// transposing read hands lane (32*(q/2) + 16*(q%2) + s) feature 32*db + 16*(q%2) + s
// of rows slab + 8h + 4*(q/2) + {0..3}: the k-slot order of an operand that
// comes straight out of an MFMA accumulator.  Slabs add 32*D bytes (an immediate).
template <int D>
struct TrFrag {
  int off[2][D / 32];  // bytes
  __device__ __forceinline__ void init(int lane) {
    const int q16 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        off[h][db] = 2 * sw_off<D>(8 * h + 4 * (q16 >> 1) + (s16 >> 2), db * 32 + 16 * (q16 & 1) + 4 * (s16 & 3));
  }
  __device__ __forceinline__ bf16x8 get(const u16* t, int slab, int db) const {
    const char* tb = (const char*)t + slab * 32 * D;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + off[0][db]));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + off[1][db]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  // Based form, as in RowFrag.
  __device__ __forceinline__ void rebase(const u16* t) {
    const unsigned a = lds_addr(t);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) off[h][db] += (int)a;
  }
  __device__ __forceinline__ bf16x8 get_at(int o, int slab, int db) const {
    const int tb = o + slab * 32 * D;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(unsigned)(tb + off[0][db]));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(unsigned)(tb + off[1][db]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) asm volatile("" : "+v"(off[h][db]));
  }
};

}  // namespace attn
