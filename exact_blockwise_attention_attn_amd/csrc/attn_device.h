// Device-side helpers for gfx950 (CDNA4): vector types, bf16 conversion,
// MFMA wrappers, cross-lane helpers and the XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }
__device__ __forceinline__ float pos_inf() { return __builtin_huge_valf(); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(u16 x) { return __uint_as_float((uint32_t)x << 16); }

// fp32 -> bf16 with round-to-nearest-even (hardware conversion on gfx950).
__device__ __forceinline__ u16 f32_to_bf16(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ bf16x8 cvt_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                             float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// D = A(32x16) * B(16x32) + C.  Lane l supplies A[l%32][8*(l/32) .. +7] and
// B[8*(l/32) .. +7][l%32]; it receives C[8*(i/4) + 4*(l/32) + i%4][l%32], i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C.  Lane l supplies A[l%16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l%16]; it receives C[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane l ^ 32 (the other half of the wavefront).
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

// Sum over each aligned group of 16 lanes (a DPP row), the result in every lane
// of the group: swaps within quads, then rotations of the row by 4 and 8 lanes.
// Vector-ALU moves only (no LDS crossbar round trip).  Every lane of the row
// must be active.
__device__ __forceinline__ float sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lanes 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lanes 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror 4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror 8
  return x;
}

// Position of key k (within a tile) in the MFMA k-slot order used for operands
// that come straight out of an MFMA accumulator: slot (g, s) of a 16-key slab
// holds key 8*(s/4) + 4*g + s%4, so the 8 keys a lane contributes are
// contiguous in LDS.
__device__ __forceinline__ int slot_pos(int k) {
  return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Map hardware id -> logical id so that consecutive logical ids run on the
// same XCD: logical work that shares K/V then shares an L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int kXcd = 8;
  if (n % kXcd) return bid;
  return (bid % kXcd) * (n / kXcd) + bid / kXcd;
}

// Packed variable-length batches: the sequences differ in work, so giving each
// XCD a contiguous range of them (as xcd_remap does) unbalances the XCDs.
// Instead XCD x takes the heads h = x (mod 8) of every sequence, in (sequence,
// head, unit) order, so every XCD carries the same share of every sequence
// while the units of one (sequence, head) still share an XCD and its L2.  With
// a head count that is not a multiple of 8 the order is the plain one.
struct SeqHeadUnit {
  int b, h, unit;
};
__device__ __forceinline__ SeqHeadUnit varlen_order(int bid, int H, int n_units) {
  constexpr int kXcd = 8;
  if (H % kXcd) return SeqHeadUnit{bid / (H * n_units), (bid / n_units) % H, bid % n_units};
  const int x = bid % kXcd, s = bid / kXcd;
  const int per_b = (H / kXcd) * n_units;  // workgroups of one sequence on one XCD
  const int r = s % per_b;
  return SeqHeadUnit{s / per_b, (r / n_units) * kXcd + x, r % n_units};
}

// Log-sum-exp merge of (La, Oa) with (Lb, Ob); -inf parts contribute nothing.
// A NaN on either side makes both weights and L NaN (fmaxf alone would drop it).
__device__ __forceinline__ void merge_weights(float La, float Lb, float& wa, float& wb, float& L) {
  float mx = fmaxf(La, Lb);
  if ((La == neg_inf()) & (Lb == neg_inf())) {
    wa = 0.f;
    wb = 0.f;
    L = neg_inf();
    return;
  }
  float ea = expf(La - mx);
  float eb = expf(Lb - mx);
  float tot = ea + eb;
  float inv = 1.0f / tot;
  wa = ea * inv;
  wb = eb * inv;
  L = mx + logf(tot);
}

}  // namespace attn
