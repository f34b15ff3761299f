// Device helpers for the gfx950 (CDNA4) attention kernels: MFMA wrappers,
// bf16 packing, fast exp2/log2, and the LDS layouts shared by the kernels.
//
// MFMA lane layout (v_mfma_f32_32x32x16_bf16, one 64-lane wavefront):
//   A (32 x 16): lane l holds A[l % 32][8*(l/32) + j],  j = 0..7
//   B (16 x 32): lane l holds B[8*(l/32) + j][l % 32],  j = 0..7
//   C (32 x 32): lane l, register i holds C[8*(i/4) + 4*(l/32) + (i%4)][l % 32]
// so every lane owns one column of C and 16 of its rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> one word of two bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 ld_lds16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void st_lds16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ void st_lds8(uint16_t* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}

// Exchange with the lane 32 positions away (the other half of the wavefront).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// ---------------------------------------------------------------------------
// Transposed tiles in LDS.
//
// The P.V product (and, in the backward pass, dO^T.P and Q^T.dS) reduces over
// the token index, which is the row index of V / dO / Q in memory.  MFMA
// operands must hold 8 consecutive reduction-index values per lane, so these
// tiles are stored transposed, [feature row][token], 64 tokens per row.
//
// Token order inside a row: the MFMA accumulator that produces P holds, in
// lane half h, the tokens {4h..4h+3, 8+4h..8+4h+3} of each group of 16 (see the
// C layout above).  Storing tokens with the middle two groups of four swapped
// puts exactly those eight tokens side by side, so one 16-byte LDS read feeds
// the operand.  The summation order of the product is irrelevant, so this
// permutation changes nothing in the result beyond fp32 rounding order.
//
// Bank spreading: rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r
// is stored at chunk slot c ^ ((r + r/8) & 7).  Readers take 32 consecutive
// rows at one chunk, writers 8-rows-apart rows at one chunk; both land on
// different slots.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tok_perm(int t) {
  // swap groups 1 and 2 (of four tokens) inside every group of sixteen
  const int g = (t >> 2) & 3;
  const int ng = (g == 1) ? 2 : (g == 2) ? 1 : g;
  return (t & ~15) | (ng << 2) | (t & 3);
}
__device__ __forceinline__ int tr64_offset(int row, int pos) {
  const int chunk = (pos >> 3) ^ ((row + (row >> 3)) & 7);
  return row * 64 + chunk * 8 + (pos & 7);
}

}  // namespace fa2
