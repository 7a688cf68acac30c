// Device-side helpers shared by the gfx950 attention kernels: vector types,
// bf16 packing, MFMA wrappers and wave-level exchanges.
//
// Lane layouts used throughout (wave64, checked on gfx950):
//  * v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8*(l/32) + j] and
//    B[8*(l/32) + j][l%32] for j = 0..7; the 16 accumulators of lane l are
//    C[8*(i/4) + 4*(l/32) + i%4][l%32], i = 0..15.
//  * v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + j],
//    B[8*(l/16) + j][l%16]; accumulators C[4*(l/16) + i][l%16], i = 0..3.
//  * ds_read_b64_tr_b16: inside each 16-lane group, output lane j receives, as
//    element r, the 16-bit word j%4 of the 8 bytes addressed by lane 4*r + j/4
//    of the same group.  Pointing lane i at row (i/4), column 4*(i%4) of a
//    4 x 16 block therefore hands lane j that block's column j.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace paa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define PAA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// Two fp32 -> two bf16 (round to nearest even), packed low/high in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// acc + the two bf16 values packed in w (one v_dot2 against 1.0 in both halves, fp32 accumulation).
// The kernels sum the probabilities as rounded to bf16 for the product with V this way, so that O is
// divided by the same weights its numerator used.
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc,
                                         false);
}

// acc + the 16 bf16 values of four packed operand registers, in one chain seeded with acc (a dependent
// VALU chain costs no extra issue cycles, and the seed saves the moves and adds of separate partials).
__device__ __forceinline__ float add_bf16x16(const u32x4_t (&pf)[4], float acc) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = add_bf16_pair(pf[k][j], acc);
  return acc;
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Transposed 8-byte LDS read (see the layout note above); returns two dwords.
__device__ __forceinline__ u32x2_t lds_read_tr16(const PAA_LDS uint16_t* p) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PAA_LDS i16x4_t*)p);
  return __builtin_bit_cast(u32x2_t, v);
}

// Value held by lane l ^ 32 (upper = this lane is in 32..63).
__device__ __forceinline__ float swap_halves(float x, bool upper) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, upper ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Stores a wave's 32 x D output tile through LDS, so that every store instruction writes whole rows
// (D / 8 lanes x 16 bytes per row) instead of 8 bytes in each of 32 rows.  acc is O^T in the
// 32x32x16 accumulator layout (lane l, block db, element i: row l % 32, column 32db + 8(i/4) +
// 4(l/32) + i%4), scaled by f and rounded to bf16; the tile is staged at `ot` (32 rows of 2D bytes,
// the wave's own) with 16-byte chunk c of row r at position c ^ (r % (D / 8)), which keeps the
// 8-byte writes and the 16-byte reads free of most bank conflicts, then read back row by row.  Rows
// at or past `rows` are not written.
template <int D>
__device__ __forceinline__ void store_o_tile(PAA_LDS char* ot, const f32x16_t (&acc)[D / 32], float f, int lane,
                                             uint16_t* o_row0, size_t row_stride, int rows) {
  constexpr int kRowBytes = 2 * D, kCpr = D / 8, kRowsPerBlock = 64 / kCpr;
  const int l32 = lane % 32, half = lane / 32;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int chunk = 4 * db + gq;  // columns 32db + 8gq .. +7; this half-wave's 4 start at 4 * half
      const u32x2_t w = {pack_bf16x2(acc[db][4 * gq + 0] * f, acc[db][4 * gq + 1] * f),
                         pack_bf16x2(acc[db][4 * gq + 2] * f, acc[db][4 * gq + 3] * f)};
      *(PAA_LDS u32x2_t*)(ot + l32 * kRowBytes + ((chunk ^ (l32 % kCpr)) * 16) + 8 * half) = w;
    }
  }
#pragma unroll
  for (int k = 0; k < 32 / kRowsPerBlock; ++k) {
    const int r = k * kRowsPerBlock + lane / kCpr;  // tile row
    const int c = lane % kCpr;                        // 16-byte chunk of the row
    const u32x4_t v = *(const PAA_LDS u32x4_t*)(ot + r * kRowBytes + ((c ^ (r % kCpr)) * 16));
    if (r < rows) *(u32x4_t*)(o_row0 + (size_t)r * row_stride + c * 8) = v;
  }
}

}  // namespace paa
