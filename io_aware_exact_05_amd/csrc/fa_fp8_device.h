// Device helpers of the fp8 (OCP e4m3) attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef i32x2 __attribute__((address_space(3))) lds_i32x2;

// XOR swizzle of the 16-byte chunk inside an fp8 row of D bytes; the value
// is below D / 16, so XOR with it permutes the row's chunks.
//   D = 128 (two rows per 256-byte bank line): for the K reads (16 rows, one
//     chunk) every (row parity, chunk) pair is distinct, and for the
//     transposed V reads (8 consecutive rows x 2 adjacent chunks per
//     half-wave) so is every one of the 16 (row, chunk) pairs.
//   D = 64 (four rows per line): rows r, r + 4, r + 8, r + 12, which share
//     their place in the line, get distinct chunks.
//   D = 256 (one row per line): the swizzle of 256-byte rows of the 16-bit
//     kernels (chunk_swz<128>).
template <int D>
__device__ __forceinline__ int swz8(int row) {
  if constexpr (D == 64) return (row >> 2) & 3;
  else if constexpr (D == 128) return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
  else return chunk_swz<128>(row);
}

// Format 0 (e4m3) for both operands, no block scales.  Constant zero scale
// operands make the compiler emit the unscaled v_mfma_f32_32x32x64_f8f6f4
// (measured equal to the scaled form with E8M0 scales 127 = 2^0), which
// issues without the scaled form's extra scale-operand cycles on the VALU
// issue port.
__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Same product with A scaled by 2^(sa - 127) and each lane's B block by
// 2^(sb - 127) (E8M0 biased exponents; sa wave-uniform, sb per lane).
__device__ __forceinline__ f32x16 mfma8_sab(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Two values -> the low two bytes of a word; the high half is whatever the
// destination register held (the builtin's form takes that half as an
// operand, and the compiler clears a register for it).
__device__ __forceinline__ int cvt_pk_e4m3_lo(float a, float b) {
  int w;
  asm("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(w) : "v"(a), "v"(b));
  return w;
}

// The second conversion overwrites the high half the first one left undefined.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, cvt_pk_e4m3_lo(a, b), true);
}

// x rounded to e4m3 (the conversion that packs P~), returned as fp32
__device__ __forceinline__ float round_e4m3(float x) {
  return __builtin_amdgcn_cvt_f32_fp8(cvt_pk_e4m3_lo(x, x), 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// V descale split as 2^e f with f in (1/2, 1]: the E8M0 scale 127 + e of the
// V^T operand (kept in [0, 254]; 255 encodes NaN) and f.
__device__ __forceinline__ int vscale_split(float vdj, float& f) {
  int ex = __builtin_amdgcn_frexp_expf(vdj);
  const float mant = __builtin_amdgcn_frexp_mantf(vdj);  // [1/2, 1)
  f = (mant == 0.5f) ? 1.0f : mant;
  ex -= (mant == 0.5f) ? 1 : 0;
  return min(max(127 + ex, 0), 254);
}

}  // namespace fa
