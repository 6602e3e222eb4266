// Block quantiser fp32 -> OCP e4m3fn for the fp8 attention path (gfx950).
//
// The fp8 path of "FlashAttention-3 (BN)" / "FlashAttention-3 (FA)" (section
// on low precision and reducing quantisation error) quantises Q, K, V to
// 8-bit floats and, for Q and K, first multiplies by a random orthogonal
// matrix so that outliers spread over all coordinates ("incoherent
// processing").  Here:
//   * rotation (optional): x <- x H_d diag(signs) / sqrt(d), H_d the
//     Sylvester Hadamard matrix, computed as a fast Walsh-Hadamard transform
//     of each row (d log2 d additions) followed by one multiply per element;
//   * a block is 128 consecutive rows of one (b, h), all d columns: amax over
//     the block; the descale is the smallest power of two 2^e with
//     amax <= 448 2^e, and codes = e4m3(clamp(x 2^-e, +-448)) rounded to
//     nearest even by v_cvt_pk_fp8_f32 (which does not saturate by itself,
//     hence the clamp).  Scaling by a power of two is exact, so each code is
//     one rounding of x / descale and the descale can later be applied
//     exactly (as an MFMA block scale or an fp32 factor).  An all-zero block
//     stores descale 1 and zero codes.
// One workgroup (256 threads) per block: thread t holds half of row t / 2
// in registers; the last butterfly stage of the transform pairs the two
// halves across neighbouring lanes.  The pass is bound by HBM traffic:
// 4 bytes read and 1 byte written per element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kBlockRows = 128;

template <int D, bool ROT>
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(QuantParams p) {
  constexpr int E = D / 2;  // elements per thread (half a row)
  const int t = threadIdx.x, r = t >> 1, hf = t & 1;
  const int bh = blockIdx.x / p.nblk, blk = blockIdx.x % p.nblk;
  const int row = blk * kBlockRows + r;
  const bool valid = row < p.N;
  const size_t base = ((size_t)bh * p.N + (valid ? row : 0)) * D + hf * E;

  float x[E];
  if (valid) {
    const float4* src = (const float4*)(p.x + base);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 v = src[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = 0.f;
  }

  if constexpr (ROT) {
    // Walsh-Hadamard butterflies (a, b) -> (a + b, a - b) at strides 1 .. E/2
    // inside the thread, then stride E across the lane pair.
#pragma unroll
    for (int h = 1; h < E; h <<= 1)
#pragma unroll
      for (int i = 0; i < E; ++i)
        if ((i & h) == 0) {
          const float a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float o = __shfl_xor(x[i], 1);
      x[i] = hf ? (o - x[i]) : (x[i] + o);
    }
    const float inv_sqrt_d = p.inv_sqrt_d;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float s = p.signs ? p.signs[hf * E + i] : 1.0f;
      x[i] = x[i] * (s * inv_sqrt_d);
    }
  }

  // amax over the block: thread, wave (64 lanes), then the four waves.
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  __shared__ float wmax[4];
  if ((t & 63) == 0) wmax[t >> 6] = a;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // smallest e with amax <= 448 2^e: with amax = m 2^k (m in [1/2, 1)),
  // 448 = 7/8 2^9 gives e = k - 9 when m <= 7/8, else k - 8
  const bool zero = amax == 0.f;
  int e = __builtin_amdgcn_frexp_expf(amax) - 9;
  e += (__builtin_amdgcn_frexp_mantf(amax) > 0.875f) ? 1 : 0;
  if (t == 0) p.descale[(size_t)bh * p.nblk + blk] = zero ? 1.0f : __builtin_amdgcn_ldexpf(1.0f, e);
  const int ne = zero ? 0 : -e;  // x 2^-e by exponent arithmetic (exact)

  if (valid) {
    uint32_t packed[E / 4];
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[k] = fminf(fmaxf(__builtin_amdgcn_ldexpf(x[4 * i + k], ne), -448.0f), 448.0f);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
      packed[i] = (uint32_t)w;
    }
    uint4* dst = (uint4*)(p.x8 + base);
#pragma unroll
    for (int i = 0; i < E / 16; ++i)
      dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
  }
}

template <int D>
hipError_t launch_q(const QuantParams& p, int rotate, hipStream_t s) {
  const unsigned grid = (unsigned)(p.BH * p.nblk);
  if (rotate)
    hipLaunchKernelGGL((quantize_e4m3_kernel<D, true>), dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((quantize_e4m3_kernel<D, false>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_e4m3(const QuantParams& p, int d, int rotate, hipStream_t s) {
  switch (d) {
    case 64: return launch_q<64>(p, rotate, s);
    case 128: return launch_q<128>(p, rotate, s);
    case 256: return launch_q<256>(p, rotate, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
