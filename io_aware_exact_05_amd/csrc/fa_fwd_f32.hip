// Fused exact attention forward for gfx950, fp32 inputs and outputs.
//
// The same tiled online-softmax pass as the 16-bit kernel ("FlashAttention
// (HI)", tiling and online-softmax sections), kept simple because fp32 is the
// small exactness check rather than a throughput path: one wave64 per
// workgroup owns 32 query rows; Q, K and V tiles sit in LDS (rows padded by
// one float so that 32 lanes reading one column hit 32 banks); both products
// run on v_mfma_f32_32x32x2f32 with fp32 operands, so P is never rounded
// below fp32.  S^T = K Q^T puts one query per lane; O^T = V^T P^T takes P
// straight from the S^T accumulators, one register (two keys) per k-step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

namespace {

constexpr float kNegInf32 = -__builtin_huge_valf();

__device__ __forceinline__ float pair_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_f32(FwdParams p) {
  constexpr int BR = 32, BC = 32, STR = D + 1, ND = D / 32;
  __shared__ float sq[BR * STR];
  __shared__ float sk[BC * STR];
  __shared__ float sv[BC * D];

  const int lane = threadIdx.x, ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  const int bh = blockIdx.x % p.BH;
  const int qt = blockIdx.x / p.BH;
  const size_t head = (size_t)bh * N * D;
  const float* __restrict__ qh = (const float*)p.q + head;
  const size_t kvhead = (size_t)kv_head(p, bh) * N * D;  // K/V head shared by a group of query heads
  const float* __restrict__ kh = (const float*)p.k + kvhead;
  const float* __restrict__ vh = (const float*)p.v + kvhead;
  const int q0 = qt * BR, myq = q0 + ql;

  for (int e = lane; e < BR * D; e += 64) {
    const int r = e / D, col = e % D;
    sq[r * STR + col] = (q0 + r < N) ? qh[(size_t)(q0 + r) * D + col] : 0.f;
  }

  f32x16 oacc[ND];
  for (int b = 0; b < ND; ++b)
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m = -1.0e30f, l = 0.f;
  const float c = p.scale_log2, cabs = fabsf(c);
  const bool neg = c < 0.f;
  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int lim = CAUSAL ? min(myq, N - 1) : N - 1;

  for (int key0 = 0; key0 < kv_end; key0 += BC) {
    __syncthreads();
    for (int e = lane; e < BC * D; e += 64) {
      const int r = e / D, col = e % D;
      const bool ok = key0 + r < N;
      sk[r * STR + col] = ok ? kh[(size_t)(key0 + r) * D + col] : 0.f;
      sv[r * D + col] = ok ? vh[(size_t)(key0 + r) * D + col] : 0.f;
    }
    __syncthreads();
    // S^T = K Q^T: row (key) 8(r/4) + 4g + r%4, column (query) ql.
    f32x16 s;
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    for (int t = 0; t < D / 2; ++t)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(sk[ql * STR + 2 * t + g], sq[ql * STR + 2 * t + g], s, 0, 0, 0);
    float mx = kNegInf32;
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * g + (r & 3);
      const float x = neg ? -s[r] : s[r];
      mx = key <= lim ? fmaxf(mx, x) : mx;
    }
    mx = pair_max(mx);
    const float mt = (mx == kNegInf32) ? kNegInf32 : mx * cabs;
    const float mnew = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    float rs = 0.f;
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * g + (r & 3);
      float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mnew));
      pr = key <= lim ? pr : 0.f;
      s[r] = pr;
      rs += pr;
    }
    l = l * alpha + rs;
    for (int b = 0; b < ND; ++b) {
      for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
      // k-step r: half-wave g contributes key 8(r/4) + 4g + r%4.
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + 4 * g + (r & 3);
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(sv[kk * D + 32 * b + ql], s[r], oacc[b], 0, 0, 0);
      }
    }
  }

  const float lt = pair_sum(l);
  if (myq < N) {
    const float inv = 1.0f / lt;
    float* orow = (float*)p.o + head + (size_t)myq * D;
    for (int b = 0; b < ND; ++b)
      for (int a = 0; a < 4; ++a) {
        float4 v4 = make_float4(oacc[b][4 * a] * inv, oacc[b][4 * a + 1] * inv,
                                oacc[b][4 * a + 2] * inv, oacc[b][4 * a + 3] * inv);
        *(float4*)(orow + 32 * b + 8 * a + 4 * g) = v4;
      }
    if (g == 0)
      p.lse[(size_t)bh * N + myq] = (m + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_f32_one(const FwdParams& p, hipStream_t s) {
  const int nq = (p.N + 31) / 32;
  hipLaunchKernelGGL((fwd_f32<D, CAUSAL>), dim3((unsigned)(nq * p.BH)), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d, int causal, hipStream_t s) {
  switch (d) {
    case 64:  return causal ? launch_f32_one<64, true>(p, s) : launch_f32_one<64, false>(p, s);
    case 128: return causal ? launch_f32_one<128, true>(p, s) : launch_f32_one<128, false>(p, s);
    case 256: return causal ? launch_f32_one<256, true>(p, s) : launch_f32_one<256, false>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
