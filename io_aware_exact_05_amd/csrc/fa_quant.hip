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
// 4 bytes read and 1 byte written per element.  For d <= 128 the block
// moves through LDS both ways, so that every global access instruction
// covers whole contiguous rows: the fp32 rows arrive by direct global -> LDS
// copies (16-byte chunks XOR-swizzled within each half row; 64 rows at a
// time with the rotation), and the codes are staged row-major before
// 16-byte stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"
#include "fa_quant_index.h"

namespace fa {
namespace {

using qidx::kBlockRows;

// 16-byte buffer -> LDS copy per lane (lane i's bytes land at lds_addr + 16 i;
// offsets past the resource read zeros); the caller waits on vmcnt.
__device__ __forceinline__ void q_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

template <int D, bool ROT>
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(QuantParams p) {
  using G = qidx::Geo<D, ROT>;
  constexpr int E = G::E;  // elements per thread (half a row)
  constexpr bool STAGE = G::STAGE;  // rows staged through LDS
  constexpr int RB = G::RB, HC = G::HC;  // row bytes, chunks per half row
  // rows per staging pass: two passes of 64 rows with the rotation (32 KiB
  // at d = 128, so that more workgroups share a CU while they transform),
  // one pass of 128 without (measured: each is the faster choice there)
  constexpr int NPASS = G::NPASS, SR = G::SR;
  __shared__ __attribute__((aligned(1024))) char tile[G::TILE_BYTES];
  const int t = threadIdx.x, r = t >> 1, hf = t & 1;
  const int bh = blockIdx.x / p.nblk, blk = blockIdx.x % p.nblk;
  const int row = blk * kBlockRows + r;
  const bool valid = row < p.N;
  const size_t base = ((size_t)bh * p.N + (valid ? row : 0)) * D + hf * E;

  float x[E];
  if constexpr (STAGE) {
    // slot s of the tile (row s / CPR, position s % CPR) receives chunk
    // position ^ (row % HC) of that row; rows past N read as zeros
    const size_t blk_elem = ((size_t)bh * p.N + (size_t)blk * kBlockRows) * D;
    const int rows_left = min(kBlockRows, p.N - blk * kBlockRows);
    // base address made wave-uniform word by word; each word stays unsigned
    // (readfirstlane returns int, which must not be sign-extended)
    const uint64_t a = (uint64_t)(uintptr_t)(p.x + blk_elem);
    const uint32_t a_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t a_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* ub = (void*)(uintptr_t)qidx::join_words(a_lo, a_hi);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        ub, 0, (int)__builtin_amdgcn_readfirstlane((uint32_t)(rows_left * RB)), 0x00020000);
    const int w = t >> 6, lane = t & 63;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)tile;
    constexpr int NI = G::NI;  // copies per thread and pass
    // with two passes, waves 0-1 take their rows from the first and waves
    // 2-3 from the second
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      if (ps == 1) __syncthreads();  // the first pass's rows have been read
#pragma unroll
      for (int u = 0; u < NI; ++u)
        q_dma16(rs, qidx::dma_src<D, ROT>(ps, u, w, lane), lds0 + qidx::dma_dst<D, ROT>(u, w));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (r / SR == ps) {
        const int lr = r - ps * SR;
#pragma unroll
        for (int k = 0; k < HC; ++k) {
          const float4 v = *(const float4*)(tile + qidx::stage_read<D, ROT>(lr, hf, k));
          x[4 * k] = v.x;
          x[4 * k + 1] = v.y;
          x[4 * k + 2] = v.z;
          x[4 * k + 3] = v.w;
        }
      }
    }
  } else if (valid) {
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
    // column factors signs[c] / sqrt(d), read once per workgroup into LDS
    // (all lanes of a half then read the same words: broadcast)
    __shared__ __attribute__((aligned(16))) float colf[D];
    if (t < D) colf[t] = (p.signs ? p.signs[t] : 1.0f) * p.inv_sqrt_d;
    // Walsh-Hadamard butterflies (a, b) -> (a + b, a - b) at strides 1 .. E/2
    // inside the thread, then stride E across the lane pair: the lower lane
    // keeps a + b, the upper one a - b = o - x (o = the partner's value,
    // fetched by a DPP quad permutation [1, 0, 3, 2]).
#pragma unroll
    for (int h = 1; h < E; h <<= 1)
#pragma unroll
      for (int i = 0; i < E; ++i)
        if ((i & h) == 0) {
          const float a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
    const float sx = hf ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float o = __builtin_bit_cast(
          float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[i]), 0xB1, 0xF, 0xF, false));
      x[i] = __builtin_fmaf(sx, x[i], o);
    }
    __syncthreads();  // colf written
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 f4 = *(const float4*)(colf + hf * E + 4 * i);
      x[4 * i] *= f4.x;
      x[4 * i + 1] *= f4.y;
      x[4 * i + 2] *= f4.z;
      x[4 * i + 3] *= f4.w;
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
  if constexpr (STAGE) {
    // codes row-major in LDS (D bytes per row; the 16-byte chunks of a row
    // XOR-swizzled by row), then 16-byte stores of whole rows
    constexpr int CR = G::CR;  // code chunks per row
    __syncthreads();  // every thread has read its fp32 half row
#pragma unroll
    for (int i = 0; i < E / 16; ++i)
      *(uint4*)(tile + qidx::code_write<D>(r, hf, i)) =
          make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
    __syncthreads();
    const int rows_left = min(kBlockRows, p.N - blk * kBlockRows);
    uint8_t* dst = p.x8 + ((size_t)bh * p.N + (size_t)blk * kBlockRows) * D;
#pragma unroll
    for (int u = 0; u < kBlockRows * CR / 256; ++u) {
      const int sl = u * 256 + t, rr = sl / CR, c = sl % CR;
      const uint4 val = *(const uint4*)(tile + qidx::code_read<D>(rr, c));
      if (rr < rows_left) *(uint4*)(dst + (size_t)rr * D + c * 16) = val;
    }
  } else if (valid) {
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
