// Fused exact attention forward for gfx950 (MI355X), fp16/bf16 inputs.
//
// One workgroup owns BR = 128 query rows of one (batch, head): four wave64s,
// each holding 32 rows for the whole pass.  The key/value sequence streams
// through LDS in tiles of BC rows, double-buffered: the next tile's global
// loads are issued before the current tile is consumed and land in the other
// buffer afterwards, so one barrier per tile suffices ("FlashAttention (HI)",
// tiling section: inputs split into tiles that fit on-chip memory, loaded in
// turn, the final result updated; "FlashAttention-3 (BN)", memory-operations
// section: the next block loads while the current one is computed).
//
// Per tile and wave (all on-chip; the score tile never reaches HBM):
//   S^T = K_j Q^T   on v_mfma_f32_32x32x16_{bf16,f16}: keys on the MFMA rows,
//                   queries on the columns, so each lane owns ONE query and a
//                   set of keys — row max / row sum are in-lane reductions plus
//                   one v_permlane32_swap with the other half-wave.
//   online softmax  running max m and running sum l per query in base 2, the
//                   scale folded into one FMA per score before v_exp_f32
//                   ("FlashAttention (HI)", online-softmax section;
//                   "FlashAttention-2 (BN)", fewer non-matmul operations).
//   O^T += V_j^T P^T  P stays in registers: the S^T accumulator layout is
//                   exactly the B-operand layout of this MFMA once the key
//                   order inside each 32-key block is permuted (bits 2 and 3 of
//                   the row index swapped when K is read); V is read from LDS
//                   already transposed with ds_read_b64_tr_b16.
// The epilogue divides by l once per row and writes O and the logsumexp once
// ("FlashAttention (HI)", one-kernel section: only the final result is
// written).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;

typedef i16x4 __attribute__((address_space(3))) lds_i16x4;

// 16-bit element traits: the MFMA and the fp32 -> 16-bit packing (RNE).
template <typename T> struct Half;
template <> struct Half<__bf16> {
  static __device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
};
template <> struct Half<_Float16> {
  static __device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
};

// Key held by MFMA row i of a 32-key block: bits 2 and 3 of i swapped.  The
// map is its own inverse.  With it, accumulator register r of half-wave g
// holds key 16*(r/8) + 8*g + (r%8): eight consecutive keys per register group.
__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ float wave_pair_max(float x) {
  // lanes l and l^32 hold the same query: v_permlane32_swap exchanges halves.
  auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
}
__device__ __forceinline__ float wave_pair_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMInit = -1.0e30f;  // finite start of the running max

// Block index -> (head, query tile).  Workgroups are dispatched round-robin
// over the 8 XCDs (block b runs on XCD b % 8).  When the head count divides
// by 8, each XCD gets a contiguous range of heads so that all query tiles of
// a head share that XCD's L2 for K and V.  Within an XCD tiles go out in
// tile-major order; for causal masking the heaviest (last) query tiles first.
__device__ __forceinline__ void decode_block(int bid, int BH, int nq, bool causal,
                                             int& bh, int& qt) {
  int t;
  if ((BH & 7) == 0) {
    const int hx = BH >> 3, xcd = bid & 7, loc = bid >> 3;
    t = loc / hx;
    bh = xcd * hx + loc % hx;
  } else {
    t = bid / BH;
    bh = bid % BH;
  }
  qt = causal ? nq - 1 - t : t;
}

template <typename T, int D, int BC, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_mfma16(FwdParams p) {
  constexpr int NW = 4, BR = 32 * NW;
  constexpr int KSTR = D + 8;    // K row stride in elements (+16 B)
  constexpr int VSTR = D + 16;   // V row stride in elements (+32 B)
  constexpr int KT = BC * KSTR, VT = BC * VSTR;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int CPT = BC * CPR / 256;     // chunks per thread per tensor
  constexpr int NS = D / 16;              // MFMA k-steps of Q K^T
  constexpr int NKB = BC / 32;            // 32-key blocks per tile
  constexpr int ND = D / 32;              // 32-column blocks of O
  static_assert(BC * CPR % 256 == 0, "tile must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) short smem[2 * (KT + VT)];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  int bh, qt;
  decode_block(blockIdx.x, p.BH, p.nq, CAUSAL, bh, qt);

  const size_t head = (size_t)bh * N * D;
  const T* __restrict__ qh = (const T*)p.q + head;
  const T* __restrict__ kh = (const T*)p.k + head;
  const T* __restrict__ vh = (const T*)p.v + head;

  const int qrow0 = qt * BR + w * 32;  // first query row of this wave
  const int myq = qrow0 + ql;          // this lane's query

  // Q operand (B of S^T = K Q^T): lane holds Q[myq][16 s + 8 g .. +8].
  i32x4 qop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (myq < N) qop[s] = *(const i32x4*)(qh + (size_t)myq * D + 16 * s + 8 * g);
    else qop[s] = i32x4{0, 0, 0, 0};
  }

  const int kv_end = CAUSAL ? min(N, (qt + 1) * BR) : N;
  const int nt = (kv_end + BC - 1) / BC;

  i32x4 kreg[CPT], vreg[CPT];
  auto gload = [&](int j) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 256 * u, row = c / CPR, col = c % CPR;
      const int key = j * BC + row;
      if (key < N) {
        kreg[u] = *(const i32x4*)(kh + (size_t)key * D + col * 8);
        vreg[u] = *(const i32x4*)(vh + (size_t)key * D + col * 8);
      } else {
        kreg[u] = i32x4{0, 0, 0, 0};
        vreg[u] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto swrite = [&](int st) {
    short* sk = smem + st * (KT + VT);
    short* sv = sk + KT;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 256 * u, row = c / CPR, col = c % CPR;
      *(i32x4*)(sk + row * KSTR + col * 8) = kreg[u];
      *(i32x4*)(sv + row * VSTR + col * 8) = vreg[u];
    }
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m = kMInit, l = 0.f;
  const float c = p.scale_log2;
  const float cabs = fabsf(c);
  const bool neg = c < 0.f;

  // transposed-read geometry for the V operand (A of O^T = V^T P^T): in each
  // 16-lane group, lane i points at row (i/4) and column 4*(i%4) of a 4 x 16
  // block; the hardware returns to lane i the 4 values of column i.
  const int trow = (lane & 15) >> 2;
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int krow = swap_bits23(ql);

  gload(0);
  swrite(0);
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    const int st = j & 1;
    if (j + 1 < nt) gload(j + 1);
    const int key0 = j * BC;
    const bool active = !CAUSAL || key0 <= qrow0 + 31;
    if (active) {
      const short* sk = smem + st * (KT + VT);
      const short* sv = sk + KT;
      // ---- S^T = K_j Q^T ----
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
        const short* kr = sk + (kb * 32 + krow) * KSTR + 8 * g;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          sacc[kb] = Half<T>::mfma(*(const i32x4*)(kr + 16 * s), qop[s], sacc[kb]);
      }
      // ---- scale, mask, online softmax ----
      const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > qrow0);
      // key of accumulator (kb, r) on this lane: key0 + 32 kb + 16 (r/8) + 8 g + r%8
      float mx = kNegInf;
      if (need_mask) {
        const int lim = CAUSAL ? min(myq, N - 1) : N - 1;  // last visible key
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 16 * (r >> 3) + 8 * g + (r & 7);
            float x = neg ? -sacc[kb][r] : sacc[kb][r];
            mx = key <= lim ? fmaxf(mx, x) : mx;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, neg ? -sacc[kb][r] : sacc[kb][r]);
      }
      mx = wave_pair_max(mx);
      const float mt = (mx == kNegInf) ? kNegInf : mx * cabs;
      const float mnew = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      const float negm = -mnew;
      float rs = 0.f;
      if (need_mask) {
        const int lim = CAUSAL ? min(myq, N - 1) : N - 1;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 16 * (r >> 3) + 8 * g + (r & 7);
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, negm));
            pr = key <= lim ? pr : 0.f;
            sacc[kb][r] = pr;
            rs += pr;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, negm));
            sacc[kb][r] = pr;
            rs += pr;
          }
      }
      l = l * alpha + rs;
#pragma unroll
      for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
      // ---- O^T += V_j^T P^T ----
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          i32x4 pop;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pop[e] = (int)Half<T>::pack2(sacc[kb][8 * h + 2 * e], sacc[kb][8 * h + 2 * e + 1]);
          const int kbase = kb * 32 + 16 * h + 8 * g;
#pragma unroll
          for (int b = 0; b < ND; ++b) {
            const short* vp = sv + (kbase + trow) * VSTR + 32 * b + tcol;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 4 * VSTR));
            const i16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[b] = Half<T>::mfma(__builtin_bit_cast(i32x4, v8), pop, oacc[b]);
          }
        }
    }
    if (j + 1 < nt) swrite(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 (m + log2 l) ----
  const float lt = wave_pair_sum(l);
  if (myq < N) {
    const float inv = 1.0f / lt;
    T* orow = (T*)p.o + head + (size_t)myq * D;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        // registers 4a..4a+3 hold columns 32 b + 8 a + 4 g + 0..3
        uint2 st;
        st.x = Half<T>::pack2(oacc[b][4 * a] * inv, oacc[b][4 * a + 1] * inv);
        st.y = Half<T>::pack2(oacc[b][4 * a + 2] * inv, oacc[b][4 * a + 3] * inv);
        *(uint2*)(orow + 32 * b + 8 * a + 4 * g) = st;
      }
    if (g == 0)
      p.lse[(size_t)bh * N + myq] = (m + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
  }
}

template <typename T, int D, int BC, bool CAUSAL>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  constexpr int BR = 128;
  FwdParams q = p;
  q.nq = (p.N + BR - 1) / BR;
  const unsigned grid = (unsigned)(q.nq * p.BH);
  hipLaunchKernelGGL((fwd_mfma16<T, D, BC, CAUSAL>), dim3(grid), dim3(256), 0, stream, q);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(const FwdParams& p, int d, int causal, hipStream_t s) {
  switch (d) {
    case 64:  return causal ? launch_one<T, 64, 64, true>(p, s) : launch_one<T, 64, 64, false>(p, s);
    case 128: return causal ? launch_one<T, 128, 64, true>(p, s) : launch_one<T, 128, 64, false>(p, s);
    case 256: return causal ? launch_one<T, 256, 32, true>(p, s) : launch_one<T, 256, 32, false>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_half(const FwdParams& p, int d, int causal, int is_bf16, hipStream_t s) {
  return is_bf16 ? launch_t<__bf16>(p, d, causal, s) : launch_t<_Float16>(p, d, causal, s);
}

}  // namespace fa
