// Attention backward pass for gfx950 (MI355X), fp16/bf16 inputs.
//
// The pages print the forward formula only ("FlashAttention (HI)" / "(TL)",
// section on the problems of standard attention) and report training
// speed-ups that need its gradient.  Differentiating O = softmax(S) V,
// S = scale Q K^T, for an upstream gradient dO gives, per (batch, head) and
// with P recomputed from the forward's logsumexp (P_ij = exp(S_ij - lse_i),
// zero for hidden keys):
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = dO_i . O_i,
//     dQ = scale dS K,  dK = scale dS^T Q.
// As in the forward, no N x N matrix reaches HBM: scores are recomputed tile
// by tile on chip ("FlashAttention (HI)", tiling section: inputs split into
// tiles that fit on-chip memory and streamed through it).
//
// Two kernels, launched in this order on one stream; neither uses atomics,
// so results are the same run to run:
//   bwd_dq    one workgroup per 128 query rows of a head (32 rows per wave).
//             Q and dO rows sit in registers as MFMA B operands; K and V
//             tiles stream through an LDS ring (global_load_lds_dwordx4).
//             Per tile: S^T = K Q^T and dP^T = V dO^T (one query per lane,
//             like the forward), dS^T in registers, dQ^T += K^T dS^T with K
//             read transposed from LDS.  Its prologue computes D_i from O
//             and dO and writes D and the base-2 logsumexp into the
//             workspace for the second kernel.
//   bwd_dkdv  one workgroup per 128 keys of a K/V head (32 keys per wave),
//             looping over every query head that shares that K/V head, so
//             a shared head's gradients are summed in registers.  K and V
//             rows sit in registers; Q, dO and the row statistics stream
//             through LDS.  Per tile: S = Q K^T and dP = dO V^T (one key per
//             lane), dV^T += dO^T P and dK^T += Q^T dS with Q and dO read
//             transposed from LDS.
// The MFMA is v_mfma_f32_32x32x16_{bf16,f16}; P and dS are rounded to the
// input type for the second products, accumulation is fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kBwdNW = 4;  // waves per workgroup (32 rows or keys each)

// BC: key rows per bwd_dq tile; BQ: query rows per bwd_dkdv tile; OCC: waves
// per SIMD the register budget of each kernel is cut to; ST_*: LDS ring
// stages of each kernel (tiles are prefetched ST - 1 ahead).  At d = 128,
// bwd_dq streams 64-key tiles through a 2-stage ring (the same 64 KiB of LDS
// as 32-key tiles in 4 stages, which had been 5-7% faster while the loop ran
// over a run-time ring stage; with the loops unrolled over the stages the
// 64-key tiles are 2% faster without masking, equal with it); bwd_dkdv takes
// 32-query tiles with V in LDS at two waves per SIMD (see bwd_dkdv).  At
// d = 64 bwd_dq fits three waves per SIMD (138 registers): up to 10% over two
// (bwd_dkdv at three, with 32-query tiles, did not add to it).  The FA_BWD_*
// macros exist for tuning builds only.
#ifndef FA_BWD_D64_BC
#define FA_BWD_D64_BC 64
#endif
#ifndef FA_BWD_D64_BQ
#define FA_BWD_D64_BQ 64
#endif
#ifndef FA_BWD_D128_BC
#define FA_BWD_D128_BC 64
#endif
#ifndef FA_BWD_D128_BQ
#define FA_BWD_D128_BQ 32
#endif
#ifndef FA_BWD_D64_STDQ
#define FA_BWD_D64_STDQ 2
#endif
#ifndef FA_BWD_D64_STKV
#define FA_BWD_D64_STKV 2
#endif
#ifndef FA_BWD_D128_STDQ
#define FA_BWD_D128_STDQ 2
#endif
#ifndef FA_BWD_D128_STKV
#define FA_BWD_D128_STKV 2
#endif
template <int D> struct BwdCfg;
template <> struct BwdCfg<64> {
  static constexpr int BC = FA_BWD_D64_BC, BQ = FA_BWD_D64_BQ, OCC_DQ = 3, OCC_KV = 2;
  static constexpr int ST_DQ = FA_BWD_D64_STDQ, ST_KV = FA_BWD_D64_STKV;
};
template <> struct BwdCfg<128> {
  static constexpr int BC = FA_BWD_D128_BC, BQ = FA_BWD_D128_BQ, OCC_DQ = 2, OCC_KV = 2;
  static constexpr int ST_DQ = FA_BWD_D128_STDQ, ST_KV = FA_BWD_D128_STKV;
};
template <> struct BwdCfg<256> {
  static constexpr int BC = 32, BQ = 32, OCC_DQ = 1, OCC_KV = 1, ST_DQ = 2, ST_KV = 2;
};

// Per-lane LDS read geometry for tiles of 32-row blocks with D columns,
// unpadded, 16-byte chunks XOR-swizzled by chunk_swz<D>.
template <int D> struct Geom {
  int roff, ry;            // row operand: row swap_bits23(lane%32), chunk (2s+g)^swz
  int toff[2], tx[2];      // transposed operand (ds_read_b64_tr_b16)
  __device__ __forceinline__ explicit Geom(int lane) {
    const int ql = lane & 31, g = lane >> 5;
    const int r = swap_bits23(ql);
    roff = r * 2 * D;
    ry = g ^ chunk_swz<D>(r);
    // In each 16-lane group, lane i addresses row i/4 and columns 4 (i%4) of a
    // 4 x 16 block; the hardware hands lane i the 4 values of column i.  Rows
    // 8 g + 4 t + 0..3 of a 16-row half block, columns 32 b + lane % 32.
    const int trow = (lane & 15) >> 2;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rr = 8 * g + 4 * t + trow;
      toff[t] = rr * 2 * D + 8 * (lane & 1);
      tx[t] = (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ chunk_swz<D>(rr);
    }
  }
};

// C[32 x 32] = A B^T over D: A = 32 rows of an LDS tile block (row i of the
// MFMA reads tile row swap_bits23(i)), B = 32 rows held in registers (lane
// l: row l%32, columns 16 s + 8 g .. +8).  Register r of half-wave g of the
// result is tile row 16 (r/8) + 8 g + r%8, column l%32.
template <typename T, int D, bool PIN>
__device__ __forceinline__ f32x16 mm_rows(const char* blk, const Geom<D>& G,
                                          const i32x4 (&b)[D / 16]) {
  // Operands are read PF steps ahead of their MFMA: enough to cover LDS
  // latency, few enough that two of these in flight do not crowd out the
  // accumulators at d = 256.  With PIN, scheduling barriers keep the reads
  // ahead (left alone, the compiler may move each read next to its MFMA and
  // wait for it there); without, the register allocator has the last word
  // (bwd_dkdv at d = 128 and 256 spills with the barriers).
  constexpr int NS = D / 16, PF = NS < 4 ? NS : 4;
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = 0.f;
  i32x4 a[NS];
#pragma unroll
  for (int s = 0; s < PF; ++s) a[s] = *(const i32x4*)(blk + G.roff + (((2 * s) ^ G.ry) << 4));
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s + PF < NS) a[s + PF] = *(const i32x4*)(blk + G.roff + (((2 * (s + PF)) ^ G.ry) << 4));
    if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
    c = Half<T>::mfma(a[s], b[s], c);
  }
  return c;
}

// mm_rows with B read from LDS as well: row boff of a tile (lane l%32's
// row), chunk (2 s + g) ^ by.
template <typename T, int D, bool PIN>
__device__ __forceinline__ f32x16 mm_rows_lds(const char* blk, const Geom<D>& G, const char* bt,
                                              int boff, int by) {
  constexpr int NS = D / 16;
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = 0.f;
  // operands of step s + 1 are read before the MFMA of step s
  auto rd = [&](int s, i32x4& a, i32x4& b) __attribute__((always_inline)) {
    a = *(const i32x4*)(blk + G.roff + (((2 * s) ^ G.ry) << 4));
    b = *(const i32x4*)(bt + boff + (((2 * s) ^ by) << 4));
  };
  i32x4 a0, b0, a1, b1;
  rd(0, a0, b0);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s + 1 < NS) rd(s + 1, a1, b1);
    if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
    c = Half<T>::mfma(a0, b0, c);
    a0 = a1;
    b0 = b1;
  }
  return c;
}

// acc[b] += A_b X over the 32 rows of an LDS tile block: A_b = columns
// 32 b .. +32 of the block, transposed (MFMA row = tile column); X = the
// 32 x 32 result of mm_rows (its row index runs over the block's rows),
// rounded to T.  Register r of the result is column 32 b + 8 (r/4) + 4 g +
// r%4 of the tile, lane l%32 is X's column.
template <typename T, int D>
__device__ __forceinline__ void mm_tr(const char* blk, const Geom<D>& G, const f32x16& x,
                                      f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    i32x4 xop;
#pragma unroll
    for (int e = 0; e < 4; ++e) xop[e] = (int)Half<T>::pack2(x[8 * h + 2 * e], x[8 * h + 2 * e + 1]);
    const char* hb = blk + 16 * h * 2 * D;
    // transposed reads issued TPF column blocks ahead of their MFMA
    constexpr int NB = D / 32, TPF = NB < 4 ? NB : 4;
    i16x4 lo[NB], hi[NB];
    auto rd = [&](int b) __attribute__((always_inline)) {
      lo[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(hb + G.toff[0] + (((4 * b) ^ G.tx[0]) << 4)));
      hi[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(hb + G.toff[1] + (((4 * b) ^ G.tx[1]) << 4)));
    };
#pragma unroll
    for (int b = 0; b < TPF; ++b) rd(b);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + TPF < NB) rd(b + TPF);
      const i16x8 a8 = {lo[b][0], lo[b][1], lo[b][2], lo[b][3], hi[b][0], hi[b][1], hi[b][2], hi[b][3]};
      acc[b] = Half<T>::mfma(__builtin_bit_cast(i32x4, a8), xop, acc[b]);
    }
  }
}

// Store a D-column row from accumulators laid out as mm_tr leaves them
// (lane = row, register r of block b = column 32 b + 8 (r/4) + 4 g + r%4),
// times f.
template <typename T, int D>
__device__ __forceinline__ void store_row(T* row, const f32x16 (&acc)[D / 32], float f, int g) {
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint2 v;
      v.x = Half<T>::pack2(acc[b][4 * a] * f, acc[b][4 * a + 1] * f);
      v.y = Half<T>::pack2(acc[b][4 * a + 2] * f, acc[b][4 * a + 3] * f);
      *(uint2*)(row + 32 * b + 8 * a + 4 * g) = v;
    }
}

__device__ __forceinline__ float lo16(int x, bool bf) {
  const unsigned short h = (unsigned short)(x & 0xffff);
  return bf ? __builtin_bit_cast(float, (unsigned)h << 16) : (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float hi16(int x, bool bf) {
  const unsigned short h = (unsigned short)((unsigned)x >> 16);
  return bf ? __builtin_bit_cast(float, (unsigned)h << 16) : (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------------------
// dQ (and the row statistics for bwd_dkdv)
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kBwdNW) __attribute__((amdgpu_waves_per_eu(BwdCfg<D>::OCC_DQ, BwdCfg<D>::OCC_DQ)))
void bwd_dq(BwdParams p) {
  constexpr int NW = kBwdNW, BR = 32 * NW, BC = BwdCfg<D>::BC, ST = BwdCfg<D>::ST_DQ;
  constexpr int RB = 2 * D, TB = BC * RB, CPR = D / 8, CPT = BC * CPR / (64 * NW);
  constexpr int NS = D / 16, NKB = BC / 32, ND = D / 32;
  constexpr bool BF = __is_same(T, __bf16);
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char smem[ST * 2 * TB];  // [stage][K, V]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  int bh, qt;
  // causal: the first passes over an XCD's CUs alternate direction (workgroups per CU)
  decode_block(blockIdx.x, p.BH, p.nq, CAUSAL, bh, qt, BwdCfg<D>::OCC_DQ * 4 / kBwdNW);
  const size_t head = (size_t)bh * N * D;
  const size_t kvhead = (size_t)kv_head_of(p.H, p.Hkv, bh) * N * D;
  const T* __restrict__ kh = (const T*)p.k + kvhead;
  const T* __restrict__ vh = (const T*)p.v + kvhead;

  const int qrow0 = qt * BR + w * 32;
  const int myq = qrow0 + ql;
  const int rq = min(myq, N - 1);

  // B operands: Q and dO rows of this lane's query; D_i = dO_i . O_i from
  // this lane's half of the columns plus the other half-wave's.
  i32x4 qop[NS], dop[NS];
  float dl = 0.f;
  {
    const size_t ro = head + (size_t)rq * D + 8 * g;
    const T* qr = (const T*)p.q + ro;
    const T* dr = (const T*)p.dout + ro;
    const T* orow = (const T*)p.o + ro;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qop[s] = *(const i32x4*)(qr + 16 * s);
      dop[s] = *(const i32x4*)(dr + 16 * s);
      const i32x4 ov = *(const i32x4*)(orow + 16 * s);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dl += lo16(dop[s][e], BF) * lo16(ov[e], BF) + hi16(dop[s][e], BF) * hi16(ov[e], BF);
    }
  }
  dl = pair_sum(dl);
  const float lse2 = p.lse[(size_t)bh * N + rq] * 1.44269504088896340736f;  // log2(e)
  if (g == 0) {  // rows N .. Npad-1: P = 2^-inf = 0 and D = 0 in bwd_dkdv
    p.ws_lse2[(size_t)bh * p.Npad + myq] = myq < N ? lse2 : __builtin_huge_valf();
    p.ws_delta[(size_t)bh * p.Npad + myq] = myq < N ? dl : 0.f;
  }
  // Drain this wave's own loads and stores: the tile copies below are counted
  // on the same vmcnt and the waits in the loop count only those.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  landed(qop);
  landed(dop);

  const int kv_end = CAUSAL ? min(N, (qt + 1) * BR) : N;
  const int nt = (kv_end + BC - 1) / BC;
  const int jlast = qrow0 >= N ? -1 : CAUSAL ? min(nt - 1, (qrow0 + 31) / BC) : nt - 1;

  // Tile copies through per-tile buffer resources that end with the head:
  // key rows past N read as zeros (their scores are masked, and zero K rows
  // add nothing to dQ), and a copy's address is a constant per-lane offset.
  uint32_t ld_voff[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int s = (u * NW + w) * 64 + lane, row = s / CPR, c = s % CPR;
    ld_voff[u] = (uint32_t)(row * RB + (c ^ chunk_swz<D>(row)) * 16);
  }

  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto issue_tile = [&](int j, int stage) __attribute__((always_inline)) {
    const uint32_t dst = smem_base + stage * 2 * TB;
    const uint32_t t0 = (uint32_t)j * TB;
    const __amdgpu_buffer_rsrc_t kbuf = tile_rsrc(kh, (uint32_t)N * RB, t0);
    const __amdgpu_buffer_rsrc_t vbuf = tile_rsrc(vh, (uint32_t)N * RB, t0);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const uint32_t lo = dst + (u * NW + w) * 1024;
      buf_dma16(kbuf, ld_voff[u], lo);
      buf_dma16(vbuf, ld_voff[u], lo + TB);
    }
  };

  const Geom<D> G(lane);
  f32x16 acc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  const float c = p.scale_log2;

  // Ring of ST stages, prefetch distance PD = ST - 1: iteration j copies
  // tile j + PD into the stage tile j - 1 used (everyone finished it before
  // the last barrier) and ends once tile j + 1 has landed.  Copies complete
  // in order, PT per tile and wave, so that is vmcnt <= PT * (tiles issued
  // after j + 1).
  constexpr int PD = ST - 1, PT = 2 * CPT;
  static_assert(PT * (PD - 1) <= 31, "pending copies must fit wait_vmcnt");
  for (int t = 0; t < PD && t < nt; ++t) issue_tile(t, t);
  wait_vmcnt(PT * (min(PD, nt) - 1));
  __syncthreads();
  // One tile; with a compile-time ring stage SG (the loop below is unrolled
  // over the stages) every LDS read is a register plus an immediate offset.
  auto step = [&](int j, auto SG) __attribute__((always_inline)) {
    const int sg = (int)SG;
    if (j + PD < nt) issue_tile(j + PD, (sg + PD) % ST);
    if (j <= jlast) {
      const char* sk = smem + sg * 2 * TB;
      const char* sv = sk + TB;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f32x16 s = mm_rows<T, D, true>(sk + kb * 32 * RB, G, qop);
        const f32x16 dp = mm_rows<T, D, true>(sv + kb * 32 * RB, G, dop);
        // register r holds key key0 + 16 (r/8) + r%8
        const int key0 = j * BC + kb * 32 + 8 * g;
        // visible iff 16 (r/8) + r%8 <= rel.  Only blocks that reach past N
        // or (causal) past the wave's first row hide keys; the test is
        // wave-uniform, so other blocks skip the selects.
        const int rel = (CAUSAL ? min(myq, N - 1) : N - 1) - key0;
        const bool hides = j * BC + kb * 32 + 31 > (CAUSAL ? min(qrow0, N - 1) : N - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(s[r], c, -lse2);
        if (hides) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = (16 * (r >> 3) + (r & 7) <= rel) ? s[r] : kNegInf;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(s[r]) * (dp[r] - dl);
        mm_tr<T, D>(sk + kb * 32 * RB, G, s, acc);
      }
    }
    wait_vmcnt(PT * max(0, min(j + PD, nt - 1) - (j + 1)));
    __syncthreads();
  };
#ifndef FA_BWD_DQ_UNROLL
#define FA_BWD_DQ_UNROLL 1
#endif
  if constexpr (FA_BWD_DQ_UNROLL && D <= 128) {
    static_assert(ST >= 2 && ST <= 4, "the unrolled loop covers rings of 2 to 4 stages");
    for (int j = 0; j < nt; j += ST) {
      step(j, std::integral_constant<int, 0>());
      if (j + 1 >= nt) break;
      step(j + 1, std::integral_constant<int, 1>());
      if constexpr (ST > 2) {
        if (j + 2 >= nt) break;
        step(j + 2, std::integral_constant<int, 2 % ST>());
        if constexpr (ST > 3) {
          if (j + 3 >= nt) break;
          step(j + 3, std::integral_constant<int, 3 % ST>());
        }
      }
    }
  } else {
    for (int j = 0; j < nt; ++j) step(j, j % ST);
  }
  if (myq < N) store_row<T, D>((T*)p.dq + head + (size_t)myq * D, acc, p.scale, g);
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kBwdNW) __attribute__((amdgpu_waves_per_eu(BwdCfg<D>::OCC_KV, BwdCfg<D>::OCC_KV)))
void bwd_dkdv(BwdParams p) {
  constexpr int NW = kBwdNW, BK = 32 * NW, BQ = BwdCfg<D>::BQ, ST = BwdCfg<D>::ST_KV;
  constexpr int RB = 2 * D, TB = BQ * RB, CPR = D / 8, CPT = BQ * CPR / (64 * NW);
  constexpr int NS = D / 16, NQB = BQ / 32, ND = D / 32;
  constexpr int SB = 2 * BQ * 4;          // row statistics per tile: base-2 lse, then D
  constexpr int STB = 2 * TB + SB;        // bytes per stage: Q, dO, statistics
  constexpr int SL = SB / 16 / NW;        // statistics chunks per wave
  static_assert(BQ * CPR % (64 * NW) == 0 && SB % (16 * NW) == 0 && SL <= 64, "tile split");
  // At d = 128 and 256 V's rows live in LDS (read as B operands) instead of
  // registers: at d = 256 the accumulators alone take 256 registers per lane;
  // at d = 128 it brings the kernel (with 32-query tiles) from 348 registers,
  // one wave per SIMD, to 253, two waves per SIMD: 15-23% faster.
  constexpr bool VLDS = D >= 128;
  constexpr int VB = VLDS ? BK * RB : 0;
  __shared__ __attribute__((aligned(1024))) char smem[ST * STB + VB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  const int BHkv = p.BH / (p.H / p.Hkv), grp = p.H / p.Hkv;
  int kvbh, t;
  decode_block(blockIdx.x, BHkv, p.nq, CAUSAL, kvbh, t, BwdCfg<D>::OCC_KV * 4 / kBwdNW);
  const int kblk = CAUSAL ? p.nq - 1 - t : t;  // causal: low key blocks (most work) first
  const int b = kvbh / p.Hkv, gk = kvbh % p.Hkv;
  const int qh0 = b * p.H + gk * grp;          // first query head of the group
  const size_t kvhead = (size_t)kvbh * N * D;

  const int k0 = kblk * BK + w * 32;
  const int mykey = k0 + ql;
  i32x4 kop[NS], vop[VLDS ? 1 : NS];
  {
    const size_t ro = kvhead + (size_t)min(mykey, N - 1) * D + 8 * g;
    const T* kr = (const T*)p.k + ro;
    const T* vr = (const T*)p.v + ro;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kop[s] = *(const i32x4*)(kr + 16 * s);
      if constexpr (!VLDS) vop[s] = *(const i32x4*)(vr + 16 * s);
    }
  }
  const char* vlds = smem + ST * STB;  // VLDS: the block's BK rows of V, chunk-swizzled
  const int vboff = (w * 32 + ql) * RB, vby = g ^ chunk_swz<D>(ql);
  if constexpr (VLDS) {
    constexpr int CPV = BK * CPR / (64 * NW);
    const uint32_t vdst = (uint32_t)(uintptr_t)(lds_void*)vlds;
    const T* vb = (const T*)p.v + kvhead;
#pragma unroll
    for (int u = 0; u < CPV; ++u) {
      const int sl = (u * NW + w) * 64 + lane, row = sl / CPR, cc = sl % CPR;
      const size_t r = (size_t)min(kblk * BK + row, N - 1);
      dma16(vb + r * D + (cc ^ chunk_swz<D>(row)) * 8, vdst + (u * NW + w) * 1024);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  landed(kop);
  if constexpr (!VLDS) landed(vop);

  const int nqt = (N + BQ - 1) / BQ;
  const int qs = CAUSAL ? (kblk * BK) / BQ : 0;  // first query tile that sees a key of the block
  const int cnt = nqt - qs;
  const int ntile = grp * cnt;

  // Q and dO tiles through per-tile buffer resources that end with the query
  // head: rows past N read as zeros (their base-2 lse is +inf, so P = 0
  // there).
  uint32_t ld_voff[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int s = (u * NW + w) * 64 + lane, row = s / CPR, cc = s % CPR;
    ld_voff[u] = (uint32_t)(row * RB + (cc ^ chunk_swz<D>(row)) * 16);
  }
  // statistics chunk of this lane (lanes < SL): chunk w SL + lane of
  // [lse2 (BQ floats), D (BQ floats)]
  const int sci = w * SL + lane;
  const int s_arr = sci / (BQ / 4), s_off = (sci % (BQ / 4)) * 4;
  const float* s_src = (s_arr == 0 ? p.ws_lse2 : p.ws_delta) + s_off;
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto issue_tile = [&](int j, int stage) __attribute__((always_inline)) {
    const int hh = j / cnt, qt = qs + j % cnt;
    const int bhq = qh0 + hh;
    const size_t hq = (size_t)bhq * N * D;
    const __amdgpu_buffer_rsrc_t qbuf = tile_rsrc((const T*)p.q + hq, (uint32_t)N * RB, (uint32_t)qt * TB);
    const __amdgpu_buffer_rsrc_t dbuf = tile_rsrc((const T*)p.dout + hq, (uint32_t)N * RB, (uint32_t)qt * TB);
    const uint32_t dst = smem_base + stage * STB;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const uint32_t lo = dst + (u * NW + w) * 1024;
      buf_dma16(qbuf, ld_voff[u], lo);
      buf_dma16(dbuf, ld_voff[u], lo + TB);
    }
    if (lane < SL) dma16(s_src + (size_t)bhq * p.Npad + qt * BQ, dst + 2 * TB + w * SL * 16);
  };

  const Geom<D> G(lane);
  f32x16 acck[ND], accv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acck[d][r] = accv[d][r] = 0.f;
  const float c = p.scale_log2;

  // Ring as in bwd_dq; PT copies per tile and wave (the statistics chunk
  // is one more instruction in every wave).
  constexpr int PD = ST - 1, PT = 2 * CPT + 1;
  static_assert(PT * (PD - 1) <= 31, "pending copies must fit wait_vmcnt");
  for (int t = 0; t < PD && t < ntile; ++t) issue_tile(t, t);
  wait_vmcnt(PT * (min(PD, ntile) - 1));
  __syncthreads();
  // One tile; the ring stage SG is a compile-time constant (the loop below is
  // unrolled over the stages), so every LDS read is a register plus an
  // immediate offset.
  // DIAG: the causal selects run only on blocks that cross the diagonal (a
  // wave-uniform branch).  At d = 128 that branch pushes the causal kernel,
  // already at 256 registers, into spills inside the loop, so there every
  // block takes the selects.
  constexpr bool DIAG = D != 128;
  // Operand reads held ahead of their MFMAs by scheduling barriers (at
  // d = 128 and 256 the barriers cost this kernel spills).
  constexpr bool PIN = D == 64;
  auto step = [&](int j, auto SG) __attribute__((always_inline)) {
    const int sg = (int)SG;
    if (j + PD < ntile) issue_tile(j + PD, (sg + PD) % ST);
    const int q0 = (qs + j % cnt) * BQ;
    // Causal: skip a tile whose every query precedes every key of this wave
    // (the mask would zero it).  Not at d = 256, where the branch around the
    // accumulators costs the register allocator ~100 spilled registers; the
    // masked tiles are computed and contribute zero there.
    constexpr bool SKIP = CAUSAL && D != 256;
    if (!SKIP || q0 + BQ - 1 >= k0) {
      const char* sq = smem + sg * STB;
      const char* sd = sq + TB;
      const float* sst = (const float*)(sq + 2 * TB);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        f32x16 s = mm_rows<T, D, PIN>(sq + qb * 32 * RB, G, kop);
        f32x16 dp;
        if constexpr (VLDS) dp = mm_rows_lds<T, D, PIN>(sd + qb * 32 * RB, G, vlds, vboff, vby);
        else dp = mm_rows<T, D, PIN>(sd + qb * 32 * RB, G, vop);
        // register r holds query q0 + 32 qb + 16 (r/8) + 8 g + r%8
        float l2[16], dd[16];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float4* a = (const float4*)(sst + 32 * qb + 16 * hh + 8 * g);
          const float4* bq = (const float4*)(sst + BQ + 32 * qb + 16 * hh + 8 * g);
          const float4 a0 = a[0], a1 = a[1], b0 = bq[0], b1 = bq[1];
          l2[8 * hh + 0] = a0.x; l2[8 * hh + 1] = a0.y; l2[8 * hh + 2] = a0.z; l2[8 * hh + 3] = a0.w;
          l2[8 * hh + 4] = a1.x; l2[8 * hh + 5] = a1.y; l2[8 * hh + 6] = a1.z; l2[8 * hh + 7] = a1.w;
          dd[8 * hh + 0] = b0.x; dd[8 * hh + 1] = b0.y; dd[8 * hh + 2] = b0.z; dd[8 * hh + 3] = b0.w;
          dd[8 * hh + 4] = b1.x; dd[8 * hh + 5] = b1.y; dd[8 * hh + 6] = b1.z; dd[8 * hh + 7] = b1.w;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(s[r], c, -l2[r]);
        // Causal: only a block some of whose queries precede some key of the
        // wave hides pairs (query < key); the test is wave-uniform, so every
        // other block skips the selects.  Visible iff 16 (r/8) + r%8 >= lo.
        if (CAUSAL && (!DIAG || q0 + 32 * qb < k0 + 31)) {
          const int lo = mykey - (q0 + 32 * qb + 8 * g);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = (16 * (r >> 3) + (r & 7) >= lo) ? s[r] : kNegInf;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(s[r]);
          s[r] = pr;
          dp[r] = pr * (dp[r] - dd[r]);
        }
        mm_tr<T, D>(sd + qb * 32 * RB, G, s, accv);
        mm_tr<T, D>(sq + qb * 32 * RB, G, dp, acck);
      }
    }
    wait_vmcnt(PT * max(0, min(j + PD, ntile - 1) - (j + 1)));
    __syncthreads();
  };
#ifndef FA_BWD_KV_UNROLL
#define FA_BWD_KV_UNROLL 1
#endif
#ifndef FA_BWD_KV_UNROLL_CAUSAL
#define FA_BWD_KV_UNROLL_CAUSAL 1
#endif
  constexpr bool UNROLL = D <= 128 && ST == 2 && (CAUSAL ? FA_BWD_KV_UNROLL_CAUSAL : FA_BWD_KV_UNROLL);
  if constexpr (UNROLL) {
    for (int j = 0; j < ntile; j += 2) {
      step(j, std::integral_constant<int, 0>());
      if (j + 1 < ntile) step(j + 1, std::integral_constant<int, 1>());
    }
  } else {
    for (int j = 0; j < ntile; ++j) step(j, j % ST);
  }
  if (mykey < N) {
    store_row<T, D>((T*)p.dk + kvhead + (size_t)mykey * D, acck, p.scale, g);
    store_row<T, D>((T*)p.dv + kvhead + (size_t)mykey * D, accv, 1.0f, g);
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
  constexpr int BR = 32 * kBwdNW;
  BwdParams a = p;
  a.nq = p.Npad / BR;  // bwd_dq covers every workspace row
  hipLaunchKernelGGL((bwd_dq<T, D, CAUSAL>), dim3((unsigned)(a.nq * p.BH)), dim3(64 * kBwdNW), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int BHkv = p.BH / (p.H / p.Hkv);
  BwdParams b = p;
  b.nq = (p.N + BR - 1) / BR;  // key blocks per K/V head
  hipLaunchKernelGGL((bwd_dkdv<T, D, CAUSAL>), dim3((unsigned)(b.nq * BHkv)), dim3(64 * kBwdNW), 0, s, b);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_d(const BwdParams& p, int d, int causal, hipStream_t s) {
  switch (d) {
    case 64:  return causal ? launch_bwd_t<T, 64, true>(p, s) : launch_bwd_t<T, 64, false>(p, s);
    case 128: return causal ? launch_bwd_t<T, 128, true>(p, s) : launch_bwd_t<T, 128, false>(p, s);
    case 256: return causal ? launch_bwd_t<T, 256, true>(p, s) : launch_bwd_t<T, 256, false>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_half(const BwdParams& p, int d, int causal, int is_bf16, hipStream_t s) {
  return is_bf16 ? launch_bwd_d<__bf16>(p, d, causal, s) : launch_bwd_d<_Float16>(p, d, causal, s);
}

}  // namespace fa
