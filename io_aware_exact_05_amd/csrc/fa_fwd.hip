// Fused exact attention forward for gfx950 (MI355X), fp16/bf16 inputs.
//
// One workgroup owns BR = 32 NW query rows of one (batch, head): NW wave64s
// (8 at d = 128, 4 at d = 64 and 256), each holding 32 rows for the whole
// pass.  The key/value sequence streams through LDS in tiles of BC rows, in a
// ring of ST stages: later tiles' loads go straight from HBM/L2 into free
// stages (global_load_lds_dwordx4, no staging registers) while the current
// tile is consumed, with one barrier per tile ("FlashAttention (HI)", tiling
// section: inputs split into tiles that fit on-chip memory, loaded in turn,
// the final result updated; "FlashAttention-3 (BN)", memory-operations
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
//                   m is only moved when a tile's max exceeds it by more than
//                   2^8, so most tiles skip the O rescale; exp2(s - m) <= 256
//                   then, and the result is the same softmax.
//   O^T += V_j^T P^T  P stays in registers: the S^T accumulator layout is
//                   exactly the B-operand layout of this MFMA once the key
//                   order inside each 32-key block is permuted (bits 2 and 3 of
//                   the row index swapped when K is read); V is read from LDS
//                   already transposed with ds_read_b64_tr_b16.
// LDS tiles are unpadded, 16-byte chunks XOR-swizzled per row so that both
// the K operand reads (16 rows, one chunk column) and the transposed V reads
// (4 rows x 4 chunks per half-wave) spread over all banks.
// The epilogue divides by l once per row and writes O and the logsumexp once
// ("FlashAttention (HI)", one-kernel section: only the final result is
// written).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// Key-tile rows BC and waves per SIMD (occupancy the register budget is cut
// to) per head dimension.  The FA_D*_BC / FA_D*_OCC macros exist for tuning
// builds only.
#ifndef FA_D64_BC
#define FA_D64_BC 128
#endif
#ifndef FA_D64_OCC
#define FA_D64_OCC 2
#endif
#ifndef FA_D128_BC
#define FA_D128_BC 64
#endif
#ifndef FA_D128_OCC
#define FA_D128_OCC 2
#endif
#ifndef FA_D256_BC
#define FA_D256_BC 32
#endif
#ifndef FA_D256_OCC
#define FA_D256_OCC 1
#endif
// Which head dimensions run fwd_wide (fa_fwd_wide.hip) instead of the kernel
// below (see use_wide for the causal case).
#ifndef FA_D64_WIDE
#define FA_D64_WIDE 1
#endif
#ifndef FA_D128_WIDE
#define FA_D128_WIDE 1
#endif
#ifndef FA_D256_WIDE
#define FA_D256_WIDE 1
#endif
#ifndef FA_D64_NW
#define FA_D64_NW 4
#endif
#ifndef FA_D128_NW
#define FA_D128_NW 8
#endif
#ifndef FA_D256_NW
#define FA_D256_NW 4
#endif
#ifndef FA_D64_ST
#define FA_D64_ST 2
#endif
#ifndef FA_D128_ST
#define FA_D128_ST 4
#endif
#ifndef FA_D256_ST
#define FA_D256_ST 4
#endif
// BC: key rows per tile; OCC: waves per SIMD the registers are budgeted
// for; NW: waves per workgroup (32 query rows each); ST: LDS ring stages.
// With two waves of the workgroup on each SIMD (NW = 8, OCC = 2) the upper
// half of the workgroup runs half a tile behind the lower half ("ping-pong",
// see the loop) and the ring prefetches ST - 2 tiles ahead, else ST - 1.
template <int D> struct TileCfg;
template <> struct TileCfg<64> {
  static constexpr int BC = FA_D64_BC, OCC = FA_D64_OCC, NW = FA_D64_NW, ST = FA_D64_ST;
};
template <> struct TileCfg<128> {
  static constexpr int BC = FA_D128_BC, OCC = FA_D128_OCC, NW = FA_D128_NW, ST = FA_D128_ST;
};
template <> struct TileCfg<256> {
  static constexpr int BC = FA_D256_BC, OCC = FA_D256_OCC, NW = FA_D256_NW, ST = FA_D256_ST;
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * TileCfg<D>::NW) __attribute__((amdgpu_waves_per_eu(TileCfg<D>::OCC, TileCfg<D>::OCC)))
void fwd_mfma16(FwdParams p) {
  constexpr int BC = TileCfg<D>::BC;
  constexpr int NW = TileCfg<D>::NW, BR = 32 * NW, ST = TileCfg<D>::ST;
  constexpr int RB = D * 2;                 // bytes per K/V row
  constexpr int TB = BC * RB;               // bytes per K or V tile
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int CPT = BC * CPR / (64 * NW); // load instructions per wave per tensor
  constexpr int NS = D / 16;                // MFMA k-steps of Q K^T
  constexpr int NKB = BC / 32;              // 32-key blocks per tile
  constexpr int ND = D / 32;                // 32-column blocks of O
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
  constexpr bool PINGPONG = TileCfg<D>::OCC >= 2 && NW == 8;
  constexpr int PD = PINGPONG ? ST - 2 : ST - 1;  // prefetch distance in tiles
  static_assert(PD >= 1, "the ring is too short");
  static_assert(2 * CPT * (PD - 1) <= 31, "pending copies must fit wait_vmcnt");
  __shared__ __attribute__((aligned(1024))) char smem[ST * 2 * TB];  // [stage][K,V]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  int bh, qt;
  decode_block(blockIdx.x, p.BH, p.nq, CAUSAL, bh, qt);

  const size_t head = (size_t)bh * N * D;
  const T* __restrict__ qh = (const T*)p.q + head;
  const size_t kvhead = (size_t)kv_head(p, bh) * N * D;  // K/V head shared by a group of query heads
  const T* __restrict__ kh = (const T*)p.k + kvhead;
  const T* __restrict__ vh = (const T*)p.v + kvhead;

  const int qrow0 = qt * BR + w * 32;  // first query row of this wave
  const int myq = qrow0 + ql;          // this lane's query

  // Q operand (B of S^T = K Q^T): lane holds Q[myq][16 s + 8 g .. +8].
  // Rows past the end read row N-1 (finite data; never stored).
  i32x4 qop[NS];
  {
    const T* qr = qh + (size_t)min(myq, N - 1) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) qop[s] = *(const i32x4*)(qr + 16 * s);
    // Consume the loads here: the tile copies below also count on vmcnt and
    // the compiler does not see them, so no load of its own may stay pending
    // into the loop (its waits would then also wait for the copies).
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" ::"v"(qop[s]));
    // A negative scale is moved into Q: scale*(q.k) = |scale|*((-q).k), and
    // flipping the sign bit of a 16-bit float is exact.  The loop below then
    // always sees a non-negative multiplier.
    if (p.scale_log2 < 0.f) {
#pragma unroll
      for (int s = 0; s < NS; ++s) qop[s] ^= (int)0x80008000u;
    }
  }

  const int kv_end = CAUSAL ? min(N, (qt + 1) * BR) : N;
  const int nt = (kv_end + BC - 1) / BC;
  // Last tile this wave computes: with causal masking, tiles wholly above the
  // wave's diagonal are skipped (the wave still helps copy them).
  const int jlast = CAUSAL ? min(nt - 1, (qrow0 + 31) / BC) : nt - 1;

  // ---- tile loader: wave w, instruction u fills LDS slots (u*NW + w)*64 + lane
  // of a tile; slot -> (row, chunk), and the lane fetches the logical chunk
  // that the swizzle stores there.  Rows past N re-read row N-1: finite values
  // that the mask zeroes.
  int ld_off[CPT];   // element offset of this lane's chunk within a tile
  int ld_row[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int s = (u * NW + w) * 64 + lane, row = s / CPR, c = s % CPR;
    ld_row[u] = row;
    ld_off[u] = (c ^ chunk_swz<D>(row)) * 8;
  }
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto issue_tile = [&](int j, int stage) {
    const uint32_t kdst = smem_base + stage * 2 * TB;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const size_t row = (size_t)min(j * BC + ld_row[u], N - 1);
      const uint32_t lds_off = kdst + (u * NW + w) * 1024;
      dma16(kh + row * D + ld_off[u], lds_off);
      dma16(vh + row * D + ld_off[u], lds_off + TB);
    }
  };

  // ---- per-lane LDS read geometry (byte offsets within a tile) ----
  // K operand (A of S^T): row kb*32 + swap_bits23(ql), logical chunk 2 s + g.
  const int krow = swap_bits23(ql);
  const int kbase_off = krow * RB;
  const int ky = g ^ chunk_swz<D>(krow);        // chunk(s) = (2 s) ^ ky
  // V operand (A of O^T = V^T P^T), transposed read: in each 16-lane group,
  // lane i points at row (i/4) and column 4*(i%4) of a 4 x 16 block; the
  // hardware returns to lane i the 4 values of column i.  Rows kbase + trow
  // (+4 for the second read), columns 32 b + 16 (lane/16 % 2) + 4 (i%4).
  const int trow = (lane & 15) >> 2;
  int vrow_off[2], vx[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 8 * g + 4 * t + trow;  // row within the 16-key half block
    vrow_off[t] = r * RB + 8 * (lane & 1);
    vx[t] = (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ chunk_swz<D>(r);
  }

  f32x16 oacc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m = kMInit, l = 0.f;
  // Multiplier of the scores in base 2.  A negative sign went into Q; a zero
  // scale is raised to 1e-30, which moves no finite score's exponent by a
  // representable amount but keeps -inf * c = -inf for hidden keys.
  const float c = fmaxf(fabsf(p.scale_log2), 1.0e-30f);

  // ---- the three per-tile steps ----
  // S^T = K_j Q^T from LDS stage `st` into S.
  auto qk = [&](int st, f32x16(&S)[NKB]) {
    const char* sk = smem + st * 2 * TB;
    __builtin_amdgcn_s_setprio(1);  // MFMA phase: issue ahead of the other wave's softmax
    // K operands are read KPF MFMAs ahead of their use, so LDS latency hides
    // behind the MFMA chain; the 32-key blocks' accumulation chains are
    // interleaved (i % NKB is the block) so consecutive MFMAs are independent.
    constexpr int NM = NKB * NS, KPF = NS;
    i32x4 kop[NM];
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int kb = i % NKB, s = i / NKB;
      kop[i] = *(const i32x4*)(sk + kb * 32 * RB + kbase_off + (((2 * s) ^ ky) << 4));
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
#pragma unroll
    for (int i = 0; i < NM; ++i) S[i % NKB] = Half<T>::mfma(kop[i], qop[i / NKB], S[i % NKB]);
    __builtin_amdgcn_sched_group_barrier(0x100, KPF, 0);  // first KPF LDS reads
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (i + KPF < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // next read
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Online-softmax update with the scores S of tile jj; S becomes P.
  auto softmax = [&](int jj, f32x16(&S)[NKB]) {
    const int key0 = jj * BC;
    const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > qrow0);
    if (need_mask) {
      // Accumulator (kb, r) of this lane holds key key0 + 8 g + kofs with
      // kofs = 32 kb + 16 (r/8) + r%8 (a constant); it is visible iff
      // kofs <= rel.  Hidden scores become -inf: the max ignores them and
      // exp2 maps them to 0 (c > 0).
      const int lim = CAUSAL ? min(myq, N - 1) : N - 1;  // last visible key
      const int rel = lim - key0 - 8 * g;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          S[kb][r] = (32 * kb + 16 * (r >> 3) + (r & 7) <= rel) ? S[kb][r] : kNegInf;
    }
    // Four independent partial maxima/sums keep the reduction chains short.
    float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx4[r & 3] = fmaxf(mx4[r & 3], S[kb][r]);
    const float mx = pair_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
    const float mt = (mx == kNegInf) ? kNegInf : mx * c;
    const bool upd = mt > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float mnew = upd ? mt : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
    }
    const float negm = -m;
    float rs4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, negm));
        S[kb][r] = pr;
        rs4[r & 3] += pr;
      }
    l += (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);
  };

  // O^T += V^T P^T with V from LDS stage `st` and P in S.
  auto pv = [&](int st, f32x16(&S)[NKB]) {
    const char* sv = smem + st * 2 * TB + TB;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        i32x4 pop;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pop[e] = (int)Half<T>::pack2(S[kb][8 * h + 2 * e], S[kb][8 * h + 2 * e + 1]);
        const char* vb = sv + (kb * 32 + 16 * h) * RB;
        i16x4 vlo[ND], vhi[ND];
#pragma unroll
        for (int b = 0; b < ND; ++b) {
          vlo[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vb + vrow_off[0] + (((4 * b) ^ vx[0]) << 4)));
          vhi[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vb + vrow_off[1] + (((4 * b) ^ vx[1]) << 4)));
        }
#pragma unroll
        for (int b = 0; b < ND; ++b) {
          const i16x8 v8 = {vlo[b][0], vlo[b][1], vlo[b][2], vlo[b][3],
                            vhi[b][0], vhi[b][1], vhi[b][2], vhi[b][3]};
          oacc[b] = Half<T>::mfma(__builtin_bit_cast(i32x4, v8), pop, oacc[b]);
        }
      }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- ping-pong over key tiles ----
  // The barrier at the end of every tile would otherwise put the two waves
  // sharing a SIMD (waves w and w + 4: waves go round-robin over the four
  // SIMDs of the CU) into the same phase, both on MFMAs or both on the
  // softmax.  With PINGPONG the upper half of the workgroup therefore runs
  // half a tile behind: in iteration j the lower half does QK_j, softmax_j,
  // PV_j while the upper half does softmax_{j-1}, PV_{j-1}, QK_j, so one
  // wave's exponentials overlap the other's matrix products.
  //
  // LDS ring of ST stages, prefetch distance PD: in iteration j tile j + PD
  // is copied into the stage of tile j + PD - ST, which nobody reads any more
  // (the lagging half finished PV_{j-2} before the last barrier); tile j + 1
  // must have landed before the barrier that ends iteration j.  Each wave
  // issues 2*CPT copies per tile and copies complete in order, so "tile j+1
  // landed" is vmcnt <= 2*CPT * (tiles issued after it).
  const bool lag = PINGPONG && w >= NW / 2;
  for (int t = 0; t < PD && t < nt; ++t) issue_tile(t, t);
  wait_vmcnt(2 * CPT * (min(nt, PD) - 1));
  __syncthreads();

  f32x16 sacc[NKB];
  for (int j = 0; j < nt; ++j) {
    if (j + PD < nt) issue_tile(j + PD, (j + PD) % ST);
    if (!lag) {
      if (j <= jlast) {
        qk(j % ST, sacc);
        softmax(j, sacc);
        pv(j % ST, sacc);
      }
    } else {
      if (j >= 1 && j - 1 <= jlast) {
        softmax(j - 1, sacc);
        pv((j - 1) % ST, sacc);
      }
      if (j <= jlast) qk(j % ST, sacc);
    }
    if (j + PD < nt) {  // steady state: tiles j+2 .. j+PD may stay in flight
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * CPT * (PD - 1)) : "memory");
    } else {
      wait_vmcnt(2 * CPT * max(0, nt - 1 - (j + 1)));
    }
    __syncthreads();
  }
  if (lag && nt - 1 <= jlast) {  // the upper half's last tile (no copy can overwrite it now)
    softmax(nt - 1, sacc);
    pv((nt - 1) % ST, sacc);
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 (m + log2 l) ----
  const float lt = pair_sum(l);
  if (myq < N) {
    const float inv = 1.0f / lt;
    T* orow = (T*)p.o + head + (size_t)myq * D;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        // registers 4a..4a+3 hold columns 32 b + 8 a + 4 g + 0..3
        uint2 stv;
        stv.x = Half<T>::pack2(oacc[b][4 * a] * inv, oacc[b][4 * a + 1] * inv);
        stv.y = Half<T>::pack2(oacc[b][4 * a + 2] * inv, oacc[b][4 * a + 3] * inv);
        *(uint2*)(orow + 32 * b + 8 * a + 4 * g) = stv;
      }
    if (g == 0)
      p.lse[(size_t)bh * N + myq] = (m + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  constexpr int NW = TileCfg<D>::NW, BR = 32 * NW;
  FwdParams q = p;
  q.nq = (p.N + BR - 1) / BR;
  const unsigned grid = (unsigned)(q.nq * p.BH);
  hipLaunchKernelGGL((fwd_mfma16<T, D, CAUSAL>), dim3(grid), dim3(64 * NW), 0, stream, q);
  return hipGetLastError();
}

// Causal work per query tile grows with the tile index.  fwd_wide runs a few
// 4-wave workgroups per CU; when its whole grid fits in one round of those
// slots the heaviest tiles alone set the runtime, and fwd_mfma16 (one 8-wave
// workgroup per CU, more rounds, heaviest tiles first) balances better.  With
// at least two rounds of the long-causal configuration's 512-row workgroups
// (one per CU) those balance too, and its 64-row waves run faster.
// Returns 0 (fwd_mfma16), 1 (fwd_wide) or 2 (fwd_wide, long causal).
static int wide_kind(const FwdParams& p, int d, int causal) {
  const bool enabled = d == 64 ? FA_D64_WIDE : d == 128 ? FA_D128_WIDE : FA_D256_WIDE;
  if (!enabled) return 0;
  if (!causal) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int lr = wide_long_causal_rows(d);
  if (lr > 0 && (long long)((p.N + lr - 1) / lr) * p.BH >= 2LL * cus) return 2;
  const int br = wide_rows_per_block(d, causal);
  const long long grid = (long long)((p.N + br - 1) / br) * p.BH;
  return grid > (long long)wide_blocks_per_cu(d, causal) * cus ? 1 : 0;
}

#ifndef FA_PIPE_D128
#define FA_PIPE_D128 1
#endif

template <typename T>
static hipError_t launch_t(const FwdParams& p, int d, int causal, hipStream_t s) {
  if (FA_PIPE_D128 && d == 128) return launch_fwd_pipe(p, d, causal, std::is_same<T, __bf16>::value, s);
  const int kind = wide_kind(p, d, causal);
  if (kind) return launch_fwd_wide(p, d, causal, kind == 2, std::is_same<T, __bf16>::value, s);
  switch (d) {
    case 64:  return causal ? launch_one<T, 64, true>(p, s) : launch_one<T, 64, false>(p, s);
    case 128: return causal ? launch_one<T, 128, true>(p, s) : launch_one<T, 128, false>(p, s);
    case 256: return causal ? launch_one<T, 256, true>(p, s) : launch_one<T, 256, false>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_half(const FwdParams& p, int d, int causal, int is_bf16, hipStream_t s) {
  return is_bf16 ? launch_t<__bf16>(p, d, causal, s) : launch_t<_Float16>(p, d, causal, s);
}

}  // namespace fa
