// Fused exact attention forward for gfx950, fp16/bf16 inputs (d = 128 and
// d = 256): few waves per SIMD, each owning 32 or 64 query rows.
//
// The method is that of "FlashAttention (HI)" (tiling, online softmax, one
// kernel writing only O and the logsumexp); the tile shapes are chosen for
// CDNA4.  Each wave owns 32 QB query rows (QB 32-row MFMA blocks) and streams
// 32-key tiles of K and V through LDS:
//   * d = 128, QB = 2: every K or V operand read from LDS feeds two MFMAs
//     (one per query block), half the LDS traffic per flop of a 32-row wave;
//     the whole state (O 64 x 128 fp32, the score tile, Q) fits in 256 VGPRs,
//     so each SIMD runs two waves, one from each half of an 8-wave workgroup,
//     offset by half a tile so one's softmax overlaps the other's MFMAs;
//   * d = 256, QB = 1: O 32 x 256 and Q still fit two waves per SIMD, which
//     the 8-wave kernel cannot reach at this width.
// MFMAs are built in VGPR form (compiler flag for this file), which keeps the
// accumulators out of the AGPRs and avoids copies between the two files.
// Score layout, key permutation, transposed V reads, chunk swizzle, lazy
// running max and masking follow fwd_mfma16 (fa_fwd.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

// True when, for every row r of a transposed V read (r = 8 g + i, i < 4), the
// swizzle of row r + 4 is that of row r with bit 0 flipped.
template <int D>
constexpr bool swz_step4_is_xor1() {
  for (int g = 0; g < 2; ++g)
    for (int i = 0; i < 4; ++i)
      if (chunk_swz<D>(8 * g + i + 4) != (chunk_swz<D>(8 * g + i) ^ 1)) return false;
  return true;
}

// Per head dimension and masking: QB 32-row query blocks per wave, BC keys
// per tile, ST ring stages, OCC waves per SIMD the registers are budgeted for,
// NW waves per workgroup (4 when not named); XK / XV: K / V LDS addresses
// formed inside the loop from one base register (XORs per tile) rather than
// kept as eight loop-invariant registers each.  Measured choices:
//   d = 128 without masking: 64 rows per wave (half the LDS reads per flop),
//           one 8-wave workgroup per CU whose two halves run half a tile
//           apart (the lagging half keeps its packed P across the barrier;
//           3.5-5% over two uncoordinated 4-wave workgroups);
//   d = 128 causal: 32 rows per wave at three waves per SIMD (twice as many
//           workgroups, so the unequal causal tiles balance over rounds);
//   d = 128 causal with many query tiles (LONG: at least two rounds of
//           512-row workgroups, one per CU): the non-causal configuration,
//           whose heavy-first rounds then balance (6-8% over the 32-row
//           kernel at 4096-16384 tokens);
//   d = 256: 32 rows per wave, one 8-wave workgroup per CU with ping-pong
//           halves (+1-2% over two 4-wave workgroups);
//   d = 64: 64 rows per wave and 64-key tiles (the state is small), one
//           8-wave workgroup per CU with ping-pong halves (+10-12% over the
//           32-row 8-wave kernel); causal launches with fewer than two rounds
//           of those 512-row workgroups take 32 rows per wave at three waves
//           per SIMD instead (15-18% over the 8-wave 32-row kernel they used
//           to fall back to at 1024-2048 tokens).
template <int D, bool CAUSAL, bool LONG = false> struct WideCfg;
template <> struct WideCfg<64, false> {
  static constexpr int QB = 2, BC = 64, ST = 3, OCC = 2, NW = 8;
  static constexpr bool XK = false, XV = false;
};
template <> struct WideCfg<64, true> {
  static constexpr int QB = 1, BC = 64, ST = 3, OCC = 3;
  static constexpr bool XK = false, XV = false;
};
template <> struct WideCfg<64, true, true> {
  static constexpr int QB = 2, BC = 64, ST = 3, OCC = 2, NW = 8;
  static constexpr bool XK = false, XV = false;
};
template <> struct WideCfg<128, false> {
  static constexpr int QB = 2, BC = 32, ST = 4, OCC = 2, NW = 8;
  static constexpr bool XK = false, XV = false;
};
template <> struct WideCfg<128, true> {
  static constexpr int QB = 1, BC = 32, ST = 3, OCC = 3;
  static constexpr bool XK = false, XV = false;
};
template <> struct WideCfg<128, true, true> {
  static constexpr int QB = 2, BC = 32, ST = 4, OCC = 2, NW = 8;
  static constexpr bool XK = false, XV = false;
};
template <bool C> struct WideCfg<256, C> {
  static constexpr int QB = 1, BC = 32, ST = 4, OCC = 2, NW = 8;
  static constexpr bool XK = true, XV = true;
};

// Waves per workgroup: 4 unless the configuration names 8 (ping-pong halves).
template <typename C, typename = void> struct NWOf { static constexpr int v = 4; };
template <typename C> struct NWOf<C, std::void_t<decltype(C::NW)>> { static constexpr int v = C::NW; };
template <typename T, int D, bool CAUSAL, bool LONG>
__global__ __launch_bounds__((64 * NWOf<WideCfg<D, CAUSAL, LONG>>::v))
__attribute__((amdgpu_waves_per_eu(WideCfg<D, CAUSAL, LONG>::OCC, WideCfg<D, CAUSAL, LONG>::OCC)))
void fwd_wide(FwdParams p) {
  using Cfg = WideCfg<D, CAUSAL, LONG>;
  constexpr int NW = NWOf<Cfg>::v;
  constexpr bool PP = NW == 8;
  constexpr int BC = Cfg::BC, QB = Cfg::QB, WR = 32 * QB, BR = WR * NW;
  constexpr int ST = Cfg::ST, PD = PP ? ST - 2 : ST - 1;
  constexpr int RB = D * 2;                  // bytes per K/V row
  constexpr int TB = BC * RB;                // bytes per K or V tile
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int CPT = BC * CPR / (64 * NW);  // copies per wave per tile and tensor
  constexpr int NS = D / 16;                 // MFMA k-steps of K Q^T
  constexpr int NKB = BC / 32;               // 32-key blocks per tile
  constexpr int ND = D / 32;                 // 32-column blocks of O
  static_assert(CPT * 64 * NW == BC * CPR, "tile must split evenly over the waves");
  static_assert(PD >= 1 && 2 * CPT * (PD - 1) <= 31, "ring depth");
  __shared__ __attribute__((aligned(1024))) char smem[ST * 2 * TB];  // [stage][K, V]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  int bh, qt;
  decode_block(blockIdx.x, p.BH, p.nq, CAUSAL, bh, qt, (CAUSAL && NW == 4) ? Cfg::OCC : 0);

  const size_t head = (size_t)bh * N * D;
  const T* __restrict__ qh = (const T*)p.q + head;
  const size_t kvhead = (size_t)kv_head(p, bh) * N * D;  // K/V head shared by a group of query heads
  const T* __restrict__ kh = (const T*)p.k + kvhead;
  const T* __restrict__ vh = (const T*)p.v + kvhead;

  const int qrow0 = qt * BR + w * WR;  // first query row of this wave
  // Q operands (B of S^T = K Q^T): block qb, lane holds
  // Q[qrow0 + 32 qb + ql][16 s + 8 g .. +8]; rows past the end read row N-1.
  // Loaded after the first tile copies are issued (below).
  i32x4 qop[QB][NS];
  const float c = fmaxf(fabsf(p.scale_log2), 1.0e-30f);

  const int kv_end = CAUSAL ? min(N, (qt + 1) * BR) : N;
  const int nt = (kv_end + BC - 1) / BC;
  // Last tile this wave computes (-1: the wave's rows are all past N and it
  // only helps with the copies).
  const int jlast = qrow0 >= N ? -1 : (CAUSAL ? min(nt - 1, (qrow0 + WR - 1) / BC) : nt - 1);

  // ---- tile copies: wave w, instruction u fills slots (u NW + w) 64 + lane ----
  // Buffer loads against a resource from the tile to the end of this head's
  // K (or V), built per tile in scalar registers: rows past N fail the
  // hardware range check and read as zeros, and a copy's address is a
  // constant per-lane offset.
  uint32_t ld_voff[CPT];  // byte offset of this lane's chunk within a tile
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int s = (u * NW + w) * 64 + lane, row = s / CPR, ch = s % CPR;
    ld_voff[u] = row * RB + (ch ^ chunk_swz<D>(row)) * 16;
  }
  const uint32_t head_bytes = (uint32_t)N * RB;
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto issue_tile = [&](int j) __attribute__((always_inline)) {
    const uint32_t kdst = smem_base + (j % ST) * 2 * TB + w * 1024;
    const uint32_t t0 = (uint32_t)j * TB;
    const __amdgpu_buffer_rsrc_t kbuf = tile_rsrc(kh, head_bytes, t0);
    const __amdgpu_buffer_rsrc_t vbuf = tile_rsrc(vh, head_bytes, t0);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      buf_dma16(kbuf, ld_voff[u], kdst + u * NW * 1024);
      buf_dma16(vbuf, ld_voff[u], kdst + u * NW * 1024 + TB);
    }
  };

  // ---- LDS read geometry ----
  // K operand (A of S^T): row kb*32 + swap_bits23(ql), logical chunk 2 s + g.
  // V operand (A of O^T = V^T P^T), transposed read: in each 16-lane group,
  // lane i points at row (i/4) and column 4*(i%4) of a 4 x 16 block; the
  // hardware returns to lane i the 4 values of column i.
  // Per-lane byte offsets inside a stage; the stage and the 16-key half are
  // compile-time and go into the instructions' immediate offsets.
  // K chunk 2 s + g of row krow sits at chunk (2 s + g) ^ swz(krow); the
  // XOR with 2 s only touches byte-offset bits 5..7, so one base register
  // serves every k-step: address = kbase ^ (s << 5).
  const int krow = swap_bits23(ql);
  const int kbase = krow * RB + ((g ^ chunk_swz<D>(krow)) << 4);
  // One base register serves all of them.  Rows r + 4 t (t = 0, 1): r has
  // bit 2 clear, and adding 4 to r flips bit 0 of its swizzle, so the second
  // group sits at vaddr ^ (4 RB + 16).  Column block b sits at ^ (b << 6):
  // the chunk index 4 b + c' is XORed with the swizzle, which only touches
  // offset bits 4..7 (4..8 at d = 256), below the row's bits.
  const int trow = (lane & 15) >> 2;
  const int vrow = 8 * g + trow;
  const int vaddr = vrow * RB + 8 * (lane & 1) +
                    (((2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ chunk_swz<D>(vrow)) << 4);
  static_assert(swz_step4_is_xor1<D>(), "rows r and r + 4 differ in bit 0 of the swizzle");

  f32x16 oacc[QB][ND];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][b][r] = 0.f;
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = kMInit;
    l[qb] = 0.f;
  }

  typedef f32x16 STile[QB][NKB];
  typedef i32x4 PTile[QB][NKB][2];

  // S^T = K_j Q^T for both query blocks; each K operand read feeds two MFMAs
  // (the first k-step starts from a zero accumulator).  SG = stage of tile j.
  auto qk = [&](auto SG, STile& S) __attribute__((always_inline)) {
    const char* sk = smem + decltype(SG)::value * 2 * TB;
    const f32x16 zero = {};
    // With XK the per-step addresses are formed here, not hoisted out of the
    // loop as eight loop-invariant registers: the empty asm makes the base opaque.
    int kb0 = kbase;
    if constexpr (Cfg::XK) asm volatile("" : "+v"(kb0));
    constexpr int NM = NKB * NS;
    i32x4 kop[NM];
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int kb = i % NKB, s = i / NKB;
      kop[i] = *(const i32x4*)(sk + kb * 32 * RB + (kb0 ^ (s << 5)));
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int kb = i % NKB, s = i / NKB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        S[qb][kb] = Half<T>::mfma(kop[i], qop[qb][s], s == 0 ? zero : S[qb][kb]);
    }
  };

  // Hidden keys of tile j become -inf (tiles crossing the diagonal or N).
  auto mask = [&](int j, STile& S) __attribute__((always_inline)) {
    const int key0 = j * BC;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int lim = CAUSAL ? min(qrow0 + 32 * qb + ql, N - 1) : N - 1;
      const int rel = lim - key0 - 8 * g;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          S[qb][kb][r] = (32 * kb + 16 * (r >> 3) + (r & 7) <= rel) ? S[qb][kb][r] : kNegInf;
    }
  };
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    return (j * BC + BC > N) || (CAUSAL && j * BC + BC - 1 > qrow0);
  };

  // Online softmax of S (branch-free): running max with lazy moves, P packed
  // to 16-bit for the second product, alpha = factor O must be scaled by.
  auto softmax = [&](STile& S, PTile& P, float (&alpha)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // four independent chains, started from the first four scores
      float mx4[4] = {S[qb][0][0], S[qb][0][1], S[qb][0][2], S[qb][0][3]};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = (kb == 0 ? 4 : 0); r < 16; ++r) mx4[r & 3] = fmaxf(mx4[r & 3], S[qb][kb][r]);
      const float mx = pair_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
      const float mt = (mx == kNegInf) ? kNegInf : mx * c;
      const float mnew = (mt > m[qb] + kLazy) ? mt : m[qb];
      alpha[qb] = __builtin_amdgcn_exp2f(m[qb] - mnew);
      m[qb] = mnew;
      const float negm = -mnew;
      float rs4[4];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][kb][r], c, negm));
          S[qb][kb][r] = pr;
          if (kb == 0 && r < 4) rs4[r] = pr;
          else rs4[r & 3] += pr;
        }
      l[qb] = l[qb] * alpha[qb] + ((rs4[0] + rs4[1]) + (rs4[2] + rs4[3]));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            P[qb][kb][h][e] =
                (int)Half<T>::pack2(S[qb][kb][8 * h + 2 * e], S[qb][kb][8 * h + 2 * e + 1]);
    }
  };

  auto rescale = [&](const float (&alpha)[QB]) __attribute__((always_inline)) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) any = any || alpha[qb] != 1.0f;
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int b = 0; b < ND; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][b][r] *= alpha[qb];
    }
  };

  // O^T += V_j^T P^T; each V operand read feeds both query blocks.
  auto pv = [&](auto SG, const PTile& P) __attribute__((always_inline)) {
    const char* sv = smem + decltype(SG)::value * 2 * TB + TB;
    int va0 = vaddr;
    if constexpr (Cfg::XV) asm volatile("" : "+v"(va0));  // as in qk
    const int va[2] = {va0, va0 ^ (4 * RB + 16)};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const char* vb = sv + (kb * 32 + 16 * h) * RB;
        i16x4 vlo[ND], vhi[ND];
#pragma unroll
        for (int b = 0; b < ND; ++b) {
          vlo[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + (va[0] ^ (b << 6))));
          vhi[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + (va[1] ^ (b << 6))));
        }
#pragma unroll
        for (int b = 0; b < ND; ++b) {
          const i16x8 v8 = {vlo[b][0], vlo[b][1], vlo[b][2], vlo[b][3],
                            vhi[b][0], vhi[b][1], vhi[b][2], vhi[b][3]};
          const i32x4 va = __builtin_bit_cast(i32x4, v8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][b] = Half<T>::mfma(va, P[qb][kb][h], oacc[qb][b]);
        }
      }
  };

  // ---- main loop: ring of ST stages, tile t copied during iteration t - PD ----
  // Tile j + PD goes into the stage of tile j - 1 (j - 2 with ping-pong
  // halves, whose upper half reads tile j - 1 in iteration j), which every
  // wave finished before the barrier that ended iteration j - 1.  Copies
  // complete in order, so "tile j + 1 has landed" is vmcnt <= 2 CPT x (tiles
  // issued after it).
  // The first tiles are issued before Q is read, so that both latencies
  // overlap; Q's loads are the newest, and draining them drains the copies.
  for (int t = 0; t < PD && t < nt; ++t) issue_tile(t);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const T* qr = qh + (size_t)min(qrow0 + 32 * qb + ql, N - 1) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) qop[qb][s] = *(const i32x4*)(qr + 16 * s);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" ::"v"(qop[qb][s]));  // drain: Q and the first tiles
  if (p.scale_log2 < 0.f) {  // a negative scale moves into Q's sign (exact)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < NS; ++s) qop[qb][s] ^= (int)0x80008000u;
  }

  wait_vmcnt(0);
  __syncthreads();

  STile sacc;
  PTile pt;
  float alpha[QB];
  // Ping-pong halves (8-wave workgroups; waves w and w + NW/2 share a SIMD):
  // the upper half runs mode 1 (P V of tile j - 1, then scores and softmax
  // of tile j; its packed P waits across the barrier), the lower half mode 0
  // (scores, softmax and P V of tile j), so the two halves' matrix products
  // and softmaxes fall half a tile apart.
  const bool upper = PP && w >= NW / 2;
  // One iteration; SG = j % ST as a compile-time constant (the loop below is
  // unrolled over the ring) so that every LDS address is register + immediate.
  auto step = [&](int j, auto SG, auto MODE) __attribute__((always_inline)) {
    constexpr int sp = (decltype(SG)::value + ST - 1) % ST;
    constexpr int md = decltype(MODE)::value;
    if (j + PD < nt) issue_tile(j + PD);
    if constexpr (md == 0) {
      if (j <= jlast) {
        qk(SG, sacc);
        if (needs_mask(j)) mask(j, sacc);
        softmax(sacc, pt, alpha);
        rescale(alpha);
        pv(SG, pt);
      }
    } else {
      if (j >= 1 && j - 1 <= jlast) pv(std::integral_constant<int, sp>(), pt);
      if (j <= jlast) {
        qk(SG, sacc);
        if (needs_mask(j)) mask(j, sacc);
        softmax(sacc, pt, alpha);
        rescale(alpha);
      }
    }
    if (j + PD < nt) {  // steady state: tiles j + 2 .. j + PD may stay in flight
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * CPT * (PD - 1)) : "memory");
    } else {
      wait_vmcnt(2 * CPT * max(0, nt - 1 - (j + 1)));
    }
    __syncthreads();
  };
  static_assert(ST >= 2 && ST <= 6, "the loop below is unrolled over 2 to 6 ring stages");
  // With ping-pong halves both run one extra iteration (j = nt): the lagging
  // half does its last P V there, the leading half only meets the barrier.
  const int nsteps = PP ? nt + 1 : nt;
  auto run = [&](auto MODE) __attribute__((always_inline)) {
    for (int j = 0; j < nsteps; j += ST) {
      step(j, std::integral_constant<int, 0>(), MODE);
      if (j + 1 < nsteps) step(j + 1, std::integral_constant<int, 1>(), MODE);
      if constexpr (ST > 2) { if (j + 2 < nsteps) step(j + 2, std::integral_constant<int, 2 % ST>(), MODE); }
      if constexpr (ST > 3) { if (j + 3 < nsteps) step(j + 3, std::integral_constant<int, 3 % ST>(), MODE); }
      if constexpr (ST > 4) { if (j + 4 < nsteps) step(j + 4, std::integral_constant<int, 4 % ST>(), MODE); }
      if constexpr (ST > 5) { if (j + 5 < nsteps) step(j + 5, std::integral_constant<int, 5 % ST>(), MODE); }
    }
  };
  if constexpr (PP) {
    if (upper) run(std::integral_constant<int, 1>());
    else run(std::integral_constant<int, 0>());
  } else {
    run(std::integral_constant<int, 0>());
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 (m + log2 l) ----
  // A lane holds one query's O row in 8-byte pieces.  Each wave stages its 32
  // rows of a query block in LDS (the ring is idle after the last barrier),
  // then writes whole rows: every store instruction covers 64 / CPR rows of
  // contiguous memory.  Chunks are XOR-swizzled by row in the staging buffer.
  static_assert(NW * 32 * RB <= ST * 2 * TB, "staging fits in the ring");
  char* stg = smem + w * (32 * RB);
  T* __restrict__ oh = (T*)p.o + head;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int myq = qrow0 + 32 * qb + ql;
    const float lt = pair_sum(l[qb]);
    const float inv = 1.0f / lt;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 stv;
        stv.x = Half<T>::pack2(oacc[qb][b][4 * a] * inv, oacc[qb][b][4 * a + 1] * inv);
        stv.y = Half<T>::pack2(oacc[qb][b][4 * a + 2] * inv, oacc[qb][b][4 * a + 3] * inv);
        *(uint2*)(stg + ql * RB + (((4 * b + a) ^ (ql & (CPR - 1))) << 4) + 8 * g) = stv;
      }
    if (g == 0 && myq < N)
      p.lse[(size_t)bh * N + myq] = (m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are staged
#pragma unroll
    for (int it = 0; it < 32 * CPR / 64; ++it) {
      const int idx = it * 64 + lane, row = idx / CPR, ch = idx % CPR;
      const i32x4 val = *(const i32x4*)(stg + row * RB + ((ch ^ (row & (CPR - 1))) << 4));
      const int grow = qrow0 + 32 * qb + row;
      if (grow < N) *(i32x4*)(oh + (size_t)grow * D + ch * 8) = val;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next block's writes
  }
}

template <typename T, int D, bool CAUSAL, bool LONG = false>
hipError_t launch_wide(const FwdParams& p, hipStream_t stream) {
  constexpr int NW = NWOf<WideCfg<D, CAUSAL, LONG>>::v;
  constexpr int BR = 32 * WideCfg<D, CAUSAL, LONG>::QB * NW;
  FwdParams q = p;
  q.nq = (p.N + BR - 1) / BR;
  const unsigned grid = (unsigned)(q.nq * p.BH);
  hipLaunchKernelGGL((fwd_wide<T, D, CAUSAL, LONG>), dim3(grid), dim3(64 * NW), 0, stream, q);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_wide_t(const FwdParams& p, int d, int causal, int long_causal, hipStream_t s) {
  switch (d) {
    case 64:
      if (causal && long_causal) return launch_wide<T, 64, true, true>(p, s);
      return causal ? launch_wide<T, 64, true>(p, s) : launch_wide<T, 64, false>(p, s);
    case 128:
      if (causal && long_causal) return launch_wide<T, 128, true, true>(p, s);
      return causal ? launch_wide<T, 128, true>(p, s) : launch_wide<T, 128, false>(p, s);
    case 256: return causal ? launch_wide<T, 256, true>(p, s) : launch_wide<T, 256, false>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int D, bool C>
static constexpr int rows_of() {
  return 32 * NWOf<WideCfg<D, C>>::v * WideCfg<D, C>::QB;
}
template <bool C>
static int rows_per_block(int d) {
  switch (d) {
    case 64: return rows_of<64, C>();
    case 128: return rows_of<128, C>();
    case 256: return rows_of<256, C>();
  }
  return 0;
}
// Workgroups per CU: OCC waves per SIMD, four SIMDs, NW waves per workgroup.
template <int D, bool C>
static constexpr int wgs_per_cu() {
  return WideCfg<D, C>::OCC * 4 / NWOf<WideCfg<D, C>>::v;
}
template <bool C>
static int blocks_per_cu(int d) {
  switch (d) {
    case 64: return wgs_per_cu<64, C>();
    case 128: return wgs_per_cu<128, C>();
    case 256: return wgs_per_cu<256, C>();
  }
  return 0;
}
int wide_rows_per_block(int d, int causal) {
  return causal ? rows_per_block<true>(d) : rows_per_block<false>(d);
}
int wide_long_causal_rows(int d) {
  switch (d) {
    case 64: return 32 * NWOf<WideCfg<64, true, true>>::v * WideCfg<64, true, true>::QB;
    case 128: return 32 * NWOf<WideCfg<128, true, true>>::v * WideCfg<128, true, true>::QB;
  }
  return 0;
}
int wide_blocks_per_cu(int d, int causal) {
  return causal ? blocks_per_cu<true>(d) : blocks_per_cu<false>(d);
}

hipError_t launch_fwd_wide(const FwdParams& p, int d, int causal, int long_causal, int is_bf16,
                           hipStream_t s) {
  return is_bf16 ? launch_wide_t<__bf16>(p, d, causal, long_causal, s)
                 : launch_wide_t<_Float16>(p, d, causal, long_causal, s);
}


}  // namespace fa
