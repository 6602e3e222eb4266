// Fused exact attention forward with OCP e4m3 operands for gfx950.
//
// The fp8 variant of the method ("FlashAttention-3 (BN)" / "(FA)", sections
// on new hardware capabilities and on low precision): both products run on
// 8-bit floats, v_mfma_scale_f32_32x32x64_f8f6f4 at twice the bf16 rate, with
// per-128-row fp32 descales for Q, K and V.
//
// Same tiling and online softmax as the 16-bit kernel: each wave owns 32
// query rows (within one descale block), a workgroup of 8 (4 with causal
// masking) waves 256 (128) rows; K/V tiles of 128 rows (one descale block
// each; 64 rows, half a block, at d = 256) stream through an LDS ring filled
// by direct global -> LDS copies; d is 64, 128 or 256;
// S^T = K8 Q8^T keeps one query per lane.
//   scores    t = s8 * (scale log2 e * q_descale[query block] *
//             k_descale[tile]): one per-tile multiplier folded into the FMA.
//   V descale each tile's descale is split as v_descale = 2^e f with f in
//             (1/2, 1]: 2^e enters the second product exactly as the MFMA's
//             E8M0 block scale of the V^T operand, f is folded into P.  The
//             block quantiser of this library emits powers of two (f = 1),
//             for which the whole descale is applied without rounding.
//   P         each row's P of a tile is scaled by a power of two to its own
//             tile maximum before rounding: with sigma = ceil(tile max - m)
//             the rounded P is P~ = e4m3(exp2(t - m + 8 - sigma + log2 f)),
//             whose row maximum lies in (2^7, 2^8], so it never saturates
//             (448), and a tile far below the running max keeps e4m3's full
//             precision instead of falling into its subnormal range; the
//             MFMA's per-lane E8M0 scale of the P~ operand, 2^(sigma - 8),
//             undoes the shift exactly.  The running max m moves once a tile
//             exceeds it by lazy = 8 (log2 units; with the rare outlier
//             entries of the fp8 workload a headroom of 2 rescaled O at half
//             of the tiles).  The running sum l counts the unrounded P (it
//             gives the logsumexp); E sums the rounding error of each tile's
//             largest P~, and O = O~ / (l + E): a row that one key decides,
//             whose P~ is off a power of two under the lazy max, gets that
//             key's value row back without the rounding of its weight.
//   P V       O^T += V8^T P~^T with V8 read transposed from LDS by
//             ds_read_b64_tr_b8 (lane i of a 16-lane group receives byte
//             i % 8 of the rows addressed by lanes 2e + i/8, e = 0..7).
// Output O is bf16, the logsumexp fp32 in natural log.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_fp8_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr float kLazy8 = 8.0f;  // log2 headroom of the running max on this path

// Key-tile rows (64 or 128) per head dimension and waves per SIMD (tuning
// builds may override them).  Measured at d = 128: 128-key tiles beat 64-key
// tiles (about 12%).  At d = 256 a 128-key score tile (64 registers) next to
// O (128) and Q (32) does not fit two waves per SIMD, so tiles are 64 keys.
// Waves per workgroup NW: 8 without masking (the two halves of the
// workgroup, waves w and w + 4 sharing a SIMD, run half a tile apart: +5%),
// 4 with causal masking (more, smaller workgroups balance the unequal causal
// tiles).
#ifndef FA_FP8_BC
#define FA_FP8_BC 128
#endif
#ifndef FA_FP8_OCC
#define FA_FP8_OCC 2
#endif
template <int D> constexpr int fp8_bc() { return D == 256 ? 64 : FA_FP8_BC; }
// d = 64 (153 registers): 4-wave workgroups at three waves per SIMD for both
// maskings, 9% (non-causal) and 14% (causal) over two 8-wave ping-pong ones:
// its softmax dominates and a third wave hides more of it.
template <int D, bool CAUSAL> constexpr int fp8_nw() { return (CAUSAL || D == 64) ? 4 : 8; }
template <int D> constexpr int fp8_occ() { return D == 64 ? 3 : FA_FP8_OCC; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__((64 * fp8_nw<D, CAUSAL>())) __attribute__((amdgpu_waves_per_eu(fp8_occ<D>(), fp8_occ<D>())))
void fwd_fp8(Fp8Params p) {
  constexpr int NW = fp8_nw<D, CAUSAL>();
  constexpr int BC = fp8_bc<D>(), BR = 32 * NW, ST = NW == 8 ? 4 : 2;
  constexpr bool PP = NW == 8;
  constexpr int PD = PP ? ST - 2 : ST - 1;   // tiles copied ahead
  constexpr int RB = D;                      // bytes per fp8 row
  constexpr int TB = BC * RB;                // bytes per K or V tile
  constexpr int SB = 2 * TB;                 // ring stage: K tile, then V tile
  constexpr int CPR = RB / 16;               // 16-byte chunks per row
  constexpr int CPT = BC * CPR / (64 * NW);  // copies per wave per tile and tensor
  constexpr int NS = D / 64;                 // MFMA k-steps of K Q^T
  constexpr int NKB = BC / 32;               // 32-key blocks per tile
  constexpr int NKS = BC / 64;               // MFMA k-steps of V^T P^T
  constexpr int ND = D / 32;                 // 32-column blocks of O
  static_assert((BC == 64 || BC == 128) && BR % 128 == 0,
                "query tiles are whole 128-row descale blocks, key tiles a half or whole one");
  static_assert(CPT * 64 * NW == BC * CPR, "tile must split evenly over the waves");
  static_assert(PD >= 1 && 2 * CPT * (PD - 1) <= 31, "ring depth");
  __shared__ __attribute__((aligned(1024))) char smem[ST * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  int bh, qt;
  // causal: the first passes over an XCD's CUs alternate direction (workgroups per CU)
  decode_block(blockIdx.x, p.BH, p.nq, CAUSAL, bh, qt, fp8_occ<D>() * 4 / NW);
  const size_t head = (size_t)bh * N * D;
  const uint8_t* __restrict__ qh = p.q + head;
  const uint8_t* __restrict__ kh = p.k + head;
  const uint8_t* __restrict__ vh = p.v + head;
  // Descales are read through the constant address space: wave-uniform
  // scalar loads, counted apart from the tile copies (a vector load here
  // would make each tile's softmax wait for every copy in flight).
  typedef const __attribute__((address_space(4))) float cfloat;
  const cfloat* qd = (const cfloat*)(p.q_descale + (size_t)bh * p.nblk);
  const cfloat* kd = (const cfloat*)(p.k_descale + (size_t)bh * p.nblk);
  const cfloat* vd = (const cfloat*)(p.v_descale + (size_t)bh * p.nblk);

  const int qrow0 = qt * BR + w * 32;
  const int myq = qrow0 + ql;

  // Q operand (B of S^T = K Q^T): lane holds Q8[myq][64 s + 32 g .. +32];
  // loaded after the first tile copies are issued (below).
  i32x8 qop[NS];
  const float c = fmaxf(fabsf(p.scale_log2), 1.0e-30f);
  // this wave's 32 rows lie in one 128-row descale block (rows past N use
  // the last block: their results are not stored)
  const float cq = c * qd[min(qrow0, N - 1) >> 7];

  const int kv_end = CAUSAL ? min(N, (qt + 1) * BR) : N;
  const int nt = (kv_end + BC - 1) / BC;
  // last tile this wave computes (-1: all its rows are past N)
  const int jlast = qrow0 >= N ? -1 : (CAUSAL ? min(nt - 1, (qrow0 + 31) / BC) : nt - 1);

  // ---- copies (as in the 16-bit kernel, D-byte rows) ----
  // Per tile, buffer resources from the tile to the end of the head: rows
  // past N read as zeros (their keys are masked), and a copy's address is a
  // constant per-lane offset.
  uint32_t ld_voff[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int s = (u * NW + w) * 64 + lane, row = s / CPR, ch16 = s % CPR;
    ld_voff[u] = (uint32_t)(row * RB + (ch16 ^ swz8<D>(row)) * 16);
  }
  const uint32_t head_bytes = (uint32_t)N * RB;
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto issue_tile = [&](int j) __attribute__((always_inline)) {
    const uint32_t dst = smem_base + (j % ST) * SB + w * 1024;
    const uint32_t t0 = (uint32_t)j * TB;
    const __amdgpu_buffer_rsrc_t kbuf = tile_rsrc(kh, head_bytes, t0);
    const __amdgpu_buffer_rsrc_t vbuf = tile_rsrc(vh, head_bytes, t0);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      buf_dma16(kbuf, ld_voff[u], dst + u * NW * 1024);
      buf_dma16(vbuf, ld_voff[u], dst + u * NW * 1024 + TB);
    }
  };

  // K operand (A of S^T): row kb*32 + swap_bits23(ql), logical chunks
  // 4 s + 2 g and 4 s + 2 g + 1.
  const int krow = swap_bits23(ql);
  const int kx = swz8<D>(krow);
  // V operand (A of O^T = V^T P~^T), transposed byte reads: lane r of each
  // 16-lane group addresses row 32 kb + 16 h + 8 g + r/2, chunk 2 b + lane/16 % 2,
  // byte 8 (r % 2) of that chunk.
  const int tr = (lane & 15) >> 1;
  const int vrow_off = (8 * g + tr) * RB + 8 * (lane & 1);
  const int vx = ((lane >> 4) & 1) ^ swz8<D>(8 * g + tr);

  f32x16 oacc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  // l: fp32 sum of the unrounded P (for the LSE); E: sum over tiles of the
  // rounding error of each tile's largest P~, in l's units.  O is divided by
  // l + E, so a row that one key decides gets that key's value row back
  // without the rounding of its weight.
  float m = kMInit, l = 0.f, E = 0.f;

  // ---- S^T = K8 Q8^T for tile j (stage st) ----
  auto qk = [&](int st, f32x16 (&S)[NKB]) __attribute__((always_inline)) {
    const char* sk = smem + st * SB;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const char* kr = sk + (kb * 32 + krow) * RB;
        const i32x4 lo = *(const i32x4*)(kr + (((4 * s + 2 * g) ^ kx) << 4));
        const i32x4 hi = *(const i32x4*)(kr + (((4 * s + 2 * g + 1) ^ kx) << 4));
        S[kb] = mfma8(i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, qop[s], S[kb]);
      }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- scale, mask, online softmax of tile j; P~ packed to e4m3 ----
  // Rescales O when the running max moves; returns the tile's V scale
  // (E8M0) and sets this lane's P~ scale sb (E8M0).
  auto softmax = [&](int j, f32x16 (&S)[NKB], i32x8 (&P)[NKS], int& sb) __attribute__((always_inline)) -> int {
    const int key0 = j * BC;
    const int blk = (j * BC) >> 7;  // the 128-row descale block of tile j
    const float ct = cq * kd[blk];
    if ((key0 + BC > N) || (CAUSAL && key0 + BC - 1 > qrow0)) {
      const int lim = CAUSAL ? min(myq, N - 1) : N - 1;
      const int rel = lim - key0 - 8 * g;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          S[kb][r] = (32 * kb + 16 * (r >> 3) + (r & 7) <= rel) ? S[kb][r] : kNegInf;
    }
    float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx4[r & 3] = fmaxf(mx4[r & 3], S[kb][r]);
    const float mx = pair_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
    const float mt = (mx == kNegInf) ? kNegInf : mx * ct;
    const bool upd = mt > m + kLazy8;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float mnew = upd ? mt : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      l *= alpha;
      E *= alpha;
#pragma unroll
      for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
    }
    // v_descale = 2^e f, f in (1/2, 1]
    float f;
    const int vsa = vscale_split(vd[blk], f);
    // this row's shift: its tile maximum in (2^7, 2^8] before rounding.
    // sigma <= lazy after the update above; below -100 the tile's P are
    // under 2^-100 of P's at the running max and any shift serves, as for
    // rows with no visible key (P = 0).  The scale 127 + sigma - 8 then lies
    // in [19, 127], a valid E8M0 exponent.
    const float sig = (mt == kNegInf) ? 0.0f : fmaxf(__builtin_ceilf(mt - m), -100.0f);
    const int isig = (int)sig;
    sb = 127 + isig - 8;
    const float beta = (8.0f - sig) + __builtin_amdgcn_logf(f) - m;
    const float lsc = __builtin_amdgcn_ldexpf(__builtin_amdgcn_rcpf(f), isig - 8);
    float rs4[4];  // four partial row sums; the first four P start them
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], ct, beta));
        S[kb][r] = pr;
        rs4[r & 3] = (kb == 0 && r < 4) ? pr : rs4[r & 3] + pr;
      }
    l += ((rs4[0] + rs4[1]) + (rs4[2] + rs4[3])) * lsc;
    // the row's largest P~ of this tile (0 if all keys are hidden)
    const float pm = (mt == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(__builtin_fmaf(mx, ct, beta));
    E = __builtin_fmaf(round_e4m3(pm) - pm, lsc, E);
    // P~ operand of k-step ks: bytes 16 kbh + 8 h + e <- S[2 ks + kbh][8 h + e]
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kbh = 0; kbh < 2; ++kbh)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q4 = 0; q4 < 2; ++q4) {
            const f32x16& sv16 = S[2 * ks + kbh];
            const int r0 = 8 * h + 4 * q4;
            P[ks][4 * kbh + 2 * h + q4] =
                (int)pack4_e4m3(sv16[r0], sv16[r0 + 1], sv16[r0 + 2], sv16[r0 + 3]);
          }
    return vsa;
  };

  // ---- O^T += V8^T P~^T for the tile in stage st, V scale sa, P~ scale sb ----
  // The V^T operand of each MFMA is read one MFMA ahead (its four transposed
  // reads are in flight while the previous product runs).
  auto pv = [&](int st, const i32x8 (&P)[NKS], int sa, int sb) __attribute__((always_inline)) {
    const char* sv = smem + st * SB + TB;
    auto vread = [&](int i) __attribute__((always_inline)) {
      const int ks = i / ND, b = i % ND;
      i32x2 part[4];
#pragma unroll
      for (int kbh = 0; kbh < 2; ++kbh)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const char* a = sv + (32 * (2 * ks + kbh) + 16 * h) * RB + vrow_off + (((2 * b) ^ vx) << 4);
          part[2 * kbh + h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)a);
        }
      return i32x8{part[0][0], part[0][1], part[1][0], part[1][1],
                   part[2][0], part[2][1], part[3][0], part[3][1]};
    };
    __builtin_amdgcn_s_setprio(1);
    i32x8 va = vread(0);
#pragma unroll
    for (int i = 0; i < NKS * ND; ++i) {
      const i32x8 vn = i + 1 < NKS * ND ? vread(i + 1) : va;
      __builtin_amdgcn_sched_barrier(0);  // keep the next reads ahead of this MFMA
      oacc[i % ND] = mfma8_sab(va, P[i / ND], oacc[i % ND], sa, sb);
      va = vn;
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Ring of ST stages: tile t is copied during iteration t - PD into the stage
  // of tile t - ST, which every wave finished before the barrier that ended
  // iteration t - PD - 1 (with ping-pong halves the upper half reads tile
  // j - 1 in iteration j, hence PD = ST - 2).  Copies complete in order:
  // "tile j + 1 has landed" is vmcnt <= 2 CPT x (tiles issued after it).
  // The first tiles are issued before Q is read, so that both latencies
  // overlap; Q's loads are the newest, and draining them drains the copies.
  for (int t = 0; t < PD && t < nt; ++t) issue_tile(t);
  {  // a negative scale is moved into Q (flip the e4m3 sign bits, exact)
    const uint8_t* qr = qh + (size_t)min(myq, N - 1) * D + 32 * g;
    const int flip = p.scale_log2 < 0.f ? (int)0x80808080u : 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const i32x4 lo = *(const i32x4*)(qr + 64 * s), hi = *(const i32x4*)(qr + 64 * s + 16);
      qop[s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[s][e] ^= flip;
    }
    // drain: Q and the first tiles (16-byte register operands, which the
    // host pass of a kernel template also accepts)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const i32x4 a = {qop[s][0], qop[s][1], qop[s][2], qop[s][3]};
      const i32x4 b = {qop[s][4], qop[s][5], qop[s][6], qop[s][7]};
      asm volatile("" ::"v"(a), "v"(b));
    }
  }
  wait_vmcnt(0);
  __syncthreads();

  // Lower half (and 4-wave workgroups): scores, softmax and P V of tile j.
  // Upper half of an 8-wave workgroup: P V of tile j - 1, then scores and
  // softmax of tile j; its packed P~ and V scale wait across the barrier.
  const bool upper = PP && w >= NW / 2;
  f32x16 S[NKB];
  i32x8 P[NKS];
  int sa = 127, sb = 127;
  auto step = [&](int j, auto LAG) __attribute__((always_inline)) {
    const int st = j % ST;
    if (j + PD < nt) issue_tile(j + PD);
    if constexpr (!decltype(LAG)::value) {
      if (j <= jlast) {
        qk(st, S);
        sa = softmax(j, S, P, sb);
        pv(st, P, sa, sb);
      }
    } else {
      if (j >= 1 && j - 1 <= jlast) pv((j + ST - 1) % ST, P, sa, sb);
      if (j <= jlast) {
        qk(st, S);
        sa = softmax(j, S, P, sb);
      }
    }
    if (j + PD < nt) {  // steady state: tiles j + 2 .. j + PD may stay in flight
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * CPT * (PD - 1)) : "memory");
    } else {
      wait_vmcnt(2 * CPT * max(0, nt - 1 - (j + 1)));
    }
    __syncthreads();
  };
  // With ping-pong halves both run one extra iteration (j = nt): the upper
  // half does its last P V there, the lower half only meets the barrier.
  const int nsteps = PP ? nt + 1 : nt;
  if (upper) {
    for (int j = 0; j < nsteps; ++j) step(j, std::true_type());
  } else {
    for (int j = 0; j < nsteps; ++j) step(j, std::false_type());
  }

  // ---- epilogue: O = O~ / l, LSE = ln2 (m + log2 l) ----
  // A lane holds one query's O row in 8-byte pieces; each wave stages its 32
  // bf16 rows in LDS (the ring is idle after the last barrier) and writes
  // whole 2D-byte rows, 16-byte chunks XOR-swizzled by row.
  constexpr int ORB = D * 2, OCPR = ORB / 16;
  static_assert(NW * 32 * ORB <= ST * SB, "staging fits in the ring");
  char* stg = smem + w * (32 * ORB);
  const float lt = pair_sum(l);
  const float inv = 1.0f / (lt + E);  // E is the same on both lanes of a row
#pragma unroll
  for (int b = 0; b < ND; ++b)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint2 stv;
      stv.x = pack_bf16x2(oacc[b][4 * a] * inv, oacc[b][4 * a + 1] * inv);
      stv.y = pack_bf16x2(oacc[b][4 * a + 2] * inv, oacc[b][4 * a + 3] * inv);
      *(uint2*)(stg + ql * ORB + (((4 * b + a) ^ (ql & (OCPR - 1))) << 4) + 8 * g) = stv;
    }
  if (g == 0 && myq < N)
    p.lse[(size_t)bh * N + myq] = (m + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are staged
  __bf16* __restrict__ oh = (__bf16*)p.o + head;
#pragma unroll
  for (int it = 0; it < 32 * OCPR / 64; ++it) {
    const int idx = it * 64 + lane, row = idx / OCPR, ch = idx % OCPR;
    const i32x4 val = *(const i32x4*)(stg + row * ORB + ((ch ^ (row & (OCPR - 1))) << 4));
    const int grow = qrow0 + row;
    if (grow < N) *(i32x4*)(oh + (size_t)grow * D + ch * 8) = val;
  }
}

template <int D>
hipError_t launch_fp8_d(const Fp8Params& p, int causal, hipStream_t s) {
  const int nw = causal ? fp8_nw<D, true>() : fp8_nw<D, false>();
  Fp8Params q = p;
  q.nq = (p.N + 32 * nw - 1) / (32 * nw);
  const unsigned grid = (unsigned)(q.nq * p.BH);
  if (causal)
    hipLaunchKernelGGL((fwd_fp8<D, true>), dim3(grid), dim3(64 * nw), 0, s, q);
  else
    hipLaunchKernelGGL((fwd_fp8<D, false>), dim3(grid), dim3(64 * nw), 0, s, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, int d, int causal, hipStream_t s) {
  switch (d) {
    case 64: return launch_fp8_d<64>(p, causal, s);
    case 128: return launch_fp8_d<128>(p, causal, s);
    case 256: return launch_fp8_d<256>(p, causal, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
