// Fused exact attention forward for gfx950, fp16/bf16 inputs, d = 128, with
// the online softmax software-pipelined against the matrix products inside
// every wave.
//
// The method is that of "FlashAttention (HI)" (tiling, online softmax, one
// kernel writing only O and the logsumexp) with the non-matmul work kept off
// the matrix cores' critical path, the aim stated in "FlashAttention-2 (BN)"
// (section 1, fewer non-matrix operations) and "FlashAttention-3 (BN)"
// (overlapping softmax with the matrix products).  On CDNA4 a single wave can
// issue about one instruction every 4-5 cycles while one 32x32x16 MFMA keeps
// the matrix core busy for 32, so a wave that alternates its own MFMAs with
// vector work hides most of that work under its matrix products.
//
// Each wave owns 32 QB query rows; K and V stream through two separate
// ST-stage LDS rings of BC-key tiles.  Iteration j of a wave:
//   phase A: S(j+1) = K(j+1) Q^T on MFMA, interleaved with the second half of
//            the softmax of tile j (exp2, row sums, packing P(j) to 16 bits);
//   barrier: copies of K(j+ST) and V(j+ST-1) are issued into the stages that
//            every wave has finished reading;
//   phase B: O^T += V(j)^T P(j)^T on MFMA, interleaved with the first half of
//            the softmax of tile j+1 (row maximum, lazy running-max update,
//            the scaled and shifted exponent argument).
// Each phase has 16 MFMA slots; a slot holds one MFMA and the vector and LDS
// instructions issued under it, and scheduling barriers keep the slots in
// program order.  Score layout (S^T = K Q^T, one query per lane), key
// permutation, transposed V reads, chunk swizzle and lazy running max are
// those of fwd_wide.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kD = 128;         // head dimension
constexpr int kRB = kD * 2;     // bytes per K/V row
constexpr int kCPR = kD / 8;    // 16-byte chunks per row
constexpr int kNS = kD / 16;    // k-steps of K Q^T
constexpr int kND = kD / 32;    // 32-column blocks of O

// QB 32-row query blocks per wave, BC keys per tile, NW waves per workgroup,
// ST ring stages (each of K and V), OCC waves per SIMD the registers are
// budgeted for, KR / VR: K and V operands in flight.
//   Wide32: 32 rows per wave, 64-key tiles, two waves per SIMD (8-wave
//           workgroups) that run half an iteration apart;
template <int QB_, int BC_, int NW_, int ST_, int OCC_, int KR_, int VR_>
struct PipeCfg {
  static constexpr int QB = QB_, BC = BC_, NW = NW_, ST = ST_, OCC = OCC_, KR = KR_, VR = VR_;
};
using Wide32 = PipeCfg<1, 64, 8, 4, 2, 4, 3>;

template <int D>
constexpr bool swz_step4_is_xor1_p() {
  for (int g = 0; g < 2; ++g)
    for (int i = 0; i < 4; ++i)
      if (chunk_swz<D>(8 * g + i + 4) != (chunk_swz<D>(8 * g + i) ^ 1)) return false;
  return true;
}
static_assert(swz_step4_is_xor1_p<kD>(), "rows r and r + 4 differ in bit 0 of the swizzle");

#define FA_SLOT_END() __builtin_amdgcn_sched_barrier(0)

// Ties a value to this point of the program: IR passes may otherwise sink
// the vector work of a slot to the first use of its result, a whole phase
// later, which keeps 32 more values live and breaks the interleaving.
template <typename V>
__device__ __forceinline__ void pin(V& x) {
  asm volatile("" : "+v"(x));
}

template <typename T, bool CAUSAL, typename Cfg>
__global__ __launch_bounds__(64 * Cfg::NW) __attribute__((amdgpu_waves_per_eu(Cfg::OCC, Cfg::OCC)))
void fwd_pipe(FwdParams p) {
  constexpr int QB = Cfg::QB, BC = Cfg::BC, NW = Cfg::NW, ST = Cfg::ST, KR = Cfg::KR, VR = Cfg::VR;
  constexpr int WR = 32 * QB, BR = WR * NW;
  constexpr int TB = BC * kRB;                  // bytes per K or V tile
  constexpr int CPT = BC * kCPR / (64 * NW);    // copies per wave per tile and tensor
  constexpr int NKB = BC / 32;                  // 32-key blocks per tile
  constexpr int NK = NKB * kNS;                 // K operands per tile (each feeds QB MFMAs)
  constexpr int NV = (BC / 16) * kND;           // V^T operands per tile (each feeds QB MFMAs)
  constexpr int NSC = QB * NKB * 16;            // scores per lane per tile
  constexpr int SPQ = NKB * 16;                 // scores per lane and query block
  constexpr int VBASE = ST * TB;                // V ring after the K ring
  static_assert(NK * QB == 16 && NV * QB == 16, "16 MFMA slots per phase");
  static_assert(NSC == 32, "32 scores per lane and tile");
  static_assert(CPT * 64 * NW == BC * kCPR, "tile must split evenly over the waves");
  static_assert(ST % 2 == 0 && ST >= 4 && ST <= 8, "the loop is unrolled over the ring");
  static_assert(2 * CPT * (ST - 3) <= 15, "copies in flight at a barrier");
  __shared__ __attribute__((aligned(1024))) char smem[2 * ST * TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  int bh, qt;
  decode_block(blockIdx.x, p.BH, p.nq, CAUSAL, bh, qt, 0);

  const size_t head = (size_t)bh * N * kD;
  const T* __restrict__ qh = (const T*)p.q + head;
  const size_t kvhead = (size_t)kv_head(p, bh) * N * kD;
  const T* __restrict__ kh = (const T*)p.k + kvhead;
  const T* __restrict__ vh = (const T*)p.v + kvhead;

  // With two waves per SIMD (w and w + NW/2) and causal masking, each SIMD
  // gets one early and one late row block so the diagonal work spreads evenly.
  const int rblk = (CAUSAL && NW == 8 && w >= NW / 2) ? (NW + NW / 2 - 1 - w) : w;
  const int qrow0 = qt * BR + rblk * WR;
  const float c = fmaxf(fabsf(p.scale_log2), 1.0e-30f);

  const int kv_end = CAUSAL ? min(N, (qt + 1) * BR) : N;
  const int nt = (kv_end + BC - 1) / BC;
  const int jlast = qrow0 >= N ? -1 : (CAUSAL ? min(nt - 1, (qrow0 + WR - 1) / BC) : nt - 1);

  // ---- tile copies (wave w, instruction u fills LDS slots (u NW + w) 64 + lane) ----
  uint32_t ld_voff[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int s = (u * NW + w) * 64 + lane, row = s / kCPR, ch = s % kCPR;
    ld_voff[u] = row * kRB + (ch ^ chunk_swz<kD>(row)) * 16;
  }
  const uint32_t head_bytes = (uint32_t)N * kRB;
  const __amdgpu_buffer_rsrc_t kbuf = make_rsrc(kh, head_bytes);
  const __amdgpu_buffer_rsrc_t vbuf = make_rsrc(vh, head_bytes);
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  // Tiles past the end of the head read as zeros (hardware range check), so
  // every barrier issues the same number of copies and the wait counts stay
  // constant.
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    const uint32_t dst = smem_base + (uint32_t)(t % ST) * TB + w * 1024;
    const uint32_t t0 = (uint32_t)t * TB;
#pragma unroll
    for (int u = 0; u < CPT; ++u) buf_dma16(kbuf, t0 + ld_voff[u], dst + u * NW * 1024);
  };
  auto issue_v = [&](int t) __attribute__((always_inline)) {
    const uint32_t dst = smem_base + VBASE + (uint32_t)(t % ST) * TB + w * 1024;
    const uint32_t t0 = (uint32_t)t * TB;
#pragma unroll
    for (int u = 0; u < CPT; ++u) buf_dma16(vbuf, t0 + ld_voff[u], dst + u * NW * 1024);
  };

  // ---- LDS read geometry (as in fwd_wide) ----
  const int krow = swap_bits23(ql);
  const int kbase = krow * kRB + ((g ^ chunk_swz<kD>(krow)) << 4);
  const int trow = (lane & 15) >> 2;
  const int vrow = 8 * g + trow;
  const int vaddr0 = vrow * kRB + 8 * (lane & 1) +
                     (((2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ chunk_swz<kD>(vrow)) << 4);
  const int vaddr1 = vaddr0 ^ (4 * kRB + 16);
  // Per-lane LDS base addresses, kept in registers: the ring stage and tile
  // offsets then fit the instructions' 16-bit immediate offsets.
  uint32_t kaddr[kNS], vaddr[2][4];
#pragma unroll
  for (int s2 = 0; s2 < kNS; ++s2) {
    kaddr[s2] = smem_base + (uint32_t)(kbase ^ (s2 << 5));
    pin(kaddr[s2]);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    vaddr[0][b] = smem_base + VBASE + (uint32_t)(vaddr0 ^ (b << 6));
    vaddr[1][b] = smem_base + VBASE + (uint32_t)(vaddr1 ^ (b << 6));
    pin(vaddr[0][b]);
    pin(vaddr[1][b]);
  }

  // K operand r of a tile (r = s NKB + kb: k-step s, key block kb).
  auto kread = [&](int stage, int r) __attribute__((always_inline)) -> i32x4 {
    return *(const i32x4*)((lds_void*)(uintptr_t)(kaddr[r / NKB] + stage * TB + (r % NKB) * 32 * kRB));
  };
  // V^T operand r of a tile (r = 4 kh + b: 16-key group kh, column block b).
  typedef i16x4 VHalf[2];
  auto vread = [&](int stage, int r, VHalf& v) __attribute__((always_inline)) {
    const uint32_t off = stage * TB + (r >> 2) * 16 * kRB;
    const int b = r & 3;
    v[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[0][b] + off));
    v[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vaddr[1][b] + off));
  };
  auto vjoin = [](const VHalf& v) __attribute__((always_inline)) -> i32x4 {
    const i16x8 v8 = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
    return __builtin_bit_cast(i32x4, v8);
  };
  i32x4 qop[QB][kNS];
  f32x16 oacc[QB][kND];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int b = 0; b < kND; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][b][r] = 0.f;
  // l: fp32 sum of P (for the LSE).  E: sum over tiles of the rounding
  // error of each tile's largest P, in the units of l; O is divided by
  // l + E, so the weight of a row's dominant key (its tile's largest P) is
  // counted in the divisor exactly as it entered P V and such a row gets
  // that key's value row back without the rounding of its weight.
  float m[QB], l[QB], E[QB], alpha[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = kMInit;
    l[qb] = 0.f;
    E[qb] = 0.f;
    alpha[qb] = 1.f;
  }
  bool rescale_pending = false;

  typedef f32x16 STile[QB][NKB];
  STile sa, sb;             // score tiles of alternate iterations
  i32x4 pk[QB][NKB][2];     // packed P of the tile being multiplied by V
  i32x4 kop[KR];            // K operands in flight (ring)
  VHalf vop[VR];            // V^T operands in flight (ring)

  // Score f of a lane (f < 32): query block f / SPQ, key block, register.
#define FA_SREF(S, f) S[(f) / SPQ][((f) % SPQ) / 16][(f) % 16]

  // Hidden keys of tile t become -inf (tiles crossing the diagonal or N).
  auto mask = [&](int t, STile& S) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int lim = CAUSAL ? min(qrow0 + 32 * qb + ql, N - 1) : N - 1;
      const int rel = lim - t * BC - 8 * g;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          S[qb][kb][r] = (32 * kb + 16 * (r >> 3) + (r & 7) <= rel) ? S[qb][kb][r] : kNegInf;
    }
  };
  auto needs_mask = [&](int t) __attribute__((always_inline)) {
    return (t * BC + BC > N) || (CAUSAL && t * BC + BC - 1 > qrow0);
  };

  // Lazy running-max update of query block qb from its tile maximum mx
  // (lane-local; combined with the partner lane here), and the rounding
  // error of the tile's largest P (the same exponent argument as its
  // exponential: one FMA of the raw score).
  auto max_update = [&](int qb, float mx) __attribute__((always_inline)) {
    const float mxp = pair_max(mx);
    const float mt = mxp * c;
    const float mnew = (mt > m[qb] + kLazy) ? mt : m[qb];
    alpha[qb] = __builtin_amdgcn_exp2f(m[qb] - mnew);
    m[qb] = mnew;
    const float pm = __builtin_amdgcn_exp2f(__builtin_fmaf(mxp, c, -mnew));
    E[qb] = __builtin_fmaf(E[qb], alpha[qb], Half<T>::round1(pm) - pm);
  };

  // ================= prologue =================
  // Copies: K0, then Q (registers), then K(t), V(t-1) for t = 1 .. ST-1 (the
  // groups the barriers before iteration 0 would have issued).
  issue_k(0);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const T* qr = qh + (size_t)min(qrow0 + 32 * qb + ql, N - 1) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < kNS; ++s) qop[qb][s] = *(const i32x4*)(qr + 16 * s);
  }
#pragma unroll
  for (int t = 1; t < ST; ++t) {
    issue_k(t);
    issue_v(t - 1);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < kNS; ++s) asm volatile("" ::"v"(qop[qb][s]));  // Q has landed
  if (p.scale_log2 < 0.f) {  // a negative scale moves into Q's sign (exact)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < kNS; ++s) qop[qb][s] ^= (int)0x80008000u;
  }
  // Copies land in issue order: once only the last ST - 2 groups (K(t), V(t-1)
  // for t = 2 .. ST-1) may be in flight, K0, K1 and V0 are in LDS, which is
  // all that S(0) and phase A of iteration 0 read; the first barrier waits
  // for K2 and V1.
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * CPT * (ST - 2)) : "memory");
  __syncthreads();

  if (jlast >= 0) {
    // S(0), its maximum and exponent arguments; first K(1) operands.
    const f32x16 zero = {};
#pragma unroll
    for (int r = 0; r < NK; ++r) {
      const i32x4 kv = kread(0, r);
      const int s = r / NKB, kb = r % NKB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sa[qb][kb] = Half<T>::mfma(kv, qop[qb][s], s == 0 ? zero : sa[qb][kb]);
    }
    if (needs_mask(0)) mask(0, sa);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = sa[qb][0][0];
#pragma unroll
      for (int f = 1; f < SPQ; ++f) mx = fmaxf(mx, sa[qb][f / 16][f % 16]);
      max_update(qb, mx);
      alpha[qb] = 1.f;  // O and l are still zero
      const float negm = -m[qb];
#pragma unroll
      for (int f = 0; f < SPQ; ++f) sa[qb][f / 16][f % 16] = __builtin_fmaf(sa[qb][f / 16][f % 16], c, negm);
    }
#pragma unroll
    for (int i = 0; i < KR - 1; ++i) kop[i] = kread(1 % ST, i);  // harmless past the last tile
  }

  // ================= main loop =================
  // Phase A of iteration j (stage of K(j+1): KS, of V(j): VS).  SC holds the
  // exponent arguments of tile j, SN receives S(j+1).  DO_QK: tile j+1
  // exists for this wave.
  auto phase_a = [&](auto KS, auto VS, auto DO_QK, STile& SC, STile& SN) __attribute__((always_inline)) {
    constexpr int ks = decltype(KS)::value, vs = decltype(VS)::value;
    constexpr bool qk = decltype(DO_QK)::value;
    if (rescale_pending) {  // the running max moved at tile j: rescale O first
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int b = 0; b < kND; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][b][r] *= alpha[qb];
    }
    const f32x16 zero = {};
    constexpr int CH = 4 / QB;  // partial row-sum chains per query block
    float rs[QB][CH];
    // pair q: scores 2q and 2q + 1 of the lane -> one packed P register
    auto expq = [&](int q) __attribute__((always_inline)) {
      float x0 = __builtin_amdgcn_exp2f(FA_SREF(SC, 2 * q));
      float x1 = __builtin_amdgcn_exp2f(FA_SREF(SC, 2 * q + 1));
      pin(x0);
      pin(x1);
      FA_SREF(SC, 2 * q) = x0;
      FA_SREF(SC, 2 * q + 1) = x1;
    };
    auto sumcvt = [&](int q) __attribute__((always_inline)) {
      const int f = 2 * q, qb = f / SPQ, kb = (f % SPQ) / 16, e = (f % 16) / 2;
      const int qq = q % (SPQ / 2), ch = qq % CH;
      const float s2 = FA_SREF(SC, f) + FA_SREF(SC, f + 1);
      rs[qb][ch] = qq < CH ? s2 : rs[qb][ch] + s2;
      int pv2 = (int)Half<T>::pack2(FA_SREF(SC, f), FA_SREF(SC, f + 1));
      pin(rs[qb][ch]);
      pin(pv2);
      pk[qb][kb][e >> 2][e & 3] = pv2;
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (qk) {
        const int r = i / QB, qb = i % QB, s = r / NKB, kb = r % NKB;
        if (qb == 0 && r + KR - 1 < NK) kop[(r + KR - 1) % KR] = kread(ks, r + KR - 1);
        SN[qb][kb] = Half<T>::mfma(kop[r % KR], qop[qb][s], s == 0 ? zero : SN[qb][kb]);
      }
      expq(i);
      if (i >= 1) sumcvt(i - 1);
      if (i >= 16 - (VR - 1)) vread(vs, i - (16 - (VR - 1)), vop[i - (16 - (VR - 1))]);  // first V(j) operands
      FA_SLOT_END();
    }
    sumcvt(15);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float t = rs[qb][0];
#pragma unroll
      for (int ch = 1; ch < CH; ++ch) t += rs[qb][ch];
      l[qb] = __builtin_fmaf(l[qb], alpha[qb], t);
      pin(l[qb]);
    }
  };

  // Phase B of iteration j (stage of V(j): VS; stage of K(j+2): K2S).
  // DO_SM: tile j+1 exists (softmax head on SN).
  auto phase_b = [&](int j, auto VS, auto K2S, auto DO_SM, STile& SN) __attribute__((always_inline)) {
    constexpr int vs = decltype(VS)::value, k2s = decltype(K2S)::value;
    constexpr bool sm = decltype(DO_SM)::value;
    if constexpr (sm) {
      if (needs_mask(j + 1)) mask(j + 1, SN);
    }
    float mx[QB], negm[QB];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = i / QB, qb = i % QB;
      if (qb == 0 && r + VR - 1 < NV) vread(vs, r + VR - 1, vop[(r + VR - 1) % VR]);
      {
        const int kh = r >> 2, b = r & 3;  // kh: 16-key group of the tile
        oacc[qb][b] = Half<T>::mfma(vjoin(vop[r % VR]), pk[qb][kh >> 1][kh & 1], oacc[qb][b]);
      }
      if constexpr (sm) {
        if (i < 8) {  // row maxima: 4 scores per slot
          const int f = 4 * i, q = f / SPQ;
          float a = (f % SPQ == 0) ? fmaxf(FA_SREF(SN, f), FA_SREF(SN, f + 1))
                                   : fmaxf(fmaxf(mx[q], FA_SREF(SN, f)), FA_SREF(SN, f + 1));
          a = fmaxf(fmaxf(a, FA_SREF(SN, f + 2)), FA_SREF(SN, f + 3));
          pin(a);
          mx[q] = a;
        } else if (i == 8) {
#pragma unroll
          for (int q = 0; q < QB; ++q) {
            max_update(q, mx[q]);
            negm[q] = -m[q];
            pin(negm[q]);
          }
        }
        if (i >= 8) {  // exponent arguments: 4 per slot
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int f = 4 * (i - 8) + e;
            float t = __builtin_fmaf(FA_SREF(SN, f), c, negm[f / SPQ]);
            pin(t);
            FA_SREF(SN, f) = t;
          }
        }
      }
      if (i >= 16 - (KR - 1)) {  // first K(j+2) operands; harmless past the last tile
        const int k2 = i - (16 - (KR - 1));
        kop[k2] = kread(k2s, k2);
      }
      FA_SLOT_END();
    }
    if constexpr (sm) {
      // rows whose running max moved need O rescaled before P(j+1) V(j+1)
      bool any = false;
#pragma unroll
      for (int q = 0; q < QB; ++q) any = any || alpha[q] != 1.0f;
      rescale_pending = __builtin_amdgcn_ballot_w64(any) != 0;
    }
  };

  // Barrier between the phases of iteration j: own copies of K(j+2) and
  // V(j+1) have landed (only those of the ST - 3 previous barriers may be in
  // flight), and every wave has finished reading K(j) (phase A of iteration
  // j - 1, or the prologue) and V(j-1); refill those two stages.
  auto barrier_step = [&](int j) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * CPT * (ST - 3)) : "memory");
    __builtin_amdgcn_s_barrier();
    issue_k(j + ST);
    issue_v(j + ST - 1);
  };

  // Full iteration (tiles j and j + 1 exist for this wave) or last
  // iteration (tile j only), with compile-time ring stages u = j % ST.  With
  // two waves per SIMD, waves 0 .. NW/2-1 do phase A, barrier, phase B, and
  // the others barrier, phase A, phase B: between two barriers one wave of
  // each SIMD is in its exponential-heavy phase A while the other is in its
  // LDS-heavy phase B.
  const bool lag = NW == 8 && w >= NW / 2;  // wave-uniform
  auto step = [&](int j, auto U, auto FULL) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    using F = decltype(FULL);
    using KS = std::integral_constant<int, (u + 1) % ST>;
    using VS = std::integral_constant<int, u>;
    using K2S = std::integral_constant<int, (u + 2) % ST>;
    if (lag) barrier_step(j);
    if constexpr (u & 1) phase_a(KS(), VS(), F(), sb, sa);
    else phase_a(KS(), VS(), F(), sa, sb);
    if (!lag) barrier_step(j);
    if constexpr (u & 1) phase_b(j, VS(), K2S(), F(), sa);
    else phase_b(j, VS(), K2S(), F(), sb);
  };
  using TF = std::true_type;
  using FF = std::false_type;
  // Every wave passes nt barriers: jlast full iterations, one last
  // iteration, then barriers only (rows whose keys all lie before the
  // workgroup's last tiles, or rows past N).
  auto unrolled = [&](int j0, auto FULL, int count) __attribute__((always_inline)) {
    // count (< ST + 1) iterations starting at j0 (j0 % ST == 0)
    step(j0, std::integral_constant<int, 0>(), FULL);
    if (count > 1) step(j0 + 1, std::integral_constant<int, 1>(), FULL);
    if (count > 2) step(j0 + 2, std::integral_constant<int, 2 % ST>(), FULL);
    if (count > 3) step(j0 + 3, std::integral_constant<int, 3 % ST>(), FULL);
    if constexpr (ST > 4) {
      if (count > 4) step(j0 + 4, std::integral_constant<int, 4 % ST>(), FULL);
      if (count > 5) step(j0 + 5, std::integral_constant<int, 5 % ST>(), FULL);
    }
    if constexpr (ST > 6) {
      if (count > 6) step(j0 + 6, std::integral_constant<int, 6 % ST>(), FULL);
      if (count > 7) step(j0 + 7, std::integral_constant<int, 7 % ST>(), FULL);
    }
  };
  int j = 0;
  for (; j + ST <= jlast; j += ST) unrolled(j, TF(), ST);
  const int rem = jlast - j;  // full iterations left (0 .. ST-1); -1: none at all
  if (rem >= 1) unrolled(j, TF(), rem);
  switch (rem) {
    case 0: step(j, std::integral_constant<int, 0>(), FF()); break;
    case 1: step(j + 1, std::integral_constant<int, 1>(), FF()); break;
    case 2: step(j + 2, std::integral_constant<int, 2 % ST>(), FF()); break;
    case 3: step(j + 3, std::integral_constant<int, 3 % ST>(), FF()); break;
    case 4: if constexpr (ST > 4) step(j + 4, std::integral_constant<int, 4 % ST>(), FF()); break;
    case 5: if constexpr (ST > 5) step(j + 5, std::integral_constant<int, 5 % ST>(), FF()); break;
    case 6: if constexpr (ST > 6) step(j + 6, std::integral_constant<int, 6 % ST>(), FF()); break;
    case 7: if constexpr (ST > 7) step(j + 7, std::integral_constant<int, 7 % ST>(), FF()); break;
    default: break;
  }
  for (j = jlast + 1; j < nt; ++j) barrier_step(j);

  // ================= epilogue: O = O^T / (l + E), LSE = ln2 (m + log2 l) =================
  // Every copy (including the zero-filled ones past the end) has landed and
  // every wave is done with the rings before they become the staging area.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  static_assert(NW * 32 * kRB <= 2 * ST * TB, "staging fits in the rings");
  char* stg = smem + w * (32 * kRB);
  T* __restrict__ oh = (T*)p.o + head;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int myq = qrow0 + 32 * qb + ql;
    const float lt = pair_sum(l[qb]);
    const float inv = 1.0f / (lt + E[qb]);  // E is the same on both lanes of a row
#pragma unroll
    for (int b = 0; b < kND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 stv;
        stv.x = Half<T>::pack2(oacc[qb][b][4 * a] * inv, oacc[qb][b][4 * a + 1] * inv);
        stv.y = Half<T>::pack2(oacc[qb][b][4 * a + 2] * inv, oacc[qb][b][4 * a + 3] * inv);
        *(uint2*)(stg + ql * kRB + (((4 * b + a) ^ (ql & (kCPR - 1))) << 4) + 8 * g) = stv;
      }
    if (g == 0 && myq < N)
      p.lse[(size_t)bh * N + myq] = (m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int it = 0; it < 32 * kCPR / 64; ++it) {
      const int idx = it * 64 + lane, row = idx / kCPR, ch = idx % kCPR;
      const i32x4 val = *(const i32x4*)(stg + row * kRB + ((ch ^ (row & (kCPR - 1))) << 4));
      const int grow = qrow0 + 32 * qb + row;
      if (grow < N) *(i32x4*)(oh + (size_t)grow * kD + ch * 8) = val;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next block's writes
  }
}

#undef FA_SREF

template <typename T, bool CAUSAL, typename Cfg>
hipError_t launch_pipe(const FwdParams& p, hipStream_t stream) {
  constexpr int BR = 32 * Cfg::QB * Cfg::NW;
  FwdParams q = p;
  q.nq = (p.N + BR - 1) / BR;
  const unsigned grid = (unsigned)(q.nq * p.BH);
  hipLaunchKernelGGL((fwd_pipe<T, CAUSAL, Cfg>), dim3(grid), dim3(64 * Cfg::NW), 0, stream, q);
  return hipGetLastError();
}

#ifndef FA_PIPE_CFG
#define FA_PIPE_CFG Wide32
#endif

}  // namespace

hipError_t launch_fwd_pipe(const FwdParams& p, int d, int causal, int is_bf16, hipStream_t s) {
  if (d != kD) return hipErrorInvalidValue;
  using C = FA_PIPE_CFG;
  if (is_bf16) return causal ? launch_pipe<__bf16, true, C>(p, s) : launch_pipe<__bf16, false, C>(p, s);
  return causal ? launch_pipe<_Float16, true, C>(p, s) : launch_pipe<_Float16, false, C>(p, s);
}

}  // namespace fa
