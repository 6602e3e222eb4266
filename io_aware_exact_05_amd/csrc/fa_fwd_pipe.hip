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
//
// Work items.  When the grid has at least as many pairs of query tiles as
// there are CUs, a workgroup takes two (the parallelism over query tiles of
// "FlashAttention-2 (BN)", section 2): with causal masking tiles i and
// nq - 1 - i of one head, so that every workgroup's load is nq + 1 tiles'
// worth of key tiles; without it the same tile of two heads of one XCD.
// The second tile's first ST K tiles and ST - 1 V tiles are copied by the
// first tile's last barriers, so its start costs only its Q load; each wave
// writes its output rows through its own LDS staging area, apart from the
// rings.
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
//           workgroups) that run half an iteration apart; four K and four V
//           operands in flight (248 registers; three V operands measured
//           0.7% slower, two 2%);
template <int QB_, int BC_, int NW_, int ST_, int OCC_, int KR_, int VR_>
struct PipeCfg {
  static constexpr int QB = QB_, BC = BC_, NW = NW_, ST = ST_, OCC = OCC_, KR = KR_, VR = VR_;
};
using Wide32 = PipeCfg<1, 64, 8, 4, 2, 4, 4>;

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

template <typename T, bool CAUSAL, bool PAIR, typename Cfg>
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
  constexpr int SGB = 32 * kRB / 2;             // staging bytes per wave: 32 rows, half of d
  static_assert(NK * QB == 16 && NV * QB == 16, "16 MFMA slots per phase");
  static_assert(NSC == 32, "32 scores per lane and tile");
  static_assert(CPT * 64 * NW == BC * kCPR, "tile must split evenly over the waves");
  static_assert(ST % 2 == 0 && ST >= 4 && ST <= 8, "the loop is unrolled over the ring");
  static_assert(2 * CPT * (ST - 3) <= 15, "copies in flight at a barrier");
  static_assert(!PAIR || (BR / BC) % ST == 0, "a causal first item spans a whole number of ring turns");
  // K ring, V ring, then one output staging area per wave, apart from the
  // rings so that a wave can write out one query tile while the copies of
  // the next tile's first K/V tiles are still landing.
  __shared__ __attribute__((aligned(1024))) char smem[2 * ST * TB + NW * SGB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;
  const int N = p.N;
  // Work items: one query tile, or (PAIR) two.  With causal masking, query
  // tiles i and nq - 1 - i of one head, i first: every pair holds nq + 1
  // tiles' worth of key tiles, so all workgroups carry the same load.
  // Without masking (head count a multiple of 16), the same query tile of
  // two heads of one XCD: an XCD's workgroups first run every tile of half
  // of its heads, then every tile of the other half, so each head's K and V
  // still stream from HBM once, shared in L2 by its query tiles.
  int bh, qt, bh2 = -1, qt2 = -1;
  if constexpr (PAIR) {
    if constexpr (CAUSAL) {
      int pi;
      decode_block(blockIdx.x, p.BH, (p.nq + 1) / 2, false, bh, pi, 0);
      qt = pi;
      if (p.nq - 1 - pi != pi) {
        bh2 = bh;
        qt2 = p.nq - 1 - pi;
      }
    } else {
      const int hx = p.BH >> 3, loc = blockIdx.x >> 3;
      bh = (blockIdx.x & 7) * hx + loc / p.nq;
      qt = loc % p.nq;
      bh2 = bh + hx / 2;
      qt2 = qt;
    }
  } else {
    decode_block(blockIdx.x, p.BH, p.nq, CAUSAL, bh, qt, 0);
  }

  // With two waves per SIMD (w and w + NW/2) and causal masking, each SIMD
  // gets one early and one late row block so the diagonal work spreads evenly.
  const int rblk = (CAUSAL && NW == 8 && w >= NW / 2) ? (NW + NW / 2 - 1 - w) : w;
  const float c = fmaxf(fabsf(p.scale_log2), 1.0e-30f);

  // Per-item geometry: first query row of this wave, key tiles of the
  // workgroup (nt) and of this wave (jlast: its last key tile, -1: none).
  int qrow0, nt, jlast;
  auto set_item = [&](int t) __attribute__((always_inline)) {
    qrow0 = t * BR + rblk * WR;
    const int kv_end = CAUSAL ? min(N, (t + 1) * BR) : N;
    nt = (kv_end + BC - 1) / BC;
    jlast = qrow0 >= N ? -1 : (CAUSAL ? min(nt - 1, (qrow0 + WR - 1) / BC) : nt - 1);
  };
  set_item(qt);
  bool has_next = qt2 >= 0;  // wave-uniform

  // ---- tile copies (wave w, instruction u fills LDS slots (u NW + w) 64 + lane) ----
  // Per-lane byte offsets of the copies (ld_voff) and LDS base addresses of
  // the K and V^T operand reads (kaddr, vaddr), kept in registers: the ring
  // stage and tile offsets then fit the instructions' 16-bit immediate
  // offsets.  Computed afresh for each work item from a lane index the
  // compiler cannot see through, so none of them stays live across items.
  uint32_t ld_voff[CPT], kaddr[kNS], vaddr[2][4];
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto set_addrs = [&]() __attribute__((always_inline)) {
    int ln = lane;
    pin(ln);
    const int lq = ln & 31, lg = ln >> 5;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int s = (u * NW + w) * 64 + ln, row = s / kCPR, ch = s % kCPR;
      ld_voff[u] = row * kRB + (ch ^ chunk_swz<kD>(row)) * 16;
    }
    const int krow = swap_bits23(lq);
    const int kbase = krow * kRB + ((lg ^ chunk_swz<kD>(krow)) << 4);
    const int trow = (ln & 15) >> 2;
    const int vrow = 8 * lg + trow;
    const int vaddr0 = vrow * kRB + 8 * (ln & 1) +
                       (((2 * ((ln >> 4) & 1) + ((ln & 3) >> 1)) ^ chunk_swz<kD>(vrow)) << 4);
    const int vaddr1 = vaddr0 ^ (4 * kRB + 16);
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
  };
  set_addrs();
  // Buffer resources over one head's rows: O and the logsumexp of the
  // current item; K and V (of the current item and of the next one) get one
  // per copied tile, starting at the tile (see issue_k).
  const uint32_t head_bytes = (uint32_t)N * kRB;
  const T* qh;
  __amdgpu_buffer_rsrc_t obuf, lbuf;
  const T *kp, *vp, *kp_n, *vp_n;
  auto kv_rsrc = [&](int h, const T*& kr, const T*& vr) __attribute__((always_inline)) {
    const size_t kvhead = (size_t)kv_head(p, h) * N * kD;
    kr = (const T*)p.k + kvhead;
    vr = (const T*)p.v + kvhead;
  };
  auto set_head = [&](int h) __attribute__((always_inline)) {
    const size_t head = (size_t)h * N * kD;
    qh = (const T*)p.q + head;
    obuf = make_rsrc((const T*)p.o + head, head_bytes);
    lbuf = make_rsrc(p.lse + (size_t)h * N, (uint32_t)N * 4u);
  };
  set_head(bh);
  kv_rsrc(bh, kp, vp);
  if constexpr (PAIR) {
    if (has_next) kv_rsrc(bh2, kp_n, vp_n);
  }
  // Tile t of the current item sits in ring stage t % ST.  Past the item's
  // last tile the copies continue with the next item's first tiles (the
  // first item's tile count is a multiple of ST, so they land in the stages
  // the next item expects), or, after the last item, read as zeros
  // (hardware range check): every barrier issues the same number of copies
  // and the wait counts stay constant.  Each tile's copies go through a
  // resource that starts at the tile and ends with the head (empty past
  // it), so the per-lane offsets ld_voff serve every tile unchanged: the
  // tile's offset is scalar work, not a vector add per copy.
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    const uint32_t dst = smem_base + (uint32_t)(t % ST) * TB + w * 1024;
    const bool nx = PAIR && t >= nt && has_next;
    const uint32_t t0 = (uint32_t)(nx ? t - nt : t) * TB;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(nx ? kp_n : kp, head_bytes, t0);
#pragma unroll
    for (int u = 0; u < CPT; ++u) buf_dma16(r, ld_voff[u], dst + u * NW * 1024);
  };
  auto issue_v = [&](int t) __attribute__((always_inline)) {
    const uint32_t dst = smem_base + VBASE + (uint32_t)(t % ST) * TB + w * 1024;
    const bool nx = PAIR && t >= nt && has_next;
    const uint32_t t0 = (uint32_t)(nx ? t - nt : t) * TB;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(nx ? vp_n : vp, head_bytes, t0);
#pragma unroll
    for (int u = 0; u < CPT; ++u) buf_dma16(r, ld_voff[u], dst + u * NW * 1024);
  };

  // LDS read geometry (as in fwd_wide): see set_addrs.

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
  // l: fp32 sum of P (for the LSE).  E: sum over tiles of the rounding
  // error of each tile's largest P, in the units of l; O is divided by
  // l + E, so the weight of a row's dominant key (its tile's largest P) is
  // counted in the divisor exactly as it entered P V and such a row gets
  // that key's value row back without the rounding of its weight.
  float m[QB], l[QB], E[QB], alpha[QB];
  bool rescale_pending;
  auto reset_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int b = 0; b < kND; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][b][r] = 0.f;
      m[qb] = kMInit;
      l[qb] = 0.f;
      E[qb] = 0.f;
      alpha[qb] = 1.f;
    }
    rescale_pending = false;
  };
  // Q rows of the wave's query blocks starting at row q0 (rows past N
  // repeat row N - 1; their results are never stored).
  auto load_q = [&](int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const T* qr = qh + (size_t)min(q0 + 32 * qb + ql, N - 1) * kD + 8 * g;
#pragma unroll
      for (int s = 0; s < kNS; ++s) qop[qb][s] = *(const i32x4*)(qr + 16 * s);
    }
  };

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
  // K0, K1, V0 (what S(0) and phase A of iteration 0 read) and Q are waited
  // for before the copies of K(t), V(t-1), t = 2 .. ST-1 (the groups the
  // barriers before iteration 0 would have issued) start: the compiler's
  // wait for Q counts only the loads it knows of, so later copies would be
  // waited for as well.  The first barrier waits for K2 and V1.
  auto q_landed = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < kNS; ++s) asm volatile("" ::"v"(qop[qb][s]));  // the compiler waits here
    if (p.scale_log2 < 0.f) {  // a negative scale moves into Q's sign (exact)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int s = 0; s < kNS; ++s) qop[qb][s] ^= (int)0x80008000u;
    }
  };
  issue_k(0);
  issue_k(1);
  issue_v(0);
  load_q(qrow0);
  q_landed();
  __syncthreads();
#pragma unroll
  for (int t = 2; t < ST; ++t) {
    issue_k(t);
    issue_v(t - 1);
  }

  // ================= work items =================
  auto run_item = [&]() __attribute__((always_inline)) {
  if constexpr (PAIR) set_addrs();
  // The previous item's score tiles and operands are dead; without this the
  // compiler keeps them live into this item (it cannot tell that every read
  // below follows a write of this item).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      asm volatile("" : "=v"(sa[qb][kb]));
      asm volatile("" : "=v"(sb[qb][kb]));
      asm volatile("" : "=v"(pk[qb][kb][0]));
      asm volatile("" : "=v"(pk[qb][kb][1]));
    }
#pragma unroll
  for (int i = 0; i < KR; ++i) asm volatile("" : "=v"(kop[i]));
#pragma unroll
  for (int i = 0; i < VR; ++i) {
    asm volatile("" : "=v"(vop[i][0]));
    asm volatile("" : "=v"(vop[i][1]));
  }
  reset_rows();
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

  // After the last item only the zero-filled copies of the last barriers
  // are in flight: they land before the workgroup's LDS is released.
  if (!has_next) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ================= epilogue: O = O^T / (l + E), LSE = ln2 (m + log2 l) =================
  // Each wave stages its rows in its own LDS area, half of d at a time, and
  // stores whole half rows.  Buffer stores with a resource over this head's
  // rows: the range check drops rows past N.  The stores are marked
  // non-temporal (nothing in this launch reads O back), which measured
  // 1-3% faster launches back to back than stores left in L2.
  constexpr int kNT = 2;  // cache-policy operand: nt
  char* stg = smem + 2 * ST * TB + w * SGB;
  constexpr int HRB = kRB / 2, HC = kCPR / 2;  // bytes and 16-byte chunks per half row
  int eln = lane;  // as in set_addrs: no offset below is shared between items
  pin(eln);
  const int eq = eln & 31, eg = eln >> 5;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r0 = qrow0 + 32 * qb;
    const float lt = pair_sum(l[qb]);
    const float inv = 1.0f / (lt + E[qb]);  // E is the same on both lanes of a row
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int bb = 0; bb < kND / 2; ++bb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int b = h * (kND / 2) + bb;
          uint2 stv;
          stv.x = Half<T>::pack2(oacc[qb][b][4 * a] * inv, oacc[qb][b][4 * a + 1] * inv);
          stv.y = Half<T>::pack2(oacc[qb][b][4 * a + 2] * inv, oacc[qb][b][4 * a + 3] * inv);
          *(uint2*)(stg + eq * HRB + (((4 * bb + a) ^ (eq & (HC - 1))) << 4) + 8 * eg) = stv;
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < 32 * HC / 64; ++it) {
        const int idx = it * 64 + eln, row = idx / HC, ch = idx % HC;
        const i32x4 val = *(const i32x4*)(stg + row * HRB + ((ch ^ (row & (HC - 1))) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(val, obuf, (uint32_t)(r0 + row) * kRB + h * HRB + ch * 16, 0, kNT);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next half's writes
    }
    const float lse = (m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, lse), lbuf, (uint32_t)(r0 + eq) * 4u, 0, kNT);
  }
  };
  run_item();
  if constexpr (PAIR) {
    if (has_next) {
      set_item(qt2);
      set_head(bh2);
      kp = kp_n;
      vp = vp_n;
      has_next = false;
      load_q(qrow0);
      q_landed();
      run_item();
    }
  }
}

#undef FA_SREF

// Two query tiles go to one workgroup when that does not add a round of
// workgroups per CU (the pairs' rounds take two items' time); without
// masking, when the head count is a multiple of 16 (two heads per pair,
// same XCD) and a tile's key tiles fill whole turns of the ring.
template <typename Cfg>
bool pipe_pairs(const FwdParams& p, int nq, bool causal) {
  if (causal ? nq < 2 : (p.BH % 16 != 0 || ((p.N + Cfg::BC - 1) / Cfg::BC) % Cfg::ST != 0)) return false;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return false;
  const long long items = (long long)nq * p.BH;
  const long long pairs = causal ? (long long)((nq + 1) / 2) * p.BH : items / 2;
  return 2 * ((pairs + cus - 1) / cus) <= (items + cus - 1) / cus;
}

template <typename T, bool CAUSAL, typename Cfg>
hipError_t launch_pipe(const FwdParams& p, hipStream_t stream) {
  constexpr int BR = 32 * Cfg::QB * Cfg::NW;
  FwdParams q = p;
  q.nq = (p.N + BR - 1) / BR;
  if (pipe_pairs<Cfg>(q, q.nq, CAUSAL)) {
    const unsigned grid = CAUSAL ? (unsigned)(((q.nq + 1) / 2) * p.BH) : (unsigned)(q.nq * (p.BH / 2));
    hipLaunchKernelGGL((fwd_pipe<T, CAUSAL, true, Cfg>), dim3(grid), dim3(64 * Cfg::NW), 0, stream, q);
  } else {
    const unsigned grid = (unsigned)(q.nq * p.BH);
    hipLaunchKernelGGL((fwd_pipe<T, CAUSAL, false, Cfg>), dim3(grid), dim3(64 * Cfg::NW), 0, stream, q);
  }
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
