// Attention of a short query block against a long key/value cache (decoding)
// for gfx950 (MI355X), fp16/bf16 inputs, split over the cache.
//
// The workload is the KV-cache inference of "FlashAttention (HI)" (section on
// specialised solutions: streaming generation over a KV cache): per head, Nq
// new queries (one decoded token, or a few) attend to Nkv >= Nq cached keys
// and values with the same exact formula, O = softmax(scale Q K^T) V; with
// causal masking the queries are the sequence's last Nq positions (query i
// sees keys j <= Nkv - Nq + i).
//
// With few queries per head the pass is bound by reading K and V from HBM, so
// the design is about keeping enough of the cache in flight:
//   - Rows: the G = H / Hkv query heads sharing a K/V head and their Nq
//     queries are consecutive rows of Q (head-major), so one wave takes up to
//     32 of them as the columns of S^T = K Q^T (one query per lane, as in the
//     forward kernel) and every K/V byte read serves all of them.
//   - Split-KV: the cache of each K/V head is cut into nsplit chunks, one
//     workgroup per (K/V head, 32-row block, chunk), so that even a single
//     sequence fills the chip.  Within a workgroup the four waves take
//     alternate 32-key tiles of the chunk, each with a private LDS ring
//     filled by global_load_lds_dwordx4 (no workgroup barrier in the loop),
//     and keep their own online softmax ("FlashAttention (HI)", tiling and
//     online-softmax sections).
//   - Merges: the waves' partial results are combined in LDS, the chunks'
//     by a second kernel, both with the exact logsumexp rule: for parts with
//     logsumexp l_s and normalised outputs O_s, l = log sum_s e^(l_s) and
//     O = sum_s e^(l_s - l) O_s.  With one chunk the first kernel writes O
//     and the logsumexp directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// Waves per workgroup and LDS ring stages per wave by head dimension: each
// wave's ring holds ST tiles of 32 keys of K and V (8, 16 or 32 KiB a tile).
template <int D> struct DecCfg;
template <> struct DecCfg<64> { static constexpr int NW = 4, ST = 4; };
template <> struct DecCfg<128> { static constexpr int NW = 4, ST = 2; };
template <> struct DecCfg<256> { static constexpr int NW = 2, ST = 2; };

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * DecCfg<D>::NW)
void decode_partial(DecodeParams p) {
  constexpr int NW = DecCfg<D>::NW, ST = DecCfg<D>::ST, BC = 32;
  constexpr int RB = 2 * D, TB = BC * RB, CPR = D / 8, CPT = BC * CPR / 64;
  constexpr int NS = D / 16, ND = D / 32;
  constexpr int WB = ST * 2 * TB;                      // ring bytes per wave
  // Merge rows are D + 4 floats apart, so the rows of a half wave start 4
  // banks apart: 16-byte accesses of 16 rows cover the 64 banks once.
  constexpr int MS = D + 4;
  static_assert(32 * MS * 4 + 256 <= WB, "the merge area must fit in a wave's ring");
  __shared__ __attribute__((aligned(1024))) char smem[NW * WB];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ql = lane & 31, g = lane >> 5;
  // block -> (split, row block, K/V head); consecutive blocks share a head
  int bid = blockIdx.x;
  const int split = bid % p.nsplit;
  bid /= p.nsplit;
  const int rb = bid % p.nrb;
  const int kvbh = bid / p.nrb;
  const int b = kvbh / p.Hkv, gk = kvbh % p.Hkv;
  const int grp = p.H / p.Hkv;
  const size_t row_base = ((size_t)b * p.H + (size_t)gk * grp) * p.Nq;  // flat row of the group's row 0
  const int rho = rb * 32 + ql;                                          // row within the group
  const size_t frow = row_base + min(rho, p.R - 1);
  const int Nkv = p.Nkv;
  const T* __restrict__ kh = (const T*)p.k + (size_t)kvbh * Nkv * D;
  const T* __restrict__ vh = (const T*)p.v + (size_t)kvbh * Nkv * D;

  // Q operand (B of S^T): lane holds Q[row][16 s + 8 g .. +8]; a negative
  // scale moves into Q's sign bit (exact) as in the forward kernel.
  i32x4 qop[NS];
  {
    const T* qr = (const T*)p.q + frow * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) qop[s] = *(const i32x4*)(qr + 16 * s);
    if (p.scale_log2 < 0.f) {
#pragma unroll
      for (int s = 0; s < NS; ++s) qop[s] ^= (int)0x80008000u;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  landed(qop);
  const float c = fmaxf(fabsf(p.scale_log2), 1.0e-30f);
  // last key this lane's query may see
  const int lim = CAUSAL ? Nkv - p.Nq + (min(rho, p.R - 1) % p.Nq) : Nkv - 1;

  const int k_begin = split * p.chunk;
  const int k_end = min(Nkv, k_begin + p.chunk);
  const int ntile = (k_end - k_begin + BC - 1) / BC;
  const int nmy = w < ntile ? (ntile - 1 - w) / NW + 1 : 0;  // tiles w, w + NW, ...

  char* ring = smem + w * WB;
  const uint32_t ring_base = (uint32_t)(uintptr_t)(lds_void*)ring;
  int ld_off[CPT], ld_row[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int sl = u * 64 + lane, row = sl / CPR, cc = sl % CPR;
    ld_row[u] = row;
    ld_off[u] = (cc ^ chunk_swz<D>(row)) * 8;
  }
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int key0 = k_begin + (w + i * NW) * BC;
    const uint32_t dst = ring_base + (i % ST) * 2 * TB;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const size_t row = (size_t)min(key0 + ld_row[u], Nkv - 1);
      dma16(kh + row * D + ld_off[u], dst + u * 1024);
      dma16(vh + row * D + ld_off[u], dst + u * 1024 + TB);
    }
  };

  // LDS read geometry (as in the forward kernel): K rows swap_bits23(ql),
  // V read transposed.
  const int krow = swap_bits23(ql);
  const int kbase_off = krow * RB;
  const int ky = g ^ chunk_swz<D>(krow);
  const int trow = (lane & 15) >> 2;
  int vrow_off[2], vx[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 8 * g + 4 * t + trow;
    vrow_off[t] = r * RB + 8 * (lane & 1);
    vx[t] = (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ chunk_swz<D>(r);
  }

  f32x16 oacc[ND];
#pragma unroll
  for (int bb = 0; bb < ND; ++bb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[bb][r] = 0.f;
  float m = kMInit, l = 0.f;

  constexpr int PD = ST - 1, PT = 2 * CPT;
  static_assert(PT * (PD - 1) <= 31, "pending copies must fit wait_vmcnt");
  for (int i = 0; i < PD && i < nmy; ++i) issue(i);
  if (nmy > 0) wait_vmcnt(PT * (min(PD, nmy) - 1));
  for (int i = 0; i < nmy; ++i) {
    // the stage refilled here held tile i - 1, whose LDS reads this wave
    // consumed (its MFMAs used them) before getting here
    if (i + PD < nmy) issue(i + PD);
    const char* sk = ring + (i % ST) * 2 * TB;
    const char* sv = sk + TB;
    const int key0 = k_begin + (w + i * NW) * BC;
    // S^T = K Q^T
    f32x16 S;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = 0.f;
    {
      i32x4 kop[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) kop[s] = *(const i32x4*)(sk + kbase_off + (((2 * s) ^ ky) << 4));
#pragma unroll
      for (int s = 0; s < NS; ++s) S = Half<T>::mfma(kop[s], qop[s], S);
    }
    // mask: register r holds key key0 + 8 g + 16 (r/8) + r%8, visible iff
    // <= min(lim, k_end - 1)
    const int rel = min(lim, k_end - 1) - key0 - 8 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = (16 * (r >> 3) + (r & 7) <= rel) ? S[r] : kNegInf;
    // online softmax in base 2 with the lazy running max
    float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int r = 0; r < 16; ++r) mx4[r & 3] = fmaxf(mx4[r & 3], S[r]);
    const float mx = pair_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
    const float mt = (mx == kNegInf) ? kNegInf : mx * c;
    const bool upd = mt > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float mnew = upd ? mt : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int bb = 0; bb < ND; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[bb][r] *= alpha;
    }
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      S[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], c, -m));
      rs += S[r];
    }
    l += rs;
    // O^T += V^T P^T
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x4 pop;
#pragma unroll
      for (int e = 0; e < 4; ++e) pop[e] = (int)Half<T>::pack2(S[8 * h + 2 * e], S[8 * h + 2 * e + 1]);
      const char* vb = sv + 16 * h * RB;
#pragma unroll
      for (int bb = 0; bb < ND; ++bb) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + vrow_off[0] + (((4 * bb) ^ vx[0]) << 4)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + vrow_off[1] + (((4 * bb) ^ vx[1]) << 4)));
        const i16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[bb] = Half<T>::mfma(__builtin_bit_cast(i32x4, v8), pop, oacc[bb]);
      }
    }
    wait_vmcnt(PT * max(0, min(i + PD, nmy - 1) - (i + 1)));
  }

  // ---- merge the waves' partial results in LDS (each wave's ring area) ----
  const float lt = pair_sum(l);
  __syncthreads();  // every wave is done with its ring
  float* mo = (float*)ring;                   // [32 rows][MS] unnormalised O of this wave
  float* ml = (float*)(ring + 32 * MS * 4);   // [32] m, then [32] l
#pragma unroll
  for (int bb = 0; bb < ND; ++bb)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float4 v4 = {oacc[bb][4 * a], oacc[bb][4 * a + 1], oacc[bb][4 * a + 2], oacc[bb][4 * a + 3]};
      *(float4*)(mo + ql * MS + 32 * bb + 8 * a + 4 * g) = v4;
    }
  if (g == 0) {
    ml[ql] = m;
    ml[32 + ql] = lt;
  }
  __syncthreads();
  // thread t: row t % 32, columns [cpt * (t / 32), + cpt)
  constexpr int CPL = D / (2 * NW);
  const int t = threadIdx.x, row = t & 31, col0 = (t >> 5) * CPL;
  float mw[NW], M = kMInit;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    mw[u] = ((const float*)(smem + u * WB + 32 * MS * 4))[row];
    M = fmaxf(M, mw[u]);
  }
  float L = 0.f, wt[NW];
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    wt[u] = __builtin_amdgcn_exp2f(mw[u] - M);
    L += wt[u] * ((const float*)(smem + u * WB + 32 * MS * 4))[32 + row];
  }
  const int rrho = rb * 32 + row;
  if (rrho >= p.R) return;
  const size_t orow = row_base + rrho;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const float lse = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * 0.69314718055994530942f : kNegInf;
  static_assert(CPL % 4 == 0, "columns per thread in 16-byte groups");
  // weighted sum over the waves of 4 columns (16-byte LDS reads)
  auto combine4 = [&](int cc) __attribute__((always_inline)) {
    float4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const float4 v = *(const float4*)((const float*)(smem + u * WB) + row * MS + col0 + cc);
      x.x += wt[u] * v.x;
      x.y += wt[u] * v.y;
      x.z += wt[u] * v.z;
      x.w += wt[u] * v.w;
    }
    return x;
  };
  if (p.nsplit == 1) {
    T* out = (T*)p.o + orow * D + col0;
#pragma unroll
    for (int cc = 0; cc < CPL; cc += 4) {
      const float4 x = combine4(cc);
      uint2 pk2;
      pk2.x = Half<T>::pack2(x.x * inv, x.y * inv);
      pk2.y = Half<T>::pack2(x.z * inv, x.w * inv);
      *(uint2*)(out + cc) = pk2;
    }
    if (col0 == 0) p.lse[orow] = lse;
  } else {
    float* out = p.ws_o + (orow * p.nsplit + split) * D + col0;
#pragma unroll
    for (int cc = 0; cc < CPL; cc += 4) {
      const float4 x = combine4(cc);
      *(float4*)(out + cc) = float4{x.x * inv, x.y * inv, x.z * inv, x.w * inv};
    }
    if (col0 == 0) p.ws_lse[orow * p.nsplit + split] = lse;
  }
}

// Combine the chunks' partial results of every row, one wave per row.  The
// wave's lanes form 64 / (D / 8) groups that walk the chunks side by side,
// lane l of a group owning columns [8 (l % (D / 8)), + 8); every chunk's O is
// read as two 16-byte loads per lane, the loads of several chunks are in
// flight together, and the groups' sums meet through lane shuffles in a fixed
// order (so results are the same run to run).
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge(DecodeParams p) {
  constexpr int LPC = D / 8;   // lanes covering one row
  constexpr int NG = 64 / LPC; // chunks read side by side
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int ns = p.nsplit;
  const float* ls = p.ws_lse + row * ns;
  float M = kNegInf;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, ls[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const int grp = lane / LPC, c0 = (lane % LPC) * 8;
  float acc[8], L = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const float* base = p.ws_o + row * ns * D + c0;
#pragma unroll 4
  for (int s = grp; s < ns; s += NG) {
    const float l_s = ls[s];
    const float4 a = *(const float4*)(base + (size_t)s * D);
    const float4 b = *(const float4*)(base + (size_t)s * D + 4);
    const float w = l_s == kNegInf ? 0.f : __expf(l_s - M);
    L += w;
    acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
    acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
  }
#pragma unroll
  for (int off = LPC; off < 64; off <<= 1) {
    L += __shfl_xor(L, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (grp != 0) return;
  const float inv = 1.0f / L;  // L >= 1: the chunk holding the maximum has weight 1
  i32x4 pk;
#pragma unroll
  for (int e = 0; e < 4; ++e) pk[e] = (int)Half<T>::pack2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *(i32x4*)((T*)p.o + row * D + c0) = pk;
  if (lane == 0) p.lse[row] = M + __logf(L);
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_dec(const DecodeParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)p.B * p.Hkv * p.nrb * p.nsplit);
  hipLaunchKernelGGL((decode_partial<T, D, CAUSAL>), dim3(grid), dim3(64 * DecCfg<D>::NW), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL((decode_merge<T, D>), dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_dec_d(const DecodeParams& p, int d, int causal, hipStream_t s) {
  switch (d) {
    case 64:  return causal ? launch_dec<T, 64, true>(p, s) : launch_dec<T, 64, false>(p, s);
    case 128: return causal ? launch_dec<T, 128, true>(p, s) : launch_dec<T, 128, false>(p, s);
    case 256: return causal ? launch_dec<T, 256, true>(p, s) : launch_dec<T, 256, false>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_half(const DecodeParams& p, int d, int causal, int is_bf16, hipStream_t s) {
  return is_bf16 ? launch_dec_d<__bf16>(p, d, causal, s) : launch_dec_d<_Float16>(p, d, causal, s);
}

// Workspace of the passes that may not allocate (fa_fwd_kvcache_noalloc):
// the partial results of the cache chunks.  Each device holds its own copy
// from the code object's load until the process ends.  The partial kernel
// writes every entry the merge kernel reads, so nothing needs clearing
// between calls; calls that overlap on one device share it and race.
static __device__ __align__(256) char scratch[FA_KVCACHE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; the array's name is only a host-side stand-in
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
