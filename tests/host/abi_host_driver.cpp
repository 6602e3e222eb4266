// Host-only driver of the C ABI's argument validation and dispatch, built by
// tests/test_abi_host_sanitized.py with the address and undefined-behaviour
// sanitizers.  The kernel launchers and the one HIP runtime call of the ABI
// layer are replaced by stubs that record what they were given, so no device
// (and no GPU code) is involved: pointers are fake addresses never
// dereferenced.  Exit status 0 when every case returns the expected status.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "fa.h"
#include "fa_kernels.h"

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace {
int g_calls = 0;
fa::DecodeParams g_dec{};
fa::BwdParams g_bwd{};
}  // namespace

namespace fa {
hipError_t launch_fwd_half(const FwdParams&, int, int, int, hipStream_t) { ++g_calls; return hipSuccess; }
hipError_t launch_fwd_wide(const FwdParams&, int, int, int, int, hipStream_t) { ++g_calls; return hipSuccess; }
int wide_rows_per_block(int, int) { return 128; }
int wide_blocks_per_cu(int, int) { return 1; }
int wide_long_causal_rows(int) { return 512; }
hipError_t launch_fwd_f32(const FwdParams&, int, int, hipStream_t) { ++g_calls; return hipSuccess; }
hipError_t launch_fwd_fp8(const Fp8Params&, int, int, hipStream_t) { ++g_calls; return hipSuccess; }
hipError_t launch_bwd_half(const BwdParams& p, int, int, int, hipStream_t) {
  ++g_calls;
  g_bwd = p;
  return hipSuccess;
}
hipError_t launch_decode_half(const DecodeParams& p, int, int, int, hipStream_t) {
  ++g_calls;
  g_dec = p;
  return hipSuccess;
}
hipError_t launch_quantize_e4m3(const QuantParams&, int, int, hipStream_t) { ++g_calls; return hipSuccess; }
// the static scratch of the no-allocation pass, at a fake 256-byte-aligned address
constexpr uintptr_t kScratchAddr = uintptr_t(11) << 36;
int g_scratch_lookups = 0;
hipError_t decode_scratch(void** ptr) {
  ++g_scratch_lookups;
  *ptr = reinterpret_cast<void*>(kScratchAddr);
  return hipSuccess;
}
}  // namespace fa

namespace {
int g_fail = 0;
void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, got, want);
    ++g_fail;
  }
}
void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }
// fake, 16-byte aligned base addresses 64 GiB apart (no two buffers of any
// case below overlap unless a case places them so on purpose)
constexpr uintptr_t G64 = uintptr_t(1) << 36;
const uintptr_t Q = 1 * G64, K = 2 * G64, V = 3 * G64, O = 4 * G64, L = 5 * G64, WS = 6 * G64,
                DO = 7 * G64, DQ = 8 * G64, DK = 9 * G64, DV = 10 * G64;
const float NaN = std::numeric_limits<float>::quiet_NaN();
const float Inf = std::numeric_limits<float>::infinity();
}  // namespace

int main() {
  // ---- fa_fwd / fa_fwd_gqa ----
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, 100, 128, 0, 0.1f, FA_BF16, nullptr), FA_OK, "fwd ok");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, 100, 64, 1, -0.3f, FA_F32, nullptr), FA_OK, "fwd f32 ok");
  expect(fa_fwd(nullptr, P(K), P(V), P(O), F(L), 2, 3, 100, 128, 0, 0.1f, FA_BF16, nullptr), FA_ERR_NULL, "fwd null q");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 0, 3, 100, 128, 0, 0.1f, FA_BF16, nullptr), FA_ERR_SHAPE, "fwd B=0");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, -5, 128, 0, 0.1f, FA_BF16, nullptr), FA_ERR_SHAPE, "fwd N<0");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, 100, 96, 0, 0.1f, FA_BF16, nullptr), FA_ERR_HEADDIM, "fwd d=96");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, 100, 128, 0, 0.1f, FA_E4M3, nullptr), FA_ERR_DTYPE, "fwd e4m3");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, 100, 128, 0, 0.1f, 7, nullptr), FA_ERR_DTYPE, "fwd dtype 7");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, 100, 128, 2, 0.1f, FA_BF16, nullptr), FA_ERR_ARG, "fwd causal 2");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, 100, 128, 0, NaN, FA_BF16, nullptr), FA_ERR_ARG, "fwd nan scale");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 2, 3, 100, 128, 0, Inf, FA_BF16, nullptr), FA_ERR_ARG, "fwd inf scale");
  expect(fa_fwd(P(Q + 8), P(K), P(V), P(O), F(L), 2, 3, 100, 128, 0, 0.1f, FA_BF16, nullptr), FA_ERR_ALIGN, "fwd align q");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L + 2), 2, 3, 100, 128, 0, 0.1f, FA_BF16, nullptr), FA_ERR_ALIGN, "fwd align lse");
  expect(fa_fwd(P(Q), P(K), P(V), P(Q + 1024), F(L), 2, 3, 100, 128, 0, 0.1f, FA_BF16, nullptr), FA_ERR_ALIAS, "fwd o in q");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(O + 16), 2, 3, 100, 128, 0, 0.1f, FA_BF16, nullptr), FA_ERR_ALIAS, "fwd lse in o");
  // sizes at and past the indexing limits (one head below 2^31 elements)
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 1, 1, 16777215, 128, 0, 0.1f, FA_BF16, nullptr), FA_OK,
         "fwd largest head");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 1, 1, 16777216, 128, 0, 0.1f, FA_BF16, nullptr), FA_ERR_SHAPE, "fwd head 2^31");
  expect(fa_fwd(P(Q), P(K), P(V), P(O), F(L), 65536, 65536, 1, 64, 0, 0.1f, FA_BF16, nullptr), FA_ERR_SHAPE, "fwd BH 2^32");
  expect(fa_fwd_gqa(P(Q), P(K), P(V), P(O), F(L), 2, 8, 2, 100, 128, 1, 0.1f, FA_F16, nullptr), FA_OK, "gqa ok");
  expect(fa_fwd_gqa(P(Q), P(K), P(V), P(O), F(L), 2, 8, 3, 100, 128, 1, 0.1f, FA_F16, nullptr), FA_ERR_SHAPE, "gqa 8/3");
  expect(fa_fwd_gqa(P(Q), P(K), P(V), P(O), F(L), 2, 8, 0, 100, 128, 1, 0.1f, FA_F16, nullptr), FA_ERR_SHAPE, "gqa Hkv 0");

  // ---- fa_bwd ----
  const size_t wsb = fa_bwd_workspace_bytes(2, 3, 100);
  expect((int)(wsb == 8u * 2 * 3 * 128), 1, "bwd workspace size");
  expect((int)(fa_bwd_workspace_bytes(0, 3, 100) == 0), 1, "bwd workspace size of B=0");
  expect(fa_bwd(P(Q), P(K), P(V), P(O), P(DO), F(L), P(DQ), P(DK), P(DV), P(WS), wsb, 2, 3, 100, 128, 1,
                0.1f, FA_BF16, nullptr), FA_OK, "bwd ok");
  expect((int)(g_bwd.Npad == 128), 1, "bwd padded rows");
  expect(fa_bwd(P(Q), P(K), P(V), P(O), P(DO), F(L), P(DQ), P(DK), P(DV), P(WS), wsb - 16, 2, 3, 100, 128, 1,
                0.1f, FA_BF16, nullptr), FA_ERR_ARG, "bwd small workspace");
  expect(fa_bwd(P(Q), P(K), P(V), P(O), P(DO), F(L), P(DQ), P(DK), P(DV), P(WS), wsb, 2, 3, 100, 128, 1,
                0.1f, FA_F32, nullptr), FA_ERR_DTYPE, "bwd f32");
  expect(fa_bwd(P(Q), P(K), P(V), P(O), P(DO), F(L), P(Q), P(DK), P(DV), P(WS), wsb, 2, 3, 100, 128, 1,
                0.1f, FA_BF16, nullptr), FA_ERR_ALIAS, "bwd dq on q");
  expect(fa_bwd(P(Q), P(K), P(V), P(O), P(DO), F(L), P(DQ), P(DK), P(DV), P(DK), wsb, 2, 3, 100, 128, 1,
                0.1f, FA_BF16, nullptr), FA_ERR_ALIAS, "bwd workspace on dk");

  // ---- fa_fwd_kvcache: the cut of the cache covers it with whole chunks ----
  const int shapes[][5] = {{1, 32, 32, 1, 16384}, {8, 32, 8, 4, 16384}, {1, 8, 8, 1, 131072},
                           {2, 4, 4, 1, 100}, {1, 16, 1, 5, 3001}, {3, 6, 3, 2, 20000}, {1, 2, 2, 64, 64}};
  for (const auto& s : shapes) {
    const int B = s[0], H = s[1], Hkv = s[2], Nq = s[3], Nkv = s[4];
    const size_t wb = fa_fwd_kvcache_workspace_bytes(B, H, Hkv, Nq, Nkv, 128);
    g_dec = fa::DecodeParams{};
    expect(fa_fwd_kvcache(P(Q), P(K), P(V), P(O), F(L), wb ? P(WS) : nullptr, wb, B, H, Hkv, Nq, Nkv,
                          128, 1, 0.1f, FA_BF16, nullptr), FA_OK, "kvcache ok");
    const bool covers = g_dec.nsplit >= 1 && g_dec.chunk % 128 == 0 &&
                        (long long)g_dec.nsplit * g_dec.chunk >= Nkv &&
                        (long long)(g_dec.nsplit - 1) * g_dec.chunk < Nkv;
    expect((int)covers, 1, "kvcache cut covers the cache with non-empty chunks");
    expect((int)(g_dec.R == (H / Hkv) * Nq && g_dec.nrb == (g_dec.R + 31) / 32), 1, "kvcache rows");
    const size_t need = g_dec.nsplit > 1 ? (size_t)B * H * Nq * g_dec.nsplit * (128 + 1) * 4 : 0;
    expect((int)(wb == need), 1, "kvcache workspace size");
    if (wb)
      expect(fa_fwd_kvcache(P(Q), P(K), P(V), P(O), F(L), P(WS), wb - 4, B, H, Hkv, Nq, Nkv, 128, 1,
                            0.1f, FA_BF16, nullptr), FA_ERR_ARG, "kvcache small workspace");
  }
  expect(fa_fwd_kvcache(P(Q), P(K), P(V), P(O), F(L), nullptr, 0, 1, 4, 4, 9, 8, 128, 1, 0.1f, FA_BF16,
                        nullptr), FA_ERR_SHAPE, "kvcache Nq > Nkv");

  // ---- fa_fwd_kvcache_noalloc: same cut, workspace = the static scratch ----
  for (const auto& s : shapes) {
    const int B = s[0], H = s[1], Hkv = s[2], Nq = s[3], Nkv = s[4];
    const size_t wb = fa_fwd_kvcache_workspace_bytes(B, H, Hkv, Nq, Nkv, 256);
    g_dec = fa::DecodeParams{};
    const int before = fa::g_scratch_lookups;
    expect(fa_fwd_kvcache_noalloc(P(Q), P(K), P(V), P(O), F(L), B, H, Hkv, Nq, Nkv, 256, 1, 0.1f, FA_F16,
                                  nullptr), FA_OK, "noalloc ok");
    const uintptr_t wso = reinterpret_cast<uintptr_t>(g_dec.ws_o), wsl = reinterpret_cast<uintptr_t>(g_dec.ws_lse);
    if (wb) {
      expect((int)(wso == fa::kScratchAddr), 1, "noalloc partial O in the scratch");
      expect((int)(wsl + (uint64_t)B * H * Nq * g_dec.nsplit * 4 == fa::kScratchAddr + wb), 1,
             "noalloc partial LSE ends the workspace");
      expect(fa::g_scratch_lookups - before, 1, "noalloc looks the scratch up");
    } else {
      expect((int)(wso == 0 && wsl == 0), 1, "noalloc single chunk uses no workspace");
      expect(fa::g_scratch_lookups - before, 0, "noalloc single chunk needs no scratch");
    }
  }
  expect(fa_fwd_kvcache_noalloc(nullptr, P(K), P(V), P(O), F(L), 1, 4, 4, 1, 4096, 128, 0, 0.1f, FA_BF16,
                                nullptr), FA_ERR_NULL, "noalloc null q");
  expect(fa_fwd_kvcache_noalloc(P(Q), P(K), P(V), P(O), F(L), 1, 4, 4, 1, 4096, 96, 0, 0.1f, FA_BF16,
                                nullptr), FA_ERR_HEADDIM, "noalloc d96");
  expect(fa_fwd_kvcache_noalloc(P(Q), P(K), P(V), P(O), F(L), 1, 4, 4, 1, 4096, 128, 0, 0.1f, FA_F32,
                                nullptr), FA_ERR_DTYPE, "noalloc f32");
  expect(fa_fwd_kvcache_noalloc(P(Q), P(K), P(V), P(K), F(L), 1, 4, 4, 1, 4096, 128, 0, 0.1f, FA_BF16,
                                nullptr), FA_ERR_ALIAS, "noalloc o on k");
  expect(fa_fwd_kvcache_noalloc(P(Q + 8), P(K), P(V), P(O), F(L), 1, 4, 4, 1, 4096, 128, 0, 0.1f, FA_BF16,
                                nullptr), FA_ERR_ALIGN, "noalloc misaligned q");
  // The cut keeps (rows) x (chunks) <= 32 base ceil(256 / base) <= 16320 with
  // base = B Hkv ceil(R / 32) < 256 (one chunk otherwise), so every shape with
  // d <= 256 fits the scratch; the worst case is base = 255 with two chunks.
  size_t worst = 0;
  for (int base = 1; base <= 300; ++base)
    for (int G : {1, 2, 4, 8, 32})
      for (int Nq : {1, 3, 8, 31, 32}) {
        const int R = G * Nq, nrb = (R + 31) / 32;
        if (base % nrb) continue;
        const int BHkv = base / nrb;
        const size_t w = fa_fwd_kvcache_workspace_bytes(BHkv, G, 1, Nq, 1 << 20, 256);
        if (w > worst) worst = w;
      }
  expect((int)(worst <= FA_KVCACHE_SCRATCH_BYTES), 1, "every cut fits the static scratch");
  expect((int)(worst == (size_t)16320 * 257 * 4), 1, "worst cut is 16320 partial rows of d = 256");

  // ---- fp8 ----
  expect(fa_fwd_fp8(P(Q), P(K), P(V), F(WS), F(WS + 4096), F(WS + 8192), P(O), F(L), 2, 3, 300, 256, 1,
                    0.1f, nullptr), FA_OK, "fp8 d256 ok");
  expect(fa_fwd_fp8(P(Q), P(K), P(V), F(WS), F(WS + 4096), F(WS + 8192), P(O), F(L), 2, 3, 300, 32, 1,
                    0.1f, nullptr), FA_ERR_HEADDIM, "fp8 d32");
  expect(fa_quantize_e4m3(F(Q), P(K), F(V), 2, 3, 300, 128, 128, 1, nullptr, nullptr), FA_OK, "quant ok");
  expect(fa_quantize_e4m3(F(Q), P(K), F(V), 2, 3, 300, 128, 64, 1, nullptr, nullptr), FA_ERR_ARG, "quant 64 rows");

  std::printf("%d launches, %d failures\n", g_calls, g_fail);
  return g_fail == 0 ? 0 : 1;
}
