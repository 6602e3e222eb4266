// C ABI of the attention forward pass: argument validation, dispatch to the
// gfx950 kernels, launch-error mapping.  Declared in include/fa.h.
//
// Validation runs entirely on the host before any HIP call, so every invalid
// argument is reported without touching (or needing) a device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_kernels.h"

namespace {

constexpr int kAbiMajor = 1, kAbiMinor = 5;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, uint64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + static_cast<uintptr_t>(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int elem_bytes(int dtype) {
  switch (dtype) {
    case FA_F32: return 4;
    case FA_F16: return 2;
    case FA_BF16: return 2;
    case FA_E4M3: return 1;
  }
  return 0;
}

// Shape checks common to the entry points.  Sizes must index with 64-bit
// offsets, B*H query tiles must fit one grid dimension, and one head must
// stay below 2^31 elements (row offsets inside a head are 32-bit).
int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  if (bh > (uint64_t)INT32_MAX) return FA_ERR_SHAPE;
  if ((uint64_t)N * (uint64_t)d > (uint64_t)INT32_MAX) return FA_ERR_SHAPE;
  const uint64_t tiles = bh * (((uint64_t)N + 31) / 32);  // finest tiling used
  if (tiles > (uint64_t)INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

// Rows per head of the backward workspace: N rounded up to 128.
uint64_t bwd_npad(int N) { return ((uint64_t)N + 127) / 128 * 128; }

// How attention over a key/value cache is cut: rows of a K/V group in
// 32-row blocks, the cache in nsplit chunks (multiples of 128 keys, at least
// 512 keys each) so that about 256 workgroups run when the cache is long
// enough: one per CU of an MI355X (the partial kernel's 128 KiB of LDS
// admits one per CU), each streaming a long chunk, which measured 16-19%
// faster than four rounds of 1024 shorter ones.
// Depends on the shape only, so the workspace size is known before any
// device call and results do not depend on the device.
struct DecPlan {
  int R, nrb, nsplit, chunk;
};
DecPlan dec_plan(int B, int H, int Hkv, int Nq, int Nkv) {
  DecPlan d{};
  d.R = (H / Hkv) * Nq;
  d.nrb = (d.R + 31) / 32;
  const uint64_t base = (uint64_t)B * Hkv * d.nrb;
  const uint64_t max_split = std::max<uint64_t>(1, ((uint64_t)Nkv + 511) / 512);
  const uint64_t want = std::max<uint64_t>(1, (256 + base - 1) / base);
  uint64_t ns = std::min(want, max_split);
  const uint64_t per = ((uint64_t)Nkv + ns - 1) / ns;
  const uint64_t chunk = (per + 127) / 128 * 128;
  d.chunk = (int)chunk;
  d.nsplit = (int)(((uint64_t)Nkv + chunk - 1) / chunk);
  return d;
}

// Argument checks of the key/value-cache pass up to its cut (shared by
// fa_fwd_kvcache and fa_fwd_kvcache_noalloc, in the order of the statuses).
int kvcache_check(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                  int H, int Hkv, int Nq, int Nkv, int d, int causal, float scale, int dtype,
                  DecPlan* pl) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || Nq < 1 || Nkv < Nq) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_SHAPE;
  if ((uint64_t)Nkv * d > (uint64_t)INT32_MAX || (uint64_t)B * H > (uint64_t)INT32_MAX)
    return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  *pl = dec_plan(B, H, Hkv, Nq, Nkv);
  if ((uint64_t)B * Hkv * pl->nrb * pl->nsplit > (uint64_t)INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

// Alignment and overlap of the pass's buffers; ws (need bytes) may be NULL.
int kvcache_check_buffers(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* ws, size_t need, int B, int H, int Hkv, int Nq, int Nkv, int d) {
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      (ws && !aligned(ws, 16)))
    return FA_ERR_ALIGN;
  const uint64_t rows = (uint64_t)B * H * Nq, kv_rows = (uint64_t)B * Hkv * Nkv;
  const uint64_t eb = (uint64_t)d * 2;
  const Range in[3] = {range_of(q, rows * eb), range_of(k, kv_rows * eb), range_of(v, kv_rows * eb)};
  const Range out[3] = {range_of(o, rows * eb), range_of(lse, rows * 4), range_of(ws, ws ? need : 0)};
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(out[i], out[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// Parameters and launch of the pass; ws holds the chunks' partial results
// when the cut has more than one chunk.
int kvcache_launch(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                   const DecPlan& pl, int B, int H, int Hkv, int Nq, int Nkv, int d, int causal,
                   float scale, int dtype, void* stream) {
  const uint64_t rows = (uint64_t)B * H * Nq;
  fa::DecodeParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.ws_o = pl.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  p.ws_lse = pl.nsplit > 1 ? p.ws_o + rows * pl.nsplit * (uint64_t)d : nullptr;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.R = pl.R;
  p.nrb = pl.nrb;
  p.nsplit = pl.nsplit;
  p.chunk = pl.chunk;
  p.rows = rows;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  (void)hipGetLastError();
  const hipError_t e = fa::launch_decode_half(p, d, causal, dtype == FA_BF16,
                                              reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return (kAbiMajor << 16) | kAbiMinor; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: B, H or N < 1, or the tensors are too large to index";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: dtype not accepted by this entry point";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension must be 64, 128 or 256";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a tensor base pointer is misaligned";
    case FA_ERR_ARG: return "FA_ERR_ARG: invalid option (causal, scale or similar)";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps an input or another output";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime rejected the kernel launch";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: the shape needs more workspace than the static scratch";
  }
  return "unknown fa_status";
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int N, int d, int causal, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  const int sc = check_shape(B, H, N, d);
  if (sc != FA_OK) return sc;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  const uint64_t rows = (uint64_t)B * H * N, kv_rows = (uint64_t)B * Hkv * N;
  const uint64_t eb = (uint64_t)d * elem_bytes(dtype);
  const Range rq = range_of(q, rows * eb), rk = range_of(k, kv_rows * eb), rv = range_of(v, kv_rows * eb);
  const Range ro = range_of(o, rows * eb), rl = range_of(lse, rows * 4);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) ||
      overlap(rl, rk) || overlap(rl, rv) || overlap(ro, rl))
    return FA_ERR_ALIAS;

  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = B * H;
  p.N = N;
  p.H = H;
  p.Hkv = Hkv;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);  // log2(e)
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  hipError_t e = (dtype == FA_F32) ? fa::launch_fwd_f32(p, d, causal, s)
                                   : fa::launch_fwd_half(p, d, causal, dtype == FA_BF16, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, int causal, float scale, int dtype, void* stream) {
  return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return (size_t)(2 * 4 * (uint64_t)B * (uint64_t)H * bwd_npad(N));
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int H, int Hkv, int N, int d, int causal, float scale,
               int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  const int sc = check_shape(B, H, N, d);
  if (sc != FA_OK) return sc;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_SHAPE;
  const uint64_t npad = bwd_npad(N);
  if ((uint64_t)B * H * npad > (uint64_t)INT32_MAX) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (workspace_bytes < fa_bwd_workspace_bytes(B, H, N)) return FA_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  const uint64_t rows = (uint64_t)B * H * N, kv_rows = (uint64_t)B * Hkv * N;
  const uint64_t eb = (uint64_t)d * 2;
  const Range in[6] = {range_of(q, rows * eb),  range_of(k, kv_rows * eb),
                       range_of(v, kv_rows * eb), range_of(o, rows * eb),
                       range_of(dout, rows * eb), range_of(lse, rows * 4)};
  const Range out[4] = {range_of(dq, rows * eb), range_of(dk, kv_rows * eb),
                        range_of(dv, kv_rows * eb),
                        range_of(workspace, fa_bwd_workspace_bytes(B, H, N))};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(out[i], out[j])) return FA_ERR_ALIAS;
  }

  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws_lse2 = static_cast<float*>(workspace);
  p.ws_delta = p.ws_lse2 + (uint64_t)B * H * npad;
  p.BH = B * H;
  p.N = N;
  p.H = H;
  p.Hkv = Hkv;
  p.Npad = (int)npad;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  (void)hipGetLastError();
  const hipError_t e = fa::launch_bwd_half(p, d, causal, dtype == FA_BF16,
                                           reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
           int B, int H, int N, int d, int causal, float scale, int dtype, void* stream) {
  return fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N, d,
                    causal, scale, dtype, stream);
}

size_t fa_fwd_kvcache_workspace_bytes(int B, int H, int Hkv, int Nq, int Nkv, int d) {
  if (B < 1 || H < 1 || Hkv < 1 || Hkv > H || H % Hkv != 0 || Nq < 1 || Nkv < Nq || d < 1) return 0;
  const DecPlan pl = dec_plan(B, H, Hkv, Nq, Nkv);
  if (pl.nsplit == 1) return 0;
  return (size_t)((uint64_t)B * H * Nq * pl.nsplit * ((uint64_t)d + 1) * 4);
}

int fa_fwd_kvcache(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int Nq, int Nkv,
                   int d, int causal, float scale, int dtype, void* stream) {
  DecPlan pl{};
  const int st = kvcache_check(q, k, v, o, lse, B, H, Hkv, Nq, Nkv, d, causal, scale, dtype, &pl);
  if (st != FA_OK) return st;
  const size_t need = fa_fwd_kvcache_workspace_bytes(B, H, Hkv, Nq, Nkv, d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return workspace ? FA_ERR_ARG : FA_ERR_NULL;
  const int sb = kvcache_check_buffers(q, k, v, o, lse, need > 0 ? workspace : nullptr, need, B, H, Hkv,
                                       Nq, Nkv, d);
  if (sb != FA_OK) return sb;
  return kvcache_launch(q, k, v, o, lse, need > 0 ? workspace : nullptr, pl, B, H, Hkv, Nq, Nkv, d,
                        causal, scale, dtype, stream);
}

int fa_fwd_kvcache_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int Hkv, int Nq, int Nkv, int d, int causal, float scale, int dtype,
                           void* stream) {
  DecPlan pl{};
  const int st = kvcache_check(q, k, v, o, lse, B, H, Hkv, Nq, Nkv, d, causal, scale, dtype, &pl);
  if (st != FA_OK) return st;
  const size_t need = fa_fwd_kvcache_workspace_bytes(B, H, Hkv, Nq, Nkv, d);
  if (need > FA_KVCACHE_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  const int sb = kvcache_check_buffers(q, k, v, o, lse, nullptr, 0, B, H, Hkv, Nq, Nkv, d);
  if (sb != FA_OK) return sb;
  void* ws = nullptr;
  if (need > 0 && (fa::decode_scratch(&ws) != hipSuccess || !ws)) return FA_ERR_LAUNCH;
  return kvcache_launch(q, k, v, o, lse, ws, pl, B, H, Hkv, Nq, Nkv, d, causal, scale, dtype, stream);
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_descale,
               const float* k_descale, const float* v_descale, void* o_bf16, float* lse, int B,
               int H, int N, int d, int causal, float scale, void* stream) {
  if (!q8 || !k8 || !v8 || !q_descale || !k_descale || !v_descale || !o_bf16 || !lse)
    return FA_ERR_NULL;
  const int sc = check_shape(B, H, N, d);
  if (sc != FA_OK) return sc;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o_bf16, 16) ||
      !aligned(lse, 4) || !aligned(q_descale, 4) || !aligned(k_descale, 4) || !aligned(v_descale, 4))
    return FA_ERR_ALIGN;
  const uint64_t rows = (uint64_t)B * H * N;
  const uint64_t nblk = ((uint64_t)N + 127) / 128;
  const uint64_t dbytes = (uint64_t)B * H * nblk * 4;
  const Range in[6] = {range_of(q8, rows * d), range_of(k8, rows * d), range_of(v8, rows * d),
                       range_of(q_descale, dbytes), range_of(k_descale, dbytes),
                       range_of(v_descale, dbytes)};
  const Range ro = range_of(o_bf16, rows * d * 2), rl = range_of(lse, rows * 4);
  for (const Range& r : in)
    if (overlap(ro, r) || overlap(rl, r)) return FA_ERR_ALIAS;
  if (overlap(ro, rl)) return FA_ERR_ALIAS;

  fa::Fp8Params p{};
  p.q = static_cast<const uint8_t*>(q8);
  p.k = static_cast<const uint8_t*>(k8);
  p.v = static_cast<const uint8_t*>(v8);
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  p.o = o_bf16;
  p.lse = lse;
  p.BH = B * H;
  p.N = N;
  p.nblk = (int)nblk;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  (void)hipGetLastError();
  const hipError_t e = fa::launch_fwd_fp8(p, d, causal, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_quantize_e4m3(const float* x, void* x8, float* descale, int B, int H, int N, int d,
                     int block_rows, int rotate, const float* signs, void* stream) {
  if (!x || !x8 || !descale) return FA_ERR_NULL;
  const int sc = check_shape(B, H, N, d);
  if (sc != FA_OK) return sc;
  if (block_rows != 128 || (rotate != 0 && rotate != 1)) return FA_ERR_ARG;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(descale, 4) || (signs && !aligned(signs, 4)))
    return FA_ERR_ALIGN;
  const uint64_t elems = (uint64_t)B * H * N * d;
  const uint64_t nblk = ((uint64_t)N + 127) / 128;
  const Range rx = range_of(x, elems * 4), r8 = range_of(x8, elems),
              rd = range_of(descale, (uint64_t)B * H * nblk * 4);
  const Range rs = range_of(signs, signs ? (uint64_t)d * 4 : 0);
  if (overlap(r8, rx) || overlap(rd, rx) || overlap(r8, rd) || overlap(r8, rs) || overlap(rd, rs))
    return FA_ERR_ALIAS;
  fa::QuantParams p{};
  p.x = x;
  p.x8 = static_cast<uint8_t*>(x8);
  p.descale = descale;
  p.BH = B * H;
  p.N = N;
  p.nblk = (int)nblk;
  p.signs = rotate ? signs : nullptr;
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)d));
  (void)hipGetLastError();
  const hipError_t e =
      fa::launch_quantize_e4m3(p, d, rotate, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
