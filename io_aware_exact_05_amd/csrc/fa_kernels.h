// Internal interface between the C ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Arguments of one forward launch.  Tensors are contiguous [B*H, N, d].
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;            // B * H
  int N;             // sequence length
  int nq;            // query tiles per head (set by the launcher)
  float scale_log2;  // scale * log2(e): scores go straight into exp2
  int H;             // query heads per batch entry
  int Hkv;           // K/V heads per batch entry (divides H)
};

// K/V head of the flattened query head bh = b H + h: b Hkv + h / (H / Hkv).
__host__ __device__ inline int kv_head(const FwdParams& p, int bh) {
  return (bh / p.H) * p.Hkv + (bh % p.H) / (p.H / p.Hkv);
}

// K/V head of flattened query head bh when Hkv K/V heads serve H query heads.
__host__ __device__ inline int kv_head_of(int H, int Hkv, int bh) {
  return (bh / H) * Hkv + (bh % H) / (H / Hkv);
}

// Arguments of the backward pass.  q, o, dout, dq: [B*H, N, d]; k, v, dk,
// dv: [B*Hkv, N, d]; lse fp32 [B*H, N] from the forward.  ws_lse2 and
// ws_delta are the two halves of the caller's workspace, fp32 [B*H, Npad]
// each (Npad = N rounded up to 128): bwd_dq writes the base-2 logsumexp and
// D_i = dO_i . O_i of every row there (rows >= N: +inf and 0), bwd_dkdv
// reads them.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* ws_lse2;
  float* ws_delta;
  int BH;            // B * H
  int N;
  int H;
  int Hkv;
  int Npad;
  int nq;            // tiles per head of the kernel being launched (set by the launcher)
  float scale;
  float scale_log2;  // scale * log2(e)
};

// Arguments of attention over a key/value cache (fa_decode.hip).  q, o:
// [B*H*Nq, d] (rows of a head consecutive, heads of a K/V group consecutive);
// k, v: [B*Hkv, Nkv, d]; lse [B*H*Nq].  The cache of each K/V head is cut
// into nsplit chunks of `chunk` keys; with nsplit > 1 the partial results go
// to ws_o [rows, nsplit, d] and ws_lse [rows, nsplit] (fp32) and a second
// kernel merges them.
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* ws_o;
  float* ws_lse;
  int B;
  int H;
  int Hkv;
  int Nq;
  int Nkv;
  int R;        // rows per K/V head: (H / Hkv) * Nq
  int nrb;      // 32-row blocks per K/V head
  int nsplit;
  int chunk;    // keys per split
  size_t rows;  // B * H * Nq
  float scale_log2;
};

// Arguments of the fp8 forward: q8/k8/v8 e4m3fn [B*H, N, d], per-128-row
// fp32 descales [B*H, nblk], o bf16 [B*H, N, d], lse fp32 [B*H, N].
struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  void* o;
  float* lse;
  int BH;
  int N;
  int nq;            // query tiles per head (set by the launcher)
  int nblk;          // 128-row descale blocks per head
  float scale_log2;  // scale * log2(e)
};

// Arguments of the block quantiser: x fp32 [B*H, N, d] -> x8 e4m3fn, descale
// fp32 [B*H, nblk]; optional rotation signs (NULL = all +1).
struct QuantParams {
  const float* x;
  uint8_t* x8;
  float* descale;
  int BH;
  int N;
  int nblk;
  const float* signs;
  float inv_sqrt_d;
};

// fp16 / bf16 inputs, MFMA path.  d in {64, 128, 256}.
hipError_t launch_fwd_half(const FwdParams& p, int d, int causal, int is_bf16, hipStream_t s);
// fp16 / bf16 with 32 or 64 query rows per wave and one wave of each
// workgroup per SIMD (fa_fwd_wide.hip).  d in {64, 128, 256}; long_causal
// (d = 64 or 128, causal) selects the configuration for many query tiles.
hipError_t launch_fwd_wide(const FwdParams& p, int d, int causal, int long_causal, int is_bf16,
                           hipStream_t s);
// Query rows per workgroup and workgroups per CU of that kernel; rows per
// workgroup of the long-causal configuration (0 where there is none).
int wide_rows_per_block(int d, int causal);
int wide_blocks_per_cu(int d, int causal);
int wide_long_causal_rows(int d);
// fp16 / bf16, d = 128, softmax software-pipelined against the matrix
// products inside each wave (fa_fwd_pipe.hip).
hipError_t launch_fwd_pipe(const FwdParams& p, int d, int causal, int is_bf16, hipStream_t s);
// fp32 inputs (v_mfma_f32_32x32x2f32).  d in {64, 128, 256}.
hipError_t launch_fwd_f32(const FwdParams& p, int d, int causal, hipStream_t s);
// e4m3 inputs (v_mfma_scale_f32_32x32x64_f8f6f4).  d = 128.
hipError_t launch_fwd_fp8(const Fp8Params& p, int d, int causal, hipStream_t s);
// Backward pass, fp16 / bf16 (fa_bwd.hip): bwd_dq then bwd_dkdv on stream s.
hipError_t launch_bwd_half(const BwdParams& p, int d, int causal, int is_bf16, hipStream_t s);
// Attention over a key/value cache, fp16 / bf16, split over the cache.
hipError_t launch_decode_half(const DecodeParams& p, int d, int causal, int is_bf16, hipStream_t s);
// Device address, on the current device, of the library's static scratch of
// FA_KVCACHE_SCRATCH_BYTES bytes that fa_fwd_kvcache_noalloc uses as its
// workspace (fa_decode.hip); looked up once per device.
hipError_t decode_scratch(void** ptr);
// fp32 -> e4m3 block quantiser, optional randomised Hadamard rotation.
hipError_t launch_quantize_e4m3(const QuantParams& p, int d, int rotate, hipStream_t s);

}  // namespace fa
