/*
 * fa.h — C ABI of the exact attention forward pass for AMD Instinct MI355X
 * (gfx950).  Library: io_aware_exact_05_amd/libfa.so.
 *
 * The operation is the one formula printed on the pages "FlashAttention (HI)"
 * and "FlashAttention (TL)" (section on the problems of standard attention):
 *
 *     O = softmax(scale * Q K^T) V        (softmax along each query row)
 *
 * with optional causal masking (masking is one of the fused operations in the
 * same pages' section on combining everything into one kernel; here query i
 * sees key j iff j <= i), computed tile by tile with an online softmax that
 * keeps a running maximum and a running sum of exponentials per row (same
 * pages, "online softmax" section), in one fused kernel that writes only the
 * final result (O) and the per-row logsumexp, never the N x N score matrix.
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers owned by the caller.  The library allocates
 *     nothing, frees nothing and keeps no mutable global state, so calls are
 *     thread-safe; calls that write the same buffers concurrently race.
 *   - Tensors are contiguous, row-major: q, k, v, o are [B, H, N, d] (each
 *     (b, h) pair is one N x d matrix of the formula); lse is [B, H, N] fp32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.
 *   - Arguments are validated before any HIP call; a failure returns a
 *     negative status and enqueues nothing.  No entry point prints or throws.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_F32 = 0,  /* IEEE binary32                                  */
  FA_F16 = 1,  /* IEEE binary16                                  */
  FA_BF16 = 2, /* bfloat16                                       */
  FA_E4M3 = 3  /* OCP fp8 e4m3fn (finite-only, max 448); fp8 API */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,    /* a required pointer is NULL                     */
  FA_ERR_SHAPE = -2,   /* B, H or N < 1, or a tensor too large to index  */
  FA_ERR_DTYPE = -3,   /* dtype not accepted by this entry point         */
  FA_ERR_HEADDIM = -4, /* d not in {64, 128, 256}                        */
  FA_ERR_ALIGN = -5,   /* q/k/v/o not 16-byte or lse not 4-byte aligned  */
  FA_ERR_ARG = -6,     /* causal not 0/1, scale not finite, bad option   */
  FA_ERR_ALIAS = -7,   /* an output overlaps an input or another output  */
  FA_ERR_LAUNCH = -8   /* the HIP runtime rejected the launch            */
} fa_status;

/*
 * fa_fwd — exact attention forward pass.
 *   q, k, v : inputs [B,H,N,d] of `dtype` (FA_F32, FA_F16 or FA_BF16).
 *   o       : output [B,H,N,d] of the same dtype, rounded to nearest-even
 *             from the fp32 accumulator.
 *   lse     : output [B,H,N] fp32, natural-log logsumexp of each masked,
 *             scaled score row: lse[i] = ln sum_{j visible} exp(scale*q_i.k_j).
 *   causal  : 0 = every key visible; 1 = key j visible to query i iff j <= i.
 *   scale   : finite multiplier of the scores (1/sqrt(d) in the formula).
 *   d       : head dimension, one of 64, 128, 256.  Any N >= 1 is accepted;
 *             partial tiles are masked inside the kernel.
 * Returns FA_OK or a negative fa_status.  E4M3 inputs return FA_ERR_DTYPE
 * (they go through an fp8 entry point).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, int dtype,
           void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
