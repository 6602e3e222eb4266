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
 *     nothing and frees nothing; calls that write the same buffers
 *     concurrently race.  The one piece of mutable global state is the static
 *     scratch of fa_fwd_kvcache_noalloc (one per device); every other entry
 *     point keeps none.
 *   - Tensors are contiguous, row-major: q, k, v, o are [B, H, N, d] (each
 *     (b, h) pair is one N x d matrix of the formula); lse is [B, H, N] fp32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.
 *   - Arguments are validated before any HIP call; a failure returns a
 *     negative status and enqueues nothing.  No entry point prints or throws.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

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
  FA_ERR_LAUNCH = -8,  /* the HIP runtime rejected the launch            */
  FA_ERR_SCRATCH = -9  /* the shape needs more than the static scratch  */
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

/*
 * fa_fwd_gqa — fa_fwd with K and V shared by groups of query heads
 * (multi-query and grouped-query attention; "FlashAttention (HI)", section on
 * development and further research, where FlashAttention-2 extends to
 * multi-query architectures).
 *   q, o    : [B,H,N,d];  k, v : [B,Hkv,N,d];  lse : [B,H,N] fp32.
 *   Hkv     : number of K/V heads, 1 <= Hkv <= H with H % Hkv == 0 (else
 *             FA_ERR_SHAPE).  Query head h of batch b attends with K/V head
 *             h / (H / Hkv) of batch b: consecutive query heads share one
 *             K/V head (Hkv = 1: one K/V head for all; Hkv = H: fa_fwd).
 * Every other argument, the results and the errors are those of fa_fwd.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, int causal, float scale, int dtype,
               void* stream);

/*
 * fa_bwd — backward pass of fa_fwd: the gradients of L = sum(dout * O) with
 * respect to q, k and v.  The pages print only the forward formula (section
 * on the problems of standard attention) and report training speed-ups on
 * "FlashAttention (HI)" (section on FlashAttention-2) that need its
 * gradient; differentiating O = softmax(S) V, S = scale Q K^T gives, per
 * (b, h), with P recomputed from lse (P_ij = exp(S_ij - lse_i), zero for
 * hidden keys) and D_i = dout_i . O_i:
 *     dV = P^T dout,  dS = P o (dout V^T - D),  dQ = scale dS K,
 *     dK = scale dS^T Q.
 *   q, k, v      : the forward's inputs [B,H,N,d], dtype FA_F16 or FA_BF16
 *                  (FA_F32 and FA_E4M3 return FA_ERR_DTYPE).
 *   o, lse       : the forward's outputs for these inputs, causal and scale
 *                  (o [B,H,N,d] of dtype, lse [B,H,N] fp32).
 *   dout         : upstream gradient dL/dO [B,H,N,d] of dtype.
 *   dq, dk, dv   : outputs [B,H,N,d] of dtype, rounded to nearest-even from
 *                  fp32 accumulators.  P and dS enter the second products
 *                  rounded to dtype.
 *   workspace    : device buffer of at least fa_bwd_workspace_bytes(B,H,N)
 *                  bytes, 16-byte aligned (else FA_ERR_ARG / FA_ERR_ALIGN),
 *                  owned by the caller; overwritten with per-row statistics
 *                  (base-2 logsumexp, D).  Its contents between calls carry
 *                  no meaning.
 *   causal, scale, d : as in fa_fwd.
 * Two kernels run in order on `stream`; no atomics, so results are the same
 * run to run.  Outputs must not overlap the inputs, each other or the
 * workspace (FA_ERR_ALIAS).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale,
           int dtype, void* stream);

/*
 * fa_bwd_gqa — fa_bwd with K/V heads shared as in fa_fwd_gqa: k, v, dk, dv are
 * [B,Hkv,N,d]; q, o, dout, dq are [B,H,N,d].  A shared K/V head's gradients
 * are the sums over the H / Hkv query heads of its group (accumulated in
 * registers, in a fixed order).  Other arguments as fa_bwd.
 */
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int H, int Hkv, int N, int d, int causal,
               float scale, int dtype, void* stream);

/*
 * Bytes of workspace fa_bwd needs: 8 * B * H * (N rounded up to 128), or 0
 * when B, H or N < 1.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_fwd_kvcache — attention of a short block of new queries against a long
 * key/value cache (decoding), the KV-cache inference of "FlashAttention
 * (HI)" (section on specialised solutions).  Same formula as fa_fwd with
 * different query and key counts:
 *   q, o    : [B,H,Nq,d] of dtype (FA_F16 or FA_BF16; others FA_ERR_DTYPE).
 *   k, v    : the cache, [B,Hkv,Nkv,d] of dtype, Nkv >= Nq >= 1 (else
 *             FA_ERR_SHAPE); K/V heads shared as in fa_fwd_gqa (Hkv = H:
 *             one per query head).
 *   lse     : output [B,H,Nq] fp32, natural-log logsumexp of each row.
 *   causal  : 1 = the queries are the sequence's last Nq positions: query i
 *             sees keys j <= Nkv - Nq + i (with Nq = 1, the whole cache).
 *   workspace, workspace_bytes : device buffer of at least
 *             fa_fwd_kvcache_workspace_bytes(...) bytes, 16-byte aligned,
 *             owned by the caller, overwritten (partial results of the
 *             cache chunks); may be NULL when that size is 0.
 * The cache is cut into chunks processed by separate workgroups and merged
 * exactly through their logsumexps; the cut depends only on the shape.
 */
int fa_fwd_kvcache(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int Nq,
                   int Nkv, int d, int causal, float scale, int dtype, void* stream);

/*
 * Workspace bytes fa_fwd_kvcache needs for this shape (0 when the cache is
 * not cut, and for invalid shapes).
 */
size_t fa_fwd_kvcache_workspace_bytes(int B, int H, int Hkv, int Nq, int Nkv, int d);

/* Size of the static scratch of fa_fwd_kvcache_noalloc, per device. */
#define FA_KVCACHE_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * fa_fwd_kvcache_noalloc — fa_fwd_kvcache for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same kernels, arguments and results, but the
 * workspace is the library's static scratch of FA_KVCACHE_SCRATCH_BYTES
 * bytes (a device array each GPU holds until the process ends) instead of a
 * caller buffer.  The caller still passes q, k, v, o and lse.
 *   - The scratch is the current device's (hipGetDevice); `stream` must
 *     belong to that device.  Its address is looked up on the first call on
 *     each device; no call allocates or frees memory.
 *   - Every call on one device uses the same scratch and leaves its partial
 *     results there; nothing in it needs to start at zero.  Calls that
 *     overlap in time on one device (other streams, other threads) race.
 *   - Status: those of fa_fwd_kvcache, and FA_ERR_SCRATCH when
 *     fa_fwd_kvcache_workspace_bytes(...) exceeds FA_KVCACHE_SCRATCH_BYTES
 *     (the cache cut keeps rows x chunks <= 16320, so no valid shape with
 *     d <= 256 does); FA_ERR_LAUNCH also when the scratch address cannot
 *     be obtained.
 */
int fa_fwd_kvcache_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Hkv, int Nq, int Nkv, int d, int causal, float scale,
                           int dtype, void* stream);

/*
 * fa_fwd_fp8 — the same pass with OCP e4m3fn (finite-only, max 448) inputs,
 * the 8-bit path of "FlashAttention-3 (BN)" / "(FA)" (sections on new
 * hardware capabilities and on low precision).
 *   q8, k8, v8          : [B,H,N,d] e4m3fn codes (one byte each).
 *   q/k/v_descale        : fp32 [B,H,ceil(N/128)]; the value of element
 *                          (b,h,i,c) is code * descale[b,h,i/128] (as written by
 *                          fa_quantize_e4m3).  Each must be a positive
 *                          normal fp32 value below 2^127 (not checked: they
 *                          live in device memory; other values give
 *                          unspecified output, never a fault).  Powers of two,
 *                          as fa_quantize_e4m3 writes, are applied exactly.
 *   o_bf16               : output [B,H,N,d] bfloat16.
 *   lse                  : output [B,H,N] fp32, natural-log logsumexp of the
 *                          scaled scores of the dequantised inputs.
 *   causal, scale, d     : as in fa_fwd (d in {64, 128, 256}, else
 *                          FA_ERR_HEADDIM).
 * P is rounded to e4m3 for the second product; before rounding it is scaled
 * by 2^6 (and by the non-power-of-two part of the V descale), which keeps it
 * <= 256 (no saturation) and mostly above e4m3's subnormal range.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_descale,
               const float* k_descale, const float* v_descale, void* o_bf16, float* lse,
               int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * fa_quantize_e4m3 — fp32 [B,H,N,d] -> e4m3fn codes x8 [B,H,N,d] and fp32
 * descale [B,H,ceil(N/block_rows)].  A block is block_rows (must be 128)
 * consecutive rows of one (b,h) with all d columns.  The descale is the
 * smallest power of two 2^e with amax <= 448 * 2^e (1 for an all-zero block)
 * and code = e4m3(clamp(x * 2^-e, -448, 448)) rounded to nearest even; the
 * power-of-two scaling is exact, so each code is a single rounding of
 * x / descale (the reading of the pages' per-block fp32 scale used here).
 *   rotate = 1 first applies x <- x H_d diag(signs) / sqrt(d) to every row
 *   (H_d the Sylvester Hadamard matrix; signs: device float[d] of +-1, NULL =
 *   all +1): the "incoherent processing" of the FlashAttention-3 pages, to be
 *   applied with the same signs to Q and K and never to V.
 * d in {64, 128, 256}.  x must not overlap x8 or descale.
 */
int fa_quantize_e4m3(const float* x, void* x8, float* descale, int B, int H, int N, int d,
                     int block_rows, int rotate, const float* signs, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
