// Internal interface between the C ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>

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
};

// fp16 / bf16 inputs, MFMA path.  d in {64, 128, 256}.
hipError_t launch_fwd_half(const FwdParams& p, int d, int causal, int is_bf16, hipStream_t s);
// fp32 inputs (v_mfma_f32_32x32x2f32).  d in {64, 128, 256}.
hipError_t launch_fwd_f32(const FwdParams& p, int d, int causal, hipStream_t s);

}  // namespace fa
