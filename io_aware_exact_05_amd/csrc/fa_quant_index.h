// Index arithmetic of the block quantiser (fa_quant.hip), kept apart so that
// a host program can enumerate every address the kernel forms and check it
// (tests/host/quant_index_check.cpp).  One workgroup of 256 threads handles
// a block of 128 rows of one (b, h); for d <= 128 the fp32 rows are staged in
// LDS by direct global -> LDS copies (SR rows per pass) and the codes leave
// through an LDS staging area as 16-byte stores of whole rows.
#pragma once
#include <stdint.h>

#ifndef __HIPCC__
#ifndef __host__
#define __host__
#endif
#ifndef __device__
#define __device__
#endif
#endif

namespace fa {
namespace qidx {

constexpr int kBlockRows = 128;

template <int D, bool ROT>
struct Geo {
  static constexpr int E = D / 2;                  // fp32 elements per thread (half a row)
  static constexpr int RB = D * 4;                 // fp32 bytes per row
  static constexpr int CPR = RB / 16, HC = CPR / 2;  // 16-byte chunks per row, per half row
  static constexpr bool STAGE = D <= 128;
  // two passes of 64 rows with the rotation, one of 128 without
  static constexpr int NPASS = ROT ? 2 : 1, SR = kBlockRows / NPASS;
  static constexpr int NI = SR * CPR / 256;        // copies per thread and pass
  static constexpr int CR = D / 16, HCR = CR / 2;  // 16-byte code chunks per row, per half row
  static constexpr int TILE_BYTES = STAGE ? SR * RB : 16;
};

// A 64-bit address rebuilt from its two wave-uniform 32-bit words.  Both
// words are unsigned: a signed low word would be sign-extended into the high
// word whenever its bit 31 is set.
__host__ __device__ inline uint64_t join_words(uint32_t lo, uint32_t hi) {
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// Copy u of pass ps by lane `lane` of wave w: byte offset of the source
// chunk within the block (row ps SR + rr, chunk position ^ (rr % HC)), and
// the LDS byte offset of the 1-KiB group it lands in (lane i at + 16 i).
template <int D, bool ROT>
__host__ __device__ inline uint32_t dma_src(int ps, int u, int w, int lane) {
  using G = Geo<D, ROT>;
  const int sl = (u * 4 + w) * 64 + lane, rr = sl / G::CPR, pos = sl % G::CPR;
  return (uint32_t)((ps * G::SR + rr) * G::RB + ((pos ^ (rr % G::HC)) << 4));
}
template <int D, bool ROT>
__host__ __device__ inline uint32_t dma_dst(int u, int w) {
  return (uint32_t)((u * 4 + w) * 1024);
}

// LDS byte offset of chunk k of half row hf of staged row lr (pass-local).
template <int D, bool ROT>
__host__ __device__ inline uint32_t stage_read(int lr, int hf, int k) {
  using G = Geo<D, ROT>;
  return (uint32_t)(lr * G::RB + ((hf * G::HC + (k ^ (lr % G::HC))) << 4));
}

// Code staging (D bytes per row): where thread (row r, half hf) writes its
// code chunk i, and where the store loop reads logical chunk c of row rr.
template <int D>
__host__ __device__ inline uint32_t code_write(int r, int hf, int i) {
  constexpr int HCR = D / 32;
  return (uint32_t)(r * D + ((hf * HCR + (i ^ (r % HCR))) << 4));
}
template <int D>
__host__ __device__ inline uint32_t code_read(int rr, int c) {
  constexpr int HCR = D / 32;
  return (uint32_t)(rr * D + (((c & ~(HCR - 1)) | ((c ^ (rr % HCR)) & (HCR - 1))) << 4));
}

}  // namespace qidx
}  // namespace fa
