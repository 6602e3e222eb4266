// Device helpers shared by the attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;

typedef i16x4 __attribute__((address_space(3))) lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_cvoid;

// Key held by MFMA row i of a 32-key block: bits 2 and 3 of i swapped.  The
// map is its own inverse.  With it, accumulator register r of half-wave g
// holds key 16*(r/8) + 8*g + (r%8): eight consecutive keys per register group.
__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ float pair_max(float x) {
  // lanes l and l^32 hold the same query: v_permlane32_swap exchanges halves.
  auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

// 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane i's
// bytes land at LDS address lds_addr + 16 i; lds_addr must be wave-uniform.
// Written as inline assembly so that the compiler does not tie every later
// LDS read to this load's completion: the caller waits (s_waitcnt vmcnt(0))
// and synchronises the workgroup before any wave reads the buffer.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// Operands loaded into registers before a tile loop: a use the compiler
// sees, right after the loads have been waited for.  Without it the compiler
// takes them as still in flight at the loop head (it does not read an
// inline-assembly wait) and puts vmcnt waits before their uses inside the
// loop, which the hardware then applies to the tile copies in flight.
template <int N>
__device__ __forceinline__ void landed(const i32x4 (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(x[i]));
}

// Raw buffer resource over [base, base + bytes) (stride 0; data format 32 bit,
// the value the gfx9 family expects for untyped buffer loads).
// The base address and size go through readfirstlane: the resource must
// live in scalar registers, and this states that they are wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Raw buffer resource over [base + off, base + bytes), empty when off >= bytes,
// built in scalar registers: the copies of a tile at byte offset off then
// use per-lane offsets relative to the tile, and the tile offset costs no
// vector instruction.  The saturating subtract is written out because the
// compiler's form of it is a vector instruction (which would then put the
// whole resource in vector registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes, uint32_t off) {
  const uint32_t o = __builtin_amdgcn_readfirstlane(off);
  const uint32_t b = __builtin_amdgcn_readfirstlane(bytes);
  uint32_t left;
  asm("s_sub_u32 %0, %1, %2\n\ts_cselect_b32 %0, 0, %0" : "=s"(left) : "s"(b), "s"(o) : "scc");
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)base + o), 0, (int)left, 0x00020000);
}

// 16-byte buffer -> LDS copy per lane (buffer_load_dwordx4 ... lds): lane i's
// bytes land at LDS address lds_addr + 16 i.  An offset past the resource's
// size reads zeros instead of memory.  Inline assembly for the same reason
// as dma16: the caller does its own vmcnt accounting.
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMInit = -1.0e30f;  // finite start of the running max
constexpr float kLazy = 8.0f;       // log2 headroom before the running max moves

// s_waitcnt vmcnt(n) for a run-time n in [0, 31] (the counter's immediate is
// a compile-time field; gfx9 counts up to 63).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define FA_VMW(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    FA_VMW(0) FA_VMW(1) FA_VMW(2) FA_VMW(3) FA_VMW(4) FA_VMW(5) FA_VMW(6) FA_VMW(7)
    FA_VMW(8) FA_VMW(9) FA_VMW(10) FA_VMW(11) FA_VMW(12) FA_VMW(13) FA_VMW(14) FA_VMW(15)
    FA_VMW(16) FA_VMW(17) FA_VMW(18) FA_VMW(19) FA_VMW(20) FA_VMW(21) FA_VMW(22) FA_VMW(23)
    FA_VMW(24) FA_VMW(25) FA_VMW(26) FA_VMW(27) FA_VMW(28) FA_VMW(29) FA_VMW(30) FA_VMW(31)
#undef FA_VMW
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// Block index -> (head, query tile).  Workgroups are dispatched round-robin
// over the 8 XCDs (block b runs on XCD b % 8).  When the head count divides
// by 8, each XCD gets a contiguous range of heads so that all query tiles of
// a head share that XCD's L2 for K and V.  Without masking, an XCD runs its
// heads one after another (the tiles of a head stream the same K/V tiles at
// about the same time); with causal masking it goes tile-major, heaviest
// (last) query tiles of every head first, for load balance.  snake > 0 (the
// workgroups per CU of the launch): the first snake passes over an XCD's 32
// CUs, which fill the CUs' slots, alternate direction, so that a CU that
// receives one of the heaviest tiles in the first pass receives one of the
// lighter tiles of the second (2% on the 2048-token causal training shape
// at three workgroups per CU, 7% for its backward at two, 3-4% for fp8 at
// d = 64 and 256).
__device__ __forceinline__ void decode_block(int bid, int BH, int nq, bool causal,
                                             int& bh, int& qt, int snake = 0) {
  int t;
  if ((BH & 7) == 0) {
    const int hx = BH >> 3, xcd = bid & 7;
    int loc = bid >> 3;
    if (causal) {  // tile-major: heavy tiles of every head first
      const int pass = loc >> 5;  // complete passes only, so the map stays a bijection
      if ((pass & 1) && pass < snake && (pass + 1) * 32 <= nq * hx) loc = (pass << 5) + 31 - (loc & 31);
      t = loc / hx;
      bh = xcd * hx + loc % hx;
    } else {       // head-major: a head's tiles run together and share K/V in L2
      t = loc % nq;
      bh = xcd * hx + loc / nq;
    }
  } else {
    t = bid / BH;
    bh = bid % BH;
  }
  qt = causal ? nq - 1 - t : t;
}

// 16-bit element traits: the MFMA and the fp32 -> 16-bit packing (RNE).
template <typename T> struct Half;
template <> struct Half<__bf16> {
  static __device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  // x rounded to bf16 (nearest even, as pack2), returned as fp32
  static __device__ __forceinline__ float round1(float x) { return (float)(__bf16)x; }
};
template <> struct Half<_Float16> {
  static __device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ float round1(float x) { return (float)(_Float16)x; }
};

// XOR swizzle of the 16-byte chunk index inside an LDS row.  Rows of 256 B
// (d = 128) or 512 B (d = 256): the two 2-bit halves of row%16 are swapped, a
// bijection of 0..15 whose values over any 4 consecutive rows differ in bits
// 2-3.  Rows of 128 B (d = 64, two rows per 256-byte bank line): a map of
// row%16 onto 0..7 that, paired with the row's half of the line, is again a
// bijection, and differs in bit 2 between rows r and r+2.
template <int D>
__host__ __device__ constexpr int chunk_swz(int row) {
  if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else return ((row & 3) << 2) | ((row >> 2) & 3);
}

}  // namespace fa
