// Host check of every address the block quantiser forms (fa_quant_index.h):
// built by tests/test_quant_index_host.py with g++ under the address and
// undefined-behaviour sanitizers, no device involved.  For d = 64, 128, 256,
// with and without the rotation, and ragged sequence lengths:
//   * the 64-bit base address rebuilt from two 32-bit words equals the
//     original for addresses whose low word has bit 31 set (a signed low
//     word would corrupt the high word);
//   * the direct copies of each staging pass move every chunk of the pass's
//     rows exactly once, from inside the block, into the LDS tile;
//   * each thread reads back exactly the chunks of its own half row;
//   * the code staging is a bijection whose read-back returns what was
//     written, inside the tile;
//   * every global load and store of a block stays inside the tensor.
// Exit status 0 and "0 failures" when all hold.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fa_quant_index.h"

using namespace fa::qidx;

namespace {
int g_fail = 0;
#define CHECK(c, ...)                      \
  do {                                     \
    if (!(c)) {                            \
      if (g_fail < 20) {                   \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);          \
        std::printf("\n");                 \
      }                                    \
      ++g_fail;                            \
    }                                      \
  } while (0)

void check_join() {
  const uint64_t addrs[] = {0x00007f3a80001000ull, 0x0000000180000000ull, 0x00007fffffffff00ull,
                            0x0000123400000000ull, 0x00000000fffffff0ull, 0x0000555580000010ull};
  for (uint64_t a : addrs) {
    const uint32_t lo = (uint32_t)a, hi = (uint32_t)(a >> 32);
    CHECK(join_words(lo, hi) == a, "join_words(%08x, %08x) != %016llx", lo, hi, (unsigned long long)a);
    // the former bug: a low word taken as int and widened with sign
    const int slo = (int)lo;
    const uint64_t wrong = ((uint64_t)hi << 32) | (uint64_t)(int64_t)slo;
    if ((lo >> 31) & 1) CHECK(wrong != a, "sign extension should corrupt %016llx", (unsigned long long)a);
  }
}

template <int D, bool ROT>
void check_layout() {
  using G = Geo<D, ROT>;
  if constexpr (G::STAGE) {
    // copies of each pass: slot (LDS byte / 16) <- source chunk (byte offset in the block)
    for (int ps = 0; ps < G::NPASS; ++ps) {
      std::vector<int> src_of_slot(G::TILE_BYTES / 16, -1);
      std::vector<int> seen(G::NPASS * G::SR * G::RB / 16, 0);
      for (int u = 0; u < G::NI; ++u)
        for (int w = 0; w < 4; ++w)
          for (int lane = 0; lane < 64; ++lane) {
            const uint32_t src = dma_src<D, ROT>(ps, u, w, lane);
            const uint32_t dst = dma_dst<D, ROT>(u, w) + 16u * lane;
            CHECK(src % 16 == 0 && src < (uint32_t)(kBlockRows * G::RB), "D=%d src %u out of block", D, src);
            CHECK(src / G::RB >= (uint32_t)(ps * G::SR) && src / G::RB < (uint32_t)((ps + 1) * G::SR),
                  "D=%d pass %d copies row %u", D, ps, src / G::RB);
            CHECK(dst + 16 <= (uint32_t)G::TILE_BYTES, "D=%d dst %u past the tile", D, dst);
            if (dst + 16 <= (uint32_t)G::TILE_BYTES && src < (uint32_t)(kBlockRows * G::RB)) {
              CHECK(src_of_slot[dst / 16] == -1, "D=%d slot %u written twice", D, dst / 16);
              src_of_slot[dst / 16] = (int)src;
              ++seen[src / 16];
            }
          }
      for (int c = ps * G::SR * G::RB / 16; c < (ps + 1) * G::SR * G::RB / 16; ++c)
        CHECK(seen[c] == 1, "D=%d pass %d chunk %d copied %d times", D, ps, c, seen[c]);
      // each thread of this pass reads its own half row, chunk by chunk
      for (int lr = 0; lr < G::SR; ++lr)
        for (int hf = 0; hf < 2; ++hf)
          for (int k = 0; k < G::HC; ++k) {
            const uint32_t off = stage_read<D, ROT>(lr, hf, k);
            CHECK(off % 16 == 0 && off + 16 <= (uint32_t)G::TILE_BYTES, "D=%d read %u past the tile", D, off);
            if (off + 16 <= (uint32_t)G::TILE_BYTES) {
              const int want = ((ps * G::SR + lr) * G::RB) + (hf * G::HC + k) * 16;
              CHECK(src_of_slot[off / 16] == want, "D=%d row %d half %d chunk %d reads source %d, want %d", D,
                    lr, hf, k, src_of_slot[off / 16], want);
            }
          }
    }
    // code staging: thread (r, hf) writes logical chunk hf HCR + i of row r
    std::vector<int> logical(kBlockRows * D / 16, -1);
    for (int r = 0; r < kBlockRows; ++r)
      for (int hf = 0; hf < 2; ++hf)
        for (int i = 0; i < G::HCR; ++i) {
          const uint32_t off = code_write<D>(r, hf, i);
          CHECK(off % 16 == 0 && off + 16 <= (uint32_t)(kBlockRows * D) && off + 16 <= (uint32_t)G::TILE_BYTES,
                "D=%d code write %u out of range", D, off);
          if (off + 16 <= (uint32_t)(kBlockRows * D)) {
            CHECK(logical[off / 16] == -1, "D=%d code slot %u written twice", D, off / 16);
            logical[off / 16] = r * G::CR + hf * G::HCR + i;
          }
        }
    for (int rr = 0; rr < kBlockRows; ++rr)
      for (int c = 0; c < G::CR; ++c) {
        const uint32_t off = code_read<D>(rr, c);
        CHECK(off + 16 <= (uint32_t)(kBlockRows * D), "D=%d code read %u out of range", D, off);
        if (off + 16 <= (uint32_t)(kBlockRows * D))
          CHECK(logical[off / 16] == rr * G::CR + c, "D=%d row %d chunk %d reads logical %d", D, rr, c,
                logical[off / 16]);
      }
  }
}

// Global accesses of every block for a head count BH and length N: the copy
// resource of a staged block spans rows_left rows from the block's first row
// (offsets past it read zeros and touch no memory); direct loads and stores
// of the other path and the code stores stay inside the tensor.
template <int D, bool ROT>
void check_global(int BH, int N) {
  using G = Geo<D, ROT>;
  const uint64_t elems = (uint64_t)BH * N * D;
  const int nblk = (N + kBlockRows - 1) / kBlockRows;
  for (int bh = 0; bh < BH; ++bh)
    for (int blk = 0; blk < nblk; ++blk) {
      const int rows_left = N - blk * kBlockRows < kBlockRows ? N - blk * kBlockRows : kBlockRows;
      CHECK(rows_left >= 1, "D=%d N=%d empty block", D, N);
      const uint64_t blk_elem = ((uint64_t)bh * N + (uint64_t)blk * kBlockRows) * D;
      if constexpr (G::STAGE) {
        CHECK(blk_elem + (uint64_t)rows_left * D <= elems, "D=%d N=%d copy resource past the tensor", D, N);
        for (int rr = 0; rr < rows_left; ++rr)
          for (int c = 0; c < G::CR; ++c)
            CHECK(blk_elem + (uint64_t)rr * D + c * 16 + 16 <= elems, "D=%d N=%d code store past the tensor", D,
                  N);
      } else {
        for (int t = 0; t < 256; ++t) {
          const int r = t >> 1, hf = t & 1, row = blk * kBlockRows + r;
          if (row >= N) continue;
          const uint64_t base = ((uint64_t)bh * N + row) * D + hf * G::E;
          CHECK(base + G::E <= elems, "D=%d N=%d row load past the tensor", D, N);
        }
      }
    }
}

template <int D>
void check_d() {
  check_layout<D, false>();
  check_layout<D, true>();
  const int Ns[] = {1, 7, 127, 128, 129, 300, 1000, 4096};
  for (int N : Ns)
    for (int BH : {1, 3}) {
      check_global<D, false>(BH, N);
      check_global<D, true>(BH, N);
    }
}
}  // namespace

int main() {
  check_join();
  check_d<64>();
  check_d<128>();
  check_d<256>();
  std::printf("%d failures\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
