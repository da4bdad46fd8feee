// Host build of the library's index helpers (csrc/mx_codec.hpp): checks the
// multiply-shift division against '/' and that the MXFP8 GEMM scale layout
// maps every (row, K block) of an operand to a distinct byte inside its
// storage, with the 32 rows of a row block contiguous per K step.
// Prints "ok" and exits 0, or names the first failure and exits 1.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "mx_codec.hpp"

static int fail(const char* what, uint64_t a, uint64_t b, uint64_t c) {
  std::printf("FAIL %s %llu %llu %llu\n", what, (unsigned long long)a,
              (unsigned long long)b, (unsigned long long)c);
  return 1;
}

int main() {
  std::mt19937_64 rng(7);
  std::vector<uint32_t> ds;
  for (uint32_t d = 1; d <= 2048; ++d) ds.push_back(d);
  for (int l = 0; l < 32; ++l) {
    ds.push_back(1u << l);
    if (l > 1) ds.push_back((1u << l) - 1), ds.push_back((1u << l) + 1);
  }
  for (int i = 0; i < 2000; ++i) ds.push_back((uint32_t)(rng() % 0xFFFFFFFFull) + 1);
  const uint32_t nmax = 0x7FFFFFFFu;
  for (uint32_t d : ds) {
    const moe::FastDiv f = moe::make_fastdiv(d);
    std::vector<uint32_t> ns = {0, 1, nmax, nmax - 1};
    if (d <= nmax) {
      ns.push_back(d - 1); ns.push_back(d);
      if (d < nmax) ns.push_back(d + 1);
      ns.push_back(nmax / d * d); ns.push_back(nmax / d * d - 1);
    }
    for (int i = 0; i < 200; ++i) ns.push_back((uint32_t)(rng() & nmax));
    for (uint32_t n : ns)
      if (moe::fastdiv(n, f) != n / d) return fail("fastdiv", n, d, moe::fastdiv(n, f));
  }
  const uint32_t rows_list[] = {1, 31, 32, 33, 96, 160, 257};
  const uint32_t nks_list[] = {1, 2, 3, 32};
  for (uint32_t rows : rows_list)
    for (uint32_t nks : nks_list) {
      const size_t bytes = moe::mx_tile_bytes(rows, 128ll * nks);
      std::vector<uint8_t> seen(bytes, 0);
      for (uint32_t r = 0; r < rows; ++r)
        for (uint32_t kb = 0; kb < 4 * nks; ++kb) {
          const uint32_t o = moe::mx_tile_off(r, kb, nks);
          if (o >= bytes) return fail("tile_off range", r, kb, o);
          if (seen[o]++) return fail("tile_off collision", r, kb, o);
          // the dword of (r, step) sits at 4 (r % 32) in its 128-byte line
          const uint32_t line = moe::mx_tile_off(r & ~31u, kb & ~3u, nks);
          if (line % 128 || o != line + 4 * (r % 32) + kb % 4)
            return fail("tile_off line", r, kb, o);
        }
    }
  std::printf("ok\n");
  return 0;
}
