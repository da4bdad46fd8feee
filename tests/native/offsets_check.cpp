// Host build of the library's offsets guard (csrc/offsets_check.hpp), as the
// tile-table, expert-order and segment-quantiser kernels apply it: thread e
// (0 <= e < E) tests pair e, and the array is rejected when any pair fails.
// Exhaustive over small arrays: the guard accepts exactly the arrays that
// run non-decreasing from 0 to rows, and for every accepted array each
// expert's rows [offsets[e], offsets[e+1]) lie inside [0, rows), so the
// tiles the table then describes only touch rows of the operands.  For a
// rejected array the table is all zeros: no tile and no segment.
// Prints "ok" and exits 0, or names the first failure and exits 1.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "offsets_check.hpp"

static int fail(const char* what, int E, int64_t rows,
                const std::vector<int32_t>& off) {
  std::printf("FAIL %s E=%d rows=%lld off=", what, E, (long long)rows);
  for (int32_t v : off) std::printf("%d ", v);
  std::printf("\n");
  return 1;
}

// what the kernels do with the guard's answer: tile_start[e] = prefix of
// ceil(M_e / unit) * tn, or all zeros when any pair fails
static std::vector<int64_t> tile_table(const std::vector<int32_t>& off, int E,
                                       int64_t rows, int unit, int tn) {
  bool bad = false;
  for (int e = 0; e < E; ++e) bad |= !moe::offsets_pair_ok(off.data(), e, E, rows);
  std::vector<int64_t> ts(E + 1, 0);
  if (bad) return ts;
  for (int e = 0; e < E; ++e)
    ts[e + 1] = ts[e] + (int64_t)((off[e + 1] - off[e] + unit - 1) / unit) * tn;
  return ts;
}

int main() {
  const int lo = -2, hi = 8;
  long cases = 0, accepted = 0;
  for (int E = 1; E <= 4; ++E) {
    std::vector<int32_t> off(E + 1, lo);
    for (;;) {
      for (int64_t rows = 0; rows <= 6; ++rows) {
        ++cases;
        // plain statement of validity
        bool valid = off[0] == 0 && off[E] == rows;
        for (int e = 0; e < E; ++e) valid = valid && off[e + 1] >= off[e];
        bool guard = true;
        for (int e = 0; e < E; ++e)
          guard = guard && moe::offsets_pair_ok(off.data(), e, E, rows);
        if (guard != valid) return fail("guard", E, rows, off);
        const int unit = 2, tn = 3;
        const std::vector<int64_t> ts = tile_table(off, E, rows, unit, tn);
        if (!guard) {
          for (int64_t v : ts)
            if (v != 0) return fail("rejected table not empty", E, rows, off);
          continue;
        }
        ++accepted;
        for (int e = 0; e < E; ++e) {
          if (off[e] < 0 || off[e + 1] > rows)
            return fail("segment outside rows", E, rows, off);
          // every tile of expert e starts inside its segment
          const int64_t nt = ts[e + 1] - ts[e];
          const int64_t mt = nt / tn;
          for (int64_t m = 0; m < mt; ++m)
            if (off[e] + m * unit >= off[e + 1])
              return fail("tile past its segment", E, rows, off);
        }
      }
      int i = 0;
      while (i <= E && ++off[i] > hi) off[i++] = lo;
      if (i > E) break;
    }
  }
  if (accepted == 0 || accepted == cases) {
    std::printf("FAIL coverage %ld of %ld accepted\n", accepted, cases);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
