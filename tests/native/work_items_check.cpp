// Host build of the ragged-M work items (csrc/work_items.hpp), as the
// grouped GEMM kernels decode them.  For random expert row counts, N tile
// counts, K step counts and split settings it checks:
//   - the tile table's tiles map one to one onto (expert, M tile, N tile),
//     every M tile inside its expert's rows; the decode through the M-tile
//     records gives the same coordinates as the search over the prefix;
//   - over all XCDs, every tile is one whole item or exactly S pieces whose
//     K ranges are non-empty and partition [0, nk), and no item decodes
//     past an XCD's count;
//   - split pieces use partial slots and arrival counters inside their
//     XCD's range, distinct per tile, one counter per split tile;
//   - the persistent take protocol (own counter first, then the other
//     XCDs' in turn), run by work-groups homed on random XCDs in a random
//     interleaving, hands out every item exactly once and ends every
//     work-group.
// Prints "ok" and exits 0, or names the first failure and exits 1.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <map>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "work_items.hpp"

using namespace moe::gg;

static int fails = 0;
static void fail(const char* what, int E, int tn, int nk, int C) {
  if (fails++ < 5)
    std::printf("FAIL %s (E=%d tn=%d nk=%d C=%d)\n", what, E, tn, nk, C);
}

int main() {
  std::mt19937 rng(12345);
  for (int trial = 0; trial < 3000; ++trial) {
    const int E = 1 + (int)(rng() % 40);
    const int tn = 1 + (int)(rng() % 9);
    const int nk = 1 + (int)(rng() % 300);
    const int C = (int[]){4, 8, 16, 32}[rng() % 4];
    SplitCfg sc{(rng() % 3) != 0, C, (int)(rng() % (kMaxSplitSlotsX + 1))};
    // expert rows: zeros, a few rows, around a tile, several tiles
    std::vector<int32_t> off(E + 1, 0);
    for (int e = 0; e < E; ++e) {
      const int kind = (int)(rng() % 4);
      int m = kind == 0 ? 0 : kind == 1 ? (int)(rng() % 40)
              : kind == 2 ? 200 + (int)(rng() % 120) : (int)(rng() % 3000);
      off[e + 1] = off[e] + m;
    }
    std::vector<int32_t> ts(E + 1, 0);
    for (int e = 0; e < E; ++e)
      ts[e + 1] = ts[e] + ((off[e + 1] - off[e] + BM - 1) / BM) * tn;
    const int total = ts[E];
    // M-tile records as the tile-table kernel writes them, after the prefix
    // in one array of tile_table_ints(E, rows) ints
    std::vector<int32_t> table(tile_table_ints(E, off[E]), -7);
    for (int e = 0; e <= E; ++e) table[e] = ts[e];
    int32_t* rec = table.data() + tile_rec_offset(E);
    if ((tile_rec_offset(E) & 3) != 0) fail("records not 16-byte aligned", E, tn, nk, C);
    for (int e = 0; e < E; ++e) {
      const int first = ts[e] / tn, n = (ts[e + 1] - ts[e]) / tn;
      for (int i = 0; i < n; ++i) {
        if (4 * (first + i) + 3 >= (int)table.size() - tile_rec_offset(E))
          fail("records past the table", E, tn, nk, C);
        else {
          int32_t* r = rec + 4 * (first + i);
          r[0] = e; r[1] = first; r[2] = off[e]; r[3] = off[e + 1] - off[e];
        }
      }
    }

    // tile table <-> (expert, M tile, N tile)
    std::set<std::tuple<int, int, int>> coords;
    for (int L = 0; L < total; ++L) {
      TileCoord tc, tr;
      ragged_m_tile_at(ts.data(), off.data(), E, L, tc);
      ragged_m_tile_at(ts.data(), off.data(), E, L, tr, rec, tn);
      if (tr.e != tc.e || tr.m0 != tc.m0 || tr.nt != tc.nt ||
          tr.seg0 != tc.seg0 || tr.seg_len != tc.seg_len)
        fail("record decode differs from the search", E, tn, nk, C);
      const int len = off[tc.e + 1] - off[tc.e];
      if (tc.e < 0 || tc.e >= E || tc.m0 < 0 || tc.m0 % BM || tc.m0 >= len ||
          tc.nt < 0 || tc.nt >= tn || tc.seg0 != off[tc.e] ||
          tc.seg_len != len)
        fail("tile coordinates", E, tn, nk, C);
      if (!coords.insert({tc.e, tc.m0, tc.nt}).second)
        fail("tile coordinates repeat", E, tn, nk, C);
    }

    // items of every XCD cover every tile once
    std::map<std::tuple<int, int, int>, std::vector<std::pair<int, int>>> got;
    std::map<std::tuple<int, int, int>, std::set<int>> slots, ids;
    std::set<int> used_slots;
    int items = 0;
    for (int x = 0; x < kXcds; ++x) {
      const XcdItems it = xcd_items_at(total, x, sc, nk);
      const int n = it.count();
      items += n;
      for (int idx = 0; idx < n + 3; ++idx) {
        TileCoord tc;
        SplitRange sr;
        const bool ok =
            decode_item_at(ts.data(), off.data(), E, sc, nk, x, idx, tc, sr,
                           rec, tn);
        if (idx >= n) {
          if (ok) fail("item past the count decodes", E, tn, nk, C);
          continue;
        }
        if (!ok) {
          fail("item inside the count does not decode", E, tn, nk, C);
          continue;
        }
        const auto key = std::make_tuple(tc.e, tc.m0, tc.nt);
        if (!coords.count(key)) fail("item is no tile", E, tn, nk, C);
        if (sr.ks < 0 || sr.ke > nk || sr.ks >= sr.ke)
          fail("empty or outside K range", E, tn, nk, C);
        got[key].push_back({sr.ks, sr.ke});
        if (sr.S > 1) {
          if (sr.S > kMaxSplit || sr.s < 0 || sr.s >= sr.S ||
              sr.ke - sr.ks < kMinSplitSteps - 1 || !sc.split)
            fail("split piece", E, tn, nk, C);
          const int slot = sr.slot0 + sr.s;
          if (slot < x * sc.slots_x || slot >= (x + 1) * sc.slots_x ||
              sr.id < x * sc.slots_x || sr.id >= (x + 1) * sc.slots_x)
            fail("slot outside the XCD", E, tn, nk, C);
          if (!used_slots.insert(slot).second)
            fail("slot used twice", E, tn, nk, C);
          slots[key].insert(sr.s);
          ids[key].insert(sr.id);
        }
      }
    }
    if ((int)got.size() != total) fail("tiles missing", E, tn, nk, C);
    for (auto& kv : got) {
      auto v = kv.second;
      std::sort(v.begin(), v.end());
      int at = 0;
      for (auto& r : v) {
        if (r.first != at) fail("K ranges do not partition", E, tn, nk, C);
        at = r.second;
      }
      if (at != nk) fail("K ranges do not reach nk", E, tn, nk, C);
      if (v.size() > 1 && (slots[kv.first].size() != v.size() ||
                           ids[kv.first].size() != 1))
        fail("pieces of a tile: slots or counter", E, tn, nk, C);
    }

    // persistent take protocol: workers on random home XCDs, interleaved
    uint32_t q[kXcds] = {0};
    const int workers = kXcds * (1 + (int)(rng() % 6));
    std::vector<int> home(workers);
    for (int w = 0; w < workers; ++w) home[w] = (int)(rng() % kXcds);
    std::vector<bool> done(workers, false);
    std::set<std::pair<int, int>> taken;
    int left = workers, steps = 0;
    while (left > 0 && steps < 1000000) {
      const int w = (int)(rng() % workers);
      ++steps;
      if (done[w]) continue;
      int x, idx;
      take_item_with(
          total, sc, nk, home[w], [&](int y) { return q[y]; },
          [&](int y) { return q[y]++; }, x, idx);
      if (x < 0) {
        done[w] = true;
        --left;
        continue;
      }
      if (!taken.insert({x, idx}).second)
        fail("item taken twice", E, tn, nk, C);
      if (idx >= xcd_items_at(total, x, sc, nk).count())
        fail("taken item past the count", E, tn, nk, C);
    }
    if (left > 0) fail("work-groups did not end", E, tn, nk, C);
    if ((int)taken.size() != items) fail("items not all taken", E, tn, nk, C);
  }
  if (fails) return 1;
  std::printf("ok\n");
  return 0;
}
