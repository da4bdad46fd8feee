// Work items of the ragged-M grouped GEMMs (forward and dgrad), as plain
// integer arithmetic usable from device code (hipcc) and from plain C++
// host code, where a CPU build checks that the items cover every tile once.
//
// Tile list.  Expert e owns tiles [tile_start[e], tile_start[e+1]) of the
// launch: ceil(M_e / BM) M tiles times tn N tiles, taken in groups of
// kGroupN N tiles with the M tiles fastest inside a group (so the tiles
// running together on one XCD share weight panels and token rows in L2).
//
// XCD shares.  XCD x takes the contiguous run [x per, x per + cnt) of the
// list (per = ceil(total / 8), the last XCDs fewer), one tile per CU per
// round.  When the last, partly filled round holds rem <= C / 2 tiles (C
// CUs per XCD), each of those rem tiles may be split into S ranges of K
// steps (S <= kMaxSplit, rem S <= C, at least kMinSplitSteps steps per
// range, rem S <= the XCD's partial-tile slots): the XCD's items are then
// its whole tiles followed by rem S pieces.  Piece s of the tile at rank rt
// of the remainder covers K steps [s nk / S, (s + 1) nk / S) and owns
// partial slot x slots + rt S + s and arrival counter x slots + rt.
#pragma once
#include <stdint.h>

#include "mx_codec.hpp"

namespace moe {
namespace gg {

constexpr int BM = 256, BN = 256;   // GEMM tile (rows of A, rows of B)
constexpr int kGroupN = 4;          // N tiles per scheduling group
constexpr int kXcds = 8;            // XCDs (one L2 each)
constexpr int kMaxSplit = 8;        // pieces of a split tile
constexpr int kMaxSplitSlotsX = 32; // partial-tile slots per XCD
// Fewest K steps of a split piece: the partial tile's round trip and the
// cache write-back / invalidate of the hand-over cost ~15 microseconds per
// split tile, which only long K ranges repay (the Mixtral-shaped down GEMM,
// K = 14336, gains 10% in bf16 and 4% in MXFP8; the Qwen3-shaped gate/up
// GEMM, K = 2048, loses 3% with 16-step ranges).
constexpr int kMinSplitSteps = 32;

struct TileCoord {
  int e;        // expert
  int m0;       // first row of the tile inside the expert's M range
  int seg0;     // offsets[e]
  int seg_len;  // rows of expert e
  int nt;       // N tile index
};

struct SplitRange {
  int ks, ke;    // K steps [ks, ke) of this work-group
  int S;         // work-groups sharing the tile (1: not split)
  int slot0;     // first partial slot of the tile; this one is slot0 + s
  int s;
  int id;        // arrival counter
};

MOE_HD inline int wi_min(int a, int b) { return a < b ? a : b; }

// Coordinates of tile L (0 <= L < tile_start[E]): the expert by binary
// search (experts without tiles have tile_start[e] == tile_start[e+1] and
// are never selected), then the group and the tile inside it.
// M-tile records: after the tile prefix tile_start[0..E] (at int offset
// tile_rec_offset(E), 16-byte aligned) one record per M tile of the launch
// in tile-list order, {expert e, e's first M tile, offsets[e], rows of e}.
// Tile L of a launch with tn N tiles per M tile belongs to M tile L / tn,
// so one 16-byte read replaces the search over tile_start.
MOE_HD inline int tile_rec_offset(int E) { return (E + 1 + 3) & ~3; }
// ints of a tile table with records for a launch of at most rows routed rows
MOE_HD inline int64_t tile_table_ints(int E, int64_t rows) {
  return tile_rec_offset(E) + 4 * (rows / BM + E);
}

MOE_HD inline void ragged_m_tile_at(const int32_t* tile_start,
                                    const int32_t* offsets, int E, int L,
                                    TileCoord& tc, const int32_t* mrec = nullptr,
                                    int tn = 0) {
  int e, local, len, seg0;
  if (mrec) {
    const int32_t* r = mrec + 4 * (L / tn);
    e = r[0];
    local = L - r[1] * tn;
    seg0 = r[2];
    len = r[3];
  } else {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_start[mid] <= L) lo = mid; else hi = mid;
    }
    e = lo;
    local = L - tile_start[e];
    seg0 = offsets[e];
    len = offsets[e + 1] - seg0;
  }
  const int mt_e = (len + BM - 1) / BM;
  const int ng = local / (mt_e * kGroupN);
  const int in_g = local - ng * mt_e * kGroupN;
  tc.e = e;
  tc.m0 = (in_g % mt_e) * BM;
  tc.nt = ng * kGroupN + in_g / mt_e;
  tc.seg0 = seg0;
  tc.seg_len = len;
}

// The split setting of a launch (split = false: never split).
struct SplitCfg {
  bool split;
  int cus_per_xcd;   // C
  int slots_x;       // partial-tile slots per XCD
};

// Items of XCD x: cnt tiles, all whole, or whole = cnt - rem tiles and
// rem * S pieces.
struct XcdItems {
  int per, cnt, whole, rem, S;
  MOE_HD int count() const {
    return S > 1 ? whole + rem * S : (cnt > 0 ? cnt : 0);
  }
};
MOE_HD inline XcdItems xcd_items_at(int total, int x, const SplitCfg& sc,
                                    int nk) {
  XcdItems it;
  it.per = (total + kXcds - 1) / kXcds;
  it.cnt = wi_min(it.per, total - x * it.per);
  it.S = 1;
  it.rem = 0;
  const int C = sc.cus_per_xcd;
  if (sc.split && C > 0 && it.cnt > 0) {
    it.rem = it.cnt % C;
    if (it.rem > 0 && 2 * it.rem <= C) {
      it.S = wi_min(wi_min(C / it.rem, kMaxSplit),
                    wi_min(sc.slots_x / it.rem, nk / kMinSplitSteps));
      if (it.S < 2) it.S = 1;
    }
  }
  it.whole = it.S > 1 ? it.cnt - it.rem : it.cnt;
  return it;
}

// Item idx of XCD x: false past the XCD's items.
MOE_HD inline bool decode_item_at(const int32_t* tile_start,
                                  const int32_t* offsets, int E,
                                  const SplitCfg& sc, int nk, int x, int idx,
                                  TileCoord& tc, SplitRange& sr,
                                  const int32_t* mrec = nullptr, int tn = 0) {
  const int total = tile_start[E];
  const XcdItems it = xcd_items_at(total, x, sc, nk);
  if (it.cnt <= 0 || idx < 0) return false;
  sr.ks = 0;
  sr.ke = nk;
  sr.S = 1;
  sr.slot0 = sr.s = sr.id = 0;
  int L;
  if (idx < it.whole) {
    L = x * it.per + idx;
  } else {
    if (it.S == 1) return false;
    const int c = idx - it.whole;
    if (c >= it.rem * it.S) return false;
    const int rt = c / it.S;
    sr.s = c - rt * it.S;
    sr.S = it.S;
    sr.ks = sr.s * nk / it.S;
    sr.ke = (sr.s + 1) * nk / it.S;
    sr.slot0 = x * sc.slots_x + rt * it.S;
    sr.id = x * sc.slots_x + rt;
    L = x * it.per + it.whole + rt;
  }
  ragged_m_tile_at(tile_start, offsets, E, L, tc, mrec, tn);
  return true;
}

// Persistent launches: a work-group homed on XCD xh takes the next index of
// its XCD's counter, and once that XCD's items are used up the next index
// of the other XCDs' counters in turn (peek: a plain read of counter y,
// take: its fetch-and-add).  Returns (x, idx), or x = -1 when every XCD's
// items are taken.  Counters only grow, so a work-group ends after at most
// kXcds failed takes.
template <class Peek, class Take>
MOE_HD inline void take_item_with(int total, const SplitCfg& sc, int nk,
                                  int xh, Peek peek, Take take, int& x,
                                  int& idx) {
  x = -1;
  idx = 0;
  for (int d = 0; d < kXcds; ++d) {
    const int y = (xh + d) & (kXcds - 1);
    const int n = xcd_items_at(total, y, sc, nk).count();
    if (n <= 0) continue;
    if (d > 0 && peek(y) >= (uint32_t)n) continue;
    const uint32_t i = take(y);
    if (i < (uint32_t)n) {
      x = y;
      idx = (int)i;
      return;
    }
  }
}

}  // namespace gg
}  // namespace moe
