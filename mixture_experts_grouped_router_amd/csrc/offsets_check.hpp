// Validity of a per-expert offsets array, as the grouped kernels read it.
// Usable from device code (hipcc) and from plain C++ host code (a CPU build
// checks the exact same predicate).
//
// The grouped GEMMs, the tile-table and expert-order kernels and the
// token-segment quantiser take each expert's rows as [offsets[e],
// offsets[e+1]) of a tensor with `rows` rows.  The array is valid when
// offsets[0] == 0, it never decreases and offsets[E] == rows; then every
// segment lies inside [0, rows).  Anything else is a caller error that only
// the device can see (offsets live in device memory): the kernels record
// MOE_DEVERR_OFFSETS in the context status word and run no tile.
#pragma once
#include <stdint.h>

#include "mx_codec.hpp"

namespace moe {

// device status code (include/moe.h: MOE_DEVERR_OFFSETS)
constexpr int32_t kDevErrOffsets = 2;

// Pair e (0 <= e < E) of offsets: offsets[e] <= offsets[e+1], with the
// ends pinned (offsets[0] == 0 for the first pair, offsets[E] == rows for
// the last).  The array is valid iff every pair is.
MOE_HD inline bool offsets_pair_ok(const int32_t* off, int e, int E,
                                   int64_t rows) {
  const int32_t lo = off[e], hi = off[e + 1];
  if (hi < lo) return false;
  if (e == 0 && lo != 0) return false;
  if (e == E - 1 && (int64_t)hi != rows) return false;
  return true;
}

}  // namespace moe
