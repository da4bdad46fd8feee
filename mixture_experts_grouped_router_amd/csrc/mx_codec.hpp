// MXFP8 element/scale encoding with integer operations only, and the index
// arithmetic of the GEMM scale layout.  Usable from device code (hipcc) and
// from plain C++ host code (CPU checks of the exact same functions).
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

// count of leading zero bits of a non-zero 32-bit value
MOE_HD inline int moe_clz32(uint32_t v) { return __builtin_clz(v); }

// E4M3 (OCP) code of a bfloat16 value scaled by 2^-s, computed with integer
// operations only: round to nearest even on the 3-bit mantissa grid,
// subnormals m*2^-9, saturation at 448 (0x7E), sign kept on zero results.
// `b` is the 16-bit bf16 pattern (finite), `s` the block scale exponent.
MOE_HD inline uint32_t e4m3_from_bf16(uint32_t b, int s) {
  const uint32_t sign = (b >> 8) & 0x80u;
  const int be = (int)((b >> 7) & 0xFF);
  uint32_t man = b & 0x7Fu;
  if (be == 0 && man == 0) return sign;
  // value = sig * 2^(ex - 7) with sig a 8-bit integer in [128, 256) for
  // normals; bf16 subnormals are normalised first.
  int ex;
  uint32_t sig;
  if (be == 0) {
    // subnormal: man * 2^-133; normalise to [128, 256)
    int lz = moe_clz32(man) - 24;  // leading zeros within 8 bits
    sig = man << lz;
    ex = -126 - lz;
  } else {
    sig = 0x80u | man;
    ex = be - 127;
  }
  ex -= s;  // scaled exponent: value = sig/128 * 2^ex
  // target quantum exponent: max(ex, -6) - 3; value / quantum =
  // sig * 2^(ex - 7 - q) with q = max(ex,-6)-3.
  int qe = (ex > -6 ? ex : -6) - 3;
  int shift = qe - (ex - 7);  // >= 4; right shift of sig
  uint32_t q;
  if (shift >= 32) {
    q = 0;
  } else {
    uint32_t kept = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    q = kept + ((rem > half || (rem == half && (kept & 1u))) ? 1u : 0u);
  }
  int e = (ex > -6 ? ex : -6);
  if (q >= 16u) { e += 1; q = 8u; }
  uint32_t code;
  if (q >= 8u) {
    if (e > 8) code = 0x7Eu;
    else {
      code = (uint32_t)((e + 7) << 3) | (q - 8u);
      if (code > 0x7Eu) code = 0x7Eu;
    }
  } else {
    code = q;  // subnormal (e == -6)
  }
  return code | sign;
}

// Scale exponent s of a block from the bf16 pattern of its amax (finite,
// sign cleared): floor(log2 amax) - 8 clamped to [-127, 127]; zero -> -127.
MOE_HD inline int e8m0_exp_from_bf16_amax(uint32_t a) {
  const int be = (int)((a >> 7) & 0xFF);
  // subnormal: man * 2^-133, floor(log2) = -133 + msb(man); zero gives
  // -133 here and clamps to -127 below (selects, no branches)
  const int msb = 31 - moe_clz32((a & 0x7Fu) | 1u);
  const int fl = be != 0 ? be - 127 : msb - 133;
  const int s = fl - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// E4M3 (OCP) code of a float32 value scaled by 2^-s, integer operations
// only, with the same rules as e4m3_from_bf16 (round to nearest even on the
// 3-bit mantissa grid, subnormals m*2^-9, saturation at 448, sign kept).
// `f` is the 32-bit pattern of a finite float.
MOE_HD inline uint32_t e4m3_from_f32(uint32_t f, int s) {
  const uint32_t sign = (f >> 24) & 0x80u;
  const int be = (int)((f >> 23) & 0xFF);
  const uint32_t man = f & 0x7FFFFFu;
  if (be == 0 && man == 0) return sign;
  // value = sig * 2^(ex - 23), sig in [2^23, 2^24)
  int ex;
  uint32_t sig;
  if (be == 0) {
    const int lz = moe_clz32(man) - 8;  // leading zeros within 24 bits
    sig = man << lz;
    ex = -126 - lz;
  } else {
    sig = 0x800000u | man;
    ex = be - 127;
  }
  ex -= s;
  const int e0 = ex > -6 ? ex : -6;
  // quantum 2^(e0 - 3): value / quantum = sig * 2^(ex - 23 - (e0 - 3))
  const int shift = (e0 - 3) - (ex - 23);  // >= 20
  uint32_t q;
  if (shift >= 25) {
    q = 0;  // below half a quantum (sig < 2^24)
  } else {
    const uint32_t kept = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    q = kept + ((rem > half || (rem == half && (kept & 1u))) ? 1u : 0u);
  }
  int e = e0;
  if (q >= 16u) { e += 1; q = 8u; }
  uint32_t code;
  if (q >= 8u) {
    if (e > 8) code = 0x7Eu;
    else {
      code = (uint32_t)((e + 7) << 3) | (q - 8u);
      if (code > 0x7Eu) code = 0x7Eu;
    }
  } else {
    code = q;
  }
  return code | sign;
}

// Scale exponent of a block from the float32 pattern of its amax (finite,
// sign cleared): floor(log2 amax) - 8 clamped to [-127, 127]; zero -> -127.
MOE_HD inline int e8m0_exp_from_f32_amax(uint32_t a) {
  const int be = (int)((a >> 23) & 0xFF);
  const uint32_t man = a & 0x7FFFFFu;
  int fl;
  if (be == 0) {
    if (man == 0) return -127;
    fl = -149 + (31 - moe_clz32(man));
  } else {
    fl = be - 127;
  }
  const int s = fl - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// n / d for n < 2^31 by multiply and shift: m = ceil(2^k / d) with
// k = 31 + ceil(log2 d) (so m < 2^32) is exact for every n < 2^31, since the
// rounding excess m d - 2^k is below d <= 2^(k - 31).
struct FastDiv {
  uint64_t m;
  uint32_t d;
  int k;
};
MOE_HD inline FastDiv make_fastdiv(uint32_t d) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.k = 31 + l;
  f.m = ((1ull << f.k) + d - 1) / d;
  return f;
}
MOE_HD inline uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)n * f.m) >> f.k);
}

// MXFP8 scales in the layout the scaled-MFMA GEMM reads: for an operand of
// rows r with K = 128 * nks values each, the four scale bytes of row r and
// K step s (K blocks 4s .. 4s+3) sit at ((r / 32) * nks + s) * 128 +
// (r % 32) * 4, so the 32 rows of one MFMA row block read one contiguous
// 128-byte line per K step.  Storage covers rows rounded up to 32.
MOE_HD inline uint32_t mx_tile_off(uint32_t r, uint32_t kb, uint32_t nks) {
  return ((r >> 5) * nks + (kb >> 2)) * 128u + ((r & 31u) << 2) + (kb & 3u);
}
inline size_t mx_tile_bytes(int64_t rows, int64_t k) {
  return (size_t)((rows + 31) / 32) * 32 * (size_t)(k / 32);
}

}  // namespace moe
