/*
 * MXFP8 row-wise quantisation of bfloat16 rows -- TEST INFRASTRUCTURE ONLY,
 * part of the CPU oracle.  Only tests/, __graft_entry__ and bench.py's
 * cpu_baseline may load it; the GPU library never does and shares no code
 * with it.
 *
 * The rule is the oracle's reading R7 (moe_oracle.py), written out in plain
 * C so that the full-size tests can quantise billions of weight values in
 * seconds: per block of 32 consecutive values v along a row,
 *   amax = max |v|; s = floor(log2 amax) - 8 clamped to [-127, 127]
 *   (amax = 0 -> -127); scale byte s + 127 (E8M0);
 *   code = OCP E4M3 of v * 2^-s: round to nearest even on the 3-bit mantissa
 *   grid (subnormals m * 2^-9), saturating at +-448, sign kept on zero.
 * The pages: "NVIDIA presents an efficient path for training biological MoE
 * models", section "Reducing memory and quantisation cost", and "Efficient
 * MoE training for biological foundation models (NVIDIA)", section "2) Model
 * size and activation memory" (8-bit elements, one scale per 32 consecutive
 * values).  Everything is evaluated in double, where each step is exact.
 * tests/test_oracle_pins.py checks it against moe_oracle.py bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* E4M3 code of a (finite, already scaled) double. */
static uint8_t e4m3_code(double v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs(v);
  if (a >= 448.0) return (uint8_t)(0x7E | sign);
  int ex = 0;
  int e;
  if (a > 0.0) {
    frexp(a, &ex);        /* a = m 2^ex, m in [0.5, 1) */
    e = ex - 1;           /* floor(log2 a) */
  } else {
    e = -7;
  }
  if (e < -6) e = -6;     /* below 2^-6: the subnormal grid */
  const double quantum = ldexp(1.0, e - 3);
  long q = (long)nearbyint(a / quantum);   /* exact quotient; ties to even */
  if (q >= 16) {          /* rounded up into the next binade */
    e += 1;
    q = 8;
  }
  const long code = q >= 8 ? (((long)(e + 7) << 3) | (q - 8)) : q;
  return (uint8_t)(code | sign);
}

static double e4m3_value(uint8_t c) {
  const int ef = (c >> 3) & 0xF, m = c & 7;
  const double mag = ef == 0 ? ldexp((double)m, -9)
                             : ldexp((double)(8 + m), ef - 10);
  return (c & 0x80) ? -mag : mag;
}

static int block_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int ex = 0;
  frexp(amax, &ex);
  int s = ex - 1 - 8;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

/* codes [rows, cols], scales [rows, cols / 32]; cols % 32 == 0.
 * dequant (nullable) [rows, cols] receives decode(code) * 2^s. */
static void quantize_row(const uint16_t* src, int64_t cols, uint8_t* codes,
                         uint8_t* scales, double* dequant) {
  for (int64_t b = 0; b < cols / 32; ++b) {
    double v[32];
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      v[i] = bf16_value(src[32 * b + i]);
      const double a = fabs(v[i]);
      if (a > amax) amax = a;
    }
    const int s = block_exponent(amax);
    if (scales) scales[b] = (uint8_t)(s + 127);
    for (int i = 0; i < 32; ++i) {
      const uint8_t c = e4m3_code(ldexp(v[i], -s));
      if (codes) codes[32 * b + i] = c;
      if (dequant) dequant[32 * b + i] = ldexp(e4m3_value(c), s);
    }
  }
}

void mx_fast_rows_bf16(const uint16_t* src, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales, double* dequant) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    quantize_row(src + r * cols, cols, codes ? codes + r * cols : 0,
                 scales ? scales + r * (cols / 32) : 0,
                 dequant ? dequant + r * cols : 0);
}
