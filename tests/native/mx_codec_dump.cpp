// Host build of the library's MXFP8 encode helpers (csrc/mx_codec.hpp):
// writes the E4M3 code of every bf16 pattern under every scale exponent in
// [-127, 127] (255 x 65536 bytes) and the scale exponent of every positive
// bf16 amax (32768 x int16) to the two files named on the command line.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "mx_codec.hpp"

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  std::vector<uint8_t> codes(255u * 65536u);
  for (int s = -127; s <= 127; ++s)
    for (uint32_t b = 0; b < 65536u; ++b) {
      const uint32_t e = (b >> 7) & 0xFF;
      codes[(size_t)(s + 127) * 65536u + b] =
          e == 0xFF ? 0xFF : (uint8_t)moe::e4m3_from_bf16(b, s);
    }
  std::vector<int16_t> sc(32768);
  for (uint32_t a = 0; a < 32768u; ++a)
    sc[a] = ((a >> 7) & 0xFF) == 0xFF ? 0 : (int16_t)moe::e8m0_exp_from_bf16_amax(a);
  FILE* f = std::fopen(argv[1], "wb");
  if (!f) return 1;
  std::fwrite(codes.data(), 1, codes.size(), f);
  std::fclose(f);
  f = std::fopen(argv[2], "wb");
  if (!f) return 1;
  std::fwrite(sc.data(), sizeof(int16_t), sc.size(), f);
  std::fclose(f);
  return 0;
}
