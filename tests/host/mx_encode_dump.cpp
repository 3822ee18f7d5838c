// Host build of the library's MX element encoder, used by the CPU tests to
// compare it with the oracle over every bf16 magnitude and shared exponent.
#include <cstdio>
#include <cstdint>
#include <vector>
#include "../../moe_grouped_block_mx_amd/csrc/mx_round.hpp"

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  FILE* f = std::fopen(argv[1], "wb");
  if (!f) return 3;
  std::vector<uint8_t> row(32768);
  // shared exponents of every magnitude, E2M1 then E4M3
  std::vector<int16_t> se(2 * 32768);
  for (uint32_t m = 0; m < 32768; ++m) {
    se[m] = (int16_t)mxgg::mx_shared_exp<mxgg::E2M1Fmt>(m);
    se[32768 + m] = (int16_t)mxgg::mx_shared_exp<mxgg::E4M3Fmt>(m);
  }
  std::fwrite(se.data(), 2, se.size(), f);
  for (int fmt = 0; fmt < 2; ++fmt) {
    for (int e = -127; e <= 127; ++e) {
      for (uint32_t m = 0; m < 32768; ++m) {
        // magnitudes with exponent field 255 are Inf/NaN: not inputs
        uint32_t c = ((m >> 7) == 0xFF) ? 0 : (fmt == 0 ? mxgg::mx_encode_mag<mxgg::E2M1Fmt>(m, e)
                                                         : mxgg::mx_encode_mag<mxgg::E4M3Fmt>(m, e));
        row[m] = (uint8_t)c;
      }
      std::fwrite(row.data(), 1, row.size(), f);
    }
  }
  std::fclose(f);
  return 0;
}
