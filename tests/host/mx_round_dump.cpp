// Host build of the library's MX shared-exponent rule and E4M3 saturation
// bound, dumped for the CPU tests to compare with the oracle.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../moe_grouped_block_mx_amd/csrc/mx_round.hpp"

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  FILE* f = std::fopen(argv[1], "wb");
  if (!f) return 3;
  std::vector<int16_t> se(2 * 32768);
  for (uint32_t m = 0; m < 32768; ++m) {
    se[m] = (int16_t)mxgg::mx_shared_exp<mxgg::E2M1Fmt>(m);
    se[32768 + m] = (int16_t)mxgg::mx_shared_exp<mxgg::E4M3Fmt>(m);
  }
  std::fwrite(se.data(), 2, se.size(), f);
  std::vector<uint32_t> lim(255), scl(255);
  for (int e = -127; e <= 127; ++e) {
    lim[e + 127] = mxgg::e4m3_sat_limit_bits(e);
    scl[e + 127] = mxgg::mx_scale_operand_bits(e);
  }
  std::fwrite(lim.data(), 4, lim.size(), f);
  std::fwrite(scl.data(), 4, scl.size(), f);
  std::fclose(f);
  return 0;
}
