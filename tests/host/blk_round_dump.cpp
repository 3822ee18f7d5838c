// Host build of the library's blockwise-FP8 scale rule and fp32 -> E4M3
// encoder, for the CPU tests to compare with the oracle.
//   blk_round_dump <in.f32> <out.bin>
// out: for every bf16 magnitude m (32768): floored amax bits, t, scale bits
// (3 x uint32 each), then one E4M3 code byte per fp32 value read from in.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../moe_grouped_block_mx_amd/csrc/blk_round.hpp"

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  FILE* fi = std::fopen(argv[1], "rb");
  if (!fi) return 3;
  std::vector<uint32_t> vals;
  uint32_t v;
  while (std::fread(&v, 4, 1, fi) == 1) vals.push_back(v);
  std::fclose(fi);
  FILE* f = std::fopen(argv[2], "wb");
  if (!f) return 3;
  std::vector<uint32_t> rule(3 * 32768);
  for (uint32_t m = 0; m < 32768; ++m) {
    const uint32_t a = mxgg::blk_amax_floored_bits(m);
    const int t = mxgg::blk_pow2_t(a);
    rule[3 * m] = a;
    rule[3 * m + 1] = (uint32_t)t;
    rule[3 * m + 2] = mxgg::blk_pow2_scale_bits(t);
  }
  std::fwrite(rule.data(), 4, rule.size(), f);
  std::vector<uint8_t> codes(vals.size());
  for (size_t i = 0; i < vals.size(); ++i) codes[i] = (uint8_t)mxgg::f32_to_e4m3_rne_sat(vals[i]);
  std::fwrite(codes.data(), 1, codes.size(), f);
  std::fclose(f);
  return 0;
}
