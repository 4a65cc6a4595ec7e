// Host-side probe of the kernels' packed-format helpers (place_code,
// extract_pair, pair_rows). It packs pseudo-random codes with the kernel
// packer and unpacks them with the kernel unpacker, printing codes, words and
// unpacked pairs so that the Python test can compare them with the oracle.
// Runs on the CPU only; calls no HIP runtime function.
#include <cstdio>

#include "qlinear_device.hpp"

using namespace qlinear;

static uint32_t lcg(uint32_t& s) {
  s = s * 1664525u + 1013904223u;
  return s >> 8;
}

template <int B>
static void probe(uint32_t seed, int ncols) {
  for (int c = 0; c < ncols; ++c) {
    uint32_t codes[kBlockRows];
    for (int r = 0; r < kBlockRows; ++r) codes[r] = lcg(seed) & ((1u << B) - 1u);
    if (c == 1)
      for (int r = 0; r < kBlockRows; ++r) codes[r] = (1u << B) - 1u;  // all ones
    uint32_t w[B] = {};
    for (int r = 0; r < kBlockRows; ++r) place_code<B>(w, r, codes[r]);
    uint32_t pr[kPairsPerBlock], ps[kPairsPerBlock], wsh[B];
    extract_all_pairs<B>(w, pr);
    for (int t = 0; t < B; ++t) wsh[t] = w[t] >> scaled_shift(B);
    [&]<int... P>(std::integer_sequence<int, P...>) {
      ((ps[P] = extract_pair_scaled<B, P>(w, wsh, kMagic)), ...);
    }(std::make_integer_sequence<int, kPairsPerBlock>{});
    std::printf("B %d\nC", B);
    for (int r = 0; r < kBlockRows; ++r) std::printf(" %u", codes[r]);
    std::printf("\nW");
    for (int t = 0; t < B; ++t) std::printf(" %u", w[t]);
    std::printf("\nP");
    for (int p = 0; p < kPairsPerBlock; ++p) {
      int lo, hi;
      pair_rows(B, p, lo, hi);
      std::printf(" %d:%d:%u:%u:%d", lo, hi, pr[p], ps[p], pair_exponent(B, p));
    }
    std::printf("\n");
  }
}

static int check_positions() {
  const int bs[6] = {2, 3, 4, 5, 6, 8};
  int bad = 0;
  for (int b : bs)
    for (int p = 0; p < kPairsPerBlock; ++p) {
      int lo, hi;
      pair_rows(b, p, lo, hi);
      if (pair_position(b, lo) != 2 * p || pair_position(b, hi) != 2 * p + 1) ++bad;
    }
  std::printf("POSBAD %d\n", bad);
  return bad;
}

int main() {
  check_positions();
  probe<2>(1u, 4);
  probe<3>(2u, 4);
  probe<4>(3u, 4);
  probe<5>(4u, 4);
  probe<6>(5u, 4);
  probe<8>(6u, 4);
  return 0;
}
