// B fragments of v_mfma_f32_16x16x32_f16 taken straight from the packed
// words, shared by the prefill kernel and the multi-row decode kernel.
//
// The B operand of a 16 x 16 x 32 MFMA gives lane l column l % 16 and rows
// 8 (l / 16) .. + 7 of the 32-row block, i.e. pairs 4g .. 4g + 3 of the
// block's unpacking order (g = l / 16), with the K order inside the block
// being the unpacking order (row_lo(p), row_hi(p) at k = 2p, 2p + 1). Each
// fragment is dequantized exactly: (1024 + q) - (1024 + z) in float16 is
// exact, then one rounding of s * (q - z).
#pragma once

#include <type_traits>

#include "qlinear_kernels.hpp"

namespace qlinear {
namespace frag {

constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, 32-bit data

// Native vector types: arrays of HIP's uint4 struct are kept in scratch memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

// Packed words of one (block, column) that the lanes of k-group g read, and
// the first of them (relative to the block's first packed row). Widths 2, 4
// and 8 keep a k-group's four pairs in one or two words; 3, 5 and 6 spread
// them, and all b words are read.
template <int B>
constexpr int frag_words() {
  return (B == 2 || B == 4) ? 1 : B == 8 ? 2 : B;
}
template <int B>
__device__ __forceinline__ int frag_first_word(int g) {
  return B == 4 ? g : B == 2 ? g / 2 : B == 8 ? 2 * g : 0;
}
template <unsigned BS>
constexpr int max_frag_words() {
  int m = 1;
  if ((BS >> 3) & 1u) m = m > 3 ? m : 3;
  if ((BS >> 5) & 1u) m = m > 5 ? m : 5;
  if ((BS >> 6) & 1u) m = m > 6 ? m : 6;
  if ((BS >> 8) & 1u) m = m > 2 ? m : 2;
  return m;
}

template <unsigned BS, class F>
__device__ __forceinline__ void with_width(int bits, F&& f) {
  switch (bits) {
    case 2: if constexpr ((BS >> 2) & 1u) f(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr ((BS >> 3) & 1u) f(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr ((BS >> 4) & 1u) f(std::integral_constant<int, 4>{}); break;
    case 5: if constexpr ((BS >> 5) & 1u) f(std::integral_constant<int, 5>{}); break;
    case 6: if constexpr ((BS >> 6) & 1u) f(std::integral_constant<int, 6>{}); break;
    case 8: if constexpr ((BS >> 8) & 1u) f(std::integral_constant<int, 8>{}); break;
    default: break;
  }
}

// The B fragment of k-group g from the words read for it: pairs 4g .. 4g + 3
// as 1024 + q, then (1024 + q) - (1024 + z) exactly and one rounding of s * d.
template <int B, int kW>
__device__ __forceinline__ half8_t dequant_frag(const uint32_t (&w)[kW], int g, half2_t neg_bias, half2_t scale,
                                               uint32_t magic) {
  uint32_t pr[4];
  if constexpr (B == 4 || B == 8) {
    pr[0] = extract_pair<B, 0>(w, magic);
    pr[1] = extract_pair<B, 1>(w, magic);
    pr[2] = extract_pair<B, 2>(w, magic);
    pr[3] = extract_pair<B, 3>(w, magic);
  } else if constexpr (B == 2) {
    const uint32_t ws[1] = {w[0] >> (8 * (g & 1))};
    pr[0] = extract_pair<2, 0>(ws, magic);
    pr[1] = extract_pair<2, 1>(ws, magic);
    pr[2] = extract_pair<2, 2>(ws, magic);
    pr[3] = extract_pair<2, 3>(ws, magic);
  } else {
    uint32_t all[kPairsPerBlock];
#pragma unroll
    for (int p = 0; p < kPairsPerBlock; ++p) all[p] = 0;
    static_for<0, kPairsPerBlock>([&](auto P) { all[decltype(P)::value] = extract_pair<B, decltype(P)::value>(w, magic); });
#pragma unroll
    for (int r = 0; r < 4; ++r)
      pr[r] = g == 0 ? all[r] : g == 1 ? all[4 + r] : g == 2 ? all[8 + r] : all[12 + r];
  }
  half8_t f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const half2_t d = dequant_pair(pr[r], neg_bias, scale);
    f[2 * r] = d[0];
    f[2 * r + 1] = d[1];
  }
  return f;
}

}  // namespace frag
}  // namespace qlinear
