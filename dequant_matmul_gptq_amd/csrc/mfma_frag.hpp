// B fragments of v_mfma_f32_16x16x32_f16 taken straight from the packed
// words, shared by the prefill kernel and the multi-row decode kernel.
//
// The B operand of a 16 x 16 x 32 MFMA gives lane l column l % 16 and rows
// 8 (l / 16) .. + 7 of the 32-row block, i.e. pairs 4g .. 4g + 3 of the
// block's unpacking order (g = l / 16), with the K order inside the block
// being the MFMA pair order (row_lo(p), row_hi(p) of pair p = mfma_pair(b, q)
// at k = 2q, 2q + 1; the natural unpacking order except for 3 and 5 bits). Each
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

// The B fragment of k-group g from the words read for it: the pairs at
// positions 4g .. 4g + 3 of the MFMA pair order (mfma_pair) as 1024 + q, then
// (1024 + q) - (1024 + z) exactly and one rounding of s * d.
// The words as opaque register values: a lane-dependent choice between
// elements of the array would otherwise be folded into an indexed load, which
// puts the array in scratch memory.
template <int kW>
__device__ __forceinline__ void opaque_words(const uint32_t (&w)[kW], uint32_t (&v)[kW]) {
#pragma unroll
  for (int t = 0; t < kW; ++t) {
    v[t] = w[t];
    asm("" : "+v"(v[t]));
  }
}

template <int B, int kW>
__device__ __forceinline__ half8_t dequant_frag(const uint32_t (&w_in)[kW], int g, half2_t neg_bias, half2_t scale,
                                               uint32_t magic) {
  uint32_t w[kW];
  if constexpr (B == 3 || B == 5 || B == 6) {
    opaque_words(w_in, w);
  } else {
#pragma unroll
    for (int t = 0; t < kW; ++t) w[t] = w_in[t];
  }
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
  } else if constexpr (B == 3) {
    // MFMA pair order: k-group g < 3 takes slots 0..3 of word g; k-group 3
    // takes slot 4 of words 0, 1, 2 and the spare pair. Word and shift are
    // per-lane values, so each lane unpacks only its four pairs.
    constexpr uint32_t kMask = Fmt<3>::kMask;
    const bool last = g == 3;
    const uint32_t wg = g == 0 ? w[0] : g == 1 ? w[1] : w[2];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const uint32_t src = last ? w[r] : wg;
      const uint32_t sh = last ? 12u : 3u * r;
      pr[r] = ((src >> sh) & kMask) | magic;
    }
    const uint32_t reg = ((wg >> 9) & kMask) | magic;
    pr[3] = last ? extract_pair<3, 15>(w, magic) : reg;
  } else if constexpr (B == 5) {
    // MFMA pair order: k-group g takes slots 0..2 of word g, then slot g of
    // word 4 (g < 3) or the spare pair (g = 3).
    constexpr uint32_t kMask = Fmt<5>::kMask;
    const uint32_t wg = g == 0 ? w[0] : g == 1 ? w[1] : g == 2 ? w[2] : w[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) pr[r] = ((wg >> (5u * r)) & kMask) | magic;
    const uint32_t reg = ((w[4] >> (5u * (uint32_t)g)) & kMask) | magic;
    pr[3] = g == 3 ? extract_pair<5, 15>(w, magic) : reg;
  } else {
    static_assert(B == 6, "widths 2, 3, 4, 5, 6, 8");
    // Natural order: k-group g < 3 holds slots 0, 1 of words 2g and 2g + 1;
    // k-group 3 the four spare pairs.
    constexpr uint32_t kMask = Fmt<6>::kMask;
    const uint32_t wa = g == 0 ? w[0] : g == 1 ? w[2] : w[4];
    const uint32_t wb = g == 0 ? w[1] : g == 1 ? w[3] : w[5];
    const bool last = g == 3;
    pr[0] = last ? extract_pair<6, 12>(w, magic) : (wa & kMask) | magic;
    pr[1] = last ? extract_pair<6, 13>(w, magic) : ((wa >> 6) & kMask) | magic;
    pr[2] = last ? extract_pair<6, 14>(w, magic) : (wb & kMask) | magic;
    pr[3] = last ? extract_pair<6, 15>(w, magic) : ((wb >> 6) & kMask) | magic;
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
