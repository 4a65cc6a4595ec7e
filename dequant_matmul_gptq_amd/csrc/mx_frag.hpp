// B fragments of v_mfma_f32_16x16x32_f16 in the factored form, for the
// matrix-core decode kernel: straight from the packed words, each pair of
// codes exposed as the float16 pair (1024 + q_lo * 2^e, 1024 + q_hi * 2^e) by
// one AND-OR (plus a shift shared by the pairs above bit 10), and no
// subtraction or scaling per weight. The A fragment (the gathered
// activations) carries the matching 2^-e, so that per 32-row block
//   sum_k A[m][k] * B[k][n] = sum_j x_j q_j + 1024 * X'      (X' = sum_j x_j 2^-e_j)
// and the zero point and the group scale are applied once per group and
// column, in float32: y += s * (acc - 1024 X' - z X).
//
// Lane l of the MFMA holds column l % 16 and k-group g = l / 16 (k = 8g ..
// 8g + 7 of the block). Every lane runs the same instructions: it loads the
// packed words its k-group needs (per-lane addresses, mx_word) and extracts
// its four pairs with per-lane shift and mask values that are fixed for the
// whole kernel (MxLane). The K order inside a block ("mx order") follows:
// position k = 8g + 2r + h holds half h of pair r of k-group g.
//   b = 2, 4, 6, 8: k-group g holds pairs 4g .. 4g + 3 of the block.
//   b = 3: g < 3 takes slots 0..3 of word g; g = 3 takes slot 4 of words
//          0, 1, 2 and the spare pair (rows 30, 31).
//   b = 5: g takes slots 0..2 of word g, then slot g of word 4 (g < 3) or
//          the spare pair (g = 3).
#pragma once

#include "qlinear_device.hpp"

namespace qlinear {
namespace mx {

// Loads of packed words per lane and block for width B.
__host__ __device__ constexpr int loads(int B) {
  return B == 2 || B == 4 ? 1 : B == 8 ? 2 : B == 3 ? 3 : B == 5 ? 5 : 6;
}

// Block-relative packed row of load i for a lane of k-group g.
__host__ __device__ inline int word(int B, int g, int i) {
  switch (B) {
    case 2: return g >> 1;
    case 4: return g;
    case 8: return 2 * g + i;
    case 3: return g < 3 ? g : i;
    case 5: {
      if (g < 3) return i == 0 ? g : 4;
      const int w[5] = {3, 0, 1, 2, 4};
      return w[i];
    }
    default: {   // 6
      if (g < 3) return i < 2 ? 2 * g : 2 * g + 1;
      return i;
    }
  }
}

// Exponent e of pair r (A side scales it by 2^-e), the same for every k-group.
__host__ __device__ constexpr int exponent(int B, int r) {
  if (B == 4) return (r & 1) ? 4 : 0;
  if (B == 2) return 2 * r;
  if (B == 5) return r == 1 ? 5 : 0;
  return 0;
}

// Pair of the block (unpacking order, pair_rows) that k-group g's slot r holds.
__host__ __device__ constexpr int pair_of(int B, int g, int r) {
  if (B == 3) return g < 3 ? 5 * g + r : (r < 3 ? 5 * r + 4 : 15);
  if (B == 5) return r < 3 ? 3 * g + r : (g < 3 ? 12 + g : 15);
  return 4 * g + r;
}

// Position k (0..31) in mx order of block row rho, and its exponent.
__host__ __device__ inline void position(int B, int rho, int& k, int& e) {
  const int ph = pair_position(B, rho);   // 2 * pair + half
  const int P = ph >> 1, h = ph & 1;
  int g = 0, r = 0;
  if (B == 3) {
    if (P == 15) { g = 3; r = 3; }
    else if (P % 5 == 4) { g = 3; r = P / 5; }
    else { g = P / 5; r = P % 5; }
  } else if (B == 5) {
    if (P == 15) { g = 3; r = 3; }
    else if (P >= 12) { g = P - 12; r = 3; }
    else { g = P / 3; r = P % 3; }
  } else {
    g = P >> 2;
    r = P & 3;
  }
  k = 8 * g + 2 * r + h;
  e = exponent(B, r);
}

// Per-lane extraction constants of width B (loop-invariant registers).
struct Lane3 { uint32_t sh[3], s3[3], m3[3]; };
struct Lane5 { uint32_t s[5], m[5]; };
struct Lane6 { uint32_t sa[4], ma[4], sb[4], mb[4]; };

__host__ __device__ inline Lane3 lane3(int g) {
  Lane3 c;
  for (int r = 0; r < 3; ++r) c.sh[r] = g < 3 ? 3u * r : 12u;
  if (g < 3) {
    c.s3[0] = 9; c.m3[0] = 0x00070007u;
    c.s3[1] = 0; c.m3[1] = 0;
    c.s3[2] = 0; c.m3[2] = 0;
  } else {   // spare pair: code bit k sits in word k, bit 15 of each half
    c.s3[0] = 15; c.m3[0] = 0x00010001u;
    c.s3[1] = 14; c.m3[1] = 0x00020002u;
    c.s3[2] = 13; c.m3[2] = 0x00040004u;
  }
  return c;
}

__host__ __device__ inline Lane5 lane5(int g) {
  Lane5 c;
  if (g < 3) {   // load 1 is word 4: slot g
    for (int i = 0; i < 5; ++i) { c.s[i] = 0; c.m[i] = 0; }
    c.s[1] = 5u * g;
    c.m[1] = 0x001F001Fu;
  } else {       // loads are words 3, 0, 1, 2, 4: code bit k of the spare pair in word k, bit 15
    const int wk[5] = {3, 0, 1, 2, 4};
    for (int i = 0; i < 5; ++i) {
      c.s[i] = 15u - wk[i];
      c.m[i] = 0x00010001u << wk[i];
    }
  }
  return c;
}

__host__ __device__ inline Lane6 lane6(int g) {
  Lane6 c;
  for (int r = 0; r < 4; ++r) {
    if (g < 3) {   // loads 0, 1: word 2g; loads 2, 3: word 2g + 1; slot r & 1
      c.sa[r] = (r & 1) ? 6u : 0u;
      c.ma[r] = 0x003F003Fu;
      c.sb[r] = 0;
      c.mb[r] = 0;
    } else {       // spare pair r: low nibble in word r at bit 12, top bits in word 4 + r/2
      c.sa[r] = 12;
      c.ma[r] = 0x000F000Fu;
      c.sb[r] = 8u + 2u * (r & 1);
      c.mb[r] = 0x00300030u;
    }
  }
  return c;
}

// The four pairs of a lane from its loaded words w[0 .. loads(B) - 1].
// magic is kMagic (passed in a register by the kernels).
template <int B>
__host__ __device__ __forceinline__ void extract(const uint32_t* w, uint32_t magic, uint32_t g_shift2,
                                                 const Lane3& c3, const Lane5& c5, const Lane6& c6, uint32_t (&p)[4]) {
  if constexpr (B == 4) {
    const uint32_t ws = w[0] >> 8;
    p[0] = (w[0] & 0x000F000Fu) | magic;
    p[1] = (w[0] & 0x00F000F0u) | magic;
    p[2] = (ws & 0x000F000Fu) | magic;
    p[3] = (ws & 0x00F000F0u) | magic;
  } else if constexpr (B == 2) {
    const uint32_t ws = w[0] >> g_shift2;   // 8 * (g & 1)
    p[0] = (ws & 0x00030003u) | magic;
    p[1] = (ws & 0x000C000Cu) | magic;
    p[2] = (ws & 0x00300030u) | magic;
    p[3] = (ws & 0x00C000C0u) | magic;
  } else if constexpr (B == 8) {
    p[0] = (w[0] & 0x00FF00FFu) | magic;
    p[1] = ((w[0] >> 8) & 0x00FF00FFu) | magic;
    p[2] = (w[1] & 0x00FF00FFu) | magic;
    p[3] = ((w[1] >> 8) & 0x00FF00FFu) | magic;
  } else if constexpr (B == 3) {
    for (int r = 0; r < 3; ++r) p[r] = ((w[r] >> c3.sh[r]) & 0x00070007u) | magic;
    uint32_t t = ((w[0] >> c3.s3[0]) & c3.m3[0]) | magic;
    t = ((w[1] >> c3.s3[1]) & c3.m3[1]) | t;
    p[3] = ((w[2] >> c3.s3[2]) & c3.m3[2]) | t;
  } else if constexpr (B == 5) {
    p[0] = (w[0] & 0x001F001Fu) | magic;
    p[1] = (w[0] & 0x03E003E0u) | magic;
    p[2] = ((w[0] >> 10) & 0x001F001Fu) | magic;
    uint32_t t = magic;
    for (int i = 0; i < 5; ++i) t = ((w[i] >> c5.s[i]) & c5.m[i]) | t;
    p[3] = t;
  } else {
    static_assert(B == 6, "widths 2, 3, 4, 5, 6, 8");
    for (int r = 0; r < 4; ++r) {
      const uint32_t lo = ((w[r] >> c6.sa[r]) & c6.ma[r]) | magic;
      p[r] = ((w[4 + r / 2] >> c6.sb[r]) & c6.mb[r]) | lo;
    }
  }
}

}  // namespace mx
}  // namespace qlinear
