// Device-side building blocks shared by the gfx950 kernels of the quantized
// linear layer: the run table passed as a kernel argument, the packed-format
// field placement, and the unpack of two codes at a time into a float16 pair.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <utility>

#include "qlinear.h"

namespace qlinear {

constexpr int kBlockRows = 32;          // rows per packing block (b words per block and column)
constexpr int kPanel = 16;              // output columns per storage panel
constexpr int kPairsPerBlock = 16;      // a block unpacks into 16 float16 pairs
constexpr uint32_t kMagic = 0x64006400u;  // float16 1024.0 in both halves

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Output epilogue, applied in float32 before the float16 rounding:
//   y[m][n] = RNE_fp16( act(acc + bias[n]) + residual[m][n] )
// with act the identity or SiLU, v / (1 + e^-v). Absent terms are NULL / 0.
struct Epilogue {
  const uint16_t* bias;       // float16 [N] or NULL
  const uint16_t* residual;   // float16 [M][N] or NULL (may be the output itself)
  const float* addend;        // float32 [M][N] or NULL (e.g. a LoRA update)
  int act;                    // QLINEAR_ACT_NONE or QLINEAR_ACT_SILU
  // Two-level scales: float16 q_scale_max [N], or NULL. When set, the
  // kernels read the scales operand as 4-bit codes c (uint32 [G][N/8], 8 per
  // word, column n at bits 4 (n % 8)) and weigh group g by (c + 1); the
  // remaining factor scale_max[n] / 16 is applied here, once per output.
  const uint16_t* scale_max;
};

// The float32 factor of a two-level scale code: c + 1 (exact).
__device__ __forceinline__ float qscale_factor(uint32_t word, int n) {
  return (float)(((word >> (4 * (n & 7))) & 15u) + 1u);
}

// y = act(v * scale_max / 16 + addend + bias) + residual. The operands are
// device (global) memory: read as such, also where the kernel has passed the
// pointers through registers the compiler cannot see.
__device__ __forceinline__ float apply_epilogue(const Epilogue& e, float v, int m, int n, int N) {
  typedef const __attribute__((address_space(1))) uint16_t* gptr;
  if (e.scale_max) v *= (float)__builtin_bit_cast(_Float16, ((gptr)e.scale_max)[n]) * 0.0625f;
  if (e.addend) v += ((const __attribute__((address_space(1))) float*)e.addend)[(size_t)m * N + n];
  if (e.bias) v += (float)__builtin_bit_cast(_Float16, ((gptr)e.bias)[n]);
  if (e.act == QLINEAR_ACT_SILU) v = v / (1.0f + __expf(-v));
  if (e.residual) v += (float)__builtin_bit_cast(_Float16, ((gptr)e.residual)[(size_t)m * N + n]);
  return v;
}

// Run table in units of 32-row blocks, copied into the kernel arguments.
struct Runs {
  int nruns;
  int blocks_per_group;                   // group_size / 32
  int packed_rows;                        // R
  int run_block[QLINEAR_MAX_RUNS + 1];    // first block of run r; [nruns] = K / 32
  int run_row[QLINEAR_MAX_RUNS + 1];      // first packed row of run r
  int run_bits[QLINEAR_MAX_RUNS];
};

// Storage index of word (packed row r, column n): 16-column panels, each
// holding its R rows contiguously, [ceil(N/16)][R][16].
__host__ __device__ __forceinline__ size_t word_index(int R, int r, int n) {
  return ((size_t)(n / kPanel) * R + r) * kPanel + (n % kPanel);
}

// Bit width and first packed row of 32-row block `blk`.
__device__ __forceinline__ void block_info(const Runs& R, int blk, int& bits, int& row) {
  int r = 0;
  while (r + 1 < R.nruns && blk >= R.run_block[r + 1]) ++r;
  bits = R.run_bits[r];
  row = R.run_row[r] + (blk - R.run_block[r]) * bits;
}

// Bit width of block `blk` when blk differs between lanes: a scan over the
// runs with wave-uniform indices, so the table is read with scalar loads
// (a lane-dependent index into the kernel arguments becomes a vector load,
// and waiting for it waits for every vector load issued before it).
__device__ __forceinline__ int block_bits_scan(const Runs& R, int blk) {
  int bits = R.run_bits[0];
  for (int r = 1; r < R.nruns; ++r) bits = blk >= R.run_block[r] ? R.run_bits[r] : bits;
  return bits;
}

// Last block (exclusive) of the run that contains `blk`.
__device__ __forceinline__ int run_end_block(const Runs& R, int blk) {
  int r = 0;
  while (r + 1 < R.nruns && blk >= R.run_block[r + 1]) ++r;
  return R.run_block[r + 1];
}

// ---------------------------------------------------------------------------
// Packed format. A block of 32 b-bit codes of one column is b words; every
// code lies inside one 16-bit half of a word, f = 16 / b codes per half.
// Unpacking produces 16 float16 pairs per block. Pair p holds two codes of
// the same column, one in each half, as 1024 + code: OR-ing a field that
// sits at the bottom of a half into the exponent bits of 1024.0 yields the
// float16 value 1024 + code exactly (codes are below 1024).
//
//   regular pair p < b*f: word t = p / f, slot i = p % f,
//       rows (2f*t + i, 2f*t + f + i)
//   b in {3, 5}, p = 15: rows (30, 31), code bit k in word k, bits 15 / 31
//   b = 6, p = 12 + v:   rows (24 + v, 28 + v), low nibble in word v bits
//       12..15 / 28..31, top two bits in word 4 + v/2
// ---------------------------------------------------------------------------

// Rows (within the block) held by pair p for width b; runtime version for staging.
__host__ __device__ __forceinline__ void pair_rows(int b, int p, int& lo, int& hi) {
  const int f = 16 / b;
  if (p < b * f) {
    const int t = p / f, i = p % f;
    lo = 2 * f * t + i;
    hi = lo + f;
  } else if (b == 6) {
    lo = 24 + (p - 12);
    hi = lo + 4;
  } else {
    lo = 30;
    hi = 31;
  }
}

// Pair order inside a block for the kernels that feed B fragments of a
// 16 x 16 x 32 MFMA from the packed words: position q = 4g + r (k-group g of
// the fragment, r < 4) holds pair mfma_pair(b, q). For 3 and 5 bits it keeps
// each k-group's pairs in as few words as possible, so a lane unpacks only
// its own four:
//   b = 3: g < 3 takes slots 0..3 of word g; g = 3 takes slot 4 of words
//          0, 1, 2 and the spare pair 15;
//   b = 5: g takes slots 0..2 of word g, then slot g of word 4 (g < 3) or
//          the spare pair 15 (g = 3).
// Other widths keep the natural order (for 6 bits, k-groups 0..2 hold two
// words each and k-group 3 the four spare pairs).
__host__ __device__ __forceinline__ int mfma_pair(int b, int q) {
  const int g = q >> 2, r = q & 3;
  if (b == 3) return g < 3 ? 5 * g + r : r < 3 ? 5 * r + 4 : 15;
  if (b == 5) return r < 3 ? 3 * g + r : g < 3 ? 12 + g : 15;
  return q;
}

template <int B>
struct Fmt {
  static constexpr int F = 16 / B;            // codes per half-word
  static constexpr int kRegular = B * F;      // regular pairs
  static constexpr uint32_t kMask = ((1u << B) - 1u) * 0x00010001u;
};

// Pair P of a block whose b words (one column) are w[0..B-1]; returns two
// float16 values 1024 + code packed in a uint32 (low half = lower row).
// `magic` is kMagic; kernels pass it in a VGPR so that a shift and one
// v_and_or_b32 (mask in an SGPR, magic in a VGPR) expose a pair.
template <int B, int P>
__host__ __device__ __forceinline__ uint32_t extract_pair(const uint32_t* w, uint32_t magic) {
  using Fm = Fmt<B>;
  if constexpr (P < Fm::kRegular) {
    constexpr int t = P / Fm::F, i = P % Fm::F;
    if constexpr (i == 0) {
      return (w[t] & Fm::kMask) | magic;
    } else {
      return ((w[t] >> (B * i)) & Fm::kMask) | magic;
    }
  } else if constexpr (B == 6) {
    constexpr int v = P - 12;
    const uint32_t lo = ((w[v] >> 12) & 0x000F000Fu) | magic;
    return ((w[4 + v / 2] >> (8 + 2 * (v % 2))) & 0x00300030u) | lo;
  } else {
    static_assert(B == 3 || B == 5, "spare rows exist only for 3, 5 and 6 bits");
    uint32_t r = ((w[0] >> 15) & 0x00010001u) | magic;
#pragma unroll
    for (int k = 1; k < B; ++k) r = ((w[k] >> (15 - k)) & (0x00010001u << k)) | r;
    return r;
  }
}

template <int B, int P>
__host__ __device__ __forceinline__ uint32_t extract_pair(const uint32_t* w) {
  return extract_pair<B, P>(w, kMagic);
}

// kMagic in a VGPR the compiler cannot fold back into a literal (VOP3 forms
// such as v_and_or_b32 take no literal operand on this architecture).
__device__ __forceinline__ uint32_t vgpr_magic() {
  uint32_t v;
  asm("v_mov_b32 %0, %1" : "=v"(v) : "i"(kMagic));
  return v;
}

// Scaled unpacking (decode path). A code whose field lies below bit 10 of its
// half is masked in place: (w & (mask << pos)) | 0x6400 is the float16 value
// 1024 + q * 2^pos, exactly. The activation paired with it is pre-scaled by
// 2^-pos, so the product keeps its value up to the known bias 1024 * x'.
// Fields at or above scaled_shift(b) are first moved down by one shift of the
// whole word, shared by all such fields of the word.
__host__ __device__ constexpr int scaled_shift(int b) { return b * ((10 - b) / b + 1); }

// Exponent e with pair p exposing 1024 + q * 2^e (0 for the spare pairs).
__host__ __device__ constexpr int pair_exponent(int b, int p) {
  const int f = 16 / b;
  if (p >= b * f) return 0;
  const int pos = b * (p % f);
  return pos + b <= 10 ? pos : pos - scaled_shift(b);
}

// Pair P from the block's words w[] and the same words shifted right by
// scaled_shift(B), wsh[] (only read for fields above the first 10 bits).
template <int B, int P>
__host__ __device__ __forceinline__ uint32_t extract_pair_scaled(const uint32_t* w, const uint32_t* wsh,
                                                                 uint32_t magic) {
  using Fm = Fmt<B>;
  if constexpr (P < Fm::kRegular) {
    constexpr int t = P / Fm::F, pos = B * (P % Fm::F);
    if constexpr (pos + B <= 10) {
      return (w[t] & (Fm::kMask << pos)) | magic;
    } else {
      return (wsh[t] & (Fm::kMask << (pos - scaled_shift(B)))) | magic;
    }
  } else {
    return extract_pair<B, P>(w, magic);
  }
}

// Position (2 * pair + half) of block row r in the unpacking order of width b:
// the inverse of pair_rows.
__host__ __device__ __forceinline__ int pair_position(int b, int r) {
  const int f = 16 / b;
  if (r < 2 * f * b) {
    const int t = r / (2 * f), u = r % (2 * f);
    return 2 * (t * f + u % f) + u / f;
  }
  if (b == 6) return 2 * (12 + (r - 24) % 4) + (r - 24) / 4;
  return 2 * 15 + (r - 30);
}

// Runtime-P dispatcher for the helper kernels (pack tests, dequant export).
template <int B>
__host__ __device__ __forceinline__ void extract_all_pairs(const uint32_t* w, uint32_t* out) {
  [&]<int... P>(std::integer_sequence<int, P...>) {
    ((out[P] = extract_pair<B, P>(w)), ...);
  }(std::make_integer_sequence<int, kPairsPerBlock>{});
}

// Write the code of block row r into the b words of its column (packing side).
template <int B>
__host__ __device__ __forceinline__ void place_code(uint32_t* w, int r, uint32_t code) {
  constexpr int F = 16 / B;
  code &= (1u << B) - 1u;
  if (r < 2 * F * B) {
    const int t = r / (2 * F), u = r % (2 * F);
    w[t] |= code << (16 * (u / F) + B * (u % F));
  } else if constexpr (B == 6) {
    const int h = (r - 24) / 4, v = (r - 24) % 4;
    w[v] |= (code & 0xFu) << (16 * h + 12);
    w[4 + v / 2] |= (code >> 4) << (16 * h + 12 + 2 * (v % 2));
  } else if constexpr (B == 3 || B == 5) {
    const int h = r - 30;
#pragma unroll
    for (int k = 0; k < B; ++k) w[k] |= ((code >> k) & 1u) << (16 * h + 15);
  }
}

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Exact float16 weights of a pair: RNE(s * ((1024 + q) - (1024 + z))).
// The subtraction of two integers below 2048 is exact in float16 and the
// product is rounded once, so the result is the correctly rounded s * (q - z).
__device__ __forceinline__ half2_t dequant_pair(uint32_t pair, half2_t neg_bias, half2_t scale) {
  const half2_t d = as_half2(pair) + neg_bias;
  return d * scale;
}

}  // namespace qlinear
