// Decode-sized layer (3 <= M <= 16, and 2 rows of wide 4-bit layers, as
// dispatched) on the matrix cores, in factored form.
//
// Each 32-row block is one v_mfma_f32_16x16x32_f16 step: A holds the token
// rows (M <= 16 of the MFMA's 16), B the block's codes as float16
// 1024 + q * 2^e straight out of the packed words (mx_frag.hpp), so the
// unpacking costs about one VALU operation per pair and the multiply runs on
// the matrix core. A carries the act-order-gathered activations pre-scaled by
// 2^-e, and the zero point and scale are applied once per unit of UB blocks
// that share them (a 128-row group with UB = 4, a block with UB = 1):
//   acc_u = sum_{j in u} x'_j (1024 + q_j 2^e_j) = sum_j x_j q_j + 1024 X'_u
//   y    += s * (acc_u - 1024 X'_u - z X_u)        (float32)
// with X_u the unit's sum of activations and X'_u that of the scaled ones.
// Both sums come from one more MFMA per block with a constant B (column 0
// all ones, column 1 the 2^e), broadcast across each 16-lane row by DPP.
//
// Work split: a workgroup of 8 waves owns a strip of 16 FN output columns
// (FN adjacent columns per lane, one 4 FN-byte load per packed row) and the
// whole K range, which its waves split into contiguous whole groups; their
// partial tiles are summed through LDS at the end (no split-K, no atomics).
// Strips are dealt to the 8 XCDs in contiguous ranges.
//
// Activations. In one-launch mode (M <= 8, LDS permitting) the workgroup
// gathers them itself: the x rows and the permutation are copied into LDS
// with global-to-LDS loads issued before any weight load (they use no
// registers, and complete before the weights because loads complete in
// order), then each thread builds k-group fragments (gathered by perm, in mx
// order, scaled by 2^-e), run by run with the width fixed at compile time.
// In two-launch mode the gather kernel below writes the same fragments for
// all 16 rows to the workspace and the main kernel loads them with the
// weights.
//
// The loop. A wave keeps D units of loads in flight (the unit's packed words,
// its scale and zero point; in two-launch mode also its A fragments),
// refilling a slot as soon as it is consumed. Before a unit's MFMAs it reads
// the next unit's A fragments from LDS, and it applies a unit's scale only
// after issuing the next unit's MFMAs (two accumulator sets), so that neither
// the LDS nor the matrix-core latency stalls the wave. Blocks go run by run,
// each run with its width fixed at compile time.
#pragma once

#include "mfma_frag.hpp"
#include "mx_frag.hpp"
#include "qgemv_stream.hpp"

namespace qlinear {

namespace mxk {

using frag::kRsrcWord3;
using frag::static_for;
using frag::u32x2;
using frag::u32x4;
using frag::with_width;
using stream::kMaxMats;
using stream::kXcds;
using stream::MatPtrs;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

enum Mode : int {
  kFewRows = 1,   // one launch, M <= 8
  kExact = 4,     // flag: B dequantized exactly (no sums MFMA, no per-unit epilogue)
  kGathered = 2,  // activations gathered by the gather kernel into the workspace
};

// Rows of the activations' fragments and sums per block / unit.
// The activation mode (kFewRows or kGathered) and the B form of a mode value.
constexpr int base_mode(int m) { return m & 3; }
constexpr bool exact_mode(int m) { return (m & kExact) != 0; }

// (one-launch mode: at most 8; MxArgs::ms holds the call's 4 or 8).
template <int kMode>
constexpr int rows_stored() {
  return base_mode(kMode) == kFewRows ? 8 : 16;
}

struct MxArgs {
  const uint16_t* x;     // float16 [M][K], original feature order (one-launch modes)
  const int32_t* perm;   // act-order permutation or NULL
  const uint16_t* xg;    // gathered fragments [nblk][16][32] float16 (two-launch mode)
  MatPtrs mat[kMaxMats];
  int mats, has_zeros;
  int M, K, N, bpg_shift;
  int nstrips, strips_per_xcd;
  int packed_rows;
  int64_t packed_words;
  int scale_bytes;       // bytes of the scales operand (float16 [G][N], or two-level codes [G][N/8] uint32)
  int scale_row_bytes;   // bytes per group row of the scales operand
  int two_level;         // 1: the scales operand holds two-level scale codes
  int lds_perm, lds_xg;   // byte offsets of the LDS regions (one-launch modes)
  int ms;                 // one-launch modes: fragment rows stored per block, 4 (M <= 4) or 8
  // Each wave's blocks [b0, b1) (whole groups) and its first segment (the
  // part of the run holding b0): its end block, first packed row and width.
  int wave_b0[kWaves], wave_b1[kWaves], wave_send[kWaves], wave_row0[kWaves], wave_bits0[kWaves];
  Runs runs;
  Epilogue epi;
};

template <int FN>
using WordVec = typename std::conditional<FN == 4, u32x4, typename std::conditional<FN == 2, u32x2, uint32_t>::type>::type;

template <int FN>
__device__ __forceinline__ WordVec<FN> load_vec(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t so) {
  if constexpr (FN == 4) return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, v, so, 0));
  else if constexpr (FN == 2) return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, v, so, 0));
  else return __builtin_amdgcn_raw_buffer_load_b32(r, v, so, 0);
}

template <int FN>
__device__ __forceinline__ uint32_t elem(const WordVec<FN>& w, int j) {
  if constexpr (FN == 1) return w;
  else return w[j];
}

// FN float16 scales and FN uint8 zero points of the lane's columns, loaded
// as whole aligned dwords (a 16- or 8-bit load would be re-masked where the
// ring wraps around the loop, and that use would wait for every load in
// flight); the lane picks its values with a shift (Lane::sshift, zshift).
template <int FN>
__device__ __forceinline__ uint32_t load_scales(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t so, uint32_t& hi) {
  if constexpr (FN == 4) {
    const u32x2 s = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, v, so, 0));
    hi = s[1];
    return s[0];
  } else {
    hi = 0;
    return __builtin_amdgcn_raw_buffer_load_b32(r, v, so, 0);
  }
}
__device__ __forceinline__ uint32_t load_zeros(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t so) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, v, so, 0);
}

// Slots of the load ring: one unit's packed words, scale and zero point, and
// in two-launch mode its A fragments.
template <int B, int FN, int UB>
struct Slot {
  WordVec<FN> w[UB][mx::loads(B)];
  uint32_t s0, s1, z;
  u32x4 x[UB];
};

// Units in flight per wave (even): about 32 words of codes per lane (fewer
// in two-launch mode, whose slots also hold the activations).
template <int B, int FN, int UB, int kMode>
constexpr int depth() {
  const int words = UB * mx::loads(B) * FN;
  int d = base_mode(kMode) == kGathered ? 40 / (words + 4 * UB) : 32 / words;
  d = d < 2 ? 2 : d > 8 ? 8 : d;
  return d & ~1;
}

// The lane's constant state.
struct Lane {
  __amdgpu_buffer_rsrc_t rw, rs, rz, rx;
  uint32_t wbase;     // byte offset of packed row 0 of the lane's first column (strip-relative)
  uint32_t sbase;     // byte offset of the lane's first scale in a scale row
  uint32_t zbase;
  uint32_t xoff;      // A fragment offset inside a block's fragments (bytes)
  uint32_t sshift;    // bit position of the lane's first scale (or scale code) in its loaded dword
  uint32_t zshift;    // bit position of the lane's first zero point in its loaded dword
  uint32_t srow;      // bytes per group row of the scales operand
  bool tl;            // two-level scale codes in place of float16 scales
  uint32_t magic;
  int g;              // k-group
  int n;              // column of the lane inside a 16-column fragment
};

// Lane constants of width B, fixed for a segment.
template <int B>
struct WidthConsts {
  uint32_t voff[mx::loads(B)];
  uint32_t sh2;
  mx::Lane3 c3;
  mx::Lane5 c5;
  mx::Lane6 c6;
  half8_t bsum;   // B operand of the sums MFMA
};

// The sums MFMA gives each row m, in column 0, X'_m = sum_k A[m][k] (the
// scaled activations) and in column 1 X_m = sum_k A[m][k] 2^e_k (the plain
// ones): B is 1 in column 0, 2^e in column 1 and 0 elsewhere.
template <int B>
__device__ __forceinline__ half8_t sums_operand(int n) {
  half8_t v;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const _Float16 h = n == 0 ? (_Float16)1.0f : n == 1 ? (_Float16)(float)(1 << mx::exponent(B, r)) : (_Float16)0.0f;
    v[2 * r] = h;
    v[2 * r + 1] = h;
  }
  return v;
}

template <int B>
__device__ __forceinline__ WidthConsts<B> width_consts(const Lane& L) {
  WidthConsts<B> c;
#pragma unroll
  for (int i = 0; i < mx::loads(B); ++i) c.voff[i] = L.wbase + (uint32_t)mx::word(B, L.g, i) * kPanel * 4;
  c.sh2 = 8u * (L.g & 1);
  if constexpr (B == 3) c.c3 = mx::lane3(L.g);
  if constexpr (B == 5) c.c5 = mx::lane5(L.g);
  if constexpr (B == 6) c.c6 = mx::lane6(L.g);
  c.bsum = sums_operand<B>(L.n);
  return c;
}

// A unit's packed words (its first packed row `row`).
template <int B, int FN, int UB>
__device__ __forceinline__ void issue_words(const Lane& L, const WidthConsts<B>& c, int row, Slot<B, FN, UB>& S) {
#pragma unroll
  for (int b = 0; b < UB; ++b) {
    const uint32_t ro = (uint32_t)(row + b * B) * kPanel * 4;
#pragma unroll
    for (int i = 0; i < mx::loads(B); ++i) S.w[b][i] = load_vec<FN>(L.rw, c.voff[i], ro);
  }
}

// A unit's scale and zero point (group grp), and in two-launch mode its
// activations (first block blk).
template <int B, int FN, int UB, int kMode>
__device__ __forceinline__ void issue_params(const Lane& L, int blk, int grp, int N, Slot<B, FN, UB>& S) {
  const uint32_t go = (uint32_t)grp * (uint32_t)N;
  S.s0 = load_scales<FN>(L.rs, L.sbase, (uint32_t)grp * L.srow, S.s1);
  S.z = load_zeros(L.rz, L.zbase, go);
  if constexpr (base_mode(kMode) == kGathered) {
#pragma unroll
    for (int b = 0; b < UB; ++b)
      S.x[b] = __builtin_bit_cast(u32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(L.rx, L.xoff, (uint32_t)(blk + b) * 16u * 64u, 0));
  }
}

// One-launch modes: a unit's A fragments from LDS.
template <int UB, int kMode>
__device__ __forceinline__ void lds_frags(const MxArgs& a, const Lane& L, const unsigned char* lds, int blk,
                                          half8_t (&af)[UB]) {
  const int ms = a.ms;
#pragma unroll
  for (int b = 0; b < UB; ++b) af[b] = *reinterpret_cast<const half8_t*>(lds + a.lds_xg + (blk + b) * ms * 64 + L.xoff);
}

template <int FN>
struct Acc {
  float4_t acc[2][2][FN];   // [unit parity][chain][fragment]: the unit's MFMA accumulators
  float4_t sacc[2][2];      // [unit parity][chain]: the unit's sums (columns 0 and 1)
  float4_t y[FN];           // the output rows' float32 sums
};

__device__ __forceinline__ float row_bcast(float v, int lane_in_row) {
  return __builtin_bit_cast(float, lane_in_row == 0
      ? __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150, 0xF, 0xF, false)    // row_newbcast:0
      : __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x151, 0xF, 0xF, false));  // row_newbcast:1
}

// y += s * (acc - 1024 X' - z X) for the lane's four rows, X' and X
// broadcast from columns 0 and 1 of the sums.
template <int FN, int kMode>
__device__ __forceinline__ void epilogue(uint32_t s0, uint32_t s1, uint32_t zw, uint32_t sshift, uint32_t zshift,
                                         bool tl, int zsym, int hz,
                                         const float4_t (&c0)[FN], const float4_t (&c1)[FN], const float4_t& sa0,
                                         const float4_t& sa1, bool two_chains, float4_t (&y)[FN]) {
  float Xs[4], X[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float v = two_chains ? sa0[r] + sa1[r] : sa0[r];
    Xs[r] = 1024.0f * row_bcast(v, 0);
    X[r] = row_bcast(v, 1);
  }
  const uint32_t sl = (FN == 1 || tl) ? s0 >> sshift : s0;
  const uint32_t zl = zw >> zshift;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const uint32_t sw = j < 2 ? sl : s1;
    // Two-level scales: the code's factor c + 1 (scale_max / 16 is applied
    // in the final epilogue).
    const float s = tl ? (float)(((sl >> (4 * j)) & 15u) + 1u)
                       : (float)__builtin_bit_cast(_Float16, (uint16_t)(sw >> (16 * (j & 1))));
    const float z = hz ? (float)((zl >> (8 * j)) & 0xFFu) : (float)zsym;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float t = (two_chains ? c0[j][r] + c1[j][r] : c0[j][r]) - Xs[r];
      y[j][r] = fmaf(s, fmaf(-z, X[r], t), y[j][r]);
    }
  }
}

// The units [0, n) of one width B starting at block blk0 and packed row
// row0. With kPre the packed words of the first D units are already in S.
// Unit u is consumed from slot u % D; after unit u + 1's MFMAs are issued,
// unit u's epilogue reads its scale from the slot, and only then is the slot
// refilled with unit u + D (nothing loaded is copied to other registers).
template <int B, int FN, int UB, int kMode, bool kPre>
__device__ __forceinline__ Acc<FN> segment(const MxArgs& a, const Lane& L, const unsigned char* lds, int blk0, int n,
                                           int row0, int N, int bpg_shift, int hz, Acc<FN> A,
                                           Slot<B, FN, UB> (&S)[depth<B, FN, UB, kMode>()]) {
  constexpr int D = depth<B, FN, UB, kMode>();
  constexpr bool kTwo = UB > 1;
  constexpr int zsym = 1 << (B - 1);
  const WidthConsts<B> c = width_consts<B>(L);
  auto params = [&](int i, Slot<B, FN, UB>& s) {
    const int ii = i < n ? i : n - 1;   // past the end: the last unit again (never computed)
    const int blk = blk0 + ii * UB;
    issue_params<B, FN, UB, kMode>(L, blk, blk >> bpg_shift, N, s);
  };
  auto fill = [&](int i, Slot<B, FN, UB>& s) {
    const int ii = i < n ? i : n - 1;
    issue_words<B, FN, UB>(L, c, row0 + ii * UB * B, s);
    params(i, s);
  };
  if constexpr (kPre) {
    static_for<0, D>([&](auto Dd) { params(decltype(Dd)::value, S[decltype(Dd)::value]); });
  } else {
    static_for<0, D>([&](auto Dd) { fill(decltype(Dd)::value, S[decltype(Dd)::value]); });
  }
  half8_t af[2][UB];
  if constexpr (base_mode(kMode) != kGathered) lds_frags<UB, kMode>(a, L, lds, blk0, af[0]);
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};

  if constexpr (exact_mode(kMode)) {
    // Exact B: each pair (1024 + q 2^e) - (1024 + z 2^e) = (q - z) 2^e exactly
    // (1024 + z 2^e is a multiple of 2^e below 2^15, so exact in float16 for
    // any uint8 z), times s with one rounding; the A side carries 2^-e, so
    // A B = x RNE(s (q - z)) exactly. The accumulators (two per unit parity)
    // run over all of K; there is no per-unit epilogue and no sums MFMA.
    auto unit_ex = [&](int i, auto Dd, bool steady) {
      constexpr int d = decltype(Dd)::value;
      constexpr int p = d & 1;
      Slot<B, FN, UB>& s = S[d];
      if constexpr (base_mode(kMode) != kGathered) {
        const int in = i + 1 < n ? i + 1 : i;
        lds_frags<UB, kMode>(a, L, lds, blk0 + in * UB, af[p ^ 1]);
      }
      half2_t sc2[FN], bias2[FN][4];
      {
        const uint32_t sl = (FN == 1 || L.tl) ? s.s0 >> L.sshift : s.s0;
        const uint32_t zl = s.z >> L.zshift;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint32_t sw = j < 2 ? sl : s.s1;
          const _Float16 sh = L.tl ? (_Float16)(float)(((sl >> (4 * j)) & 15u) + 1u)
                                   : __builtin_bit_cast(_Float16, (uint16_t)(sw >> (16 * (j & 1))));
          sc2[j] = half2_t{sh, sh};
          const float zf = hz ? (float)((zl >> (8 * j)) & 0xFFu) : (float)zsym;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const _Float16 bh = (_Float16)(1024.0f + zf * (float)(1 << mx::exponent(B, r)));
            bias2[j][r] = half2_t{bh, bh};
          }
        }
      }
      static_for<0, UB>([&](auto Bb) {
        constexpr int b = decltype(Bb)::value;
        constexpr int ch = b & 1;
        half8_t ab;
        if constexpr (base_mode(kMode) == kGathered) ab = __builtin_bit_cast(half8_t, s.x[b]);
        else ab = af[p][b];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          uint32_t w[mx::loads(B)];
#pragma unroll
          for (int k = 0; k < mx::loads(B); ++k) w[k] = elem<FN>(s.w[b][k], j);
          uint32_t q[4];
          mx::extract<B>(w, L.magic, c.sh2, c.c3, c.c5, c.c6, q);
          half2_t h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = (__builtin_bit_cast(half2_t, q[r]) - bias2[j][r]) * sc2[j];
          const half8_t bf = half8_t{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
          A.acc[p][ch][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, bf, A.acc[p][ch][j], 0, 0, 0);
        }
      });
      // The slot's words and parameters are read: it takes unit i + D.
      if (steady) fill(i + D, s);
      else if (i + D < n) fill(i + D, s);
    };
    int i = 0;
    for (; i + 2 * D <= n; i += D) static_for<0, D>([&](auto Dd) { unit_ex(i + decltype(Dd)::value, Dd, true); });
    static_for<0, D>([&](auto Dd) {
      if (i + (int)decltype(Dd)::value < n) unit_ex(i + decltype(Dd)::value, Dd, false);
    });
    i += D;
    static_for<0, D>([&](auto Dd) {
      if (i + (int)decltype(Dd)::value < n) unit_ex(i + decltype(Dd)::value, Dd, false);
    });
    return A;
  }

  // Unit i from slot d (its parity d & 1: D is even and rounds start at multiples of D).
  auto unit = [&](int i, auto Dd, bool steady) {
    constexpr int d = decltype(Dd)::value;
    constexpr int p = d & 1;
    constexpr int dp = (d + D - 1) % D;   // the previous unit's slot
    Slot<B, FN, UB>& s = S[d];
    if constexpr (base_mode(kMode) != kGathered) {
      const int in = i + 1 < n ? i + 1 : i;
      lds_frags<UB, kMode>(a, L, lds, blk0 + in * UB, af[p ^ 1]);
    }
    static_for<0, UB>([&](auto Bb) {
      constexpr int b = decltype(Bb)::value;
      constexpr int ch = kTwo ? (b & 1) : 0;     // two accumulation chains per unit of 4 blocks
      constexpr bool fresh = b < (kTwo ? 2 : 1);
      half8_t ab;
      if constexpr (base_mode(kMode) == kGathered) ab = __builtin_bit_cast(half8_t, s.x[b]);
      else ab = af[p][b];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        uint32_t w[mx::loads(B)];
#pragma unroll
        for (int k = 0; k < mx::loads(B); ++k) w[k] = elem<FN>(s.w[b][k], j);
        uint32_t q[4];
        mx::extract<B>(w, L.magic, c.sh2, c.c3, c.c5, c.c6, q);
        const half8_t bf = __builtin_bit_cast(half8_t, u32x4{q[0], q[1], q[2], q[3]});
        A.acc[p][ch][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, bf, fresh ? zero : A.acc[p][ch][j], 0, 0, 0);
      }
      A.sacc[p][ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, c.bsum, fresh ? zero : A.sacc[p][ch], 0, 0, 0);
    });
    if (i > 0) {
      // The previous unit: its epilogue, then its slot takes unit i - 1 + D.
      const Slot<B, FN, UB>& sp = S[dp];
      epilogue<FN, kMode>(sp.s0, sp.s1, sp.z, L.sshift, L.zshift, L.tl, zsym, hz, A.acc[p ^ 1][0], A.acc[p ^ 1][1], A.sacc[p ^ 1][0],
                          A.sacc[p ^ 1][1], kTwo, A.y);
      if (steady) fill(i - 1 + D, S[dp]);
      else if (i - 1 + D < n) fill(i - 1 + D, S[dp]);
    }
    if (i == n - 1)
      epilogue<FN, kMode>(s.s0, s.s1, s.z, L.sshift, L.zshift, L.tl, zsym, hz, A.acc[p][0], A.acc[p][1], A.sacc[p][0], A.sacc[p][1], kTwo,
                          A.y);
  };

  // Steady rounds: every slot refilled, unconditionally (clamped past the end).
  int i = 0;
  for (; i + 2 * D <= n; i += D) static_for<0, D>([&](auto Dd) { unit(i + decltype(Dd)::value, Dd, true); });
  // The last 1 .. 2D - 1 units.
  static_for<0, D>([&](auto Dd) {
    if (i + (int)decltype(Dd)::value < n) unit(i + decltype(Dd)::value, Dd, false);
  });
  i += D;
  static_for<0, D>([&](auto Dd) {
    if (i + (int)decltype(Dd)::value < n) unit(i + decltype(Dd)::value, Dd, false);
  });
  return A;
}

// The packed words of the first D units of a segment, issued before the
// activations are staged: D * UB * loads(B) loads, all from distinct rows
// (slots past the segment read the rows that follow it, or past the end of
// the buffer, which reads zeros; they are never computed), so none can be
// merged with another and the staging wait can count them.
template <int B, int FN, int UB, int kMode>
__device__ __forceinline__ void pre_issue(const Lane& L, int row0, Slot<B, FN, UB> (&S)[depth<B, FN, UB, kMode>()]) {
  const WidthConsts<B> c = width_consts<B>(L);
  static_for<0, depth<B, FN, UB, kMode>()>([&](auto Dd) {
    constexpr int d = decltype(Dd)::value;
    issue_words<B, FN, UB>(L, c, row0 + d * UB * B, S[d]);
  });
}

// Width of block blk (a loop over the runs; the two-launch gather only).
__device__ __forceinline__ int width_of(const Runs& R, int blk) {
  int bits = R.run_bits[0];
  for (int r = 1; r < R.nruns; ++r) bits = blk >= R.run_block[r] ? R.run_bits[r] : bits;
  return bits;
}

// The block rows that k-group g's fragment holds at width B, in mx order:
// pair r of the fragment is rows (row[2r], row[2r + 1]), scaled by 2^-e_r.
template <int B>
struct FragRows {
  int row[8];
};

template <int B>
__device__ __forceinline__ FragRows<B> frag_rows(int g) {
  FragRows<B> f;
#pragma unroll
  for (int r = 0; r < 4; ++r) pair_rows(B, mx::pair_of(B, g, r), f.row[2 * r], f.row[2 * r + 1]);
  return f;
}

// One k-group fragment of block blk for activation rows m < rows: the 8
// values x[m][feature(blk * 32 + row_j)], each pair times its 2^-e (exact
// unless subnormal), written as 8 float16 by put(m, fragment).
template <int B, int MS, class Feature, class Get, class Put>
__device__ __forceinline__ void gather_frag(const FragRows<B>& fr, int blk, int rows, Feature&& feature, Get&& get,
                                            Put&& put) {
  int f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = feature(blk * kBlockRows + fr.row[j]);
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    if (m < rows) {
      uint32_t pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const _Float16 sc = (_Float16)(1.0f / (float)(1 << mx::exponent(B, r)));
        const half2_t v = half2_t{get(m, f[2 * r]), get(m, f[2 * r + 1])};
        pr[r] = __builtin_bit_cast(uint32_t, v * half2_t{sc, sc});
      }
      put(m, u32x4{pr[0], pr[1], pr[2], pr[3]});
    }
  }
}

template <int FN>
struct Red {
  float4_t v[kWaves][FN][64];
};

// The kernel. BS: the code widths it may meet; FN: columns per lane; UB:
// blocks per scale unit; kMode: see Mode.
template <unsigned BS, int FN, int UB, int kMode>
__global__ __launch_bounds__(kThreads) void qgemv_mx_kernel(MxArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int MS = rows_stored<kMode>();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Every argument the first loads need, read in one scalar batch (the asm
  // takes them and hands them back, so none is read later behind another wait).
  MatPtrs mp = a.mat[blockIdx.y];
  int M = a.M, K = a.K, N = a.N, spx = a.strips_per_xcd, nstrips = a.nstrips, R = a.packed_rows;
  int bpg_shift = a.bpg_shift, scale_bytes = a.scale_bytes, hz = a.has_zeros, srow = a.scale_row_bytes,
      tl = a.two_level;
  int64_t packed_words = a.packed_words;
  int b0 = a.wave_b0[wave], b1 = a.wave_b1[wave], s_end = a.wave_send[wave], row0 = a.wave_row0[wave];
  int bits0 = a.wave_bits0[wave], lds_perm = a.lds_perm, lds_xg = a.lds_xg;
  const uint16_t* xsrc16 = a.x;
  const int32_t* perm = a.perm;
  asm volatile("" : "+s"(mp.qweight), "+s"(mp.scales), "+s"(mp.zeros), "+s"(mp.y), "+s"(M), "+s"(K), "+s"(N),
               "+s"(spx), "+s"(nstrips), "+s"(R), "+s"(bpg_shift), "+s"(scale_bytes), "+s"(hz), "+s"(srow), "+s"(tl),
               "+s"(packed_words), "+s"(b0), "+s"(b1), "+s"(s_end), "+s"(row0), "+s"(bits0), "+s"(lds_perm),
               "+s"(lds_xg), "+s"(xsrc16), "+s"(perm));

  const int bid = blockIdx.x;
  const int strip = (bid % kXcds) * spx + bid / kXcds;
  if (strip >= nstrips) return;   // the whole workgroup leaves together

  Lane L;
  L.g = lane >> 4;
  L.n = lane & 15;
  L.magic = vgpr_magic();
  // The weight buffer starts at the strip's first panel: 32-bit offsets
  // span only the strip's FN panels.
  const int64_t strip_words = (int64_t)FN * R * kPanel;
  const int64_t first_word = (int64_t)strip * strip_words;
  L.rw = __builtin_amdgcn_make_buffer_rsrc((void*)(mp.qweight + first_word), 0,
                                           (int)(min(strip_words, packed_words - first_word) * 4), kRsrcWord3);
  L.rs = __builtin_amdgcn_make_buffer_rsrc((void*)mp.scales, 0, scale_bytes, kRsrcWord3);
  // Without zero points the zero loads read the scales (the value is unused).
  L.rz = __builtin_amdgcn_make_buffer_rsrc(hz ? (void*)mp.zeros : (void*)mp.scales, 0,
                                           hz ? scale_bytes / 2 : scale_bytes, kRsrcWord3);
  const int col_req = strip * kPanel * FN + L.n * FN;
  // Lanes past N read the last columns (valid addresses) and are never stored.
  const int col = col_req < N ? col_req : N - FN;
  L.wbase = (uint32_t)(col / kPanel - strip * FN) * (uint32_t)R * kPanel * 4 + (uint32_t)(col % kPanel) * 4;
  L.srow = (uint32_t)srow;
  L.tl = tl != 0;
  if (tl) {   // the word of 8 scale codes holding the lane's columns
    L.sbase = (uint32_t)(col / 8) * 4;
    L.sshift = 4u * (uint32_t)(col & 7);
  } else {
    L.sbase = (uint32_t)(col & ~1) * 2;                     // FN >= 2: col is even
    L.sshift = (uint32_t)(col & 1) * 16;
  }
  L.zbase = hz ? (uint32_t)(col & ~3) : (uint32_t)(col & ~1) * 2;   // FN == 4: col is a multiple of 4
  L.zshift = (uint32_t)(col & 3) * 8;
  const int mrow = min(lane & 15, M - 1);   // the A row of this lane (rows past M repeat row M - 1)
  L.xoff = (uint32_t)(mrow * 32 + 8 * L.g) * 2;
  if constexpr (base_mode(kMode) == kGathered) {
    const int nblk = K / kBlockRows;
    L.rx = __builtin_amdgcn_make_buffer_rsrc((void*)a.xg, 0, (int)((size_t)nblk * MS * 64), kRsrcWord3);
  } else {
    L.rx = L.rs;
  }

  Acc<FN> A;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    A.y[j] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) A.acc[p][ch][j] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) A.sacc[p][ch] = float4_t{0.f, 0.f, 0.f, 0.f};

  // The wave's first segment: blocks [b0, s_end) of width bits0.
  const int n0 = (s_end - b0) / UB;
  auto first = [&](auto B0c) {
    constexpr int B0 = decltype(B0c)::value;
    Slot<B0, FN, UB> S0[depth<B0, FN, UB, kMode>()];

    if constexpr (base_mode(kMode) != kGathered) {
      // 1. x rows and perm into LDS, no registers: wave-wide 16-byte
      // global-to-LDS loads (lane l of a load fills bytes 16 l .. 16 l + 15
      // of a 1 KiB piece). Pieces past the end re-read the last 16 bytes and
      // land in the padding of the region.
      const int xbytes = M * K * 2;
      const int xpieces = (xbytes + 1023) / 1024;
      const char* xsrc = reinterpret_cast<const char*>(xsrc16);
      for (int i = wave; i < xpieces; i += kWaves) {
        const int off = min(i * 1024 + lane * 16, xbytes - 16);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(xsrc + off),
                                         (__attribute__((address_space(3))) void*)(lds + i * 1024), 16, 0, 0);
      }
      if (perm) {
        const int pbytes = K * 4;
        const int ppieces = (pbytes + 1023) / 1024;
        const char* psrc = reinterpret_cast<const char*>(perm);
        for (int i = wave; i < ppieces; i += kWaves) {
          const int off = min(i * 1024 + lane * 16, pbytes - 16);
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(psrc + off),
                                           (__attribute__((address_space(3))) void*)(lds + lds_perm + i * 1024), 16,
                                           0, 0);
        }
      }
      asm volatile("" ::: "memory");
    }
    // 2. The first weight loads of the wave.
    if (n0 > 0) pre_issue<B0, FN, UB, kMode>(L, row0, S0);
    asm volatile("" ::: "memory");

    if constexpr (base_mode(kMode) != kGathered) {
      // 3. Wait for the staging loads only (they precede the weight loads,
      // and loads complete in order), then gather. A wave without blocks
      // issued no weight loads and waits for all.
      constexpr int kAfter = depth<B0, FN, UB, kMode>() * UB * mx::loads(B0);
      constexpr int kWait = kAfter < 63 ? kAfter : 63;
      if (n0 > 0) __builtin_amdgcn_s_waitcnt((kWait & 15) | (0x7f << 4) | ((kWait >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt((0x7f << 4));
      __builtin_amdgcn_s_barrier();
      // Run by run with the width fixed at compile time; a thread's k-group
      // is fixed (the block count per pass is a multiple of 4), so its rows
      // are worked out once per run.
      const _Float16* xr = reinterpret_cast<const _Float16*>(lds);
      const int32_t* pl = reinterpret_cast<const int32_t*>(lds + lds_perm);
      const int gq = tid & 3;
      for (int r = 0; r < a.runs.nruns; ++r) {
        const int t0 = 4 * a.runs.run_block[r], t1 = 4 * a.runs.run_block[r + 1];
        with_width<BS>(a.runs.run_bits[r], [&](auto Bc) {
          constexpr int Bw = decltype(Bc)::value;
          const FragRows<Bw> fr = frag_rows<Bw>(gq);
          for (int t = t0 + tid; t < t1; t += kThreads) {
            const int blk = t >> 2;
            gather_frag<Bw, MS>(
                fr, blk, M,
                // perm entries clamped into [0, K): a malformed perm cannot address outside x
                [&](int j) { return perm ? (int)min((unsigned)pl[j], (unsigned)(K - 1)) : j; },
                [&](int m, int f) { return xr[m * K + f]; },
                [&](int m, u32x4 v) {
                  *reinterpret_cast<u32x4*>(lds + lds_xg + (blk * a.ms + m) * 64 + gq * 16) = v;
                });
          }
        });
      }
      __syncthreads();
    }

    // 4. The first segment (its first loads are in flight).
    if (n0 > 0) A = segment<B0, FN, UB, kMode, true>(a, L, lds, b0, n0, row0, N, bpg_shift, hz, A, S0);
  };
  with_width<BS>(bits0, first);

  // The wave's other segments.
  for (int blk = s_end; blk < b1;) {
    int r = 0;
    for (int q = 1; q < a.runs.nruns; ++q) r = blk >= a.runs.run_block[q] ? q : r;
    const int e = min(b1, a.runs.run_block[r + 1]);
    const int bits = a.runs.run_bits[r];
    const int row = a.runs.run_row[r] + (blk - a.runs.run_block[r]) * bits;
    with_width<BS>(bits, [&](auto BB) {
      constexpr int Bw = decltype(BB)::value;
      Slot<Bw, FN, UB> S[depth<Bw, FN, UB, kMode>()];
      A = segment<Bw, FN, UB, kMode, false>(a, L, lds, blk, (e - blk) / UB, row, N, bpg_shift, hz, A, S);
    });
    blk = e;
  }

  // 5. The waves' partial tiles summed through LDS, then the epilogue and
  // the float16 store. Lane l holds rows 4 (l / 16) + r of column l % 16 of
  // each fragment.
  if constexpr (exact_mode(kMode)) {
#pragma unroll
    for (int j = 0; j < FN; ++j) A.y[j] = (A.acc[0][0][j] + A.acc[0][1][j]) + (A.acc[1][0][j] + A.acc[1][1][j]);
  }
  __syncthreads();   // every wave is done with the staged activations
  Red<FN>* red = reinterpret_cast<Red<FN>*>(lds);
#pragma unroll
  for (int j = 0; j < FN; ++j) red->v[wave][j][lane] = A.y[j];
  __syncthreads();
  const Epilogue epi = a.epi;
  for (int e = tid; e < 256 * FN; e += kThreads) {
    const int j = e >> 8, l = (e >> 2) & 63, r = e & 3;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red->v[w][j][l][r];
    const int row = 4 * (l >> 4) + r;
    const int cc = strip * kPanel * FN + (l & 15) * FN + j;
    if (row < M && cc < N)
      ((__attribute__((address_space(1))) uint16_t*)mp.y)[(size_t)row * N + cc] =
          __builtin_bit_cast(uint16_t, (_Float16)apply_epilogue(epi, v, row, cc, N));
  }
}

constexpr unsigned kSet4 = 1u << 4;

template <unsigned BS, int FN, int UB, int kMode>
hipError_t launch_fn(MxArgs a, size_t lds, hipStream_t stream) {
  a.nstrips = (a.N + kPanel * FN - 1) / (kPanel * FN);
  a.strips_per_xcd = (a.nstrips + kXcds - 1) / kXcds;
  hipLaunchKernelGGL((qgemv_mx_kernel<BS, FN, UB, kMode>), dim3(kXcds * a.strips_per_xcd, a.mats), dim3(kThreads),
                     lds, stream, a);
  return hipGetLastError();
}

template <unsigned BS, int UB, int kMode>
hipError_t launch_mode(const MxArgs& a, int fn, size_t lds, hipStream_t stream) {
  if (fn == 4) return launch_fn<BS, 4, UB, kMode>(a, lds, stream);
  if (fn == 2) return launch_fn<BS, 2, UB, kMode>(a, lds, stream);
  return launch_fn<BS, 1, UB, kMode>(a, lds, stream);
}

template <unsigned BS, int UB>
hipError_t launch_set(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream) {
  switch (mode) {
    case kFewRows: return launch_mode<BS, UB, kFewRows>(a, fn, lds, stream);
    case kFewRows | kExact: return launch_mode<BS, UB, kFewRows | kExact>(a, fn, lds, stream);
    case kGathered | kExact: return launch_mode<BS, UB, kGathered | kExact>(a, fn, lds, stream);
    default: return launch_mode<BS, UB, kGathered>(a, fn, lds, stream);
  }
}

// Instances, one file per set of code widths (qgemv_mx_inst_*.hip), so
// that they compile in parallel.
hipError_t launch_set4_ub4(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream);
hipError_t launch_set4_ub1(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream);
hipError_t launch_low(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream);
hipError_t launch_mid_few(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream);
hipError_t launch_mid_gathered(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream);
hipError_t launch_all(const MxArgs& a, int fn, bool exact, size_t lds, hipStream_t stream);

}  // namespace mxk

}  // namespace qlinear
