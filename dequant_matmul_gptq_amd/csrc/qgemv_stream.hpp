// Decode-sized quantized linear layer (M <= 16) on gfx950: one pass over the
// packed weights at HBM speed, with no cross-workgroup reduction.
//
// Work split. A workgroup of 4 or 8 waves owns a strip of 16 output columns
// -- one storage panel, whose packed rows are contiguous in memory -- and the
// whole K range, so it writes its float16 outputs directly: no split-K, no
// atomics. Inside a wave, lane = (block slot ks, column quad cq): 4 column
// quads x 16 block slots. Each lane unpacks whole 32-row blocks of its 4
// columns, streaming the block's b words with b 16-byte loads; a wave step
// covers 16 consecutive blocks of one run (uniform bit width). The waves take
// contiguous parts of K; the step after the one being computed is in flight
// (double buffering), and the first step is issued before the activations
// are staged, so its HBM latency overlaps the staging.
//
// Activations. For M = 1 the kernel gathers them itself: the perm entries of
// the wave's first blocks and the whole x row are loaded first, before the
// weights (vector loads complete in issue order, so anything issued after the
// weights would wait for them), the x row goes to LDS, and each wave builds
// its own act-order-gathered, pair-ordered copy from there. For M > 1 a
// separate gather kernel writes that copy to the workspace and each wave
// copies its part into LDS.
//
// Strips are assigned XCD by XCD: workgroups are dispatched round-robin over
// the 8 XCDs, so workgroup i is given a strip from XCD (i % 8)'s contiguous
// range; neighbouring strips share the lines of the scale rows.
//
// Arithmetic per block, column and activation row. The codes come out of the
// packed words as float16 pairs 1024 + q * 2^e (mask in place; one shift per
// word for the fields above bit 10), the activations are gathered by
// act-order and pre-scaled by 2^-e, and
//   acc = sum_pairs dot2((1024 + q_lo 2^e, 1024 + q_hi 2^e), (x_lo 2^-e, x_hi 2^-e))
//       = sum_j x_j q_j + 1024 * X'_blk
//   y  += s * (acc - 1024 * X'_blk - z * X_blk)
// where X_blk is the block's sum of activations and X'_blk that of the
// scaled ones. Products of float16 values are exact in float32; accumulation
// is float32.
//
// Reduction: butterfly shuffles across the 16 block slots of a wave, then
// across the waves through LDS.
#pragma once

#include <algorithm>

#include "qlinear_kernels.hpp"

namespace qlinear {

namespace stream {

constexpr int kMaxWaves = 8;           // waves per workgroup: 4 or 8 (they split K)
constexpr int CQ = 4;                  // column quads per strip
constexpr int SC = 4 * CQ;             // 16 columns per workgroup
constexpr int KS = 64 / CQ;            // 16 blocks per wave step
constexpr int kXcds = 8;
constexpr int kStageBudget = 60 * 1024;  // bytes of LDS for staged activations

constexpr int kMaxMats = 8;   // matrices of one grouped call

// One matrix of a call: the matrices of a grouped call share the layout, the
// activations and the permutation, and have their own weights and output.
struct MatPtrs {
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint8_t* zeros;   // NULL for every matrix of the call, or for none
  uint16_t* y;
};

struct StreamArgs {
  const uint16_t* x;       // single-row kernel: the activations, float16 [K], original order
  const int32_t* perm;     // single-row kernel: act-order permutation or NULL
  const uint32_t* xq;      // gathered, scaled activations, [M][K/32][16] float16 pairs
  const float2* xsum;      // block sums (X, 1024 * X'), [M][K/32]
  int mats;                // matrices in this call, 1 .. kMaxMats
  int has_zeros;
  MatPtrs mat[kMaxMats];
  int M, K, N;
  int nstrips, strips_per_xcd;  // 16-column strips per matrix; workgroups per XCD over all matrices
  int chunk;               // blocks per wave staged at a time
  int xrow_words;          // single-row kernel: LDS words holding the x row
  int bpg_shift;           // log2(group_size / 32)
  // multi-row kernel: each wave's first run segment, set by the host (its
  // width, or 0 for a wave without blocks, its first packed row and its end
  // block, the latter also bounded by the first chunk)
  int wave_bits[kMaxWaves], wave_row[kMaxWaves], wave_end[kMaxWaves];
  // one-launch several-width kernel: wave w's blocks are [wave_begin[w], wave_begin[w + 1])
  int wave_begin[kMaxWaves + 1];
  Runs runs;
  Epilogue epi;
};

template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Bit of a kernel's width set that marks two-level scales (4-bit codes in
// place of the float16 scales; scale_max comes in the epilogue).
constexpr unsigned kTwoLevelBit = 1u << 16;
template <unsigned BS>
constexpr bool two_level() { return (BS & kTwoLevelBit) != 0; }

struct Raw {
  uint2 s;      // 4 float16 scales (two-level: the code word, and the shift of the lane's first code)
  uint32_t z;   // 4 uint8 zero points
  bool ok;      // false: the lane has no block this step (contributes nothing)
};

// Loads of one lane for one step: the b words of block `blk` (packed row
// `row`) for its 4 columns, and that block's group scales and zeros.
// `panel` points at the lane's 4 slots in row 0 of this workgroup's panel
// (the rows of a panel are 16 words apart); `scol` is the lane's first
// column, clamped into the matrix for the scale and zero reads.
// Every load is issued unconditionally, so that the compiler can count the
// loads in flight exactly (a branch around a load makes it wait for all of
// them). A lane without work (ok == false) reads the valid block `blk_safe`
// at `row_safe` instead and gets a zero scale, which zeroes its contribution.
template <int B, bool kTL = false>
__device__ __forceinline__ void issue(const StreamArgs& a, const MatPtrs& mp, const uint32_t* panel, int blk,
                                      int row, bool ok, int blk_safe, int row_safe, int scol, uint4 (&W)[B], Raw& P) {
  const uint32_t* p = panel + (size_t)(ok ? row : row_safe) * kPanel;
#pragma unroll
  for (int t = 0; t < B; ++t) W[t] = *reinterpret_cast<const uint4*>(p + t * kPanel);
  if constexpr (kTL) {
    // The word of 8 scale codes holding the lane's 4 columns (symmetric
    // groups: no zero points). The shift is applied where the code is used.
    const size_t gw = (size_t)((ok ? blk : blk_safe) >> a.bpg_shift) * (a.N / 8) + scol / 8;
    P.s.x = reinterpret_cast<const uint32_t*>(mp.scales)[gw];
    P.s.y = 4u * (uint32_t)(scol & 7);
    P.z = 0u;
    P.ok = ok;
    return;
  }
  const size_t g = (size_t)((ok ? blk : blk_safe) >> a.bpg_shift) * a.N + scol;
  const uint2 sv = *reinterpret_cast<const uint2*>(mp.scales + g);
  // Without zero points, read the scales again (any valid address): the value
  // is not used.
  const uint8_t* zp = a.has_zeros ? mp.zeros : reinterpret_cast<const uint8_t*>(mp.scales);
  const uint32_t zv = *reinterpret_cast<const uint32_t*>(zp + g);
  P.s = sv;
  P.z = zv;
  P.ok = ok;
}

// Unpack and multiply one block (this lane's 4 columns), then fold in the
// block's scale, zero point and bias. xs_blk points at pair 0 of the block for
// activation row 0; rows are `row_stride` words apart. xs_sum likewise.
template <int B, int MT, bool kTL>
__device__ __forceinline__ void compute(const StreamArgs& a, const uint4 (&W)[B], const Raw& P,
                                        const uint32_t* __restrict__ xs_blk, int row_stride,
                                        const float2* __restrict__ xsum_blk, int sum_stride, uint32_t magic,
                                        float (&yacc)[4][MT]) {
  uint32_t wc[4][B], wsh[4][B];
#pragma unroll
  for (int t = 0; t < B; ++t) {
    wc[0][t] = W[t].x;
    wc[1][t] = W[t].y;
    wc[2][t] = W[t].z;
    wc[3][t] = W[t].w;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int t = 0; t < B; ++t) wsh[c][t] = wc[c][t] >> scaled_shift(B);
  float acc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[c][m] = 0.0f;

  static_for<0, kPairsPerBlock / 4>([&](auto Q) {
    constexpr int q4 = decltype(Q)::value;
    uint4 xv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xv[m] = *reinterpret_cast<const uint4*>(xs_blk + m * row_stride + 4 * q4);
    static_for<0, 4>([&](auto R) {
      constexpr int r = decltype(R)::value;
      constexpr int Pp = 4 * q4 + r;
      uint32_t v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = extract_pair_scaled<B, Pp>(wc[c], wsh[c], magic);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t xp = r == 0 ? xv[m].x : r == 1 ? xv[m].y : r == 2 ? xv[m].z : xv[m].w;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c][m] = __builtin_amdgcn_fdot2(as_half2(v[c]), as_half2(xp), acc[c][m], false);
      }
    });
  });

  float s[4], z[4];
  if constexpr (kTL) {
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] = P.ok ? (float)(((P.s.x >> (P.s.y + 4 * c)) & 15u) + 1u) : 0.0f;
  } else {
    s[0] = P.ok ? half_lo(P.s.x) : 0.0f;
    s[1] = P.ok ? half_hi(P.s.x) : 0.0f;
    s[2] = P.ok ? half_lo(P.s.y) : 0.0f;
    s[3] = P.ok ? half_hi(P.s.y) : 0.0f;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) z[c] = a.has_zeros ? (float)((P.z >> (8 * c)) & 0xFFu) : (float)(1 << (B - 1));
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float2 X = xsum_blk[m * sum_stride];
#pragma unroll
    for (int c = 0; c < 4; ++c) yacc[c][m] = fmaf(s[c], fmaf(-z[c], X.x, acc[c][m] - X.y), yacc[c][m]);
  }
}

// All steps of one run segment [blk0, blk1) of this wave, double-buffered
// (8-bit runs single-buffered, to bound register use). The segment's first
// packed row is row0. The staged activations of block blk sit at LDS slot
// blk - lds_blk0 of this wave's area. With kPre, the first step's words and
// parameters are already in Wa / Pa.
template <int B, int MT, bool kPre, bool kTL>
__device__ __forceinline__ void run_segment(const StreamArgs& a, const MatPtrs& mp, int blk0, int blk1, int row0, int ks,
                                            const uint32_t* panel, int col, bool colv, const uint32_t* xs_w, const float2* xsum_w, int lds_blk0,
                                            uint32_t magic, float (&yacc)[4][MT], uint4 (&Wa)[B], Raw& Pa) {
  const int nsteps = (blk1 - blk0 + KS - 1) / KS;
  auto lane_issue = [&](int i, uint4 (&W)[B], Raw& P) {
    const int blk = blk0 + i * KS + ks;
    issue<B, kTL>(a, mp, panel, blk, row0 + (i * KS + ks) * B, colv && blk < blk1, blk0, row0, col, W, P);
  };
  auto lane_compute = [&](int i, const uint4 (&W)[B], const Raw& P) {
    const int bl = min(blk0 + i * KS + ks, blk1 - 1) - lds_blk0;   // clamped: idle lanes hold zeros
    compute<B, MT, kTL>(a, W, P, xs_w + bl * kPairsPerBlock, a.chunk * kPairsPerBlock, xsum_w + bl, a.chunk, magic,
                   yacc);
  };
  if constexpr (!kPre) lane_issue(0, Wa, Pa);
  if constexpr (B == 8) {
    for (int i = 0; i < nsteps; ++i) {
      if (i > 0) lane_issue(i, Wa, Pa);
      lane_compute(i, Wa, Pa);
    }
  } else {
    uint4 Wb[B];
    Raw Pb;
    for (int i = 0; i < nsteps; i += 2) {
      if (i + 1 < nsteps) lane_issue(i + 1, Wb, Pb);
      lane_compute(i, Wa, Pa);
      if (i + 1 >= nsteps) break;
      if (i + 2 < nsteps) lane_issue(i + 2, Wa, Pa);
      lane_compute(i + 1, Wb, Pb);
    }
  }
}

template <int MT, unsigned BS>
__device__ __forceinline__ void any_segment(const StreamArgs& a, const MatPtrs& mp, int bits, int blk0, int blk1, int row0, int ks,
                                            const uint32_t* panel, int col, bool colv, const uint32_t* xs_w, const float2* xsum_w,
                                            int lds_blk0, uint32_t magic, float (&yacc)[4][MT]) {
#define QLINEAR_SEGMENT(BB)                                                                                \
  case BB:                                                                                                 \
    if constexpr ((BS >> BB) & 1u) {                                                                       \
      uint4 W[BB];                                                                                         \
      Raw P;                                                                                               \
      run_segment<BB, MT, false, two_level<BS>()>(a, mp, blk0, blk1, row0, ks, panel, col, colv, xs_w, xsum_w, lds_blk0, magic, yacc, W, P); \
    }                                                                                                      \
    break;
  switch (bits) {
    QLINEAR_SEGMENT(2)
    QLINEAR_SEGMENT(3)
    QLINEAR_SEGMENT(4)
    QLINEAR_SEGMENT(5)
    QLINEAR_SEGMENT(6)
    QLINEAR_SEGMENT(8)
    default: break;
  }
#undef QLINEAR_SEGMENT
}

// 32-bit words of one wave's staging area for `chunk` blocks (16-byte aligned).
template <int MT>
__host__ __device__ constexpr int stage_words(int chunk) {
  return (chunk * MT * (kPairsPerBlock + 2) + 3) / 4 * 4;
}

// Reduce the lane sums over the 16 block slots of each wave (lanes cq,
// cq + 4, ..., cq + 60), then over the waves through LDS, and store y.
template <int MT, int WV>
__device__ __forceinline__ void reduce_store(const StreamArgs& a, uint16_t* y, float (&red)[WV][4][MT][SC],
                                             float (&yacc)[4][MT], int tid, int lane, int wave, int strip) {
  const int cq = lane % CQ;
  // The 4 block slots of each 16-lane row with two DPP row shifts (lanes
  // 12..15 of a row end up with its sums, one per column quad), then the 4
  // rows of each wave and the waves through LDS.
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = yacc[c][m];
      v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF,
                                                                 true));   // row_shr:4
      v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF,
                                                                 true));   // row_shr:8
      yacc[c][m] = v;
    }
  if ((lane & 15) >= 12) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) red[wave][lane >> 4][m][cq * 4 + c] = yacc[c][m];
  }
  __syncthreads();
  if (tid < SC * MT) {
    const int m = tid / SC, c = tid % SC;
    const int n = strip * SC + c;
    if (m < a.M && n < a.N) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < WV; ++w)
#pragma unroll
        for (int row = 0; row < 4; ++row) v += red[w][row][m][c];
      y[(size_t)m * a.N + n] = __builtin_bit_cast(uint16_t, (_Float16)apply_epilogue(a.epi, v, m, n, a.N));
    }
  }
}

// Kernel body, specialised on B0, the width of this wave's first run, so the
// first step can be issued into a typed buffer before the activation staging.
template <int MT, unsigned BS, int WV, int B0>
__device__ __forceinline__ void stream_body(const StreamArgs& a, const MatPtrs& mp, uint32_t* lds, float (&red)[WV][4][MT][SC],
                                            int tid, int lane, int wave, int strip, int wb0, int wb1, int row0,
                                            int seg0_end) {
  const int cq = lane % CQ, ks = lane / CQ;
  const int col_req = strip * SC + cq * 4;
  const bool colv = col_req < a.N;
  const int col = colv ? col_req : a.N - 4;   // scale/zero column for lanes past N
  // The lane's 4 word slots in row 0 of this strip's panel (padding slots of
  // the last panel exist and hold zeros).
  const uint32_t* panel = mp.qweight + (size_t)strip * a.runs.packed_rows * kPanel + cq * 4;
  const int nblk = a.K / kBlockRows;
  const int per_wave = (nblk + WV - 1) / WV;
  const int nchunks = (per_wave + a.chunk - 1) / a.chunk;
  const uint32_t magic = vgpr_magic();

  // This wave's LDS area: [MT][chunk][16] float16 pairs, then [MT][chunk] sums,
  // rounded up to 16 bytes.
  const int area = stage_words<MT>(a.chunk);
  uint32_t* xs_w = lds + wave * area;
  float2* xsum_w = reinterpret_cast<float2*>(xs_w + a.chunk * MT * kPairsPerBlock);

  uint4 W0[B0];
  Raw P0;
  {
    // A wave without blocks (K < 32 * waves) reads block 0 and discards it.
    const int blk = wb0 + ks;
    const bool any = wb0 < wb1;
    issue<B0, two_level<BS>()>(a, mp, panel, blk, row0 + ks * B0, any && colv && blk < seg0_end, any ? wb0 : 0, any ? row0 : 0, col, W0,
              P0);
  }

  float yacc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[c][m] = 0.0f;

  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = wb0 + ch * a.chunk;
    const int c1 = min(wb1, c0 + a.chunk);
    const int nb = c1 > c0 ? c1 - c0 : 0;
    if (ch > 0) __syncthreads();  // every wave is done with its previous chunk
    // Copy this wave's chunk of gathered activations and block sums to LDS,
    // eight 16-byte loads in flight per lane (unconditional loads from
    // clamped indices, wave-uniform trip count).
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= a.M) break;
      const int mm = m;
      const uint4* src = reinterpret_cast<const uint4*>(a.xq + ((size_t)mm * nblk + (nb > 0 ? c0 : 0)) * kPairsPerBlock);
      uint4* dst = reinterpret_cast<uint4*>(xs_w + mm * a.chunk * kPairsPerBlock);
      const int n4 = nb * (kPairsPerBlock / 4);
      constexpr int U = 8;
      const int iters = (n4 + U * 64 - 1) / (U * 64);
      for (int it = 0; it < iters; ++it) {
        const int base = it * U * 64 + lane;
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = src[min(base + u * 64, n4 - 1)];
        // Clamped lanes rewrite the last element with its own value.
#pragma unroll
        for (int u = 0; u < U; ++u) dst[min(base + u * 64, n4 - 1)] = v[u];
      }
      const float2* ssrc = a.xsum + (size_t)mm * nblk + (nb > 0 ? c0 : 0);
      const int siters = (nb + 63) / 64;
      for (int it = 0; it < siters; ++it) {
        const int i = it * 64 + lane;
        const float2 v = ssrc[min(i, nb - 1)];
        xsum_w[mm * a.chunk + min(i, nb - 1)] = v;
      }
    }
    __syncthreads();

    int blk = c0;
    if (ch == 0 && blk < seg0_end) {
      run_segment<B0, MT, true, two_level<BS>()>(a, mp, blk, seg0_end, row0, ks, panel, col, colv, xs_w, xsum_w, c0, magic, yacc, W0, P0);
      blk = seg0_end;
    }
    while (blk < c1) {
      int bits, row;
      block_info(a.runs, blk, bits, row);
      const int seg_end = min(c1, run_end_block(a.runs, blk));
      any_segment<MT, BS>(a, mp, bits, blk, seg_end, row, ks, panel, col, colv, xs_w, xsum_w, c0, magic, yacc);
      blk = seg_end;
    }
  }

  reduce_store<MT, WV>(a, mp.y, red, yacc, tid, lane, wave, strip);
}

template <int MT, unsigned BS, int WV, int B0>
__device__ __forceinline__ void dispatch_body(const StreamArgs& a, const MatPtrs& mp, uint32_t* lds, float (&red)[WV][4][MT][SC], int tid,
                                              int lane, int wave, int strip, int wb0, int wb1, int row0, int seg0_end) {
  stream_body<MT, BS, WV, B0>(a, mp, lds, red, tid, lane, wave, strip, wb0, wb1, row0, seg0_end);
}

// One kernel per (MT, set of code widths that may occur). BS has bit b set
// for every width b the matrix may contain; the host picks the smallest
// instantiated set that covers the layout's runs, which keeps the register
// budget of the common formats low.
template <int MT, unsigned BS, int WV>
__global__ __launch_bounds__(WV * 64) void qgemv_stream_kernel(StreamArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ float red[WV][4][MT][SC];   // per wave and 16-lane row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The arguments the first loads need, read in one scalar batch (the matrix
  // is blockIdx.y and the wave's first run segment comes from the host, so no
  // read waits on another); later reads of the same fields reuse these.
  const MatPtrs mp = a.mat[blockIdx.y];
  const int bits0 = a.wave_bits[wave], row0 = a.wave_row[wave], seg0_end = a.wave_end[wave];
  asm volatile("" ::"s"(mp.qweight), "s"(mp.scales), "s"(mp.zeros), "s"(mp.y), "s"(bits0), "s"(row0), "s"(seg0_end),
               "s"(a.strips_per_xcd), "s"(a.nstrips), "s"(a.K), "s"(a.N), "s"(a.M), "s"(a.chunk), "s"(a.bpg_shift),
               "s"(a.has_zeros), "s"(a.runs.packed_rows), "s"(a.xq), "s"(a.xsum));
  const int bid = blockIdx.x;
  const int strip = (bid % kXcds) * a.strips_per_xcd + bid / kXcds;
  if (strip >= a.nstrips) return;  // the whole workgroup leaves together

  const int nblk = a.K / kBlockRows;
  const int wb0 = (wave * nblk) / WV, wb1 = ((wave + 1) * nblk) / WV;

#define QLINEAR_BODY(BB)                                                                     \
  case BB:                                                                                   \
    if constexpr ((BS >> BB) & 1u) dispatch_body<MT, BS, WV, BB>(a, mp, lds, red, tid, lane, wave, strip, wb0, wb1, row0, seg0_end); \
    return;
  switch (bits0) {
    QLINEAR_BODY(2)
    QLINEAR_BODY(3)
    QLINEAR_BODY(4)
    QLINEAR_BODY(5)
    QLINEAR_BODY(6)
    QLINEAR_BODY(8)
    default: break;
  }
#undef QLINEAR_BODY
  // This wave has no blocks (K too small for every wave): it still joins the
  // barriers of the staging and the final reduction, which the other waves run.
  dispatch_body<MT, BS, WV, (BS & 16u) ? 4 : (BS & 4u) ? 2 : (BS & 8u) ? 3 : (BS & 32u) ? 5 : (BS & 64u) ? 6 : 8>(a, mp, lds, red, tid, lane, wave, strip, wb0, wb1, row0, seg0_end);
}

// Equal split of the K blocks over WV waves (wave w: [w nblk / WV, (w + 1) nblk / WV)).
inline void equal_waves(StreamArgs& a, int WV) {
  const int nblk = a.K / kBlockRows;
  for (int w = 0; w <= WV; ++w) a.wave_begin[w] = (w * nblk) / WV;
}

// Each wave's first run segment: its width (0 for a wave without blocks),
// first packed row and end block, the latter bounded by `limit` blocks; the
// waves' ranges come from wave_begin.
inline void first_segments(StreamArgs& a, int WV, int limit) {
  for (int w = 0; w < WV; ++w) {
    const int wb0 = a.wave_begin[w], wb1 = a.wave_begin[w + 1];
    a.wave_bits[w] = 0;
    a.wave_row[w] = 0;
    a.wave_end[w] = wb0;
    if (wb0 < wb1) {
      int r = 0;
      while (r + 1 < a.runs.nruns && wb0 >= a.runs.run_block[r + 1]) ++r;
      a.wave_bits[w] = a.runs.run_bits[r];
      a.wave_row[w] = a.runs.run_row[r] + (wb0 - a.runs.run_block[r]) * a.runs.run_bits[r];
      a.wave_end[w] = std::min(std::min(wb1, a.runs.run_block[r + 1]), wb0 + limit);
    }
  }
}

template <int MT, unsigned BS, int WV>
hipError_t launch_set(StreamArgs a, hipStream_t stream) {
  const int nblk = a.K / kBlockRows;
  const int per_wave = (nblk + WV - 1) / WV;
  const int max_chunk = (kStageBudget / (WV * 4) - 3) / (MT * (kPairsPerBlock + 2));
  a.chunk = per_wave < max_chunk ? per_wave : max_chunk;
  if (a.chunk < 1) a.chunk = 1;
  const size_t lds = (size_t)WV * stage_words<MT>(a.chunk) * 4;
  a.nstrips = (a.N + SC - 1) / SC;
  a.strips_per_xcd = (a.nstrips + kXcds - 1) / kXcds;
  equal_waves(a, WV);   // as the kernel splits K
  first_segments(a, WV, a.chunk);   // each bounded by the wave's first chunk
  hipLaunchKernelGGL((qgemv_stream_kernel<MT, BS, WV>), dim3(kXcds * a.strips_per_xcd, a.mats), dim3(WV * 64), lds,
                     stream, a);
  return hipGetLastError();
}

// Waves per workgroup of the multi-row kernel at M = 1 (they split K).
// Measured on MI355X: 8 waves pay off only when there are few 16-column
// strips and K is long; 4 otherwise.
inline int waves_for(int N, int K) {
  const int nstrips = (N + SC - 1) / SC;
  return (nstrips <= 512 && K / kBlockRows >= 256) ? 8 : 4;
}

// Kernels for M <= 2 with the activations gathered by the gather kernel.
template <unsigned BS>
hipError_t launch_set_small_m(const StreamArgs& a, hipStream_t stream) {
  if (a.M <= 1) {
    if (waves_for(a.N, a.K) >= 8) return launch_set<1, BS, 8>(a, stream);
    return launch_set<1, BS, 4>(a, stream);
  }
  return launch_set<2, BS, 4>(a, stream);
}

constexpr unsigned kLowBits = (1u << 2) | (1u << 3);                            // ~2-3 bpw
constexpr unsigned kMidBits = (1u << 3) | (1u << 4) | (1u << 5) | (1u << 6);   // ~3.5-5 bpw
constexpr unsigned kAllBits = (1u << 2) | (1u << 3) | (1u << 4) | (1u << 5) | (1u << 6) | (1u << 8);

// Instantiated in the qgemv_stream_*.hip files: M <= 2 per set of widths
// (larger M runs the single-row or the matrix-core decode kernel).
hipError_t launch_uniform(unsigned set, const StreamArgs& a, hipStream_t stream);
hipError_t launch_mixed(unsigned set, const StreamArgs& a, hipStream_t stream);

}  // namespace stream

}  // namespace qlinear
