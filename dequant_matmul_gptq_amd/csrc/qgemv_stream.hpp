// Decode-sized quantized linear layer (M <= 16) on gfx950: one pass over the
// packed weights at HBM speed, with no cross-workgroup reduction.
//
// Work split. A 256-thread workgroup owns a strip of 16 output columns and
// the whole K range, so it writes its float16 outputs directly: no split-K,
// no atomics, no workspace. Inside a wave, lane = (block slot ks, column quad
// cq): 4 column quads x 16 block slots. Each lane unpacks whole 32-row blocks
// of its 4 columns, streaming the block's b words with b 16-byte loads; a wave
// step covers 16 consecutive blocks of one run (uniform bit width). The 4
// waves take contiguous quarters of K, and the two steps ahead of the one
// being computed are in flight (double buffering).
//
// Strips are assigned XCD by XCD: workgroups are dispatched round-robin over
// the 8 XCDs, so workgroup i is given a strip from XCD (i % 8)'s contiguous
// range. The two 16-column strips that share each 128-byte line of a packed
// row are then read through the same L2.
//
// Arithmetic per block and column is that of the split-K decode kernel:
//   acc = sum_pairs dot2((1024 + q_lo, 1024 + q_hi), (x_lo, x_hi))
//   y  += s * (acc - (1024 + z) * X_blk)
// The activations are gathered by act-order into unpacking pair order once per
// call by the shared gather kernel (with the block sums X_blk); each
// workgroup copies them into LDS with 16-byte loads (in chunks when M * K is
// large).
// Reduction: butterfly shuffles across the 16 block slots of a wave, then
// the 4 waves through LDS.
#pragma once

#include "qlinear_kernels.hpp"

namespace qlinear {

namespace stream {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int CQ = 4;                  // column quads per strip
constexpr int SC = 4 * CQ;             // 16 columns per workgroup
constexpr int KS = 64 / CQ;            // 16 blocks per wave step
constexpr int kXcds = 8;
constexpr int kStageBudget = 60 * 1024;  // bytes of LDS for staged activations

struct StreamArgs {
  const uint32_t* xq;      // gathered activations, [M][K/32][16] float16 pairs
  const float* xsum;       // block sums, [M][K/32]
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint8_t* zeros;
  uint16_t* y;
  int M, K, N;
  int nstrips, strips_per_xcd;
  int chunk;                             // blocks per wave staged at a time
  Runs runs;
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

struct Raw {
  uint2 s;      // 4 float16 scales
  uint32_t z;   // 4 uint8 zero points
};

// One wave step: its 16 blocks start at block `blk0` and packed row `row0`
// (blocks of one run, b rows apart); `nb` of them are real.
struct Step {
  int blk0, row0, nb;
};

template <int B>
__device__ __forceinline__ void issue(const StreamArgs& a, const Step& st, int ks, int col, bool colv,
                                      int bpg, uint4 (&W)[B], Raw& P) {
  const bool ok = colv && ks < st.nb;
  const int row = st.row0 + ks * B;
#pragma unroll
  for (int t = 0; t < B; ++t)
    W[t] = ok ? *reinterpret_cast<const uint4*>(a.qweight + (size_t)(row + t) * a.N + col)
              : make_uint4(0u, 0u, 0u, 0u);
  const int g = (st.blk0 + ks) / bpg;
  P.s = ok ? *reinterpret_cast<const uint2*>(a.scales + (size_t)g * a.N + col) : make_uint2(0u, 0u);
  P.z = (ok && a.zeros) ? *reinterpret_cast<const uint32_t*>(a.zeros + (size_t)g * a.N + col) : 0u;
}

// Unpack and multiply one block (this lane's 4 columns), then fold in the
// block's scale and zero point.
template <int B, int MT>
__device__ __forceinline__ void compute(const StreamArgs& a, const uint4 (&W)[B], const Raw& P,
                                        const uint32_t* __restrict__ xs_blk, const float* __restrict__ xsum_blk,
                                        uint32_t magic, float (&yacc)[4][MT]) {
  uint32_t wc[4][B];
#pragma unroll
  for (int t = 0; t < B; ++t) {
    wc[0][t] = W[t].x;
    wc[1][t] = W[t].y;
    wc[2][t] = W[t].z;
    wc[3][t] = W[t].w;
  }
  float acc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[c][m] = 0.0f;

  static_for<0, kPairsPerBlock / 4>([&](auto Q) {
    constexpr int q4 = decltype(Q)::value;
    uint4 xv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xv[m] = *reinterpret_cast<const uint4*>(xs_blk + m * kPairsPerBlock + 4 * q4);
    static_for<0, 4>([&](auto R) {
      constexpr int r = decltype(R)::value;
      constexpr int Pp = 4 * q4 + r;
      uint32_t v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = extract_pair<B, Pp>(wc[c], magic);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t xp = r == 0 ? xv[m].x : r == 1 ? xv[m].y : r == 2 ? xv[m].z : xv[m].w;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c][m] = __builtin_amdgcn_fdot2(as_half2(v[c]), as_half2(xp), acc[c][m], false);
      }
    });
  });

  float s[4], zb[4];
  s[0] = half_lo(P.s.x);
  s[1] = half_hi(P.s.x);
  s[2] = half_lo(P.s.y);
  s[3] = half_hi(P.s.y);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    zb[c] = 1024.0f + (a.zeros ? (float)((P.z >> (8 * c)) & 0xFFu) : (float)(1 << (B - 1)));
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float X = xsum_blk[m];
#pragma unroll
    for (int c = 0; c < 4; ++c) yacc[c][m] = fmaf(s[c], fmaf(-zb[c], X, acc[c][m]), yacc[c][m]);
  }
}

// All steps of one run segment [blk0, blk1) of this wave, double-buffered
// (8-bit runs single-buffered, to bound register use). Blocks are at LDS slot
// (blk - lds_blk0) of this wave's staging area. With kPre, the first step's
// words and parameters are already in Wa / Pa.
template <int B, int MT, bool kPre>
__device__ __forceinline__ void run_segment(const StreamArgs& a, int blk0, int blk1, int row0, int ks, int col,
                                            bool colv, const uint32_t* xs_w, const float* xsum_w, int lds_blk0,
                                            uint32_t magic, float (&yacc)[4][MT], uint4 (&Wa)[B], Raw& Pa) {
  const int bpg = a.runs.blocks_per_group;
  const int nsteps = (blk1 - blk0 + KS - 1) / KS;
  auto step_of = [&](int i) {
    Step st;
    st.blk0 = blk0 + i * KS;
    st.row0 = row0 + i * KS * B;
    st.nb = min(KS, blk1 - st.blk0);
    return st;
  };
  auto lane_compute = [&](const Step& st, const uint4 (&W)[B], const Raw& P) {
    const int bl = min(st.blk0 + ks, blk1 - 1) - lds_blk0;   // clamped: idle lanes hold zeros
    compute<B, MT>(a, W, P, xs_w + bl * MT * kPairsPerBlock, xsum_w + bl * MT, magic, yacc);
  };
  if constexpr (!kPre) issue<B>(a, step_of(0), ks, col, colv, bpg, Wa, Pa);
  if constexpr (B == 8) {
    for (int i = 0; i < nsteps; ++i) {
      if (i > 0) issue<B>(a, step_of(i), ks, col, colv, bpg, Wa, Pa);
      lane_compute(step_of(i), Wa, Pa);
    }
  } else {
    uint4 Wb[B];
    Raw Pb;
    for (int i = 0; i < nsteps; i += 2) {
      if (i + 1 < nsteps) issue<B>(a, step_of(i + 1), ks, col, colv, bpg, Wb, Pb);
      lane_compute(step_of(i), Wa, Pa);
      if (i + 1 >= nsteps) break;
      if (i + 2 < nsteps) issue<B>(a, step_of(i + 2), ks, col, colv, bpg, Wa, Pa);
      lane_compute(step_of(i + 1), Wb, Pb);
    }
  }
}

template <int MT, unsigned BS>
__device__ __forceinline__ void any_segment(const StreamArgs& a, int bits, int blk0, int blk1, int row0, int ks,
                                            int col, bool colv, const uint32_t* xs_w, const float* xsum_w,
                                            int lds_blk0, uint32_t magic, float (&yacc)[4][MT]) {
#define QLINEAR_SEGMENT(BB)                                                                                \
  case BB:                                                                                                 \
    if constexpr ((BS >> BB) & 1u) {                                                                       \
      uint4 W[BB];                                                                                         \
      Raw P;                                                                                               \
      run_segment<BB, MT, false>(a, blk0, blk1, row0, ks, col, colv, xs_w, xsum_w, lds_blk0, magic, yacc, W, P); \
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

// Kernel body, specialised on B0, the width of this wave's first run, so the
// first step can be issued into a typed buffer before the activation staging
// and its HBM latency overlaps the act-order gather.
template <int MT, unsigned BS, int B0>
__device__ __forceinline__ void stream_body(const StreamArgs& a, uint32_t* lds, float (&red)[kWaves][MT][SC],
                                            int tid, int lane, int wave, int strip, int wb0, int wb1,
                                            int row0) {
  const int cq = lane % CQ, ks = lane / CQ;
  const int col = strip * SC + cq * 4;
  const bool colv = col < a.N;
  const int nblk = a.K / kBlockRows;
  const int per_wave = (nblk + kWaves - 1) / kWaves;
  const int nchunks = (per_wave + a.chunk - 1) / a.chunk;
  const uint32_t magic = vgpr_magic();

  // LDS: per wave, `chunk` blocks of MT x 16 float16 pairs, then the block sums.
  uint32_t* xs = lds;                                                                     // [kWaves][chunk][MT][16]
  float* xsum = reinterpret_cast<float*>(lds + kWaves * a.chunk * MT * kPairsPerBlock);  // [kWaves][chunk][MT]

  uint4 W0[B0];
  Raw P0;
  const int seg0_end = wb0 < wb1 ? min(min(wb1, run_end_block(a.runs, wb0)), wb0 + a.chunk) : wb0;
  if (wb0 < wb1) {
    Step st;
    st.blk0 = wb0;
    st.row0 = row0;
    st.nb = min(KS, seg0_end - wb0);
    issue<B0>(a, st, ks, col, colv, a.runs.blocks_per_group, W0, P0);
  }

  float yacc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[c][m] = 0.0f;

  for (int ch = 0; ch < nchunks; ++ch) {
    if (ch > 0) __syncthreads();  // every wave is done with the previous chunk
    // Stage chunk ch of every wave from the gathered activations: contiguous
    // 16-byte copies, eight in flight per thread.
    {
      const int per_w = a.chunk * MT * (kPairsPerBlock / 4);   // uint4 items per wave
      const int items = kWaves * per_w;
      constexpr int U = 8;
      for (int base = tid; base < items; base += U * kThreads) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int it = base + u * kThreads;
          v[u] = make_uint4(0u, 0u, 0u, 0u);
          if (it < items) {
            const int w = it / per_w, rem = it % per_w;
            const int bl = rem / (MT * 4), m = (rem / 4) % MT, q4 = rem % 4;
            const int blk = (w * nblk) / kWaves + ch * a.chunk + bl;
            if (m < a.M && blk < ((w + 1) * nblk) / kWaves)
              v[u] = *reinterpret_cast<const uint4*>(a.xq + ((size_t)m * nblk + blk) * kPairsPerBlock + 4 * q4);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int it = base + u * kThreads;
          if (it < items) *reinterpret_cast<uint4*>(xs + 4 * it) = v[u];
        }
      }
      for (int it = tid; it < kWaves * a.chunk * MT; it += kThreads) {
        const int w = it / (a.chunk * MT), rem = it % (a.chunk * MT);
        const int bl = rem / MT, m = rem % MT;
        const int blk = (w * nblk) / kWaves + ch * a.chunk + bl;
        float v = 0.0f;
        if (m < a.M && blk < ((w + 1) * nblk) / kWaves) v = a.xsum[(size_t)m * nblk + blk];
        xsum[it] = v;
      }
      __syncthreads();
    }

    const int c0 = wb0 + ch * a.chunk;
    const int c1 = min(wb1, c0 + a.chunk);
    const uint32_t* xs_w = xs + wave * a.chunk * MT * kPairsPerBlock;
    const float* xsum_w = xsum + wave * a.chunk * MT;
    int blk = c0;
    if (ch == 0 && blk < seg0_end) {
      run_segment<B0, MT, true>(a, blk, seg0_end, row0, ks, col, colv, xs_w, xsum_w, c0, magic, yacc, W0, P0);
      blk = seg0_end;
    }
    while (blk < c1) {
      int bits, row;
      block_info(a.runs, blk, bits, row);
      const int seg_end = min(c1, run_end_block(a.runs, blk));
      any_segment<MT, BS>(a, bits, blk, seg_end, row, ks, col, colv, xs_w, xsum_w, c0, magic, yacc);
      blk = seg_end;
    }
  }

  // Reduce over the 16 block slots of the wave (lanes cq, cq + 4, ..., cq + 60).
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = yacc[c][m];
#pragma unroll
      for (int off = CQ; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
      yacc[c][m] = v;
    }
  if (ks == 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) red[wave][m][cq * 4 + c] = yacc[c][m];
  }
  __syncthreads();
  if (tid < SC * MT) {
    const int m = tid / SC, c = tid % SC;
    const int n = strip * SC + c;
    if (m < a.M && n < a.N) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red[w][m][c];
      a.y[(size_t)m * a.N + n] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
  }
}

// One kernel per (MT, set of code widths that may occur). BS has bit b set
// for every width b the matrix may contain; the host picks the smallest
// instantiated set that covers the layout's runs, which keeps the register
// budget of the common formats low.
template <int MT, unsigned BS>
__global__ __launch_bounds__(kThreads) void qgemv_stream_kernel(StreamArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ float red[kWaves][MT][SC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  const int strip = (bid % kXcds) * a.strips_per_xcd + bid / kXcds;
  if (strip >= a.nstrips) return;  // the whole workgroup leaves together

  const int nblk = a.K / kBlockRows;
  const int wb0 = (wave * nblk) / kWaves, wb1 = ((wave + 1) * nblk) / kWaves;
  int bits0 = 0, row0 = 0;
  if (wb0 < wb1) block_info(a.runs, wb0, bits0, row0);
#define QLINEAR_BODY(BB)                                                                     \
  case BB:                                                                                   \
    if constexpr ((BS >> BB) & 1u) stream_body<MT, BS, BB>(a, lds, red, tid, lane, wave, strip, wb0, wb1, row0); \
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
  // This wave has no blocks (K < 128 rows): it still joins the barriers of
  // the staging and the final reduction, which stream_body's other waves run.
  stream_body<MT, BS, (BS & 16u) ? 4 : (BS & 4u) ? 2 : (BS & 8u) ? 3 : (BS & 32u) ? 5 : (BS & 64u) ? 6 : 8>(
      a, lds, red, tid, lane, wave, strip, wb0, wb1, row0);
}

template <int MT, unsigned BS>
hipError_t launch_set(StreamArgs a, hipStream_t stream) {
  const int nblk = a.K / kBlockRows;
  const int per_wave = (nblk + kWaves - 1) / kWaves;
  const int per_block_bytes = MT * (kPairsPerBlock * 4 + 4);
  const int max_chunk = kStageBudget / (kWaves * per_block_bytes);
  a.chunk = per_wave < max_chunk ? per_wave : max_chunk;
  if (a.chunk < 1) a.chunk = 1;
  a.nstrips = (a.N + SC - 1) / SC;
  a.strips_per_xcd = (a.nstrips + kXcds - 1) / kXcds;
  const size_t lds = (size_t)kWaves * a.chunk * per_block_bytes;
  hipLaunchKernelGGL((qgemv_stream_kernel<MT, BS>), dim3(kXcds * a.strips_per_xcd), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <unsigned BS>
hipError_t launch_set_any_m(const StreamArgs& a, hipStream_t stream) {
  if (a.M <= 1) return launch_set<1, BS>(a, stream);
  if (a.M <= 2) return launch_set<2, BS>(a, stream);
  return launch_set<4, BS>(a, stream);
}

constexpr unsigned kAllBits = (1u << 2) | (1u << 3) | (1u << 4) | (1u << 5) | (1u << 6) | (1u << 8);

// Instantiated in the qgemv_stream_*.hip files: M <= 4 per set of widths,
// and 4 < M <= 16 for any widths.
hipError_t launch_uniform(unsigned set, const StreamArgs& a, hipStream_t stream);
hipError_t launch_mixed(unsigned set, const StreamArgs& a, hipStream_t stream);
hipError_t launch_wide(const StreamArgs& a, hipStream_t stream);

}  // namespace stream

}  // namespace qlinear
