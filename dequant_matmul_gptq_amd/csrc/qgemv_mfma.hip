// Multi-row decode kernel (2 <= M <= 16) on gfx950: the M activation rows
// fill one 16-row tile of v_mfma_f32_16x16x32_f16, so every weight is
// dequantized once and multiplied into all M rows by the matrix core. (The
// factored VALU kernel spends one dot2 per pair and row, which at M = 16
// needs more registers than a wave has.)
//
// Work split. A workgroup of 8 waves owns a 16-column strip -- one storage
// panel -- and the whole K range; the waves take contiguous parts of K and
// their 16 x 16 partial tiles are summed through LDS, so there is no
// cross-workgroup reduction. Strips are dealt to the 8 XCDs in contiguous
// ranges, as in the other decode kernels.
//
// Per 32-row block a lane (column n = l % 16, k-group g = l / 16) loads the
// packed words that hold pairs 4g .. 4g + 3 of its column (one word at 4
// bits) and the block's A fragment, 8 gathered activations of row l % 16,
// from the workspace (rows past M read as zeros: their offsets lie beyond
// the buffer). It dequantizes its B fragment exactly in registers and issues
// one MFMA. Loads run a chunk of blocks ahead of the MFMAs; the blocks go
// run by run, each run with its width fixed at compile time.
#include "mfma_frag.hpp"
#include "qgemv_stream.hpp"

namespace qlinear {

namespace {

using namespace frag;
using stream::MatPtrs;
using stream::kMaxMats;
using stream::kXcds;

constexpr int kWaves = 8;
// Blocks of one wave whose loads are issued together: 8, or 4 where a
// k-group spreads over all b words (widths 3, 5, 6), to bound registers.
template <int kW>
constexpr int chunk_blocks() {
  return kW <= 2 ? 8 : 4;
}

struct MfmaArgs {
  const uint16_t* xq;      // gathered activations, float16 [M][K] in unpacking order
  MatPtrs mat[kMaxMats];
  int mats, has_zeros;
  int M, K, N, nstrips, strips_per_xcd;
  int xq_bytes, qweight_bytes, scale_bytes;
  Runs runs;
};

// One block's loads for one lane.
template <int kW>
struct BlockLoads {
  u32x4 x;          // A fragment: activations 8g .. 8g + 7 of row l % 16
  uint32_t w[kW];   // the k-group's packed words of column n
  uint32_t s;       // float16 scale (low half)
  uint32_t z;       // zero point (low byte)
};

struct Lane {
  __amdgpu_buffer_rsrc_t rx, rw, rs, rz;
  uint32_t xoff;   // byte offset of the lane's A piece in block 0
  uint32_t woff;   // byte offset of packed row 0 of the lane's column
  uint32_t col;    // the lane's column (beyond every buffer when past N)
  int g;
};

// Loads of block blk (packed row `row`) of width B.
template <int B>
__device__ __forceinline__ void issue_block(const MfmaArgs& a, const Lane& L, int blk, int row,
                                            BlockLoads<frag_words<B>()>& C) {
  C.x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.rx, L.xoff, blk * kBlockRows * 2, 0));
  const uint32_t v = L.woff + (uint32_t)frag_first_word<B>(L.g) * kPanel * 4;
#pragma unroll
  for (int t = 0; t < frag_words<B>(); ++t)
    C.w[t] = __builtin_amdgcn_raw_buffer_load_b32(L.rw, v, (row + t) * kPanel * 4, 0);
  const int grp = blk / a.runs.blocks_per_group;
  C.s = __builtin_amdgcn_raw_buffer_load_b16(L.rs, L.col * 2, grp * a.N * 2, 0);
  C.z = a.has_zeros ? __builtin_amdgcn_raw_buffer_load_b8(L.rz, L.col, grp * a.N, 0) : 0u;
}

template <int B>
__device__ __forceinline__ void compute_block(const MfmaArgs& a, const Lane& L, const BlockLoads<frag_words<B>()>& C,
                                              uint32_t magic, float4_t& acc) {
  constexpr int kW = frag_words<B>();
  // -(1024 + z) and the scale as float16 pairs; symmetric codes use z = 2^(b-1).
  const uint32_t z = a.has_zeros ? (C.z & 0xFFu) : (uint32_t)(1 << (B - 1));
  const uint32_t nb = (z * 0x10001u) | 0xE400E400u;
  const uint32_t sv = (C.s & 0xFFFFu) * 0x10001u;
  uint32_t w[kW];
#pragma unroll
  for (int t = 0; t < kW; ++t) w[t] = C.w[t];
  const half8_t bf = dequant_frag<B, kW>(w, L.g, as_half2(nb), as_half2(sv), magic);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, C.x), bf, acc, 0, 0, 0);
}

// Loads of the blocks c0 .. c0 + kC - 1 that lie in the segment.
template <int B, int kC>
__device__ __forceinline__ void issue_chunk(const MfmaArgs& a, const Lane& L, int s0, int s1, int row0, int c0,
                                            BlockLoads<frag_words<B>()> (&C)[kC]) {
#pragma unroll
  for (int i = 0; i < kC; ++i)
    if (c0 + i < s1) issue_block<B>(a, L, c0 + i, row0 + (c0 + i - s0) * B, C[i]);   // uniform over the wave
}

template <int B, int kC>
__device__ __forceinline__ void compute_chunk(const MfmaArgs& a, const Lane& L, int s1, int c0,
                                              const BlockLoads<frag_words<B>()> (&C)[kC], uint32_t magic,
                                              float4_t& acc) {
#pragma unroll
  for (int i = 0; i < kC; ++i)
    if (c0 + i < s1) compute_block<B>(a, L, C[i], magic, acc);   // uniform over the wave
}

// Blocks [s0, s1) of one width B, starting at packed row row0: chunks of
// blocks double-buffered.
template <int B>
__device__ __forceinline__ void segment(const MfmaArgs& a, const Lane& L, int s0, int s1, int row0, uint32_t magic,
                                        float4_t& acc) {
  constexpr int kC = chunk_blocks<frag_words<B>()>();
  BlockLoads<frag_words<B>()> C0[kC], C1[kC];
  issue_chunk<B, kC>(a, L, s0, s1, row0, s0, C0);
  for (int c = s0; c < s1; c += 2 * kC) {
    issue_chunk<B, kC>(a, L, s0, s1, row0, c + kC, C1);
    compute_chunk<B, kC>(a, L, s1, c, C0, magic, acc);
    if (c + kC >= s1) break;
    issue_chunk<B, kC>(a, L, s0, s1, row0, c + 2 * kC, C0);
    compute_chunk<B, kC>(a, L, s1, c + kC, C1, magic, acc);
  }
}

template <unsigned BS>
__global__ __launch_bounds__(kWaves * 64) void qgemv_mfma_kernel(MfmaArgs a) {
  __shared__ float4_t red[kWaves][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  const int gstrip = (bid % kXcds) * a.strips_per_xcd + bid / kXcds;
  if (gstrip >= a.mats * a.nstrips) return;   // the whole workgroup leaves together
  const int mi = gstrip / a.nstrips;
  const int strip = gstrip - mi * a.nstrips;
  const MatPtrs mp = a.mat[mi];

  Lane L;
  L.g = lane >> 4;
  L.rx = __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, 0, a.xq_bytes, kRsrcWord3);
  L.rw = __builtin_amdgcn_make_buffer_rsrc((void*)mp.qweight, 0, a.qweight_bytes, kRsrcWord3);
  L.rs = __builtin_amdgcn_make_buffer_rsrc((void*)mp.scales, 0, a.scale_bytes, kRsrcWord3);
  L.rz = __builtin_amdgcn_make_buffer_rsrc(a.has_zeros ? (void*)mp.zeros : (void*)mp.scales, 0,
                                           a.has_zeros ? a.scale_bytes / 2 : a.scale_bytes, kRsrcWord3);
  const int m = lane & 15;
  // Rows past M and columns past N read at offsets beyond every buffer: the
  // loads return zeros (zero activations, zero scales).
  L.xoff = m < a.M ? ((uint32_t)m * (uint32_t)a.K + 8u * (uint32_t)L.g) * 2u : 0x80000000u;
  const int col = strip * kPanel + (lane & 15);
  const bool cok = col < a.N;
  L.col = cok ? (uint32_t)col : 0x40000000u;
  L.woff = cok ? (uint32_t)strip * (uint32_t)a.runs.packed_rows * kPanel * 4 + (uint32_t)(col % kPanel) * 4
               : 0x80000000u;

  const int nblk = a.K / kBlockRows;
  const int b0 = (wave * nblk) / kWaves, b1 = ((wave + 1) * nblk) / kWaves;
  const uint32_t magic = vgpr_magic();
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  // The wave's blocks run segment by segment (a segment is the part of a run
  // of one width inside [b0, b1)), the width a compile-time constant inside.
  for (int blk = b0; blk < b1;) {
    int bits, row;
    if constexpr ((BS & (BS - 1)) == 0) {
      bits = __builtin_ctz(BS);
      row = blk * bits;
    } else {
      block_info(a.runs, blk, bits, row);
    }
    const int s1 = (BS & (BS - 1)) == 0 ? b1 : min(b1, run_end_block(a.runs, blk));
    with_width<BS>(bits, [&](auto BB) { segment<decltype(BB)::value>(a, L, blk, s1, row, magic, acc); });
    blk = s1;
  }

  // Lane l holds rows 4 (l / 16) + r of column l % 16 of the wave's partial
  // tile; the 8 partial tiles are summed through LDS, one thread per output.
  red[wave][lane] = acc;
  __syncthreads();
  if (tid < 256) {
    const int l = tid >> 2, r = tid & 3;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[w][l][r];
    const int row = 4 * (l >> 4) + r;
    const int c = strip * kPanel + (l & 15);
    if (row < a.M && c < a.N)
      mp.y[(size_t)row * a.N + c] = __builtin_bit_cast(uint16_t, (_Float16)v);
  }
}

template <unsigned BS>
hipError_t launch_set(const MfmaArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((qgemv_mfma_kernel<BS>), dim3(kXcds * a.strips_per_xcd), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool qgemv_mfma_supported(const qlinear_layout& L) {
  // Buffer offsets and sizes are 32-bit.
  const size_t lim = (size_t)1 << 31;
  return (size_t)L.packed_words * 4 < lim && (size_t)L.groups * L.N * 2 < lim &&
         (size_t)QLINEAR_GEMV_MAX_M * L.K * 2 < lim;
}

hipError_t launch_qgemv_mfma(const qlinear_layout& L, const Runs& runs, const uint32_t* xq, int M, int mats,
                             const uint32_t* const* qweights, const uint16_t* const* scales,
                             const uint8_t* const* zeros, uint16_t* const* ys, hipStream_t stream) {
  MfmaArgs a;
  a.xq = reinterpret_cast<const uint16_t*>(xq);
  a.mats = mats;
  a.has_zeros = zeros != nullptr && zeros[0] != nullptr;
  for (int i = 0; i < kMaxMats; ++i) {
    const int j = i < mats ? i : 0;   // unused entries repeat matrix 0
    a.mat[i].qweight = qweights[j];
    a.mat[i].scales = scales[j];
    a.mat[i].zeros = a.has_zeros ? zeros[j] : nullptr;
    a.mat[i].y = ys[j];
  }
  a.M = M;
  a.K = L.K;
  a.N = L.N;
  a.nstrips = (L.N + kPanel - 1) / kPanel;
  a.strips_per_xcd = (mats * a.nstrips + kXcds - 1) / kXcds;
  a.xq_bytes = (int)((size_t)M * L.K * 2);
  a.qweight_bytes = (int)((size_t)L.packed_words * 4);
  a.scale_bytes = (int)((size_t)L.groups * L.N * 2);
  a.runs = runs;
  unsigned set = 0;
  for (int r = 0; r < L.nruns; ++r) set |= 1u << L.run_bits[r];
  switch (set) {
    case 1u << 2: return launch_set<1u << 2>(a, stream);
    case 1u << 3: return launch_set<1u << 3>(a, stream);
    case 1u << 4: return launch_set<1u << 4>(a, stream);
    case 1u << 5: return launch_set<1u << 5>(a, stream);
    case 1u << 6: return launch_set<1u << 6>(a, stream);
    case 1u << 8: return launch_set<1u << 8>(a, stream);
    default: break;
  }
  if ((set & ~stream::kLowBits) == 0) return launch_set<stream::kLowBits>(a, stream);
  if ((set & ~stream::kMidBits) == 0) return launch_set<stream::kMidBits>(a, stream);
  return launch_set<stream::kAllBits>(a, stream);
}

}  // namespace qlinear
