// Multi-row decode kernel (3 <= M <= 16 in use) on gfx950: the M activation
// rows fill one 16-row tile of v_mfma_f32_16x16x32_f16, so every weight is
// dequantized once and multiplied into all M rows by the matrix core. (The
// factored VALU kernel spends one dot2 per pair and row, which at M = 16
// needs more registers than a wave has.)
//
// Work split. A workgroup of 8 waves owns a strip of 16 FN columns (FN = 1,
// 2 or 4 per lane, chosen on the host) and the whole K range; the waves take
// contiguous parts of K and their partial tiles are summed through LDS, so
// there is no cross-workgroup reduction. Strips are dealt to the 8 XCDs in
// contiguous ranges, as in the other decode kernels.
//
// Per 32-row block a lane (column group c = l % 16, k-group g = l / 16)
// loads the packed words that hold pairs 4g .. 4g + 3 of its FN adjacent
// columns (one 4 FN-byte load per packed row) and the block's A fragment, 8
// gathered activations of row l % 16, from the workspace (rows past M read
// as zeros: their offsets lie beyond the buffer). It dequantizes its FN B
// fragments exactly in registers and issues FN MFMAs with the one A
// fragment. Loads run a chunk of blocks ahead of the MFMAs; the blocks go run
// by run, each run with its width fixed at compile time.
#include "mfma_frag.hpp"
#include "qgemv_stream.hpp"

namespace qlinear {

namespace {

using namespace frag;
using stream::MatPtrs;
using stream::kMaxMats;
using stream::kXcds;

constexpr int kWaves = 8;

// Words a lane loads per block and packed row: FN adjacent columns.
template <int FN>
using WordVec = typename std::conditional<FN == 4, u32x4, typename std::conditional<FN == 2, u32x2, uint32_t>::type>::type;

// Blocks of one wave whose loads are issued together, bounded by the words
// per block (kW packed rows of FN columns) to stay within registers.
template <int kW, int FN>
constexpr int chunk_blocks() {
  return kW * FN <= 4 ? 8 : kW * FN <= 12 ? 4 : 2;
}

struct MfmaArgs {
  const uint16_t* xq;      // gathered activations, float16 [M][K] in unpacking order
  MatPtrs mat[kMaxMats];
  int mats, has_zeros;
  int M, K, N, nstrips, strips_per_xcd;
  int xq_bytes, scale_bytes;
  int64_t packed_words;
  Runs runs;
  Epilogue epi;
};

// One block's loads for one lane.
template <int kW, int FN>
struct BlockLoads {
  u32x4 x;                 // A fragment: activations 8g .. 8g + 7 of row l % 16
  WordVec<FN> w[kW];       // the k-group's packed words of the lane's FN columns
  WordVec<(FN + 1) / 2> s; // FN float16 scales
  uint32_t z;              // FN uint8 zero points
};

struct Lane {
  __amdgpu_buffer_rsrc_t rx, rw, rs, rz;
  uint32_t xoff;   // byte offset of the lane's A piece in block 0
  uint32_t woff;   // byte offset of packed row 0 of the lane's first column in the strip's panels
  uint32_t col;    // the lane's first column (beyond every buffer when past N)
  int g;
};

template <int FN>
__device__ __forceinline__ WordVec<FN> load_words(__amdgpu_buffer_rsrc_t r, uint32_t v, int so) {
  if constexpr (FN == 4) return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, v, so, 0));
  else if constexpr (FN == 2) return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, v, so, 0));
  else return __builtin_amdgcn_raw_buffer_load_b32(r, v, so, 0);
}

// Loads of block blk (packed row `row`) of width B.
template <int B, int FN>
__device__ __forceinline__ void issue_block(const MfmaArgs& a, const Lane& L, int blk, int row,
                                            BlockLoads<frag_words<B>(), FN>& C) {
  C.x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.rx, L.xoff, blk * kBlockRows * 2, 0));
  const uint32_t v = L.woff + (uint32_t)frag_first_word<B>(L.g) * kPanel * 4;
#pragma unroll
  for (int t = 0; t < frag_words<B>(); ++t) C.w[t] = load_words<FN>(L.rw, v, (row + t) * kPanel * 4);
  const int grp = blk / a.runs.blocks_per_group;
  if constexpr (FN == 4) {
    C.s = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(L.rs, L.col * 2, grp * a.N * 2, 0));
    C.z = a.has_zeros ? __builtin_amdgcn_raw_buffer_load_b32(L.rz, L.col, grp * a.N, 0) : 0u;
  } else if constexpr (FN == 2) {
    C.s = __builtin_amdgcn_raw_buffer_load_b32(L.rs, L.col * 2, grp * a.N * 2, 0);
    C.z = a.has_zeros ? __builtin_amdgcn_raw_buffer_load_b16(L.rz, L.col, grp * a.N, 0) : 0u;
  } else {
    C.s = __builtin_amdgcn_raw_buffer_load_b16(L.rs, L.col * 2, grp * a.N * 2, 0);
    C.z = a.has_zeros ? __builtin_amdgcn_raw_buffer_load_b8(L.rz, L.col, grp * a.N, 0) : 0u;
  }
}

template <int FN>
__device__ __forceinline__ uint32_t word_of(const WordVec<FN>& w, int j) {
  if constexpr (FN == 1) return w;
  else return w[j];
}

// Fragment j: column j of the lane's FN columns.
template <int B, int FN>
__device__ __forceinline__ void compute_block(const MfmaArgs& a, const Lane& L, const BlockLoads<frag_words<B>(), FN>& C,
                                              uint32_t magic, float4_t (&acc)[FN]) {
  constexpr int kW = frag_words<B>();
  const half8_t af = __builtin_bit_cast(half8_t, C.x);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    // -(1024 + z) and the scale as float16 pairs; symmetric codes use z = 2^(b-1).
    const uint32_t z = a.has_zeros ? ((C.z >> (8 * j)) & 0xFFu) : (uint32_t)(1 << (B - 1));
    const uint32_t nb = (z * 0x10001u) | 0xE400E400u;
    uint32_t sh;
    if constexpr (FN == 1) sh = C.s;
    else sh = word_of<(FN + 1) / 2>(C.s, j / 2) >> (16 * (j % 2));
    const uint32_t sv = (sh & 0xFFFFu) * 0x10001u;
    uint32_t w[kW];
#pragma unroll
    for (int t = 0; t < kW; ++t) w[t] = word_of<FN>(C.w[t], j);
    const half8_t bf = dequant_frag<B, kW>(w, L.g, as_half2(nb), as_half2(sv), magic);
    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[j], 0, 0, 0);
  }
}

// Loads of the blocks c0 .. c0 + kC - 1 that lie in the segment.
template <int B, int FN, int kC>
__device__ __forceinline__ void issue_chunk(const MfmaArgs& a, const Lane& L, int s0, int s1, int row0, int c0,
                                            BlockLoads<frag_words<B>(), FN> (&C)[kC]) {
#pragma unroll
  for (int i = 0; i < kC; ++i)
    if (c0 + i < s1) issue_block<B, FN>(a, L, c0 + i, row0 + (c0 + i - s0) * B, C[i]);   // uniform over the wave
}

template <int B, int FN, int kC>
__device__ __forceinline__ void compute_chunk(const MfmaArgs& a, const Lane& L, int s1, int c0,
                                              const BlockLoads<frag_words<B>(), FN> (&C)[kC], uint32_t magic,
                                              float4_t (&acc)[FN]) {
#pragma unroll
  for (int i = 0; i < kC; ++i)
    if (c0 + i < s1) compute_block<B, FN>(a, L, C[i], magic, acc);   // uniform over the wave
}

// Blocks [s0, s1) of one width B, starting at packed row row0: chunks of
// blocks double-buffered.
template <int B, int FN>
__device__ __forceinline__ void segment(const MfmaArgs& a, const Lane& L, int s0, int s1, int row0, uint32_t magic,
                                        float4_t (&acc)[FN]) {
  constexpr int kC = chunk_blocks<frag_words<B>(), FN>();
  BlockLoads<frag_words<B>(), FN> C0[kC], C1[kC];
  issue_chunk<B, FN, kC>(a, L, s0, s1, row0, s0, C0);
  for (int c = s0; c < s1; c += 2 * kC) {
    issue_chunk<B, FN, kC>(a, L, s0, s1, row0, c + kC, C1);
    compute_chunk<B, FN, kC>(a, L, s1, c, C0, magic, acc);
    if (c + kC >= s1) break;
    issue_chunk<B, FN, kC>(a, L, s0, s1, row0, c + 2 * kC, C0);
    compute_chunk<B, FN, kC>(a, L, s1, c + kC, C1, magic, acc);
  }
}

// A workgroup's strip is 16 FN columns: lane l (c = l % 16) takes columns
// 16 FN * strip + FN c + j, j < FN, and fragment j holds column j of every lane.
template <unsigned BS, int FN>
__global__ __launch_bounds__(kWaves * 64) void qgemv_mfma_kernel(MfmaArgs a) {
  __shared__ float4_t red[kWaves][FN][64];

  // Kernel arguments, all read in one batch (the matrix is blockIdx.y, so no
  // read waits on another): the empty asm takes them as operands and hands
  // them back, so they are not read again later.
  MatPtrs mp = a.mat[blockIdx.y];
  int spx = a.strips_per_xcd, nstrips = a.nstrips, M = a.M, K = a.K, N = a.N, R = a.runs.packed_rows;
  int xq_bytes = a.xq_bytes, scale_bytes = a.scale_bytes, has_zeros = a.has_zeros;
  int64_t packed_words = a.packed_words;
  const uint16_t* xq = a.xq;
  Epilogue epi = a.epi;
  asm volatile("" : "+s"(mp.qweight), "+s"(mp.scales), "+s"(mp.zeros), "+s"(mp.y), "+s"(spx), "+s"(nstrips),
               "+s"(M), "+s"(K), "+s"(N), "+s"(R), "+s"(xq_bytes), "+s"(scale_bytes), "+s"(has_zeros),
               "+s"(packed_words), "+s"(xq), "+s"(epi.bias), "+s"(epi.residual), "+s"(epi.act),
               "+s"(epi.addend)
               : "s"(a.runs.blocks_per_group));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  const int strip = (bid % kXcds) * spx + bid / kXcds;
  if (strip >= nstrips) return;   // the whole workgroup leaves together

  Lane L;
  L.g = lane >> 4;
  L.rx = __builtin_amdgcn_make_buffer_rsrc((void*)xq, 0, xq_bytes, kRsrcWord3);
  // The weight buffer starts at the strip's first panel, so 32-bit offsets
  // cover any matrix: they only span the strip's FN panels.
  const int64_t strip_words = (int64_t)FN * R * kPanel;
  const int64_t first_word = (int64_t)strip * strip_words;
  L.rw = __builtin_amdgcn_make_buffer_rsrc((void*)(mp.qweight + first_word), 0,
                                           (int)(min(strip_words, packed_words - first_word) * 4), kRsrcWord3);
  L.rs = __builtin_amdgcn_make_buffer_rsrc((void*)mp.scales, 0, scale_bytes, kRsrcWord3);
  L.rz = __builtin_amdgcn_make_buffer_rsrc(has_zeros ? (void*)mp.zeros : (void*)mp.scales, 0,
                                           has_zeros ? scale_bytes / 2 : scale_bytes, kRsrcWord3);
  const int m = lane & 15;
  // Rows past M and columns past N read at offsets beyond every buffer: the
  // loads return zeros (zero activations, zero scales). N is a multiple of 8,
  // so a lane's FN columns are in or out as a whole.
  L.xoff = m < M ? ((uint32_t)m * (uint32_t)K + 8u * (uint32_t)L.g) * 2u : 0x80000000u;
  const int col = strip * kPanel * FN + (lane & 15) * FN;
  const bool cok = col < N;
  L.col = cok ? (uint32_t)col : 0x40000000u;
  L.woff = cok ? (uint32_t)(col / kPanel - strip * FN) * (uint32_t)R * kPanel * 4 +
                     (uint32_t)(col % kPanel) * 4
               : 0x80000000u;

  const int nblk = K / kBlockRows;
  const int b0 = (wave * nblk) / kWaves, b1 = ((wave + 1) * nblk) / kWaves;
  const uint32_t magic = vgpr_magic();
  float4_t acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) acc[j] = {0.f, 0.f, 0.f, 0.f};
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
    with_width<BS>(bits, [&](auto BB) { segment<decltype(BB)::value, FN>(a, L, blk, s1, row, magic, acc); });
    blk = s1;
  }

  // Lane l holds rows 4 (l / 16) + r of column l % 16 of each fragment of the
  // wave's partial tile; the 8 partial tiles are summed through LDS.
#pragma unroll
  for (int j = 0; j < FN; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  for (int e = tid; e < 256 * FN; e += kWaves * 64) {
    const int j = e >> 8, l = (e >> 2) & 63, r = e & 3;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[w][j][l][r];
    const int row = 4 * (l >> 4) + r;
    const int c = strip * kPanel * FN + (l & 15) * FN + j;
    if (row < M && c < N)
      ((__attribute__((address_space(1))) uint16_t*)mp.y)[(size_t)row * N + c] =
          __builtin_bit_cast(uint16_t, (_Float16)apply_epilogue(epi, v, row, c, N));
  }
}

template <unsigned BS, int FN>
hipError_t launch_fn(MfmaArgs a, hipStream_t stream) {
  a.nstrips = (a.N + kPanel * FN - 1) / (kPanel * FN);
  a.strips_per_xcd = (a.nstrips + kXcds - 1) / kXcds;
  hipLaunchKernelGGL((qgemv_mfma_kernel<BS, FN>), dim3(kXcds * a.strips_per_xcd, a.mats), dim3(kWaves * 64), 0, stream,
                     a);
  return hipGetLastError();
}

// Columns per lane. Wider strips let one A fragment feed more MFMAs and
// read the activations fewer times, but leave fewer workgroups, each wave
// with its whole share of K. Measured on MI355X at M = 8 and 16: 4 columns
// when that still gives >= 128 workgroups and a wave has <= 32 blocks
// (4096 -> 11008: 17 vs 27 us; 8192 -> 28672 at 2.5 bpw: 100 vs 128 us),
// otherwise the widest with >= 256 workgroups (28672 -> 8192: 2 columns,
// 101 vs 114 us; 4096 -> 4096 and 11008 -> 4096: 1 column).
template <unsigned BS>
hipError_t launch_set(const MfmaArgs& a, hipStream_t stream) {
  const auto strips = [&](int fn) { return a.mats * ((a.N + kPanel * fn - 1) / (kPanel * fn)); };
  const int blocks_per_wave = a.K / kBlockRows / kWaves;
  if (strips(4) >= 256 || (strips(4) >= 128 && blocks_per_wave <= 32)) return launch_fn<BS, 4>(a, stream);
  if (strips(2) >= 256) return launch_fn<BS, 2>(a, stream);
  return launch_fn<BS, 1>(a, stream);
}

}  // namespace

bool qgemv_mfma_supported(const qlinear_layout& L) {
  // Buffer offsets and sizes are 32-bit: the scales and the gathered
  // activations must stay below 2^31 bytes (the weights are addressed per strip).
  const size_t lim = (size_t)1 << 31;
  return (size_t)L.groups * L.N * 2 < lim && (size_t)QLINEAR_GEMV_MAX_M * L.K * 2 < lim &&
         (size_t)4 * L.packed_rows * kPanel * 4 < lim;
}

hipError_t launch_qgemv_mfma(const qlinear_layout& L, const Runs& runs, const uint32_t* xq, int M, int mats,
                             const uint32_t* const* qweights, const uint16_t* const* scales,
                             const uint8_t* const* zeros, uint16_t* const* ys, const Epilogue& epi,
                             hipStream_t stream) {
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
  a.nstrips = 0;
  a.strips_per_xcd = 0;
  a.xq_bytes = (int)((size_t)M * L.K * 2);
  a.packed_words = L.packed_words;
  a.scale_bytes = (int)((size_t)L.groups * L.N * 2);
  a.runs = runs;
  a.epi = epi;
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
