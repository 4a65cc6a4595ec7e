// Prefill kernel for matrices with several code widths (EXL2): a 128 x 128
// tile per workgroup of 4 waves (64 x 64 each). Per K-step of 64 rows (two
// 32-row blocks) the activation tile is copied to LDS and the weight tile is
// unpacked and dequantized exactly to float16 in LDS (each block with its own
// width; w = RNE(s * (q - z)), one rounding), then v_mfma_f32_16x16x32_f16
// accumulates in float32. The activations were gathered by act-order into
// unpacking pair order beforehand, as for the single-width kernel.
//
// Every global load of a step (A pieces, packed words, scale, zero point) is
// a buffer load with a per-lane offset fixed for the whole kernel and a
// scalar per-step offset, issued unconditionally and before the first wait:
// rows past M repeat row M - 1 and columns past N repeat column N - 1 (their
// outputs are not stored), so no load sits behind a branch. The scale and
// zero-point modes are template parameters for the same reason. A block's
// width and first packed row come from a scalar run cursor that moves along K
// with the blocks.
#include <algorithm>

#include "mfma_frag.hpp"

namespace qlinear {

namespace {

using frag::kRsrcWord3;
using frag::u32x4;

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kLdsRow = BK;            // 64 halves = 128 bytes, eight 16-byte chunks
constexpr int kAPieces = BM * BK / 8 / kThreads;   // 16-byte A pieces per thread per step

// LDS tiles are rows of 64 halves without padding; 16-byte chunk c of row r
// sits at chunk position c ^ (r & 7). Measured with SQ_LDS_BANK_CONFLICT on
// gfx950: a 16-byte store is conflict-free when each 8 consecutive lanes
// write 8 distinct 16-byte slots of a 128-byte window, which holds for the
// A-tile stores (8 lanes: one row's 8 chunks) and, with this swizzle, for the
// B-tile stores (8 lanes: 8 consecutive rows at one chunk; the swizzle
// c ^ ((r >> 1) & 7) cost 8 conflict cycles per store). The fragment reads
// (16 consecutive rows at one chunk) are conflict-free with either.
__device__ __forceinline__ int lds_at(int r, int c) { return r * kLdsRow + ((c ^ (r & 7)) << 3); }

// Per-lane LDS offsets (halves) of the tile accesses, set once: the low three
// bits of the row are the same in every access a lane makes, so each access
// is one of these plus a multiple of 8 rows.
struct LdsOffsets {
  int a_st;      // A-tile store of piece 0 (piece i: + 32 i rows)
  int b_st[4];   // B-tile stores: chunks bchunk .. bchunk + 3 of the thread's row
  int a_rd[2];   // A fragment 0 at K offsets 0 and 32 (fragment i: + 16 i rows)
  int b_rd[2];   // B fragment 0, likewise
};

struct LdsGemmArgs {
  const uint16_t* xq;
  const uint32_t* qweight;
  const uint16_t* scales;   // float16 [groups][N], or packed 4-bit codes [groups][N / 8] (two-level)
  const uint8_t* zeros;
  uint16_t* y;
  int M, K, N;
  int xq_bytes, qweight_bytes, scale_bytes, zero_bytes;
  // Split K: slice blockIdx.z covers blocks [z * slice_blocks, + slice_blocks)
  // and writes float32 partial sums part[z][M][N] (the epilogue comes in
  // split_sum_kernel); part == nullptr: one slice, float16 output.
  float* part;
  int slice_blocks;
  Runs runs;
  Epilogue epi;
};

// The run of the blocks a wave is at: blocks advance along K, so the run
// index only moves forward and its table entries are read when a block
// crosses into the next run (wave-uniform, scalar registers).
struct RunCursor {
  int r;      // run index
  int b0;     // its first block
  int row0;   // its first packed row
  int bits;   // its code width
  int next;   // first block of run r + 1 (K / 32 after the last run)
};

// Width and first packed row of block blk (wave-uniform, not below the
// cursor's first block).
__device__ __forceinline__ void run_of(const LdsGemmArgs& a, RunCursor& c, int blk, int& bits, int& row) {
  while (blk >= c.next) {
    ++c.r;
    c.b0 = c.next;
    c.row0 = a.runs.run_row[c.r];
    c.bits = a.runs.run_bits[c.r];
    c.next = a.runs.run_block[c.r + 1];
  }
  bits = c.bits;
  row = c.row0 + (blk - c.b0) * c.bits;
}

// Per-lane buffer offsets (bytes) that do not change along K.
struct LaneOffsets {
  uint32_t a[kAPieces];   // A piece (row, 16-byte chunk) at K = 0
  uint32_t w;             // packed row 0 of the lane's column
  uint32_t s;             // the column's scale (or its scale code's word) in group 0
  uint32_t z;             // the column's zero point in group 0
};

struct Rsrc {
  __amdgpu_buffer_rsrc_t x, w, s, z;
};

// The packed words, scale and zero point of (block at packed row `row`, group
// g) for the lane's column: loads only.
template <int B, bool kTL, bool kZeros>
struct BLoads {
  uint32_t w[B];
  uint32_t s;
  uint32_t z;
};

template <int B, bool kTL, bool kZeros>
__device__ __forceinline__ BLoads<B, kTL, kZeros> load_b(const LdsGemmArgs& a, const Rsrc& rs, const LaneOffsets& off,
                                                         int row, int g) {
  BLoads<B, kTL, kZeros> v;
  const int wrow = row * kPanel * 4;   // rows of a panel are 16 words apart
#pragma unroll
  for (int t = 0; t < B; ++t) v.w[t] = __builtin_amdgcn_raw_buffer_load_b32(rs.w, off.w, wrow + t * kPanel * 4, 0);
  if constexpr (kTL)
    v.s = __builtin_amdgcn_raw_buffer_load_b32(rs.s, off.s, g * (a.N / 8) * 4, 0);
  else
    v.s = __builtin_amdgcn_raw_buffer_load_b16(rs.s, off.s, g * a.N * 2, 0);
  if constexpr (kZeros) v.z = __builtin_amdgcn_raw_buffer_load_b8(rs.z, off.z, g * a.N, 0);
  return v;
}

// Unpack + dequantize the loaded (block, column) into 16 float16 pairs in LDS.
// Two-level scales: the group factor c + 1, exact in float16, so that
// s * (q - z) stays an exact integer; scale_max / 16 comes in the epilogue.
template <int B, bool kTL, bool kZeros>
__device__ __forceinline__ void dequant_to_lds(const BLoads<B, kTL, kZeros>& v, int ncol, uint16_t* Bs,
                                               const LdsOffsets& lo) {
  const _Float16 s = kTL ? (_Float16)qscale_factor(v.s, ncol) : __builtin_bit_cast(_Float16, (uint16_t)v.s);
  const int z = kZeros ? (int)v.z : 1 << (B - 1);
  const _Float16 nb = (_Float16)(-(1024 + z));
  const half2_t scale = {s, s}, neg_bias = {nb, nb};
  uint32_t pr[kPairsPerBlock];
  extract_all_pairs<B>(v.w, pr);
#pragma unroll
  for (int q4 = 0; q4 < kPairsPerBlock / 4; ++q4) {
    u32x4 o;
    o[0] = as_u32(dequant_pair(pr[4 * q4 + 0], neg_bias, scale));
    o[1] = as_u32(dequant_pair(pr[4 * q4 + 1], neg_bias, scale));
    o[2] = as_u32(dequant_pair(pr[4 * q4 + 2], neg_bias, scale));
    o[3] = as_u32(dequant_pair(pr[4 * q4 + 3], neg_bias, scale));
    *reinterpret_cast<u32x4*>(Bs + lo.b_st[q4]) = o;
  }
}

// Fill the LDS tiles of the step at block kb: the A tile (128 rows x 64
// halves) and this wave's block kb + bsub of the B tile (the thread's
// column: four chunks of its row), dequantized at width B. kTail: K ends after block kb (odd block count), so the second
// half of the A tile is zero and the waves of the second block store zeros.
template <int B, bool kTL, bool kZeros, bool kTail>
__device__ __forceinline__ void fill_step(const LdsGemmArgs& a, const Rsrc& rs, const LaneOffsets& off, int tid, int kb,
                                          int blk, int row, int ncol, bool bzero, uint16_t* As, uint16_t* Bs,
                                          const LdsOffsets& lo) {
  u32x4 av[kAPieces];
#pragma unroll
  for (int i = 0; i < kAPieces; ++i)
    av[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.x, off.a[i], kb * kBlockRows * 2, 0));
  BLoads<B, kTL, kZeros> bl;
  if (!kTail || !bzero) bl = load_b<B, kTL, kZeros>(a, rs, off, row, blk / a.runs.blocks_per_group);
  // A stores wait only for the A loads (the B loads were issued after them).
#pragma unroll
  for (int i = 0; i < kAPieces; ++i) {
    u32x4 v = av[i];
    if constexpr (kTail)
      if (tid % (BK / 8) >= BK / 16) v = u32x4{0u, 0u, 0u, 0u};   // chunks of the block past K
    *reinterpret_cast<u32x4*>(As + lo.a_st + i * (kThreads / (BK / 8)) * kLdsRow) = v;
  }
  if (kTail && bzero) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) *reinterpret_cast<u32x4*>(Bs + lo.b_st[q4]) = u32x4{0u, 0u, 0u, 0u};
  } else {
    dequant_to_lds<B, kTL, kZeros>(bl, ncol, Bs, lo);
  }
}

// One K-step: both LDS tiles filled (the width's branch is uniform per wave),
// then 2 x 16 MFMAs per wave.
template <bool kTL, bool kZeros, bool kTail>
__device__ __forceinline__ void k_step(const LdsGemmArgs& a, const Rsrc& rs, RunCursor& cur, const LaneOffsets& off,
                                       const LdsOffsets& lo, int tid, int bsub, int kb, int nblk, int ncol, uint16_t* As,
                                       uint16_t* Bs, float4_t (&acc)[4][4]) {
  const int blk = __builtin_amdgcn_readfirstlane(kb + bsub);
  const bool bzero = kTail && blk >= nblk;   // wave-uniform
  int bits = 4, row = 0;
  if (!bzero) run_of(a, cur, blk, bits, row);
  switch (bits) {
    case 2: fill_step<2, kTL, kZeros, kTail>(a, rs, off, tid, kb, blk, row, ncol, bzero, As, Bs, lo); break;
    case 3: fill_step<3, kTL, kZeros, kTail>(a, rs, off, tid, kb, blk, row, ncol, bzero, As, Bs, lo); break;
    case 4: fill_step<4, kTL, kZeros, kTail>(a, rs, off, tid, kb, blk, row, ncol, bzero, As, Bs, lo); break;
    case 5: fill_step<5, kTL, kZeros, kTail>(a, rs, off, tid, kb, blk, row, ncol, bzero, As, Bs, lo); break;
    case 6: fill_step<6, kTL, kZeros, kTail>(a, rs, off, tid, kb, blk, row, ncol, bzero, As, Bs, lo); break;
    default: fill_step<8, kTL, kZeros, kTail>(a, rs, off, tid, kb, blk, row, ncol, bzero, As, Bs, lo); break;
  }
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < BK; kk += 32) {
    half8_t af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const half8_t*>(As + lo.a_rd[kk / 32] + i * 16 * kLdsRow);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const half8_t*>(Bs + lo.b_rd[kk / 32] + j * 16 * kLdsRow);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
  }
  __syncthreads();
}

template <bool kTL, bool kZeros>
__global__ __launch_bounds__(kThreads, 4) void gemm_lds_kernel(LdsGemmArgs a) {
  __shared__ __align__(16) uint16_t As[BM * kLdsRow];
  __shared__ __align__(16) uint16_t Bs[BN * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;   // 2 x 2 waves of 64 x 64
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int nblk = a.K / kBlockRows;

  Rsrc rs;
  rs.x = __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, 0, a.xq_bytes, kRsrcWord3);
  rs.w = __builtin_amdgcn_make_buffer_rsrc((void*)a.qweight, 0, a.qweight_bytes, kRsrcWord3);
  rs.s = __builtin_amdgcn_make_buffer_rsrc((void*)a.scales, 0, a.scale_bytes, kRsrcWord3);
  rs.z = __builtin_amdgcn_make_buffer_rsrc(kZeros ? (void*)a.zeros : (void*)a.scales, 0,
                                           kZeros ? a.zero_bytes : a.scale_bytes, kRsrcWord3);

  // B work item of this thread: block bsub of each step (the same for a
  // whole wave), column tid % 128 of the tile.
  const int bsub = tid / BN;
  const int ncol = n0 + tid % BN;
  const int nc = min(ncol, a.N - 1);
  LaneOffsets off;
#pragma unroll
  for (int i = 0; i < kAPieces; ++i) {
    const int lin = tid + i * kThreads;
    const int m = min(m0 + lin / (BK / 8), a.M - 1);
    off.a[i] = ((uint32_t)m * (uint32_t)a.K + (uint32_t)(lin % (BK / 8)) * 8) * 2;
  }
  off.w = (uint32_t)word_index(a.runs.packed_rows, 0, nc) * 4;
  off.s = kTL ? (uint32_t)(nc / 8) * 4 : (uint32_t)nc * 2;
  off.z = (uint32_t)nc;
  LdsOffsets lo;
  lo.a_st = lds_at(tid / (BK / 8), tid % (BK / 8));
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) lo.b_st[q4] = lds_at(tid % BN, bsub * (kBlockRows / 8) + q4);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    lo.a_rd[h] = lds_at(wr * 64 + (lane & 15), h * 4 + (lane >> 4));
    lo.b_rd[h] = lds_at(wc * 64 + (lane & 15), h * 4 + (lane >> 4));
  }

  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = {0.f, 0.f, 0.f, 0.f};

  // The blocks of this workgroup's K slice (all of K without split); slices
  // start at even blocks, so only the last can end in the odd-block tail.
  const int kb_begin = a.part ? (int)blockIdx.z * a.slice_blocks : 0;
  const int kb_end = a.part ? min(nblk, kb_begin + a.slice_blocks) : nblk;
  RunCursor cur{0, 0, a.runs.run_row[0], a.runs.run_bits[0], a.runs.run_block[1]};
  const int nfull = kb_begin + ((kb_end - kb_begin) & ~1);   // steps whose two blocks are both inside K
  for (int kb = kb_begin; kb < nfull; kb += BK / kBlockRows)
    k_step<kTL, kZeros, false>(a, rs, cur, off, lo, tid, bsub, kb, nblk, ncol, As, Bs, acc);
  if (nfull < kb_end) k_step<kTL, kZeros, true>(a, rs, cur, off, lo, tid, bsub, nfull, nblk, ncol, As, Bs, acc);

  // Epilogue: lane holds C[4*(lane/16) + r][lane % 16] of each 16 x 16 tile.
  float* const part = a.part ? a.part + (size_t)blockIdx.z * a.M * a.N : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wc * 64 + j * 16 + (lane & 15);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wr * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (m >= a.M) continue;
        if (part)
          part[(size_t)m * a.N + n] = acc[i][j][r];
        else
          a.y[(size_t)m * a.N + n] = __builtin_bit_cast(uint16_t, (_Float16)apply_epilogue(a.epi, acc[i][j][r], m, n, a.N));
      }
    }
  }
}

// The slices' partial sums added in slice order (the same order on every
// call), then the epilogue and the float16 rounding: 4 consecutive outputs
// per thread (N is a multiple of 8, so they share a row).
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int slices, int M, int N,
                                                        uint16_t* __restrict__ y, Epilogue epi) {
  const size_t total = (size_t)M * N;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= total) return;
  float4_t v = *reinterpret_cast<const float4_t*>(part + i);
  for (int s = 1; s < slices; ++s) {
    const float4_t w = *reinterpret_cast<const float4_t*>(part + (size_t)s * total + i);
    v = v + w;
  }
  const int m = (int)(i / N), n = (int)(i % N);
  uint16_t h[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) h[c] = __builtin_bit_cast(uint16_t, (_Float16)apply_epilogue(epi, v[c], m, n + c, N));
  uint2 o;
  o.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
  o.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
  *reinterpret_cast<uint2*>(y + i) = o;
}

}  // namespace

hipError_t launch_qgemm_lds(const qlinear_layout& L, const Runs& runs, const uint16_t* xq, int M,
                            const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros, uint16_t* y,
                            const Epilogue& epi, int slices, float* part, hipStream_t stream) {
  LdsGemmArgs a;
  a.xq = xq;
  a.qweight = qweight;
  a.scales = scales;
  a.zeros = zeros;
  a.y = y;
  a.M = M;
  a.K = L.K;
  a.N = L.N;
  // Byte sizes for the buffer resources: the caller keeps the activations of
  // a call below 2^31 bytes, and qgemm_supported the weights and scales.
  const bool tl = epi.scale_max != nullptr;
  a.xq_bytes = (int)((size_t)M * L.K * 2);
  a.qweight_bytes = (int)((size_t)L.packed_words * 4);
  a.scale_bytes = (int)(tl ? (size_t)L.groups * (L.N / 8) * 4 : (size_t)L.groups * L.N * 2);
  a.zero_bytes = (int)((size_t)L.groups * L.N);
  a.runs = runs;
  a.epi = epi;
  // Slices of an even number of blocks, as equal as that allows.
  const int nblk = L.K / kBlockRows;
  const int steps = (nblk + 1) / 2;
  slices = slices > 1 && part ? std::min(slices, steps) : 1;
  a.slice_blocks = 2 * ((steps + slices - 1) / slices);
  slices = (nblk + a.slice_blocks - 1) / a.slice_blocks;
  a.part = slices > 1 ? part : nullptr;
  const dim3 grid((L.N + BN - 1) / BN, (M + BM - 1) / BM, slices);
  if (tl) {
    if (zeros)
      hipLaunchKernelGGL((gemm_lds_kernel<true, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_lds_kernel<true, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (zeros)
      hipLaunchKernelGGL((gemm_lds_kernel<false, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_lds_kernel<false, false>), grid, dim3(kThreads), 0, stream, a);
  }
  if (a.part) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t quads = ((size_t)M * L.N) / 4;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream, a.part, slices, M,
                       L.N, y, epi);
  }
  return hipGetLastError();
}

}  // namespace qlinear
