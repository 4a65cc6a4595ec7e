// Packing, unpacking and float16 dequantization of whole matrices.
// One thread per (32-row block, output column); consecutive threads take
// consecutive columns so every row of codes and of packed words is read and
// written with coalesced accesses.
#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

constexpr int kColsPerCta = 256;

// n may lie past N, in the padding slots of the last panel: those words are 0.
template <int B>
__device__ void pack_block(const uint8_t* __restrict__ q, uint32_t* __restrict__ qweight, int N, int R,
                           int blk, int row, int n) {
  uint32_t w[B];
#pragma unroll
  for (int t = 0; t < B; ++t) w[t] = 0u;
  if (n < N) {
    const uint8_t* src = q + (size_t)blk * kBlockRows * N + n;
#pragma unroll
    for (int r = 0; r < kBlockRows; ++r) place_code<B>(w, r, src[(size_t)r * N]);
  }
#pragma unroll
  for (int t = 0; t < B; ++t) qweight[word_index(R, row + t, n)] = w[t];
}

template <int B>
__device__ void load_block(const uint32_t* __restrict__ qweight, int R, int row, int n, uint32_t* w) {
#pragma unroll
  for (int t = 0; t < B; ++t) w[t] = qweight[word_index(R, row + t, n)];
}

template <int B>
__device__ void unpack_block(const uint32_t* __restrict__ qweight, uint8_t* __restrict__ q, int N, int R,
                             int blk, int row, int n) {
  uint32_t w[B], pr[kPairsPerBlock];
  load_block<B>(qweight, R, row, n, w);
  extract_all_pairs<B>(w, pr);
  uint8_t* dst = q + (size_t)blk * kBlockRows * N + n;
#pragma unroll
  for (int p = 0; p < kPairsPerBlock; ++p) {
    int lo, hi;
    pair_rows(B, p, lo, hi);
    dst[(size_t)lo * N] = (uint8_t)(pr[p] & 0x3FFu);
    dst[(size_t)hi * N] = (uint8_t)((pr[p] >> 16) & 0x3FFu);
  }
}

template <int B>
__device__ void dequant_block(const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
                              const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ scale_max,
                              uint16_t* __restrict__ wout, int N, int R, int blk, int row, int g, int n) {
  uint32_t w[B], pr[kPairsPerBlock];
  load_block<B>(qweight, R, row, n, w);
  extract_all_pairs<B>(w, pr);
  const int z = zeros ? (int)zeros[(size_t)g * N + n] : (1 << (B - 1));
  // Two-level scales: d = (q - z) (c + 1) is an integer of at most 2048 in
  // magnitude (symmetric groups), exact in float16; d * scale_max / 16 is
  // exact in float32 (at most 22 significant bits) and rounded once.
  float post = 1.0f;
  _Float16 s;
  if (scale_max) {
    s = (_Float16)qscale_factor(reinterpret_cast<const uint32_t*>(scales)[(size_t)g * (N / 8) + n / 8], n);
    post = (float)__builtin_bit_cast(_Float16, scale_max[n]) * 0.0625f;
  } else {
    s = __builtin_bit_cast(_Float16, scales[(size_t)g * N + n]);
  }
  const _Float16 nb = (_Float16)(-(1024 + z));
  const half2_t scale = {s, s}, neg_bias = {nb, nb};
  uint16_t* dst = wout + (size_t)blk * kBlockRows * N + n;
#pragma unroll
  for (int p = 0; p < kPairsPerBlock; ++p) {
    uint32_t v = as_u32(dequant_pair(pr[p], neg_bias, scale));
    if (scale_max) {
      const _Float16 lo16 = (_Float16)((float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu)) * post);
      const _Float16 hi16 = (_Float16)((float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)) * post);
      v = (uint32_t)__builtin_bit_cast(uint16_t, lo16) | ((uint32_t)__builtin_bit_cast(uint16_t, hi16) << 16);
    }
    int lo, hi;
    pair_rows(B, p, lo, hi);
    dst[(size_t)lo * N] = (uint16_t)(v & 0xFFFFu);
    dst[(size_t)hi * N] = (uint16_t)(v >> 16);
  }
}

__global__ __launch_bounds__(kColsPerCta) void pack_kernel(const uint8_t* __restrict__ q,
                                                           uint32_t* __restrict__ qweight, int N,
                                                           Runs runs) {
  const int n = blockIdx.x * kColsPerCta + threadIdx.x;
  const int blk = blockIdx.y;
  if (n >= (N + kPanel - 1) / kPanel * kPanel) return;
  const int R = runs.packed_rows;
  int bits, row;
  block_info(runs, blk, bits, row);
  switch (bits) {
    case 2: pack_block<2>(q, qweight, N, R, blk, row, n); break;
    case 3: pack_block<3>(q, qweight, N, R, blk, row, n); break;
    case 4: pack_block<4>(q, qweight, N, R, blk, row, n); break;
    case 5: pack_block<5>(q, qweight, N, R, blk, row, n); break;
    case 6: pack_block<6>(q, qweight, N, R, blk, row, n); break;
    case 8: pack_block<8>(q, qweight, N, R, blk, row, n); break;
    default: break;
  }
}

__global__ __launch_bounds__(kColsPerCta) void unpack_kernel(const uint32_t* __restrict__ qweight,
                                                             uint8_t* __restrict__ q, int N, Runs runs) {
  const int n = blockIdx.x * kColsPerCta + threadIdx.x;
  const int blk = blockIdx.y;
  if (n >= N) return;
  const int R = runs.packed_rows;
  int bits, row;
  block_info(runs, blk, bits, row);
  switch (bits) {
    case 2: unpack_block<2>(qweight, q, N, R, blk, row, n); break;
    case 3: unpack_block<3>(qweight, q, N, R, blk, row, n); break;
    case 4: unpack_block<4>(qweight, q, N, R, blk, row, n); break;
    case 5: unpack_block<5>(qweight, q, N, R, blk, row, n); break;
    case 6: unpack_block<6>(qweight, q, N, R, blk, row, n); break;
    case 8: unpack_block<8>(qweight, q, N, R, blk, row, n); break;
    default: break;
  }
}

__global__ __launch_bounds__(kColsPerCta) void dequant_kernel(const uint32_t* __restrict__ qweight,
                                                              const uint16_t* __restrict__ scales,
                                                              const uint8_t* __restrict__ zeros,
                                                              const uint16_t* __restrict__ scale_max,
                                                              uint16_t* __restrict__ w, int N, Runs runs) {
  const int n = blockIdx.x * kColsPerCta + threadIdx.x;
  const int blk = blockIdx.y;
  if (n >= N) return;
  const int R = runs.packed_rows;
  int bits, row;
  block_info(runs, blk, bits, row);
  const int g = blk / runs.blocks_per_group;
  switch (bits) {
    case 2: dequant_block<2>(qweight, scales, zeros, scale_max, w, N, R, blk, row, g, n); break;
    case 3: dequant_block<3>(qweight, scales, zeros, scale_max, w, N, R, blk, row, g, n); break;
    case 4: dequant_block<4>(qweight, scales, zeros, scale_max, w, N, R, blk, row, g, n); break;
    case 5: dequant_block<5>(qweight, scales, zeros, scale_max, w, N, R, blk, row, g, n); break;
    case 6: dequant_block<6>(qweight, scales, zeros, scale_max, w, N, R, blk, row, g, n); break;
    case 8: dequant_block<8>(qweight, scales, zeros, scale_max, w, N, R, blk, row, g, n); break;
    default: break;
  }
}

// q_scale words from 4-bit scale codes: word i of group row g packs the
// codes of columns 8 i .. 8 i + 7, column 8 i + k at bits 4 k (codes are
// taken modulo 16).
__global__ __launch_bounds__(256) void pack_qscale_kernel(const uint8_t* __restrict__ codes,
                                                          uint32_t* __restrict__ words, int64_t nwords) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nwords) return;
  const uint8_t* src = codes + i * 8;   // the codes of a group row are contiguous, as are the rows
  uint32_t v = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) v |= ((uint32_t)src[k] & 15u) << (4 * k);
  words[i] = v;
}

dim3 matrix_grid(const qlinear_layout& L) {
  const int n16 = (L.N + kPanel - 1) / kPanel * kPanel;   // padded columns are packed as zeros
  return dim3((unsigned)((n16 + kColsPerCta - 1) / kColsPerCta), (unsigned)(L.K / kBlockRows), 1);
}

}  // namespace

hipError_t launch_pack(const qlinear_layout& L, const Runs& runs, const uint8_t* q, uint32_t* qweight,
                       hipStream_t stream) {
  hipLaunchKernelGGL(pack_kernel, matrix_grid(L), dim3(kColsPerCta), 0, stream, q, qweight, L.N, runs);
  return hipGetLastError();
}

hipError_t launch_unpack(const qlinear_layout& L, const Runs& runs, const uint32_t* qweight, uint8_t* q,
                         hipStream_t stream) {
  hipLaunchKernelGGL(unpack_kernel, matrix_grid(L), dim3(kColsPerCta), 0, stream, qweight, q, L.N, runs);
  return hipGetLastError();
}

hipError_t launch_dequant(const qlinear_layout& L, const Runs& runs, const uint32_t* qweight,
                          const uint16_t* scales, const uint8_t* zeros, const uint16_t* scale_max, uint16_t* w,
                          hipStream_t stream) {
  hipLaunchKernelGGL(dequant_kernel, matrix_grid(L), dim3(kColsPerCta), 0, stream, qweight, scales, zeros,
                     scale_max, w, L.N, runs);
  return hipGetLastError();
}

hipError_t launch_pack_qscale(const uint8_t* codes, int64_t groups, int64_t N, uint32_t* words,
                              hipStream_t stream) {
  const int64_t nwords = groups * (N / 8);
  if (nwords == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_qscale_kernel, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, stream, codes,
                     words, nwords);
  return hipGetLastError();
}

}  // namespace qlinear
