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
                              const uint8_t* __restrict__ zeros, uint16_t* __restrict__ wout, int N, int R,
                              int blk, int row, int g, int n) {
  uint32_t w[B], pr[kPairsPerBlock];
  load_block<B>(qweight, R, row, n, w);
  extract_all_pairs<B>(w, pr);
  const uint16_t sbits = scales[(size_t)g * N + n];
  const int z = zeros ? (int)zeros[(size_t)g * N + n] : (1 << (B - 1));
  const _Float16 s = __builtin_bit_cast(_Float16, sbits);
  const _Float16 nb = (_Float16)(-(1024 + z));
  const half2_t scale = {s, s}, neg_bias = {nb, nb};
  uint16_t* dst = wout + (size_t)blk * kBlockRows * N + n;
#pragma unroll
  for (int p = 0; p < kPairsPerBlock; ++p) {
    const uint32_t v = as_u32(dequant_pair(pr[p], neg_bias, scale));
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
                                                              uint16_t* __restrict__ w, int N, Runs runs) {
  const int n = blockIdx.x * kColsPerCta + threadIdx.x;
  const int blk = blockIdx.y;
  if (n >= N) return;
  const int R = runs.packed_rows;
  int bits, row;
  block_info(runs, blk, bits, row);
  const int g = blk / runs.blocks_per_group;
  switch (bits) {
    case 2: dequant_block<2>(qweight, scales, zeros, w, N, R, blk, row, g, n); break;
    case 3: dequant_block<3>(qweight, scales, zeros, w, N, R, blk, row, g, n); break;
    case 4: dequant_block<4>(qweight, scales, zeros, w, N, R, blk, row, g, n); break;
    case 5: dequant_block<5>(qweight, scales, zeros, w, N, R, blk, row, g, n); break;
    case 6: dequant_block<6>(qweight, scales, zeros, w, N, R, blk, row, g, n); break;
    case 8: dequant_block<8>(qweight, scales, zeros, w, N, R, blk, row, g, n); break;
    default: break;
  }
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
                          const uint16_t* scales, const uint8_t* zeros, uint16_t* w, hipStream_t stream) {
  hipLaunchKernelGGL(dequant_kernel, matrix_grid(L), dim3(kColsPerCta), 0, stream, qweight, scales, zeros, w,
                     L.N, runs);
  return hipGetLastError();
}

}  // namespace qlinear
