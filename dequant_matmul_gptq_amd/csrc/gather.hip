// Act-order gather of the activations into unpacking pair order, shared by
// the decode and prefill paths.
//
//   xq[m][blk][p]  = (x[m][perm[32*blk + lo(p)]], x[m][perm[32*blk + hi(p)]])
//   xsum[m][blk]   = sum of the 32 gathered values of block blk (optional)
//
// where (lo(p), hi(p)) are the rows that pair p of block blk unpacks to for
// that block's code width. Inside each 32-row block the K order is thus the
// order in which the weights come out of the packed words, so the weights
// never need to be reordered. One thread per (block, pair); the 16 pairs of a
// block are 16 consecutive lanes, which reduce the block sum with shuffles.
#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

__global__ __launch_bounds__(256) void gather_pairs_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ perm,
                                                           uint32_t* __restrict__ xq, float* __restrict__ xsum,
                                                           int M, int K, Runs runs) {
  const int nblk = K / kBlockRows;
  const int pairs = nblk * kPairsPerBlock;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const bool live = idx < pairs;
  const int blk = live ? idx / kPairsPerBlock : 0, p = idx % kPairsPerBlock;
  int bits, row;
  block_info(runs, blk, bits, row);
  int lo, hi;
  pair_rows(bits, p, lo, hi);
  const int jlo = blk * kBlockRows + lo, jhi = blk * kBlockRows + hi;
  // perm entries are clamped into [0, K): a malformed perm cannot address outside x.
  const int flo = perm ? (int)min((unsigned)perm[jlo], (unsigned)(K - 1)) : jlo;
  const int fhi = perm ? (int)min((unsigned)perm[jhi], (unsigned)(K - 1)) : jhi;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t* xr = x + (size_t)m * K;
    const uint16_t vl = live ? xr[flo] : (uint16_t)0, vh = live ? xr[fhi] : (uint16_t)0;
    if (live) xq[(size_t)m * pairs + idx] = (uint32_t)vl | ((uint32_t)vh << 16);
    if (xsum) {
      float s = (float)__builtin_bit_cast(_Float16, vl) + (float)__builtin_bit_cast(_Float16, vh);
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off, 16);
      if (live && p == 0) xsum[(size_t)m * nblk + blk] = s;
    }
  }
}

}  // namespace

hipError_t launch_gather_pairs(const Runs& runs, const uint16_t* x, const int32_t* perm, int M, int K,
                               uint32_t* xq, float* xsum, hipStream_t stream) {
  const int pairs = (K / kBlockRows) * kPairsPerBlock;
  const int gy = M < 65535 ? M : 65535;
  hipLaunchKernelGGL(gather_pairs_kernel, dim3((pairs + 255) / 256, gy, 1), dim3(256), 0, stream, x, perm, xq,
                     xsum, M, K, runs);
  return hipGetLastError();
}

}  // namespace qlinear
