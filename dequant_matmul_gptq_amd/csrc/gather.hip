// Act-order gather of the activations into unpacking pair order, for the
// decode and prefill paths.
//
//   xq[m][blk][p]  = (x[m][perm[32*blk + lo(p)]], x[m][perm[32*blk + hi(p)]])
//
// (for the MFMA kernels, position p holds pair mfma_pair(b, p) instead)
//   xsum[m][blk]   = (sum of the block's 32 values, 1024 * sum of the
//                     scaled values) (optional, decode path)
//
// In scaled mode (decode path) each pair is multiplied by 2^-e, e being the
// exponent at which the decode kernel unpacks that pair's codes.
// where (lo(p), hi(p)) are the rows that pair p of block blk unpacks to for
// that block's code width. Inside each 32-row block the K order is thus the
// order in which the weights come out of the packed words, so the weights
// never need to be reordered. One thread per (block, pair); the 16 pairs of a
// block are 16 consecutive lanes, which reduce the block sum with shuffles.
#include <algorithm>

#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

__global__ __launch_bounds__(256) void gather_pairs_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ perm,
                                                           uint32_t* __restrict__ xq, float2* __restrict__ xsum,
                                                           int M, int K, int scaled, int mfma, Runs runs) {
  // Every argument read in one scalar batch (the asm takes them and hands
  // them back, so none is read later behind another wait).
  // The first 8 runs' first blocks and widths are part of that batch: read
  // inside the run scan, each would be a round trip of its own (entries past
  // nruns lie inside the table and are ignored).
  int nruns = runs.nruns;
  int rb[8], rw[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    rb[r] = runs.run_block[r];
    rw[r] = runs.run_bits[r];
  }
  asm volatile("" : "+s"(M), "+s"(K), "+s"(scaled), "+s"(mfma), "+s"(nruns), "+s"(rb[1]), "+s"(rb[2]), "+s"(rb[3]),
               "+s"(rb[4]), "+s"(rb[5]), "+s"(rb[6]), "+s"(rb[7]), "+s"(rw[0]), "+s"(rw[1]), "+s"(rw[2]), "+s"(rw[3]),
               "+s"(rw[4]), "+s"(rw[5]), "+s"(rw[6]), "+s"(rw[7])
               : "s"(x), "s"(perm), "s"(xq), "s"(xsum));
  const int nblk = K / kBlockRows;
  const int pairs = nblk * kPairsPerBlock;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const bool live = idx < pairs;
  const int blk = live ? idx / kPairsPerBlock : 0, p = idx % kPairsPerBlock;
  // The width of block blk: that of the last run starting at or before it.
  int bits = rw[0];
#pragma unroll
  for (int r = 1; r < 8; ++r) bits = (r < nruns && blk >= rb[r]) ? rw[r] : bits;
  for (int r = 8; r < nruns; ++r) bits = blk >= runs.run_block[r] ? runs.run_bits[r] : bits;
  int lo, hi;
  pair_rows(bits, mfma ? mfma_pair(bits, p) : p, lo, hi);
  const int jlo = blk * kBlockRows + lo, jhi = blk * kBlockRows + hi;
  // perm entries are clamped into [0, K): a malformed perm cannot address outside x.
  const int flo = perm ? (int)min((unsigned)perm[jlo], (unsigned)(K - 1)) : jlo;
  const int fhi = perm ? (int)min((unsigned)perm[jhi], (unsigned)(K - 1)) : jhi;
  // Scaled mode: the pair is multiplied by 2^-e, the scale at which the decode
  // kernel unpacks its codes (exact unless the value becomes subnormal).
  const float sc = scaled ? __builtin_ldexpf(1.0f, -pair_exponent(bits, p)) : 1.0f;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t* xr = x + (size_t)m * K;
    const _Float16 vl = live ? __builtin_bit_cast(_Float16, xr[flo]) : (_Float16)0.0f;
    const _Float16 vh = live ? __builtin_bit_cast(_Float16, xr[fhi]) : (_Float16)0.0f;
    const _Float16 sl = (_Float16)((float)vl * sc), sh = (_Float16)((float)vh * sc);
    if (live)
      xq[(size_t)m * pairs + idx] = (uint32_t)__builtin_bit_cast(uint16_t, sl) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, sh) << 16);
    if (xsum) {
      // X = sum of the block's activations; Bsum = 1024 * sum of the scaled
      // activations, the bias the 1024 + q * 2^e pairs add to the dot products.
      float X = (float)vl + (float)vh;
      float Bs = (float)sl + (float)sh;
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {
        X += __shfl_xor(X, off, 16);
        Bs += __shfl_xor(Bs, off, 16);
      }
      if (live && p == 0) xsum[(size_t)m * nblk + blk] = make_float2(X, 1024.0f * Bs);
    }
  }
}

// Prefill variant (no scaling, no sums): a workgroup stages R whole rows of
// x in LDS with 16-byte loads. Each thread then takes quads of 4 consecutive
// pairs (one block, so one width lookup), looks their rows and perm entries
// up once for all R rows, and writes each row's quad as one 16-byte store:
// a wave writes 1 KiB of a row of xq, contiguous.
template <int kT>
__global__ __launch_bounds__(kT) void gather_rows_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                         uint32_t* __restrict__ xq, int M, int K, int R, int mfma,
                                                         int perm16, Runs runs) {
  extern __shared__ __align__(16) uint16_t xs[];   // R rows of K float16
  // Loads per thread in flight in the staging loop, quads in the gather loop.
  constexpr int kBatch = 8, kQuads = 2;
  const int m0 = blockIdx.x * R;
  const int rows = min(R, M - m0);
  const int n16 = K / 8;   // 16-byte pieces per row (K is a multiple of 32)
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)m0 * K);
  uint4* dst = reinterpret_cast<uint4*>(xs);
  const int total = rows * n16;
  for (int base = threadIdx.x; base < total; base += kT * kBatch) {
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = src[min(base + u * kT, total - 1)];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (base + u * kT < total) dst[base + u * kT] = v[u];
  }
  __syncthreads();
  const int pairs = (K / kBlockRows) * kPairsPerBlock;
  const int quads = pairs / 4;
  for (int base = threadIdx.x; base < quads; base += kT * kQuads) {
    int flo[kQuads][4], fhi[kQuads][4];
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int q = min(base + u * kT, quads - 1);
      const int blk = q / (kPairsPerBlock / 4), t = q % (kPairsPerBlock / 4);
      const int bits = block_bits_scan(runs, blk);
      const int row0 = blk * kBlockRows;
      if (perm16 && (bits == 2 || bits == 4 || bits == 8)) {
        // Both pair orders put the quad's rows in two aligned runs of 4: rows
        // 8t..8t+7 at 4 and 8 bits, 16(t/2) + 4(t%2) + 0..3 and + 8..11 at 2
        // bits. Two 16-byte perm loads instead of eight 4-byte ones.
        const int a0 = bits == 2 ? 16 * (t >> 1) + 4 * (t & 1) : 8 * t;
        const int a1 = bits == 2 ? a0 + 8 : a0 + 4;
        const int4 p0 = *reinterpret_cast<const int4*>(perm + row0 + a0);
        const int4 p1 = *reinterpret_cast<const int4*>(perm + row0 + a1);
        const auto c = [K](int v) { return (int)min((unsigned)v, (unsigned)(K - 1)); };
        if (bits == 8) {   // pair e: rows 8t + 4(e/2) + e%2 and that + 2
          flo[u][0] = c(p0.x), flo[u][1] = c(p0.y), flo[u][2] = c(p1.x), flo[u][3] = c(p1.y);
          fhi[u][0] = c(p0.z), fhi[u][1] = c(p0.w), fhi[u][2] = c(p1.z), fhi[u][3] = c(p1.w);
        } else {           // pair e: rows a0 + e and a1 + e
          flo[u][0] = c(p0.x), flo[u][1] = c(p0.y), flo[u][2] = c(p0.z), flo[u][3] = c(p0.w);
          fhi[u][0] = c(p1.x), fhi[u][1] = c(p1.y), fhi[u][2] = c(p1.z), fhi[u][3] = c(p1.w);
        }
        continue;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = t * 4 + e;
        int lo, hi;
        pair_rows(bits, mfma ? mfma_pair(bits, p) : p, lo, hi);
        const int jlo = row0 + lo, jhi = row0 + hi;
        // perm entries are clamped into [0, K): a malformed perm cannot address outside the row.
        flo[u][e] = perm ? (int)min((unsigned)perm[jlo], (unsigned)(K - 1)) : jlo;
        fhi[u][e] = perm ? (int)min((unsigned)perm[jhi], (unsigned)(K - 1)) : jhi;
      }
    }
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int q = base + u * kT;
      if (q < quads)
        for (int r = 0; r < rows; ++r) {
          const uint16_t* xr = xs + r * K;
          uint4 o;
          o.x = (uint32_t)xr[flo[u][0]] | ((uint32_t)xr[fhi[u][0]] << 16);
          o.y = (uint32_t)xr[flo[u][1]] | ((uint32_t)xr[fhi[u][1]] << 16);
          o.z = (uint32_t)xr[flo[u][2]] | ((uint32_t)xr[fhi[u][2]] << 16);
          o.w = (uint32_t)xr[flo[u][3]] | ((uint32_t)xr[fhi[u][3]] << 16);
          reinterpret_cast<uint4*>(xq + (size_t)(m0 + r) * pairs)[q] = o;
        }
    }
  }
}

}  // namespace

hipError_t launch_gather_rows(const Runs& runs, const uint16_t* x, const int32_t* perm, int M, int K,
                              uint32_t* xq, bool mfma, hipStream_t stream) {
  const size_t row_bytes = (size_t)K * 2;
  if (row_bytes > kGatherRowsLds) return launch_gather_pairs(runs, x, perm, M, K, xq, nullptr, false, mfma, stream);
  // Up to 4 rows per workgroup within 32 KiB; 2 rows within 64 KiB where
  // 32 KiB holds only one (K = 13824 at M = 2048, measured with 4-byte perm
  // loads: 47 us instead of 55-74 us with one row); at least one row.
  const size_t r32 = std::min<size_t>(4, (size_t)32768 / row_bytes), r64 = std::min<size_t>(2, kGatherRowsLds / row_bytes);
  const int R = (int)std::max<size_t>(1, std::max(r32, r64));
  const int grid = (M + R - 1) / R;
  const size_t lds = (size_t)R * row_bytes;
  const int perm16 = perm != nullptr && ((uintptr_t)perm & 15) == 0;
  // Past 40 KiB of rows a CU holds at most 3 workgroups: 1024 threads each
  // keep enough loads in flight.
  if (lds > 40 * 1024)
    hipLaunchKernelGGL(gather_rows_kernel<1024>, dim3(grid), dim3(1024), lds, stream, x, perm, xq, M, K, R,
                       mfma ? 1 : 0, perm16, runs);
  else
    hipLaunchKernelGGL(gather_rows_kernel<256>, dim3(grid), dim3(256), lds, stream, x, perm, xq, M, K, R,
                       mfma ? 1 : 0, perm16, runs);
  return hipGetLastError();
}

hipError_t launch_gather_pairs(const Runs& runs, const uint16_t* x, const int32_t* perm, int M, int K,
                               uint32_t* xq, float2* xsum, bool scaled, bool mfma, hipStream_t stream) {
  const int pairs = (K / kBlockRows) * kPairsPerBlock;
  const int gy = M < 65535 ? M : 65535;
  hipLaunchKernelGGL(gather_pairs_kernel, dim3((pairs + 255) / 256, gy, 1), dim3(256), 0, stream, x, perm, xq,
                     xsum, M, K, scaled ? 1 : 0, mfma ? 1 : 0, runs);
  return hipGetLastError();
}

}  // namespace qlinear
