// Host side of the matrix-core decode kernel (qgemv_mx.hpp): the launch
// shape and mode, and the gather kernel of the two-launch mode.
#include <string.h>
#include <algorithm>

#include "qgemv_mx.hpp"

namespace qlinear {

namespace mxk {

// Two-launch mode: the gather kernel. Thread = (block, k-group, row); the
// fragments of all 16 rows go to the workspace (rows past M as zeros, which
// the MFMA lanes of those rows read).
__global__ __launch_bounds__(256) void gather_mx_kernel(const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ perm, uint16_t* __restrict__ xg,
                                                        int M, int K, Runs runs) {
  const int nblk = K / kBlockRows;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= nblk * 4 * 16) return;
  const int m = t & 15, blk = t >> 6, gg = (t >> 4) & 3;
  u32x4* dst = reinterpret_cast<u32x4*>(xg + ((size_t)blk * 16 + m) * 32 + gg * 8);
  if (m >= M) {
    *dst = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  with_width<stream::kAllBits>(width_of(runs, blk), [&](auto Bc) {
    constexpr int Bw = decltype(Bc)::value;
    gather_frag<Bw, 1>(
        frag_rows<Bw>(gg), blk, 1,
        [&](int j) { return perm ? (int)min((unsigned)perm[j], (unsigned)(K - 1)) : j; },
        [&](int, int f) { return __builtin_bit_cast(_Float16, x[(size_t)m * K + f]); },
        [&](int, u32x4 v) { *dst = v; });
  });
}

}  // namespace mxk

// Fragment rows stored per block in the one-launch modes: 4 up to 4 rows
// (the LDS that leaves for x and perm), else 8.
static int mx_rows_per_block(int M) { return M <= 4 ? 4 : 8; }

// Bytes of LDS of the one-launch modes: x rows, perm and fragments (the
// first two rounded up to whole 1 KiB pieces of the staging loads); at
// least the partial tiles of the final reduction.
static size_t mx_lds_bytes(int M, int K, bool perm, int FN, int& off_perm, int& off_xg) {
  const int MS = mx_rows_per_block(M);
  const int nblk = K / kBlockRows;
  const size_t xb = ((size_t)M * K * 2 + 1023) / 1024 * 1024;
  const size_t pb = perm ? ((size_t)K * 4 + 1023) / 1024 * 1024 : 0;
  const size_t red = sizeof(mxk::Red<4>) / 4 * FN;
  off_perm = (int)xb;
  off_xg = (int)(xb + pb);
  const size_t total = (size_t)off_xg + (size_t)nblk * MS * 64;
  return total > red ? total : red;
}

// LDS a one-launch workgroup may take, and the CUs that share the grid.
constexpr size_t kMxLdsBudget = 160 * 1024;
constexpr int kMxCus = 256;

// When one launch beats the gather kernel + this kernel (measured on MI355X,
// us at M = 3 / 4 unless noted, weights from HBM, one launch vs two):
// - one code width, 5..8 rows: 7B 4096 -> 4096 at M = 5 / 8 9.25 / 9.37 vs
//   11.67 / 11.50, 4096 -> 11008 12.08 / 12.84 vs 13.71 / 13.88;
// - widths 2-3 (EXL2 2.5 bpw, two runs): 4096^2 9.83 / 9.54 vs 12.33 / 12.37,
//   5120^2 12.78 / 12.88 vs 15.07 / 14.47, 8192^2 17.14 / 17.16 vs 18.48 /
//   18.09, 4096 -> 11008 15.47 / 15.25 vs 16.27 / 15.74, but 8192 -> 28672
//   47.69 / 48.13 vs 44.57 / 43.86 (every workgroup gathers its x rows run by
//   run: too many workgroups);
// - widths 3-6 (EXL2 4.0 bpw, four runs): 2048 -> 8192 12.27 / 12.30 vs 13.01
//   / 12.48, 4096^2 12.79 / 12.89 vs 13.48 / 12.44, but 5120^2 17.05 / 17.26
//   vs 16.09 / 15.79, 8192^2 23.97 / 23.95 vs 23.02 / 22.61, 4096 -> 11008
//   19.70 / 19.75 vs 18.93 / 18.49 (21.49 vs 18.54 at M = 8).
bool qgemv_mx_one_launch(const qlinear_layout& L, int M, bool perm) {
  int a, b;
  unsigned set = 0;
  for (int r = 0; r < L.nruns; ++r) set |= 1u << L.run_bits[r];
  bool fast;
  if ((set & (set - 1)) == 0)
    fast = M <= 8;
  else if ((set & ~stream::kLowBits) == 0)
    fast = M <= 4 && (int64_t)L.nruns * L.N <= 32768;
  else
    fast = M <= 4 && (int64_t)L.K * L.N <= (int64_t)4096 * 4096;
  return fast && mx_lds_bytes(M, L.K, perm, 4, a, b) <= kMxLdsBudget;
}

bool qgemv_mx_supported(const qlinear_layout& L) {
  // Buffer offsets and sizes are 32-bit: the scales, and the packed words of
  // a strip of 4 panels, must stay below 2^31 bytes (the weights are
  // addressed per strip).
  const size_t lim = (size_t)1 << 31;
  return (size_t)L.groups * L.N * 2 < lim && (size_t)4 * L.packed_rows * kPanel * 4 < lim &&
         qgemv_mx_workspace_bytes(L.K) < lim;
}

size_t qgemv_mx_workspace_bytes(int K) { return ((size_t)(K / kBlockRows) * 16 * 64 + 255) / 256 * 256; }

hipError_t launch_qgemv_mx(const qlinear_layout& L, const Runs& runs, const uint16_t* x, int M,
                           const int32_t* perm, int mats, const uint32_t* const* qweights,
                           const uint16_t* const* scales, const uint8_t* const* zeros, uint16_t* const* ys,
                           void* ws, const Epilogue& epi, hipStream_t stream) {
  mxk::MxArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.perm = perm;
  a.mats = mats;
  a.has_zeros = zeros != nullptr && zeros[0] != nullptr;
  for (int i = 0; i < mxk::kMaxMats; ++i) {
    const int j = i < mats ? i : 0;   // unused entries repeat matrix 0
    a.mat[i].qweight = qweights[j];
    a.mat[i].scales = scales[j];
    a.mat[i].zeros = a.has_zeros ? zeros[j] : nullptr;
    a.mat[i].y = ys[j];
  }
  a.M = M;
  a.K = L.K;
  a.N = L.N;
  const int bpg = L.group_size / kBlockRows;
  a.bpg_shift = bpg == 4 ? 2 : bpg == 2 ? 1 : 0;
  a.packed_rows = L.packed_rows;
  a.packed_words = L.packed_words;
  a.two_level = epi.scale_max != nullptr;
  a.scale_row_bytes = a.two_level ? L.N / 2 : L.N * 2;
  a.scale_bytes = (int)((size_t)L.groups * a.scale_row_bytes);
  a.runs = runs;
  a.epi = epi;
  unsigned set = 0;
  for (int r = 0; r < L.nruns; ++r) set |= 1u << L.run_bits[r];
  // Scale units of 4 blocks for 4-bit codes in 128-row groups, else one block.
  const int ub = (set == mxk::kSet4 && bpg == 4) ? 4 : 1;
  // Each wave takes a contiguous range of whole groups; its first segment
  // is the part of the run holding its first block.
  for (int w = 0; w < mxk::kWaves; ++w) {
    const int g0 = (int)((int64_t)w * L.groups / mxk::kWaves), g1 = (int)((int64_t)(w + 1) * L.groups / mxk::kWaves);
    const int b0 = g0 * bpg, b1 = g1 * bpg;
    int r = 0;
    while (r + 1 < L.nruns && b0 >= runs.run_block[r + 1]) ++r;
    a.wave_b0[w] = b0;
    a.wave_b1[w] = b1;
    a.wave_send[w] = b1 < runs.run_block[r + 1] ? b1 : runs.run_block[r + 1];
    a.wave_bits0[w] = runs.run_bits[r];
    a.wave_row0[w] = runs.run_row[r] + (b0 - runs.run_block[r]) * runs.run_bits[r];
  }

  // Columns per lane (measured on MI355X at 1-16 rows: wider loads win while
  // the grid keeps at least ~160 workgroups of 4 columns per lane, else 2
  // columns with >= 256 workgroups, else 1).
  const auto strips = [&](int fn) { return mats * ((L.N + kPanel * fn - 1) / (kPanel * fn)); };
  int fn = strips(4) >= 160 ? 4 : strips(2) >= 256 ? 2 : 1;

  int mode;
  size_t lds = 0;
  const bool all = (set & ~stream::kMidBits) != 0 && (set & ~stream::kLowBits) != 0 && set != mxk::kSet4;
  if (!all && qgemv_mx_one_launch(L, M, perm != nullptr)) {
    mode = mxk::kFewRows;
    // The staged rows can leave room for only one workgroup per CU: then
    // take wider strips while that saves a round of workgroups (measured on
    // MI355X, us: 5120^2 at M = 5 / 6 10.43 / 10.81 with 160 workgroups of 2
    // columns per lane against 18.18 / 19.10 with 320 of 1; EXL2 4.0 bpw
    // 5120^2 at M = 3 17.07 against 23.66).
    const int per_round = kMxCus * (int)std::max<size_t>(1, kMxLdsBudget / mx_lds_bytes(M, L.K, perm != nullptr, fn, a.lds_perm, a.lds_xg));
    const auto rounds = [&](int f) { return (strips(f) + per_round - 1) / per_round; };
    while (fn < 4 && rounds(2 * fn) < rounds(fn)) fn *= 2;
    lds = mx_lds_bytes(M, L.K, perm != nullptr, fn, a.lds_perm, a.lds_xg);
    a.ms = mx_rows_per_block(M);
  } else {
    // Two launches (the set of all widths, 8-bit runs mixed with others,
    // always runs this way: its one-launch instances are not built).
    mode = mxk::kGathered;
    uint16_t* xg = reinterpret_cast<uint16_t*>(ws);
    a.xg = xg;
    const int threads = L.K / kBlockRows * 4 * 16;
    hipLaunchKernelGGL(mxk::gather_mx_kernel, dim3((threads + 255) / 256), dim3(256), 0, stream, x, perm, xg, M, L.K,
                       runs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    lds = sizeof(mxk::Red<4>) / 4 * fn;
  }
  // B dequantized exactly when every block has a scale of its own (the
  // factored form's per-unit epilogue would run per block).
  const bool exact = ub == 1;
  if (exact) mode |= mxk::kExact;
  if (set == mxk::kSet4) {
    if (ub == 4) return mxk::launch_set4_ub4(a, fn, mode, lds, stream);
    return mxk::launch_set4_ub1(a, fn, mode, lds, stream);
  }
  if ((set & ~stream::kLowBits) == 0) return mxk::launch_low(a, fn, mode, lds, stream);
  if ((set & ~stream::kMidBits) == 0) {
    if (mxk::base_mode(mode) == mxk::kFewRows) return mxk::launch_mid_few(a, fn, mode, lds, stream);
    return mxk::launch_mid_gathered(a, fn, mode, lds, stream);
  }
  return mxk::launch_all(a, fn, exact, lds, stream);
}

}  // namespace qlinear
