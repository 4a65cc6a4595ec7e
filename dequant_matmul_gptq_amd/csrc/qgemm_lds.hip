// Prefill kernel for matrices with several code widths (EXL2): a 128 x 128
// tile per workgroup of 4 waves (64 x 64 each). Per K-step of 64 rows (two
// 32-row blocks) the activation tile is copied to LDS and the weight tile is
// unpacked and dequantized exactly to float16 in LDS (each block with its own
// width; w = RNE(s * (q - z)), one rounding), then v_mfma_f32_16x16x32_f16
// accumulates in float32. The activations were gathered by act-order into
// unpacking pair order beforehand, as for the single-width kernel.
#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kPad = 8;                 // halves of padding per LDS row
constexpr int kLdsRow = BK + kPad;      // 72 halves = 144 bytes

struct LdsGemmArgs {
  const uint16_t* xq;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint8_t* zeros;
  uint16_t* y;
  int M, K, N;
  Runs runs;
  Epilogue epi;
};

// Unpack + dequantize one (block, column) into 16 float16 pairs in LDS.
template <int B>
__device__ __forceinline__ void dequant_to_lds(const LdsGemmArgs& a, int row, int g, int n, bool valid,
                                               uint32_t* dst /* 16 words */) {
  uint32_t w[B];
#pragma unroll
  for (int t = 0; t < B; ++t) w[t] = valid ? a.qweight[word_index(a.runs.packed_rows, row + t, n)] : 0u;
  _Float16 s = (_Float16)0.0f;
  int z = 1 << (B - 1);
  if (valid) {
    // Two-level scales: the group factor c + 1, exact in float16, so that
    // s * (q - z) stays an exact integer; scale_max / 16 comes in the epilogue.
    if (a.epi.scale_max)
      s = (_Float16)qscale_factor(reinterpret_cast<const uint32_t*>(a.scales)[(size_t)g * (a.N / 8) + n / 8], n);
    else
      s = __builtin_bit_cast(_Float16, a.scales[(size_t)g * a.N + n]);
    if (a.zeros) z = a.zeros[(size_t)g * a.N + n];
  }
  const _Float16 nb = (_Float16)(-(1024 + z));
  const half2_t scale = {s, s}, neg_bias = {nb, nb};
  uint32_t pr[kPairsPerBlock];
  extract_all_pairs<B>(w, pr);
#pragma unroll
  for (int q4 = 0; q4 < kPairsPerBlock / 4; ++q4) {
    uint4 v;
    v.x = as_u32(dequant_pair(pr[4 * q4 + 0], neg_bias, scale));
    v.y = as_u32(dequant_pair(pr[4 * q4 + 1], neg_bias, scale));
    v.z = as_u32(dequant_pair(pr[4 * q4 + 2], neg_bias, scale));
    v.w = as_u32(dequant_pair(pr[4 * q4 + 3], neg_bias, scale));
    *reinterpret_cast<uint4*>(dst + 4 * q4) = v;
  }
}

__global__ __launch_bounds__(kThreads) void gemm_lds_kernel(LdsGemmArgs a) {
  __shared__ __align__(16) uint16_t As[BM * kLdsRow];
  __shared__ __align__(16) uint16_t Bs[BN * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;   // 2 x 2 waves of 64 x 64
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int nblk = a.K / kBlockRows;

  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = {0.f, 0.f, 0.f, 0.f};

  // B-tile work item of this thread: block (tid / 128) of the step, column tid % 128.
  const int bsub = tid / BN;
  const int bn = tid % BN;
  const int ncol = n0 + bn;
  const bool nvalid = ncol < a.N;

  for (int kb = 0; kb < nblk; kb += BK / kBlockRows) {
    // A tile: 128 rows x 64 halves, 16 bytes per thread per pass.
#pragma unroll
    for (int i = 0; i < (BM * BK / 8) / kThreads; ++i) {
      const int lin = tid + i * kThreads;
      const int r = lin / (BK / 8), ch = lin % (BK / 8);
      const int m = m0 + r;
      const int k = kb * kBlockRows + ch * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < a.M && k < a.K) v = *reinterpret_cast<const uint4*>(a.xq + (size_t)m * a.K + k);
      *reinterpret_cast<uint4*>(As + r * kLdsRow + ch * 8) = v;
    }
    // B tile: dequantize block kb + bsub for column ncol.
    {
      const int blk = kb + bsub;
      uint32_t* dst = reinterpret_cast<uint32_t*>(Bs + bn * kLdsRow + bsub * kBlockRows);
      if (blk < nblk) {
        int bits, row;
        block_info(a.runs, blk, bits, row);
        const int g = blk / a.runs.blocks_per_group;
        switch (bits) {
          case 2: dequant_to_lds<2>(a, row, g, ncol, nvalid, dst); break;
          case 3: dequant_to_lds<3>(a, row, g, ncol, nvalid, dst); break;
          case 4: dequant_to_lds<4>(a, row, g, ncol, nvalid, dst); break;
          case 5: dequant_to_lds<5>(a, row, g, ncol, nvalid, dst); break;
          case 6: dequant_to_lds<6>(a, row, g, ncol, nvalid, dst); break;
          case 8: dequant_to_lds<8>(a, row, g, ncol, nvalid, dst); break;
          default: break;
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) *reinterpret_cast<uint4*>(dst + 4 * q4) = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      half8_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(As + (wr * 64 + i * 16 + (lane & 15)) * kLdsRow + kk +
                                                  8 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(Bs + (wc * 64 + j * 16 + (lane & 15)) * kLdsRow + kk +
                                                  8 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // Epilogue: lane holds C[4*(lane/16) + r][lane % 16] of each 16 x 16 tile.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wc * 64 + j * 16 + (lane & 15);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wr * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (m < a.M)
          a.y[(size_t)m * a.N + n] = __builtin_bit_cast(uint16_t, (_Float16)apply_epilogue(a.epi, acc[i][j][r], m, n, a.N));
      }
    }
  }
}

}  // namespace

hipError_t launch_qgemm_lds(const qlinear_layout& L, const Runs& runs, const uint16_t* xq, int M,
                            const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros, uint16_t* y,
                            const Epilogue& epi, hipStream_t stream) {
  LdsGemmArgs a;
  a.xq = xq;
  a.qweight = qweight;
  a.scales = scales;
  a.zeros = zeros;
  a.y = y;
  a.M = M;
  a.K = L.K;
  a.N = L.N;
  a.runs = runs;
  a.epi = epi;
  const int gmy = (M + BM - 1) / BM;
  hipLaunchKernelGGL(gemm_lds_kernel, dim3((L.N + BN - 1) / BN, gmy, 1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlinear
