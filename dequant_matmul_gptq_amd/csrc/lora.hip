// On-the-fly LoRA update on gfx950 (ExLlamaV2 project page, LoRA adapters:
// the low-rank pair is applied in the forward pass rather than merged into
// the weights; several adapters combine with weights):
//   delta[m][n] (+)= scale * sum_j t[m][j] * B[j][n],   t = x A.
//
// Two launches, both small next to the quantized matmul they feed:
//  1. shrink: t = x A, split along K. Workgroup (row tile, K chunk) sums
//     kLoraChunk rows of K for MB rows of x and writes its partial sums
//     tpart[chunk][m][j] to the workspace. Lanes are (k slot, j): the RP
//     lanes of a k slot read one row of A (contiguous) and share x[m][k].
//  2. expand: workgroup (row tile, column tile) sums the partials of its
//     kExpandRows rows into LDS (times scale), then each thread owns one
//     column n and runs the rank loop over B's rows (coalesced along n) for
//     all rows of the tile.
// Everything is float32 after the float16 loads. No atomics: the K split is
// reduced in the expand kernel, in a fixed order.
#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

constexpr int kLoraThreads = 256;
constexpr int kLoraChunk = 256;  // rows of K per shrink workgroup
constexpr int kExpandRows = 8;   // rows of x per expand workgroup

// RP: rank padded to 8, 16, 32 or 64. MB = 64 / RP rows of x per workgroup,
// so that each thread holds MB accumulators whatever the rank.
template <int RP>
__global__ __launch_bounds__(kLoraThreads) void lora_shrink_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                   const uint16_t* __restrict__ A, int r,
                                                                   float* __restrict__ tpart) {
  constexpr int MB = 64 / RP;
  constexpr int NKS = kLoraThreads / RP;  // k slots
  __shared__ float red[NKS * MB * RP];
  const int tid = threadIdx.x;
  const int j = tid % RP, ks = tid / RP;
  const int m0 = blockIdx.x * MB;
  const int chunk = blockIdx.y;
  const int k0 = chunk * kLoraChunk, k1 = min(k0 + kLoraChunk, K);
  float acc[MB];
#pragma unroll
  for (int mm = 0; mm < MB; ++mm) acc[mm] = 0.0f;
#pragma unroll 4
  for (int k = k0 + ks; k < k1; k += NKS) {
    const float a = j < r ? (float)__builtin_bit_cast(_Float16, A[(size_t)k * r + j]) : 0.0f;
#pragma unroll
    for (int mm = 0; mm < MB; ++mm) {
      const int m = min(m0 + mm, M - 1);  // rows past M repeat row M - 1 and are not stored
      acc[mm] += (float)__builtin_bit_cast(_Float16, x[(size_t)m * K + k]) * a;
    }
  }
#pragma unroll
  for (int mm = 0; mm < MB; ++mm) red[(ks * MB + mm) * RP + j] = acc[mm];
  __syncthreads();
  if (tid < MB * RP) {
    const int mm = tid / RP, jj = tid % RP;
    float v = 0.0f;
    for (int s = 0; s < NKS; ++s) v += red[(s * MB + mm) * RP + jj];
    const int m = m0 + mm;
    if (m < M && jj < r) tpart[((size_t)chunk * M + m) * r + jj] = v;
  }
}

__global__ __launch_bounds__(kLoraThreads) void lora_expand_kernel(const float* __restrict__ tpart, int chunks, int M,
                                                                   int r, const uint16_t* __restrict__ B, int N,
                                                                   float scale, int accumulate,
                                                                   float* __restrict__ delta) {
  __shared__ float ts[kExpandRows][64];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kExpandRows;
  for (int i = tid; i < kExpandRows * r; i += kLoraThreads) {
    const int mm = i / r, j = i % r;
    const int m = m0 + mm;
    float v = 0.0f;
    if (m < M)
      for (int c = 0; c < chunks; ++c) v += tpart[((size_t)c * M + m) * r + j];
    ts[mm][j] = scale * v;
  }
  __syncthreads();
  const int n = blockIdx.y * kLoraThreads + tid;
  if (n >= N) return;
  float acc[kExpandRows];
#pragma unroll
  for (int mm = 0; mm < kExpandRows; ++mm) acc[mm] = 0.0f;
  for (int j = 0; j < r; ++j) {
    const float b = (float)__builtin_bit_cast(_Float16, B[(size_t)j * N + n]);
#pragma unroll
    for (int mm = 0; mm < kExpandRows; ++mm) acc[mm] += ts[mm][j] * b;
  }
#pragma unroll
  for (int mm = 0; mm < kExpandRows; ++mm) {
    const int m = m0 + mm;
    if (m < M) {
      float* d = delta + (size_t)m * N + n;
      *d = accumulate ? *d + acc[mm] : acc[mm];
    }
  }
}

template <int RP>
hipError_t launch_shrink(const uint16_t* x, int M, int K, const uint16_t* A, int r, float* tpart,
                         hipStream_t stream) {
  constexpr int MB = 64 / RP;
  hipLaunchKernelGGL(lora_shrink_kernel<RP>, dim3((M + MB - 1) / MB, lora_chunks(K)), dim3(kLoraThreads), 0,
                     stream, x, M, K, A, r, tpart);
  return hipGetLastError();
}

}  // namespace

int lora_chunks(int K) { return (K + kLoraChunk - 1) / kLoraChunk; }

size_t lora_workspace_bytes(int M, int K, int rank) {
  return (size_t)lora_chunks(K) * (size_t)M * (size_t)rank * sizeof(float);
}

hipError_t launch_lora_delta(const uint16_t* x, int M, int K, const uint16_t* A, int rank, const uint16_t* B, int N,
                             float scale, bool accumulate, float* delta, void* ws, hipStream_t stream) {
  float* tpart = static_cast<float*>(ws);
  hipError_t e = rank <= 8    ? launch_shrink<8>(x, M, K, A, rank, tpart, stream)
                 : rank <= 16 ? launch_shrink<16>(x, M, K, A, rank, tpart, stream)
                 : rank <= 32 ? launch_shrink<32>(x, M, K, A, rank, tpart, stream)
                              : launch_shrink<64>(x, M, K, A, rank, tpart, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lora_expand_kernel, dim3((M + kExpandRows - 1) / kExpandRows, (N + kLoraThreads - 1) / kLoraThreads),
                     dim3(kLoraThreads), 0, stream, tpart, lora_chunks(K), M, rank, B, N, scale, accumulate ? 1 : 0,
                     delta);
  return hipGetLastError();
}

}  // namespace qlinear
