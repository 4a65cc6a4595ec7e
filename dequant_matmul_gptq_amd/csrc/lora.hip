// On-the-fly LoRA update on gfx950 (ExLlamaV2 project page, LoRA adapters:
// the low-rank pair is applied in the forward pass rather than merged into
// the weights; several adapters combine with weights):
//   delta[m][n] (+)= scale * sum_j t[m][j] * B[j][n],   t = x A.
//
// Two launches, both small next to the quantized matmul they feed:
//  1. shrink: t = x A, split along K. Workgroup (row tile, K chunk) stages
//     the chunk's kLoraChunk rows of A and the x tile (kShrinkRows rows of
//     that chunk, stored k-major so that one k's rows are one vector read)
//     in LDS with coalesced loads, then lanes (k slot, j) sum their products
//     from LDS; the k slots are reduced through LDS and the
//     partial sums tpart[chunk][m][j] go to the workspace. Each row of A is
//     read once per row tile, and x once.
//  2. expand: workgroup (row tile, column tile) sums the partials of its
//     kExpandRows rows into LDS (times scale), in a fixed order; each thread
//     owns one column n and runs the rank loop (B's rows, coalesced along n)
//     for all rows of the tile, the first 16 rows of B loaded before the
//     partial sums so that the two latencies overlap.
// Everything is float32 after the float16 loads. No atomics: the K split is
// reduced in the expand kernel, so results do not depend on timing.
#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

constexpr int kLoraThreads = 256;
constexpr int kLoraChunk = 256;   // rows of K per shrink workgroup
constexpr int kShrinkRows = 16;   // rows of x per shrink workgroup (1 for a single row)
constexpr int kExpandRows = 8;    // rows of x per expand workgroup
constexpr int kExpandPre = 16;    // ranks of B loaded ahead of the partial sums

// RP: the rank padded to 8, 16, 32 or 64. MB: rows of x per workgroup,
// kShrinkRows, or 1 when M is 1.
template <int RP, int MB>
__global__ __launch_bounds__(kLoraThreads) void lora_shrink_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                   const uint16_t* __restrict__ A, int r,
                                                                   float* __restrict__ tpart) {
  constexpr int NKS = kLoraThreads / RP;  // k slots
  __shared__ _Float16 As[kLoraChunk * RP];              // rows k0 .. k0 + kn of A, row stride r
  __shared__ __align__(16) _Float16 Xs[kLoraChunk][MB];   // transposed: the MB rows of one k are contiguous
  __shared__ float red[NKS * MB * RP];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * MB;
  const int chunk = blockIdx.y;
  const int k0 = chunk * kLoraChunk, kn = min(kLoraChunk, K - k0);
  // Staging: every load of a thread is issued before its first LDS store
  // (fixed trip counts, clamped addresses), so they are all in flight at once.
  const uint16_t* a_src = A + (size_t)k0 * r;           // the chunk's rows are contiguous
  const int na = kn * r;
  uint16_t av[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) av[u] = a_src[min(u * kLoraThreads + tid, na - 1)];
  constexpr int kXPer = MB * kLoraChunk / kLoraThreads;
  uint16_t xv[kXPer];
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    const int i = u * kLoraThreads + tid;
    const int mm = i / kLoraChunk, kk = i % kLoraChunk;
    const int m = min(m0 + mm, M - 1);                    // rows past M repeat row M - 1 and are not stored
    xv[u] = x[(size_t)m * K + k0 + min(kk, kn - 1)];
  }
#pragma unroll
  for (int u = 0; u < RP; ++u)
    if (u * kLoraThreads + tid < na) As[u * kLoraThreads + tid] = __builtin_bit_cast(_Float16, av[u]);
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    const int i = u * kLoraThreads + tid;
    Xs[i % kLoraChunk][i / kLoraChunk] = i % kLoraChunk < kn ? __builtin_bit_cast(_Float16, xv[u]) : (_Float16)0.0f;
  }
  __syncthreads();
  const int j = tid % RP, ks = tid / RP;
  float acc[MB];
#pragma unroll
  for (int mm = 0; mm < MB; ++mm) acc[mm] = 0.0f;
  if (j < r) {
    for (int k = ks; k < kn; k += NKS) {
      const float a = (float)As[k * r + j];
#pragma unroll
      for (int mm = 0; mm < MB; ++mm) acc[mm] += (float)Xs[k][mm] * a;
    }
  }
#pragma unroll
  for (int mm = 0; mm < MB; ++mm) red[(ks * MB + mm) * RP + j] = acc[mm];
  __syncthreads();
  for (int t = tid; t < MB * RP; t += kLoraThreads) {
    const int mm = t / RP, jj = t % RP;
    float v = 0.0f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) v += red[(s * MB + mm) * RP + jj];
    const int m = m0 + mm;
    if (m < M && jj < r) tpart[((size_t)chunk * M + m) * r + jj] = v;
  }
}

__global__ __launch_bounds__(kLoraThreads) void lora_expand_kernel(const float* __restrict__ tpart, int chunks, int M,
                                                                   int r, const uint16_t* __restrict__ B, int N,
                                                                   float scale, int accumulate,
                                                                   float* __restrict__ delta) {
  __shared__ float ts[kExpandRows][QLINEAR_LORA_MAX_RANK];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kExpandRows;
  const int n = blockIdx.y * kLoraThreads + tid;
  const uint16_t* bcol = B + min(n, N - 1);  // threads past N load column N - 1 and store nothing
  // B's first kExpandPre rows of this column, loaded before the partial sums
  // below so that their latency overlaps (rows past the rank repeat row r - 1).
  float bpre[kExpandPre];
#pragma unroll
  for (int j = 0; j < kExpandPre; ++j) bpre[j] = (float)__builtin_bit_cast(_Float16, bcol[(size_t)min(j, r - 1) * N]);
  for (int e = tid; e < kExpandRows * r; e += kLoraThreads) {
    const int mm = e / r, j = e % r;
    const int m = m0 + mm;
    float v = 0.0f;
    if (m < M) {
      // eight partial sums over the chunks, combined in a fixed order
      float p[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      const float* src = tpart + (size_t)m * r + j;
      const size_t stride = (size_t)M * r;
      int c = 0;
      for (; c + 8 <= chunks; c += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u] += src[(size_t)(c + u) * stride];
      }
      for (int u = 0; c < chunks; ++c, ++u) p[u] += src[(size_t)c * stride];
      v = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    ts[mm][j] = scale * v;   // zero for rows past M
  }
  __syncthreads();
  if (n >= N) return;
  float acc[kExpandRows];
#pragma unroll
  for (int mm = 0; mm < kExpandRows; ++mm) acc[mm] = 0.0f;
#pragma unroll
  for (int j = 0; j < kExpandPre; ++j) {
    if (j < r) {
#pragma unroll
      for (int mm = 0; mm < kExpandRows; ++mm) acc[mm] += ts[mm][j] * bpre[j];
    }
  }
  // Ranks past kExpandPre, unrolled by 8: the 8 loads of B of a pass are in
  // flight together, and only the accumulators live across passes.
#pragma unroll 8
  for (int j = kExpandPre; j < r; ++j) {
    const float b = (float)__builtin_bit_cast(_Float16, bcol[(size_t)j * N]);
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

// Large M with N a multiple of 4: each thread owns 4 adjacent columns, so a
// workgroup reads its rows' partial sums once per 1024 columns (not 256), and
// B and delta move as 8- and 16-byte vectors (a wave stores 1 KiB
// contiguously).
__global__ __launch_bounds__(kLoraThreads) void lora_expand4_kernel(const float* __restrict__ tpart, int chunks, int M,
                                                                    int r, const uint16_t* __restrict__ B, int N,
                                                                    float scale, int accumulate,
                                                                    float* __restrict__ delta) {
  __shared__ float ts[kExpandRows][QLINEAR_LORA_MAX_RANK];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kExpandRows;
  const int q = blockIdx.y * kLoraThreads + tid;   // column quad: columns 4q .. 4q + 3
  const int nq = N / 4;
  const uint2* bq = reinterpret_cast<const uint2*>(B) + min(q, nq - 1);   // quads past N repeat the last, not stored
  for (int e = tid; e < kExpandRows * r; e += kLoraThreads) {
    const int mm = e / r, j = e % r;
    const int m = m0 + mm;
    float v = 0.0f;
    if (m < M) {
      float p[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      const float* src = tpart + (size_t)m * r + j;
      const size_t stride = (size_t)M * r;
      int c = 0;
      for (; c + 8 <= chunks; c += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u] += src[(size_t)(c + u) * stride];
      }
      for (int u = 0; c < chunks; ++c, ++u) p[u] += src[(size_t)c * stride];
      v = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    ts[mm][j] = scale * v;
  }
  __syncthreads();
  if (q >= nq) return;
  float acc[kExpandRows][4];
#pragma unroll
  for (int mm = 0; mm < kExpandRows; ++mm)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[mm][c] = 0.0f;
#pragma unroll 4
  for (int j = 0; j < r; ++j) {
    const uint2 w = bq[(size_t)j * nq];
    const float b0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.x & 0xFFFFu));
    const float b1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.x >> 16));
    const float b2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.y & 0xFFFFu));
    const float b3 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.y >> 16));
#pragma unroll
    for (int mm = 0; mm < kExpandRows; ++mm) {
      const float t = ts[mm][j];
      acc[mm][0] += t * b0;
      acc[mm][1] += t * b1;
      acc[mm][2] += t * b2;
      acc[mm][3] += t * b3;
    }
  }
#pragma unroll
  for (int mm = 0; mm < kExpandRows; ++mm) {
    const int m = m0 + mm;
    if (m < M) {
      float4* d = reinterpret_cast<float4*>(delta + (size_t)m * N) + q;
      float4 v = make_float4(acc[mm][0], acc[mm][1], acc[mm][2], acc[mm][3]);
      if (accumulate) {
        const float4 o = *d;
        v.x += o.x;
        v.y += o.y;
        v.z += o.z;
        v.w += o.w;
      }
      *d = v;
    }
  }
}

template <int RP>
hipError_t launch_rank(const uint16_t* x, int M, int K, const uint16_t* A, int r, const uint16_t* B, int N,
                       float scale, bool accumulate, float* delta, float* tpart, hipStream_t stream) {
  const auto shrink = M == 1 ? lora_shrink_kernel<RP, 1> : lora_shrink_kernel<RP, kShrinkRows>;
  const int tiles = M == 1 ? 1 : (M + kShrinkRows - 1) / kShrinkRows;
  hipLaunchKernelGGL(shrink, dim3(tiles, lora_chunks(K)), dim3(kLoraThreads), 0, stream, x, M, K, A, r, tpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (M > 16 && N % 4 == 0) {
    const int nq = N / 4;
    hipLaunchKernelGGL(lora_expand4_kernel,
                       dim3((M + kExpandRows - 1) / kExpandRows, (nq + kLoraThreads - 1) / kLoraThreads),
                       dim3(kLoraThreads), 0, stream, tpart, lora_chunks(K), M, r, B, N, scale, accumulate ? 1 : 0,
                       delta);
  } else {
    hipLaunchKernelGGL(lora_expand_kernel,
                       dim3((M + kExpandRows - 1) / kExpandRows, (N + kLoraThreads - 1) / kLoraThreads),
                       dim3(kLoraThreads), 0, stream, tpart, lora_chunks(K), M, r, B, N, scale, accumulate ? 1 : 0,
                       delta);
  }
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
  if (rank <= 8) return launch_rank<8>(x, M, K, A, rank, B, N, scale, accumulate, delta, tpart, stream);
  if (rank <= 16) return launch_rank<16>(x, M, K, A, rank, B, N, scale, accumulate, delta, tpart, stream);
  if (rank <= 32) return launch_rank<32>(x, M, K, A, rank, B, N, scale, accumulate, delta, tpart, stream);
  return launch_rank<64>(x, M, K, A, rank, B, N, scale, accumulate, delta, tpart, stream);
}

}  // namespace qlinear
