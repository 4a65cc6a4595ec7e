// Q4 / Q6 / Q8 KV-cache codec (ExLlamaV2 blog: the Q4, Q6 and Q8 cache modes
// beside FP16, "How to Use Effectively", Step 2; their memory savings of 75%
// and 50% against FP16). The pages fix no format; this one is:
//   rows of D float16 values, cut into blocks of G in {32, 64, 128};
//   per block, in float32: s = RNE_fp16(max |x| / (2^(b-1) - 1));
//   code q = clamp(rint(x / s), -2^(b-1), 2^(b-1) - 1) + 2^(b-1) (a correctly
//   rounded float32 division, ties to even; s = 0 gives the midpoint);
//   a block's codes are a little-endian bit stream of G b / 32 words;
//   dequantized x' = RNE_fp16(s (q - 2^(b-1))) (an exact float32 product).
//
// Both kernels are streaming: one thread per 16 consecutive elements (two
// 16-byte float16 loads or stores), whose b / 2 code words are whole and
// contiguous with its neighbours', so every access is coalesced. A block's
// G / 16 threads are adjacent lanes and reduce its maximum with lane swaps.
// HBM-bound: quantize reads 2 and writes b / 8 + 2 / G bytes per element,
// dequantize the reverse.
#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

constexpr int kKvThreads = 256;

template <int B>
constexpr int kv_words() { return B / 2; }   // code words per 16 elements

// Insert the B-bit code c of element i (0..15) into the thread's words.
template <int B>
__device__ __forceinline__ void put_code(uint32_t (&w)[kv_words<B>()], int i, uint32_t c) {
  const int pos = i * B, k = pos >> 5, sh = pos & 31;
  w[k] |= c << sh;
  if (sh + B > 32) w[k + 1] |= c >> (32 - sh);
}

template <int B>
__device__ __forceinline__ uint32_t get_code(const uint32_t (&w)[kv_words<B>()], int i) {
  const int pos = i * B, k = pos >> 5, sh = pos & 31;
  uint32_t v = w[k] >> sh;
  if (sh + B > 32) v |= w[k + 1] << (32 - sh);
  return v & ((1u << B) - 1u);
}

template <int B, int G>
__global__ __launch_bounds__(kKvThreads) void kv_quant_kernel(const uint16_t* __restrict__ x,
                                                              uint32_t* __restrict__ codes,
                                                              uint16_t* __restrict__ scales, int64_t units) {
  const int64_t t = (int64_t)blockIdx.x * kKvThreads + threadIdx.x;
  // units is a multiple of G / 16, so the lanes of a block all stay or all leave.
  if (t >= units) return;
  const uint4* src = reinterpret_cast<const uint4*>(x) + 2 * t;
  const uint4 a = src[0], b = src[1];
  const uint32_t h[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(h[i] & 0xFFFFu));
    v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(h[i] >> 16));
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  // The block's G / 16 lanes are adjacent and start at a multiple of G / 16.
#pragma unroll
  for (int k = 1; k < G / 16; k <<= 1) m = fmaxf(m, __shfl_xor(m, k));
  constexpr float kQmax = (float)((1 << (B - 1)) - 1);
  const _Float16 s16 = (_Float16)(m / kQmax);
  const float s = (float)s16;
  constexpr int kHalf = 1 << (B - 1);
  uint32_t w[kv_words<B>()];
#pragma unroll
  for (int k = 0; k < kv_words<B>(); ++k) w[k] = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float r = s > 0.0f ? __builtin_rintf(v[i] / s) : 0.0f;
    r = fminf(fmaxf(r, (float)-kHalf), (float)(kHalf - 1));
    put_code<B>(w, i, (uint32_t)((int)r + kHalf));
  }
  uint32_t* dst = codes + t * kv_words<B>();
#pragma unroll
  for (int k = 0; k < kv_words<B>(); ++k) dst[k] = w[k];
  if ((t & (G / 16 - 1)) == 0) scales[t / (G / 16)] = __builtin_bit_cast(uint16_t, s16);
}

template <int B, int G>
__global__ __launch_bounds__(kKvThreads) void kv_dequant_kernel(const uint32_t* __restrict__ codes,
                                                                const uint16_t* __restrict__ scales,
                                                                uint16_t* __restrict__ x, int64_t units) {
  const int64_t t = (int64_t)blockIdx.x * kKvThreads + threadIdx.x;
  if (t >= units) return;
  uint32_t w[kv_words<B>()];
  const uint32_t* src = codes + t * kv_words<B>();
#pragma unroll
  for (int k = 0; k < kv_words<B>(); ++k) w[k] = src[k];
  const float s = (float)__builtin_bit_cast(_Float16, scales[t / (G / 16)]);
  constexpr int kHalf = 1 << (B - 1);
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 lo = (_Float16)(s * (float)((int)get_code<B>(w, 2 * i) - kHalf));
    const _Float16 hi = (_Float16)(s * (float)((int)get_code<B>(w, 2 * i + 1) - kHalf));
    h[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>(x) + 2 * t;
  dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
  dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
}

template <int B, int G>
hipError_t launch_kv(bool quant, const uint16_t* x, uint32_t* codes, uint16_t* scales, uint16_t* out,
                     int64_t units, hipStream_t stream) {
  const dim3 grid((unsigned)((units + kKvThreads - 1) / kKvThreads));
  if (quant)
    hipLaunchKernelGGL((kv_quant_kernel<B, G>), grid, dim3(kKvThreads), 0, stream, x, codes, scales, units);
  else
    hipLaunchKernelGGL((kv_dequant_kernel<B, G>), grid, dim3(kKvThreads), 0, stream, codes, scales, out, units);
  return hipGetLastError();
}

template <int B>
hipError_t launch_kv_bits(bool quant, int group, const uint16_t* x, uint32_t* codes, uint16_t* scales,
                          uint16_t* out, int64_t units, hipStream_t stream) {
  if (group == 32) return launch_kv<B, 32>(quant, x, codes, scales, out, units, stream);
  if (group == 64) return launch_kv<B, 64>(quant, x, codes, scales, out, units, stream);
  return launch_kv<B, 128>(quant, x, codes, scales, out, units, stream);
}

hipError_t launch_kv_any(bool quant, int bits, int group, const uint16_t* x, uint32_t* codes, uint16_t* scales,
                         uint16_t* out, int64_t elements, hipStream_t stream) {
  const int64_t units = elements / 16;
  if (units == 0) return hipSuccess;
  if (bits == 4) return launch_kv_bits<4>(quant, group, x, codes, scales, out, units, stream);
  if (bits == 6) return launch_kv_bits<6>(quant, group, x, codes, scales, out, units, stream);
  return launch_kv_bits<8>(quant, group, x, codes, scales, out, units, stream);
}

}  // namespace

hipError_t launch_kv_quant(const uint16_t* x, int64_t elements, int bits, int group, uint32_t* codes,
                           uint16_t* scales, hipStream_t stream) {
  return launch_kv_any(true, bits, group, x, codes, scales, nullptr, elements, stream);
}

hipError_t launch_kv_dequant(const uint32_t* codes, const uint16_t* scales, int64_t elements, int bits, int group,
                             uint16_t* x, hipStream_t stream) {
  return launch_kv_any(false, bits, group, nullptr, const_cast<uint32_t*>(codes), const_cast<uint16_t*>(scales), x,
                       elements, stream);
}

}  // namespace qlinear
