// Decode-sized quantized linear layer (M <= 16) on gfx950, bound by HBM.
//
// Work split: a 256-thread workgroup owns a strip of 256 output columns and
// a contiguous range of 32-row blocks (split-K); each lane of a wave owns 4
// adjacent columns and streams their packed words with one 16-byte load per
// packed row, so a wave reads 1 KiB contiguous per row. The 4 waves of a
// workgroup split its block range further.
//
// Arithmetic per 32-row block and column (b-bit codes, one scale group):
//   acc  = sum_pairs dot2((1024 + q_lo, 1024 + q_hi), (x_lo, x_hi))    float32
//   y   += s * (acc - (1024 + z) * X_blk),   X_blk = sum of the block's x
// which equals s * sum_j x_j (q_j - z): the float16 pairs 1024 + q come out of
// the packed word with one shift and one mask (see qlinear_device.hpp), and
// the bias 1024 and the zero point are removed once per block. Products of
// float16 values are exact in float32; accumulation is float32 throughout.
//
// The act-order gather x[m][perm[j]] is staged in LDS once per workgroup, in
// the pair order the unpacking produces, together with the block sums X_blk.
//
// Split-K partial sums go to a float32 workspace with atomic adds; the last
// workgroup of a strip to arrive (arrival counter) reads the sums back with
// atomic exchanges -- which also re-zeroes the workspace -- and stores the
// float16 result.
#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStripCols = 256;       // 64 lanes x 4 columns
constexpr int kTargetCtas = 1024;     // ~4 workgroups per CU on 256 CUs
constexpr int kMaxStageLds = 48 * 1024;  // activation staging
constexpr int kRedRows = 4;              // rows per cross-wave reduction pass

struct GemvArgs {
  const uint16_t* x;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint8_t* zeros;
  const int32_t* perm;
  uint16_t* y;
  float* acc;
  uint32_t* cnt;
  int M, K, N, nsplit, nb_max;
  Runs runs;
};

template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Per-group scale and (1024 + zero point) of the lane's 4 columns.
struct GroupParams {
  float s[4];
  float zb[4];
};

template <int B>
__device__ __forceinline__ void load_words(const GemvArgs& a, int row, int col, bool valid, uint4 (&W)[B]) {
#pragma unroll
  for (int t = 0; t < B; ++t) {
    W[t] = valid ? *reinterpret_cast<const uint4*>(a.qweight + (size_t)(row + t) * a.N + col)
                 : make_uint4(0u, 0u, 0u, 0u);
  }
}

struct RawParams {
  uint2 s;
  uint32_t z;
};

__device__ __forceinline__ RawParams load_params(const GemvArgs& a, int g, int col, bool valid) {
  RawParams r;
  r.s = valid ? *reinterpret_cast<const uint2*>(a.scales + (size_t)g * a.N + col) : make_uint2(0u, 0u);
  r.z = (valid && a.zeros) ? *reinterpret_cast<const uint32_t*>(a.zeros + (size_t)g * a.N + col) : 0u;
  return r;
}

template <int B>
__device__ __forceinline__ GroupParams decode_params(const GemvArgs& a, const RawParams& r) {
  GroupParams p;
  p.s[0] = half_lo(r.s.x);
  p.s[1] = half_hi(r.s.x);
  p.s[2] = half_lo(r.s.y);
  p.s[3] = half_hi(r.s.y);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float z = a.zeros ? (float)((r.z >> (8 * c)) & 0xFFu) : (float)(1 << (B - 1));
    p.zb[c] = 1024.0f + z;
  }
  return p;
}

// One 32-row block for the lane's 4 columns and MT activation rows.
template <int B, int MT>
__device__ __forceinline__ void block_compute(const uint4 (&W)[B], const uint32_t* __restrict__ xs_blk,
                                              const float* __restrict__ xsum_blk, const GroupParams& gp,
                                              float (&yacc)[4][MT]) {
  uint32_t wc[4][B];
#pragma unroll
  for (int t = 0; t < B; ++t) {
    wc[0][t] = W[t].x;
    wc[1][t] = W[t].y;
    wc[2][t] = W[t].z;
    wc[3][t] = W[t].w;
  }
  float acc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[c][m] = 0.0f;

  static_for<0, kPairsPerBlock / 4>([&](auto Q) {
    constexpr int q4 = decltype(Q)::value;
    uint4 xv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xv[m] = *reinterpret_cast<const uint4*>(xs_blk + m * kPairsPerBlock + 4 * q4);
    static_for<0, 4>([&](auto R) {
      constexpr int P = 4 * q4 + decltype(R)::value;
      uint32_t v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = extract_pair<B, P>(wc[c]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t xp = (decltype(R)::value == 0) ? xv[m].x
                            : (decltype(R)::value == 1) ? xv[m].y
                            : (decltype(R)::value == 2) ? xv[m].z
                                                        : xv[m].w;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c][m] = __builtin_amdgcn_fdot2(as_half2(v[c]), as_half2(xp), acc[c][m], false);
      }
    });
  });

#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float X = xsum_blk[m];
#pragma unroll
    for (int c = 0; c < 4; ++c) yacc[c][m] = fmaf(gp.s[c], fmaf(-gp.zb[c], X, acc[c][m]), yacc[c][m]);
  }
}

// Blocks [blk0, blk1) of one run (uniform width B), double-buffered: the
// words of block i+1 are in flight while block i is computed.
template <int B, int MT>
__device__ __forceinline__ void process_segment(const GemvArgs& a, int blk0, int blk1, int row0, int col,
                                                bool valid, const uint32_t* xs, const float* xsum, int wg_blk0,
                                                float (&yacc)[4][MT], bool use_pre, const uint4 (&pre)[8],
                                                const RawParams& pre_p) {
  const int bpg = a.runs.blocks_per_group;
  uint4 Wa[B], Wb[B];
  RawParams Pa, Pb;
  if (use_pre) {
#pragma unroll
    for (int t = 0; t < B; ++t) Wa[t] = pre[t];
    Pa = pre_p;
  } else {
    load_words<B>(a, row0, col, valid, Wa);
    Pa = load_params(a, blk0 / bpg, col, valid);
  }
  for (int i = blk0; i < blk1; i += 2) {
    const int ra = row0 + (i - blk0) * B;
    if (i + 1 < blk1) {
      load_words<B>(a, ra + B, col, valid, Wb);
      Pb = load_params(a, (i + 1) / bpg, col, valid);
    }
    {
      const int bl = i - wg_blk0;
      block_compute<B, MT>(Wa, xs + bl * MT * kPairsPerBlock, xsum + bl * MT, decode_params<B>(a, Pa), yacc);
    }
    if (i + 1 >= blk1) break;
    if (i + 2 < blk1) {
      load_words<B>(a, ra + 2 * B, col, valid, Wa);
      Pa = load_params(a, (i + 2) / bpg, col, valid);
    }
    {
      const int bl = i + 1 - wg_blk0;
      block_compute<B, MT>(Wb, xs + bl * MT * kPairsPerBlock, xsum + bl * MT, decode_params<B>(a, Pb), yacc);
    }
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void qgemv_kernel(GemvArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int strip = blockIdx.x;
  const int split = blockIdx.y;
  const int nblk = a.K / kBlockRows;
  const int wg_blk0 = (int)((long long)split * nblk / a.nsplit);
  const int wg_blk1 = (int)((long long)(split + 1) * nblk / a.nsplit);
  const int nb = wg_blk1 - wg_blk0;
  const int wb0 = wg_blk0 + (wave * nb) / kWaves;
  const int wb1 = wg_blk0 + ((wave + 1) * nb) / kWaves;
  const int col = strip * kStripCols + lane * 4;
  const bool valid = col < a.N;

  // Issue the loads of this wave's first block before the activation staging,
  // so that HBM latency overlaps the perm -> x gather.
  uint4 pre[8];
  RawParams pre_p = {make_uint2(0u, 0u), 0u};
#pragma unroll
  for (int t = 0; t < 8; ++t) pre[t] = make_uint4(0u, 0u, 0u, 0u);
  int first_bits = 0;
  if (wb0 < wb1) {
    int row;
    block_info(a.runs, wb0, first_bits, row);
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (t < first_bits)
        pre[t] = valid ? *reinterpret_cast<const uint4*>(a.qweight + (size_t)(row + t) * a.N + col)
                       : make_uint4(0u, 0u, 0u, 0u);
    pre_p = load_params(a, wb0 / a.runs.blocks_per_group, col, valid);
  }

  // Stage x[m][perm[j]] for the workgroup's blocks in unpacking pair order.
  uint32_t* xs = lds;                                          // [nb][MT][16] float16 pairs
  float* xsum = reinterpret_cast<float*>(lds + a.nb_max * MT * kPairsPerBlock);  // [nb][MT]
  // Walk the runs overlapping [wg_blk0, wg_blk1) with workgroup-uniform
  // (scalar) indices, so the bit width of every staged block is uniform.
  {
    int blk = wg_blk0;
    int r = 0;
    while (r + 1 < a.runs.nruns && blk >= a.runs.run_block[r + 1]) ++r;
    while (blk < wg_blk1) {
      const int bits = a.runs.run_bits[r];
      const int seg_end = min(wg_blk1, a.runs.run_block[r + 1]);
      const int items = (seg_end - blk) * kPairsPerBlock;
      for (int idx = tid; idx < items; idx += kThreads) {
        const int bl = (blk - wg_blk0) + idx / kPairsPerBlock, p = idx % kPairsPerBlock;
        int lo, hi;
        pair_rows(bits, p, lo, hi);
        const int jlo = (wg_blk0 + bl) * kBlockRows + lo, jhi = (wg_blk0 + bl) * kBlockRows + hi;
        // perm entries are clamped into [0, K) so that a malformed perm cannot
        // address outside x.
        const int flo = a.perm ? (int)min((unsigned)a.perm[jlo], (unsigned)(a.K - 1)) : jlo;
        const int fhi = a.perm ? (int)min((unsigned)a.perm[jhi], (unsigned)(a.K - 1)) : jhi;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          uint32_t v = 0u;
          if (m < a.M) v = (uint32_t)a.x[(size_t)m * a.K + flo] | ((uint32_t)a.x[(size_t)m * a.K + fhi] << 16);
          xs[(bl * MT + m) * kPairsPerBlock + p] = v;
        }
      }
      blk = seg_end;
      ++r;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nb * MT; idx += kThreads) {
    const uint32_t* src = xs + idx * kPairsPerBlock;
    float s = 0.0f;
#pragma unroll
    for (int p = 0; p < kPairsPerBlock; ++p) s += half_lo(src[p]) + half_hi(src[p]);
    xsum[idx] = s;
  }
  __syncthreads();

  float yacc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[c][m] = 0.0f;

  int blk = wb0;
  bool first = true;
  while (blk < wb1) {
    int bits, row;
    block_info(a.runs, blk, bits, row);
    const int seg_end = min(wb1, run_end_block(a.runs, blk));
    switch (bits) {
      case 2: process_segment<2, MT>(a, blk, seg_end, row, col, valid, xs, xsum, wg_blk0, yacc, first, pre, pre_p); break;
      case 3: process_segment<3, MT>(a, blk, seg_end, row, col, valid, xs, xsum, wg_blk0, yacc, first, pre, pre_p); break;
      case 4: process_segment<4, MT>(a, blk, seg_end, row, col, valid, xs, xsum, wg_blk0, yacc, first, pre, pre_p); break;
      case 5: process_segment<5, MT>(a, blk, seg_end, row, col, valid, xs, xsum, wg_blk0, yacc, first, pre, pre_p); break;
      case 6: process_segment<6, MT>(a, blk, seg_end, row, col, valid, xs, xsum, wg_blk0, yacc, first, pre, pre_p); break;
      case 8: process_segment<8, MT>(a, blk, seg_end, row, col, valid, xs, xsum, wg_blk0, yacc, first, pre, pre_p); break;
      default: break;
    }
    first = false;
    blk = seg_end;
  }

  // Cross-wave reduction through LDS, kRedRows activation rows at a time:
  // red[wave][row][256 columns].
  const int colt = strip * kStripCols + tid;
  const bool validt = colt < a.N;
  float* red = reinterpret_cast<float*>(lds);
  constexpr int RC = MT < kRedRows ? MT : kRedRows;
  float sum[MT];
#pragma unroll
  for (int m0 = 0; m0 < MT; m0 += RC) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      const int m = m0 + r;
      float4 v = make_float4(yacc[0][m], yacc[1][m], yacc[2][m], yacc[3][m]);
      *reinterpret_cast<float4*>(red + (wave * RC + r) * kStripCols + lane * 4) = v;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += red[(w * RC + r) * kStripCols + tid];
      sum[m0 + r] = t;
    }
  }

  if (a.nsplit == 1) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < a.M && validt) a.y[(size_t)m * a.N + colt] = __builtin_bit_cast(uint16_t, (_Float16)sum[m]);
    return;
  }

  // Split-K combine. The partial sums are device-scope float atomics, which
  // every XCD performs at one coherence point. The workgroup barrier waits
  // until this workgroup's atomics have been performed (vmcnt(0)) before the
  // arrival counter is bumped, so the last workgroup to arrive sees every
  // partial sum when it reads them back -- with atomic exchanges, which also
  // re-zero the workspace. No cache write-back/invalidate (a device-scope
  // fence) is needed because no plain global store takes part in the exchange.
#pragma unroll
  for (int m = 0; m < MT; ++m)
    if (m < a.M && validt) atomicAdd(a.acc + (size_t)m * a.N + colt, sum[m]);
  // vmcnt also counts no-return atomics until they complete; the barrier alone
  // does not wait for them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned old = atomicAdd(a.cnt + strip, 1u);
    s_last = (old == (unsigned)(a.nsplit - 1));
  }
  __syncthreads();
  if (s_last) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < a.M && validt) {
        const float v = atomicExch(a.acc + (size_t)m * a.N + colt, 0.0f);
        a.y[(size_t)m * a.N + colt] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
    if (tid == 0) atomicExch(a.cnt + strip, 0u);
  }
}

template <int MT>
hipError_t launch_mt(GemvArgs a, hipStream_t stream) {
  const int nstrips = (a.N + kStripCols - 1) / kStripCols;
  const int nblk = a.K / kBlockRows;
  int nsplit = (kTargetCtas + nstrips - 1) / nstrips;
  nsplit = min(nsplit, max(1, nblk / kWaves));
  const int per_block_bytes = MT * (kPairsPerBlock * 4 + 4);
  const int max_nb = kMaxStageLds / per_block_bytes;
  nsplit = max(nsplit, (nblk + max_nb - 1) / max_nb);
  nsplit = min(nsplit, nblk);
  a.nsplit = nsplit;
  a.nb_max = (nblk + nsplit - 1) / nsplit;
  const size_t stage = (size_t)a.nb_max * per_block_bytes;
  const size_t reduce = (size_t)kWaves * (MT < kRedRows ? MT : kRedRows) * kStripCols * 4;
  const size_t lds = stage > reduce ? stage : reduce;
  hipLaunchKernelGGL(qgemv_kernel<MT>, dim3(nstrips, nsplit, 1), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

size_t qgemv_workspace_bytes(int N) {
  const size_t acc = (size_t)QLINEAR_GEMV_MAX_M * N * sizeof(float);
  const size_t cnt = (size_t)((N + kStripCols - 1) / kStripCols) * sizeof(uint32_t);
  return (acc + cnt + 255) / 256 * 256;
}

hipError_t launch_qgemv(const qlinear_layout& L, const Runs& runs, const uint16_t* x, int M,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        const int32_t* perm, uint16_t* y, void* ws, hipStream_t stream) {
  GemvArgs a;
  a.x = x;
  a.qweight = qweight;
  a.scales = scales;
  a.zeros = zeros;
  a.perm = perm;
  a.y = y;
  a.acc = reinterpret_cast<float*>(ws);
  a.cnt = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) +
                                      (size_t)QLINEAR_GEMV_MAX_M * L.N * sizeof(float));
  a.M = M;
  a.K = L.K;
  a.N = L.N;
  a.nsplit = 1;
  a.nb_max = 0;
  a.runs = runs;
  if (M <= 1) return launch_mt<1>(a, stream);
  if (M <= 2) return launch_mt<2>(a, stream);
  if (M <= 4) return launch_mt<4>(a, stream);
  if (M <= 8) return launch_mt<8>(a, stream);
  return launch_mt<16>(a, stream);
}

}  // namespace qlinear
