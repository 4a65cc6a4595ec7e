// Single-launch decode kernel (M = 1 to 4) on gfx950: the act-order gather
// happens inside the kernel, so a call is one launch. For M > 1 the x rows
// (1, 2 or 4 of them) all sit in LDS and each weight pair, once unpacked, is
// used for every row.
//
// Work split as in the multi-row kernel: a workgroup of 4 waves owns a
// 16-column panel and the whole K range; lane = (block slot ks, column quad
// cq); a wave step is 16 consecutive blocks, two steps in flight.
//
// Activations. The workgroup copies the x row (float16, original order) into
// LDS; its loads are issued first, before any weight load (vector loads
// complete in issue order, so a load issued after the weights would wait for
// them). For its block, each lane of a column quad gathers 4 of the block's
// 16 pairs: the perm entries of those 8 rows are loaded with the step's
// weights, the values read from the LDS row and scaled by 2^-e (the exponent
// at which the pair's codes are unpacked), and the four lanes of the quad
// exchange their pairs with DPP broadcasts. The block sums X (activations)
// and X' (scaled activations) are reduced over the quad the same way.
// Arithmetic per block and column is that of the multi-row kernel:
//   acc = sum_pairs dot2((1024 + q_lo 2^e, 1024 + q_hi 2^e), (x_lo 2^-e, x_hi 2^-e))
//   y  += s * (acc - 1024 * X' - z * X)
#pragma once

#include "qgemv_stream.hpp"

namespace qlinear {

namespace stream {

constexpr int kRowLdsBudget = 62 * 1024;  // bytes of LDS for the x row

// LDS words of the x row (K float16, rounded up to 16 bytes).
__host__ __device__ constexpr int row_words(int K) { return (K / 2 + 3) / 4 * 4; }

// Activation rows of the kernel instance for M rows: 1, 2 or 4.
constexpr int row_mt(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

// Whether a call of M <= 4 rows runs this kernel: the x rows must fit in the
// LDS budget, and the matrix must have a single code width (one row of
// several widths runs qgemv_rowmix_kernel, qgemv_rowmix.hpp). The budget is
// below the 160 KB a workgroup may hold because the rows are staged through
// registers: 4 rows of K = 11008 would need 128 VGPRs.
inline bool single_row(int M, int K, unsigned set) {
  return M <= 4 && (size_t)row_mt(M) * row_words(K) * 4 <= kRowLdsBudget && (set & (set - 1)) == 0;
}

// Loads of one lane for one step: the block's weights, scale and zero point
// (as in the multi-row kernel) and the perm entries of the lane's 4 pairs.
struct StepRegs {
  uint4 W[8];   // entries 0 .. B-1 used
  Raw P;
  int pl[4], ph[4];
};

// The lane's 4 pairs 4 cq + r of a block of width B: their rows in the block
// and the scale 2^-e of their activations.
template <int B>
__device__ __forceinline__ void lane_pairs(int cq, int (&rlo)[4], int (&rhi)[4], float (&sc)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = 4 * cq + r;
    pair_rows(B, p, rlo[r], rhi[r]);
    sc[r] = __builtin_ldexpf(1.0f, -pair_exponent(B, p));
  }
}

// The perm entries follow the block alone (blk_ok), not the lane's columns:
// the four lanes of a quad exchange the pairs of one block, so a lane whose
// columns lie past N must still gather its quad's block.
template <int B, bool kTL = false>
__device__ __forceinline__ void issue_step(const StreamArgs& a, const MatPtrs& mp, const uint32_t* panel,
                                           const int32_t* psrc, int blk,
                                           int row, bool blk_ok, bool ok, int blk_safe, int row_safe, int col,
                                           const int (&rlo)[4], const int (&rhi)[4], StepRegs& S) {
  issue<B, kTL>(a, mp, panel, blk, row, ok, blk_safe, row_safe, col, reinterpret_cast<uint4(&)[B]>(S.W), S.P);
  const int32_t* pb = psrc + (size_t)(blk_ok ? blk : blk_safe) * kBlockRows;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    S.pl[r] = pb[rlo[r]];
    S.ph[r] = pb[rhi[r]];
  }
}

__device__ __forceinline__ float quad_sum(float v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  return v;
}

// Gather the lane's 4 pairs of block blk from each of the MT LDS rows (row m
// at xrow + m * xstride), exchange them over the quad, then unpack the
// block's pairs for the lane's 4 columns once and multiply them into every
// row. kTL: two-level scales (the block's weight is its 4-bit scale code + 1;
// the factor scale_max / 16 comes in the epilogue).
template <int B, bool kPerm, int MT, bool kTL = false>
__device__ __forceinline__ void compute_step(const StreamArgs& a, const StepRegs& S, const _Float16* xrow, int xstride,
                                             int blk, const int (&rlo)[4], const int (&rhi)[4], const float (&sc)[4],
                                             uint32_t magic, float (&yacc)[4][MT]) {
  uint32_t own[4][MT];
  float xs[MT], xss[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xs[m] = xss[m] = 0.0f;
  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // perm entries are clamped into [0, K): a malformed perm cannot address outside the row.
    const int flo = kPerm ? (int)min((unsigned)S.pl[r], (unsigned)(a.K - 1)) : blk * kBlockRows + rlo[r];
    const int fhi = kPerm ? (int)min((unsigned)S.ph[r], (unsigned)(a.K - 1)) : blk * kBlockRows + rhi[r];
    const _Float16 s16 = (_Float16)sc[r];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      // The pair in float16, scaled by 2^-e with one packed multiply (exact,
      // or the same rounding of a subnormal as float32 then float16), and
      // both added into the block sums by a dot product with (1, 1).
      const uint32_t pair = (uint32_t)__builtin_bit_cast(uint16_t, xrow[m * xstride + flo]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, xrow[m * xstride + fhi]) << 16);
      const half2_t scaled = as_half2(pair) * half2_t{s16, s16};
      own[r][m] = as_u32(scaled);
      xs[m] = __builtin_amdgcn_fdot2(as_half2(pair), ones, xs[m], false);
      xss[m] = __builtin_amdgcn_fdot2(scaled, ones, xss[m], false);
    }
  }
  float X[MT], Xs[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    X[m] = quad_sum(xs[m]);
    Xs[m] = quad_sum(xss[m]);
  }

  const uint4* W = S.W;
  uint32_t wc[4][B], wsh[4][B];
#pragma unroll
  for (int t = 0; t < B; ++t) {
    wc[0][t] = W[t].x;
    wc[1][t] = W[t].y;
    wc[2][t] = W[t].z;
    wc[3][t] = W[t].w;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int t = 0; t < B; ++t) wsh[c][t] = wc[c][t] >> scaled_shift(B);
  float acc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[c][m] = 0.0f;
  static_for<0, kPairsPerBlock>([&](auto Q) {
    constexpr int Pp = decltype(Q)::value;
    if constexpr (MT == 1) {
      // (one row: each pair unpacked right before its product)
      const uint32_t xp = (uint32_t)__builtin_amdgcn_mov_dpp((int)own[Pp % 4][0], (Pp / 4) * 0x55, 0xF, 0xF, false);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t v = extract_pair_scaled<B, Pp>(wc[c], wsh[c], magic);
        acc[c][0] = __builtin_amdgcn_fdot2(as_half2(v), as_half2(xp), acc[c][0], false);
      }
    } else {
      uint32_t v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = extract_pair_scaled<B, Pp>(wc[c], wsh[c], magic);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t xp = (uint32_t)__builtin_amdgcn_mov_dpp((int)own[Pp % 4][m], (Pp / 4) * 0x55, 0xF, 0xF, false);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c][m] = __builtin_amdgcn_fdot2(as_half2(v[c]), as_half2(xp), acc[c][m], false);
      }
    }
  });
  // A lane without a block this step (past the range or past N) adds nothing.
  if (S.P.ok) {
    float s[4];
    if constexpr (kTL) {
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] = (float)(((S.P.s.x >> (S.P.s.y + 4 * c)) & 15u) + 1u);
    } else {
      s[0] = half_lo(S.P.s.x);
      s[1] = half_hi(S.P.s.x);
      s[2] = half_lo(S.P.s.y);
      s[3] = half_hi(S.P.s.y);
    }
    // The 4 zero points as bytes of one word (symmetric: 2^(B-1) each; two-level
    // scales are symmetric).
    const uint32_t zw = (!kTL && a.has_zeros) ? S.P.z : (uint32_t)(1u << (B - 1)) * 0x01010101u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float z = (float)((zw >> (8 * c)) & 0xFFu);
#pragma unroll
      for (int m = 0; m < MT; ++m) yacc[c][m] = fmaf(s[c], fmaf(-z, X[m], acc[c][m] - 1024.0f * Xs[m]), yacc[c][m]);
    }
  }
}

// Lane context shared by the steps of a wave.
struct RowLane {
  MatPtrs mp;
  const uint32_t* panel;
  const int32_t* psrc;
  const _Float16* xrow;        // x row 0 in LDS; row m at xrow + m * xstride
  int xstride;
  int ks, cq, col;
  bool colv;
  uint32_t magic;
};

// Step i of the segment [blk0, blk1) starting at packed row row0.
template <int B, bool kTL = false>
__device__ __forceinline__ void seg_issue(const StreamArgs& a, const RowLane& L, int blk0, int blk1, int row0, int i,
                                          const int (&rlo)[4], const int (&rhi)[4], StepRegs& S) {
  const int blk = blk0 + i * KS + L.ks;
  const bool blk_ok = blk < blk1;
  issue_step<B, kTL>(a, L.mp, L.panel, L.psrc, blk, row0 + (i * KS + L.ks) * B, blk_ok, L.colv && blk_ok, blk0, row0,
                L.col, rlo, rhi, S);
}

// All steps of the wave's blocks [blk0, blk1) (at least one), D in flight;
// the first D were issued already into S[0 .. D-1]. kPerm: act-order (the
// choice is made once per launch, not per pair).
template <int B, int D, bool kPerm, int MT, bool kTL = false>
__device__ __forceinline__ void row_steps(const StreamArgs& a, const RowLane& L, int blk0, int blk1, int row0,
                                          float (&yacc)[4][MT], StepRegs (&S)[D]) {
  int rlo[4], rhi[4];
  float sc[4];
  lane_pairs<B>(L.cq, rlo, rhi, sc);
  const int nsteps = (blk1 - blk0 + KS - 1) / KS;
  auto comp = [&](int i, const StepRegs& R) {
    // Past the range the whole quad is idle (zero scale); its pairs come
    // from block blk0 (as its perm entries did).
    const int blk = blk0 + i * KS + L.ks < blk1 ? blk0 + i * KS + L.ks : blk0;
    compute_step<B, kPerm, MT, kTL>(a, R, L.xrow, L.xstride, blk, rlo, rhi, sc, L.magic, yacc);
  };
  // Steady state: every buffer is refilled on every pass. (A refill under a
  // condition turns the buffers into loop-carried copies, and a copy waits for
  // the load it copies: only one step would stay in flight.)
  int i = 0;
  for (; i + 2 * D - 1 < nsteps; i += D) {
    static_for<0, D>([&](auto Dd) {
      constexpr int d = decltype(Dd)::value;
      comp(i + d, S[d]);
      seg_issue<B, kTL>(a, L, blk0, blk1, row0, i + d + D, rlo, rhi, S[d]);
    });
  }
  // The last 1 to 2D - 1 steps; those among i .. i + D - 1 are issued.
  const int r = nsteps - i;
  static_for<0, 2 * D - 1>([&](auto Tt) {
    constexpr int t = decltype(Tt)::value;
    if (t < r) {
      comp(i + t, S[t % D]);
      if (t + D < r) seg_issue<B, kTL>(a, L, blk0, blk1, row0, i + t + D, rlo, rhi, S[t % D]);
    }
  });
}

// A pointer in the global address space: loads through it are global (not
// flat) loads, which the vector-memory counter alone tracks.
template <class T>
using global_ptr = const __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ global_ptr<T> as_global(const void* p) {
  return (global_ptr<T>)p;
}
typedef uint32_t piece_t __attribute__((ext_vector_type(4)));   // 16 bytes of the x row

// One code width B for the whole matrix (one run: block b starts at packed
// row b * B). Grid: x = 16-column strips, XCD-major; y = matrix of the group.
// Every kernel argument the first loads need is read up front, and none of
// those reads depends on another, so the weight stream starts after a single
// scalar-load round trip.
// P: sixteen-byte pieces of the x row per thread, all loaded before the
// weights; P * WV * 64 * 16 bytes cover the row. D: steps in flight per wave.
// kPerm: act-order (perm given), a kernel of its own so that the step loop
// holds no per-pair choice.
// MT: activation rows, 1, 2 or 4 (rows from M on repeat row M - 1 and are not stored).
// kAddend: the epilogue adds a float32 addend (an instance of its own: the
// pointer is read only where it is used).
template <int B, int WV, int P, int D, bool kPerm, int MT, bool kAddend = false>
__global__ __launch_bounds__(WV * 64) void qgemv_row_kernel(StreamArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ float red[WV][4][MT][SC];   // per wave and 16-lane row: the sums of the strip's columns

  // Kernel arguments, all read in one batch: the empty asm takes them as
  // operands (and hands them back, so they are not read again later).
  MatPtrs mp = a.mat[blockIdx.y];
  int K = a.K, N = a.N, M = a.M, spx = a.strips_per_xcd, xw = a.xrow_words;
  const uint16_t* xsrc = a.x;
  Epilogue epi = a.epi;
  {
    const int R = a.runs.packed_rows, bpg = a.bpg_shift, hz = a.has_zeros;
    const int32_t* const perm = a.perm;
    asm volatile("" : "+s"(K), "+s"(N), "+s"(M), "+s"(spx), "+s"(xw), "+s"(xsrc), "+s"(mp.y), "+s"(epi.bias),
                 "+s"(epi.residual), "+s"(epi.act)
                 : "s"(R), "s"(bpg), "s"(hz), "s"(perm), "s"(mp.qweight), "s"(mp.scales), "s"(mp.zeros));
  }
  const float* addp = nullptr;
  if constexpr (kAddend) {
    addp = epi.addend;
    asm volatile("" : "+s"(addp));
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  const int strip = (bid % kXcds) * spx + bid / kXcds;
  if (strip * SC >= N) return;  // the whole workgroup leaves together

  // 1. The x rows: every piece this thread copies, loaded before anything else.
  constexpr int nthr = WV * 64;
  const int n16 = K / 8;
  piece_t xr[MT][P];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const global_ptr<piece_t> xg = as_global<piece_t>(xsrc + (size_t)min(m, M - 1) * K);
#pragma unroll
    for (int u = 0; u < P; ++u) xr[m][u] = xg[min(u * nthr + tid, n16 - 1)];
  }
  // The epilogue's operands of this strip's outputs, read now rather than
  // after the final reduction (a residual that is the output itself is read
  // before the same thread writes it). Every thread loads, from y when a term
  // is absent: loads without a branch around them keep the wait before each
  // LDS store below down to that store's own piece. This kernel takes no
  // float32 addend: the dispatcher sends calls with one to the other kernels.
  // Thread tid < 16 MT stores output (row tid / 16, column tid % 16).
  const int n_out = min(strip * SC + (tid % SC), N - 1);
  const int m_out = min(tid / SC, M - 1);
  const uint16_t bias_raw = as_global<uint16_t>(epi.bias ? epi.bias : mp.y)[n_out];
  const uint16_t res_raw = as_global<uint16_t>(epi.residual ? epi.residual : mp.y)[(size_t)m_out * N + n_out];
  float add_v = 0.0f;
  if constexpr (kAddend) add_v = as_global<float>(addp)[(size_t)m_out * N + n_out];
  asm volatile("" ::: "memory");   // keep the row loads ahead of the weight loads

  // 2. The first D steps of the wave's blocks, issued by every wave (a wave
  // without blocks reads block wb0 < K / 32 and computes nothing; steps past
  // the end are duplicate reads with zero scale).
  const int nblk = K / kBlockRows;
  const int wb0 = (wave * nblk) / WV, wb1 = ((wave + 1) * nblk) / WV;
  const int row0 = wb0 * B;
  RowLane L;
  L.mp = mp;
  L.cq = lane % CQ;
  L.ks = lane / CQ;
  const int col_req = strip * SC + L.cq * 4;
  L.colv = col_req < N;
  L.col = L.colv ? col_req : N - 4;   // scale/zero column for lanes past N
  L.panel = mp.qweight + (size_t)strip * a.runs.packed_rows * kPanel + L.cq * 4;
  L.psrc = a.perm ? a.perm : reinterpret_cast<const int32_t*>(mp.qweight);   // >= K readable words
  L.xrow = reinterpret_cast<const _Float16*>(lds);
  L.xstride = xw * 2;
  L.magic = vgpr_magic();
  StepRegs S[D];
  {
    int rlo[4], rhi[4];
    float sc[4];
    lane_pairs<B>(L.cq, rlo, rhi, sc);
    static_for<0, D>([&](auto Dd) {
      constexpr int d = decltype(Dd)::value;
      seg_issue<B>(a, L, wb0, wb1, row0, d, rlo, rhi, S[d]);
    });
  }

  // 3. The rows into LDS (clamped threads rewrite the last piece with its own value).
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    piece_t* xl = reinterpret_cast<piece_t*>(lds + m * xw);
#pragma unroll
    for (int u = 0; u < P; ++u) xl[min(u * nthr + tid, n16 - 1)] = xr[m][u];
  }
  __syncthreads();

  // 4. Stream the wave's blocks.
  float yacc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[c][m] = 0.0f;
  if (wb0 < wb1) row_steps<B, D, kPerm, MT>(a, L, wb0, wb1, row0, yacc, S);

  // Reduce over the block slots: the 4 of each 16-lane row with two DPP row
  // shifts (lanes 12..15 of a row end up with its sums, one per column
  // quad), then the 4 rows of each wave and the waves through LDS; the
  // epilogue as apply_epilogue, without the addend: bias, activation, residual.
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = yacc[c][m];
      v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF,
                                                                 true));   // row_shr:4
      v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF,
                                                                 true));   // row_shr:8
      yacc[c][m] = v;
    }
  if ((lane & 15) >= 12) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) red[wave][lane >> 4][m][L.cq * 4 + c] = yacc[c][m];
  }
  __syncthreads();
  const int c_out = tid % SC;
  if (tid < SC * MT && tid / SC < M && strip * SC + c_out < N) {
    const int m = tid / SC;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WV; ++w)
#pragma unroll
      for (int row = 0; row < 4; ++row) v += red[w][row][m][c_out];
    if constexpr (kAddend) v += add_v;
    if (epi.bias) v += (float)__builtin_bit_cast(_Float16, bias_raw);
    if (epi.act == QLINEAR_ACT_SILU) v = v / (1.0f + __expf(-v));
    if (epi.residual) v += (float)__builtin_bit_cast(_Float16, res_raw);
    ((__attribute__((address_space(1))) uint16_t*)mp.y)[(size_t)m * N + strip * SC + c_out] =
        __builtin_bit_cast(uint16_t, (_Float16)v);
  }
}

template <int B, int WV, int P, int D, int MT, bool kAddend>
hipError_t launch_row(StreamArgs a, hipStream_t stream) {
  const auto kernel = a.perm ? qgemv_row_kernel<B, WV, P, D, true, MT, kAddend>
                             : qgemv_row_kernel<B, WV, P, D, false, MT, kAddend>;
  a.nstrips = (a.N + SC - 1) / SC;
  a.strips_per_xcd = (a.nstrips + kXcds - 1) / kXcds;
  a.xrow_words = row_words(a.K);
  const size_t lds = (size_t)MT * a.xrow_words * 4;
  hipLaunchKernelGGL(kernel, dim3(kXcds * a.strips_per_xcd, a.mats), dim3(WV * 64), lds, stream, a);
  return hipGetLastError();
}

// Four waves per workgroup for every shape. Measured on MI355X (7B decode
// launches, graph-timed): 8 waves take 9.29 / 5.02 / 14.99 / 8.53 us against
// 7.61 / 4.48 / 11.67 / 7.82 us on 3 x 4096^2, 4096^2, 2 x 4096 -> 11008 and
// 11008 -> 4096, although two 8-wave workgroups fit per CU (112 VGPRs for the
// 4-bit instance): a wave then holds a single step of 16 blocks.
constexpr int kRowWaves = 4;

// x-row pieces per thread: the fewest of 2, 4, 8 and 16 that cover the row
// (16 cover the whole LDS budget); a piece past the row is a duplicate load.
constexpr int kRowPiecesMax = 16;
static_assert(kRowPiecesMax * kRowWaves * 64 * 16 >= kRowLdsBudget, "x-row pieces must cover the LDS budget");

// Steps in flight per wave. Measured on MI355X: 3 instead of 2 is slower
// even where each CU holds one workgroup and each wave has 6 steps
// (11008 -> 4096: 9.1 vs 8.3 us), so every shape keeps two.
constexpr int kRowDepth = 2;

// MT rows: the pieces per thread that cover K (MT x rows must fit the LDS
// budget, which single_row() checks: 2 rows need at most 8 pieces, 4 rows 4).
template <int B, int MT, bool kAddend>
hipError_t launch_row_mt(const StreamArgs& a, hipStream_t stream) {
  constexpr int per_piece = kRowWaves * 64 * 8;   // x values per piece index
  if (a.K <= 2 * per_piece) return launch_row<B, kRowWaves, 2, kRowDepth, MT, kAddend>(a, stream);
  if (a.K <= 4 * per_piece) return launch_row<B, kRowWaves, 4, kRowDepth, MT, kAddend>(a, stream);
  if constexpr (MT <= 2) {
    if (a.K <= 8 * per_piece) return launch_row<B, kRowWaves, 8, kRowDepth, MT, kAddend>(a, stream);
  }
  if constexpr (MT == 1) return launch_row<B, kRowWaves, kRowPiecesMax, kRowDepth, 1, kAddend>(a, stream);
  return hipErrorInvalidValue;
}

template <int B, bool kAddend>
hipError_t launch_row_width(const StreamArgs& a, hipStream_t stream) {
  const int mt = row_mt(a.M);
  if (mt == 1) return launch_row_mt<B, 1, kAddend>(a, stream);
  if (mt == 2) return launch_row_mt<B, 2, kAddend>(a, stream);
  return launch_row_mt<B, 4, kAddend>(a, stream);
}

// Instantiated in qgemv_row.hip (no addend) and qgemv_row_addend.hip (with a
// float32 addend): `set` holds exactly one code width.
hipError_t launch_row_set(unsigned set, const StreamArgs& a, hipStream_t stream);
hipError_t launch_row_set_addend(unsigned set, const StreamArgs& a, hipStream_t stream);

}  // namespace stream

}  // namespace qlinear
