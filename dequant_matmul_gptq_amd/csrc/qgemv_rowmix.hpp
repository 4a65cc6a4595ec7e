// One-launch decode kernel (M = 1 or 2) for layouts of several code widths or
// with two-level scales: the single-row kernel's scheme (qgemv_m1.hpp) run
// segment by segment.
#pragma once

#include "qgemv_m1.hpp"

namespace qlinear {

namespace stream {

// Several code widths at M = 1 or 2 (EXL2 layouts), in one launch: the scheme of
// qgemv_row_kernel, run segment by segment. A wave's K range is cut at the
// run boundaries; each segment has its width fixed at compile time (a switch
// over the widths of the set BS) and refills its own D steps, so the
// pipeline restarts at a boundary. The host gives each wave its K range and
// first segment (width, first packed row, end block), so the first D steps
// are issued right after the x row loads, as in the single-width kernel.
// Register use: the first segment's issue, row staging and steps sit in one
// width branch (two branches joined by the in-flight step registers cost
// 20-40 VGPRs more), and the per-width lane constants are recomputed inside
// the segment loop rather than hoisted out of it for every width.

// Calls f(integral_constant<int, b>) for the width b = bits if BS holds it.
template <unsigned BS, class F>
__device__ __forceinline__ void for_width(int bits, F&& f) {
  switch (bits) {
    case 2: if constexpr ((BS >> 2) & 1u) f(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr ((BS >> 3) & 1u) f(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr ((BS >> 4) & 1u) f(std::integral_constant<int, 4>{}); break;
    case 5: if constexpr ((BS >> 5) & 1u) f(std::integral_constant<int, 5>{}); break;
    case 6: if constexpr ((BS >> 6) & 1u) f(std::integral_constant<int, 6>{}); break;
    case 8: if constexpr ((BS >> 8) & 1u) f(std::integral_constant<int, 8>{}); break;
    default: break;
  }
}

// Whether a call of 1 or 2 rows with several widths (or two-level scales,
// any widths) runs the one-launch kernel below: the x rows must fit the LDS
// budget, and the call must have at most 1024 strips of 16 columns (4
// workgroups per CU), or 256 where the kernel needs many registers: rows of
// more than 16384 values at M = 1 (16 x-row pieces per thread, about 200
// VGPRs), more than 8192 at M = 2 (8 pieces per row, past 256 VGPRs). Past
// that the gather kernel plus the multi-row kernel win: the latter holds more
// waves per SIMD, which pays once the grid takes several rounds. Measured on
// MI355X (graph-timed, one launch vs gather + multi-row, us):
//   M = 1  EXL2 4.0 bpw 4096 -> 11008 (688 strips)        11.9 vs 14.8
//          2.5 bpw 8192 -> 28672 (1792 strips)            31.4 vs 29.4
//          3/2-bit 16384 -> 8192 (512) / -> 2048 (128)     18.1 / 10.1 vs 18.8 / 12.1
//          3/2-bit 28672 -> 8192 (512) / -> 4096 (256)     30.9 / 17.4 vs 29.8 / 20.1
//   M = 2  3/2-bit 4096 -> 11008 (688) / -> 16384 (1024)   10.8 / 13.5 vs 15.4 / 18.0
//          3/2-bit 8192 -> 16384 (1024)                    21.4 vs 23.9
//          3/2-bit 12288 -> 8192 (512) / -> 4096 (256)     18.6 / 10.5 vs 18.5 / 14.4
inline bool mixed_row(int M, int K, int N, int mats, unsigned set, bool two_level) {
  const int64_t strips = (int64_t)((N + SC - 1) / SC) * mats;
  const int64_t max_strips = K > (M == 2 ? 8192 : 16384) ? 256 : 1024;
  return M >= 1 && M <= 2 && (size_t)M * row_words(K) * 4 <= kRowLdsBudget &&
         ((set & (set - 1)) != 0 || two_level) && strips <= max_strips;
}

template <unsigned BS, int WV, int P, int D, bool kPerm, int MT>
__global__ __launch_bounds__(WV * 64) void qgemv_rowmix_kernel(StreamArgs a) {
  constexpr bool kTL = two_level<BS>();   // two-level scales: scale codes, scale_max in the epilogue
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ float red[WV][4][MT][SC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Kernel arguments, all read in one batch (the wave's first segment too).
  MatPtrs mp = a.mat[blockIdx.y];
  int K = a.K, N = a.N, M = a.M, spx = a.strips_per_xcd, xw = a.xrow_words;
  const uint16_t* xsrc = a.x;
  Epilogue epi = a.epi;
  int bits0 = a.wave_bits[wave], row0 = a.wave_row[wave], seg0_end = a.wave_end[wave];
  int wb0 = a.wave_begin[wave], wb1 = a.wave_begin[wave + 1];
  {
    const int R = a.runs.packed_rows, bpg = a.bpg_shift, hz = a.has_zeros, nruns = a.runs.nruns;
    const int32_t* const perm = a.perm;
    asm volatile("" : "+s"(K), "+s"(N), "+s"(M), "+s"(spx), "+s"(xw), "+s"(xsrc), "+s"(mp.y), "+s"(epi.bias),
                 "+s"(epi.residual), "+s"(epi.act), "+s"(bits0), "+s"(row0), "+s"(seg0_end), "+s"(wb0), "+s"(wb1)
                 : "s"(R), "s"(bpg), "s"(hz), "s"(nruns), "s"(perm), "s"(mp.qweight), "s"(mp.scales),
                   "s"(mp.zeros));
  }
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
  // The epilogue's operands of this strip's outputs (as in qgemv_row_kernel):
  // thread tid < 16 MT stores output (row tid / 16, column tid % 16).
  const int n_out = min(strip * SC + (tid % SC), N - 1);
  const int m_out = min(tid / SC, M - 1);
  const uint16_t bias_raw = as_global<uint16_t>(epi.bias ? epi.bias : mp.y)[n_out];
  const uint16_t res_raw = as_global<uint16_t>(epi.residual ? epi.residual : mp.y)[(size_t)m_out * N + n_out];
  uint16_t smax_raw = 0;
  if constexpr (kTL) smax_raw = as_global<uint16_t>(epi.scale_max)[n_out];
  asm volatile("" ::: "memory");   // keep the row loads ahead of the weight loads

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

  // 2. The first D steps of the first segment, then 3. the row into LDS.
  // Both sit in the width's branch, so the wait before each LDS store covers
  // that store's own piece and none of the weight loads issued after it.
  // A wave without blocks has width 0 and only stores its pieces, as would a
  // wave whose width were outside BS (the host picks a BS covering every run
  // width): every wave reaches exactly one barrier here.
  auto store_row = [&]() {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      piece_t* xl = reinterpret_cast<piece_t*>(lds + m * xw);
#pragma unroll
      for (int u = 0; u < P; ++u) xl[min(u * nthr + tid, n16 - 1)] = xr[m][u];
    }
  };
  float yacc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[c][m] = 0.0f;
  if (bits0 <= 0 || bits0 > 8 || ((BS >> bits0) & 1u) == 0) {
    store_row();
    __syncthreads();
  }
  for_width<BS>(bits0, [&](auto Bc) {
    constexpr int B = decltype(Bc)::value;
    StepRegs S[D];
    int rlo[4], rhi[4];
    float sc[4];
    lane_pairs<B>(L.cq, rlo, rhi, sc);
    static_for<0, D>([&](auto Dd) {
      constexpr int d = decltype(Dd)::value;
      seg_issue<B, kTL>(a, L, wb0, seg0_end, row0, d, rlo, rhi, S[d]);
    });
    store_row();
    __syncthreads();
    row_steps<B, D, kPerm, MT, kTL>(a, L, wb0, seg0_end, row0, yacc, S);
  });
  if (wb0 < wb1) {
    for (int blk = seg0_end; blk < wb1;) {
      int bits, row;
      block_info(a.runs, blk, bits, row);
      const int seg_end = min(wb1, run_end_block(a.runs, blk));
      for_width<BS>(bits, [&](auto Bc) {
        constexpr int B = decltype(Bc)::value;
        StepRegs T[D];
        int rlo[4], rhi[4];
        float sc[4];
        int cq = L.cq;
        asm volatile("" : "+v"(cq));   // keeps the lane's pair rows inside the loop (not hoisted per width)
        lane_pairs<B>(cq, rlo, rhi, sc);
        static_for<0, D>([&](auto Dd) {
          constexpr int d = decltype(Dd)::value;
          seg_issue<B, kTL>(a, L, blk, seg_end, row, d, rlo, rhi, T[d]);
        });
        RowLane Lc = L;
        Lc.cq = cq;
        row_steps<B, D, kPerm, MT, kTL>(a, Lc, blk, seg_end, row, yacc, T);
      });
      blk = seg_end;
    }
  }

  // 5. Reduce over the block slots, the wave's rows and the waves; epilogue
  // and store, as in qgemv_row_kernel.
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
    if constexpr (kTL) v *= (float)__builtin_bit_cast(_Float16, smax_raw) * 0.0625f;
    if (epi.bias) v += (float)__builtin_bit_cast(_Float16, bias_raw);
    if (epi.act == QLINEAR_ACT_SILU) v = v / (1.0f + __expf(-v));
    if (epi.residual) v += (float)__builtin_bit_cast(_Float16, res_raw);
    ((__attribute__((address_space(1))) uint16_t*)mp.y)[(size_t)m * N + strip * SC + c_out] =
        __builtin_bit_cast(uint16_t, (_Float16)v);
  }
}

// The waves' K ranges: each point of the equal split moves to the nearest
// run boundary less than half a wave's share away (and past the previous
// point, so that no wave is left empty). A boundary
// inside a wave's range restarts its pipeline, and the wave of the most
// segments sets the workgroup's time; on EXL2 layouts (a few runs, widest
// first) the moved points also balance the weight bytes per wave better
// (EXL2 4.0 bpw 4096 -> 11008, runs of 13, 13, 64 and 38 blocks: splits
// 26 / 64 / 90 in place of 32 / 64 / 96).
inline void snapped_waves(StreamArgs& a, int WV) {
  const int nblk = a.K / kBlockRows;
  const int half = nblk / (2 * WV);
  a.wave_begin[0] = 0;
  for (int w = 1; w < WV; ++w) {
    const int eq = (w * nblk) / WV;
    int best = eq, dist = half;
    for (int r = 1; r < a.runs.nruns; ++r) {
      const int b = a.runs.run_block[r];
      const int d = b > eq ? b - eq : eq - b;
      if (d < dist && b > a.wave_begin[w - 1]) {
        dist = d;
        best = b;
      }
    }
    a.wave_begin[w] = std::max(best, a.wave_begin[w - 1]);
  }
  a.wave_begin[WV] = nblk;
}

template <unsigned BS, int P, int MT>
hipError_t launch_rowmix(StreamArgs a, hipStream_t stream) {
  const auto kernel = a.perm ? qgemv_rowmix_kernel<BS, kRowWaves, P, kRowDepth, true, MT>
                             : qgemv_rowmix_kernel<BS, kRowWaves, P, kRowDepth, false, MT>;
  a.nstrips = (a.N + SC - 1) / SC;
  a.strips_per_xcd = (a.nstrips + kXcds - 1) / kXcds;
  a.xrow_words = row_words(a.K);
  snapped_waves(a, kRowWaves);
  first_segments(a, kRowWaves, a.K / kBlockRows);
  const size_t lds = (size_t)MT * a.xrow_words * 4;
  hipLaunchKernelGGL(kernel, dim3(kXcds * a.strips_per_xcd, a.mats), dim3(kRowWaves * 64), lds, stream, a);
  return hipGetLastError();
}

// The rows (1 or 2) and the pieces per thread that cover K (mixed_row()
// bounds K by the LDS budget: 2 rows need at most 8 pieces).
template <unsigned BS>
hipError_t launch_rowmix_set(const StreamArgs& a, hipStream_t stream) {
  constexpr int per_piece = kRowWaves * 64 * 8;
  if (a.M >= 2) {
    if (a.K <= 2 * per_piece) return launch_rowmix<BS, 2, 2>(a, stream);
    if (a.K <= 4 * per_piece) return launch_rowmix<BS, 4, 2>(a, stream);
    return launch_rowmix<BS, 8, 2>(a, stream);
  }
  if (a.K <= 2 * per_piece) return launch_rowmix<BS, 2, 1>(a, stream);
  if (a.K <= 4 * per_piece) return launch_rowmix<BS, 4, 1>(a, stream);
  if (a.K <= 8 * per_piece) return launch_rowmix<BS, 8, 1>(a, stream);
  return launch_rowmix<BS, kRowPiecesMax, 1>(a, stream);
}

// Instantiated in the qgemv_rowmix_*.hip files, one per set of widths:
// the smallest instantiated set that covers `set`.
hipError_t launch_rowmix_low(const StreamArgs& a, hipStream_t stream);
hipError_t launch_rowmix_mid(const StreamArgs& a, hipStream_t stream);
hipError_t launch_rowmix_all(const StreamArgs& a, hipStream_t stream);
// The same with two-level scales (in the qgemv_rowmix_tl_*.hip files).
hipError_t launch_rowmix_low_tl(const StreamArgs& a, hipStream_t stream);
hipError_t launch_rowmix_mid_tl(const StreamArgs& a, hipStream_t stream);
hipError_t launch_rowmix_all_tl(const StreamArgs& a, hipStream_t stream);

}  // namespace stream

}  // namespace qlinear
