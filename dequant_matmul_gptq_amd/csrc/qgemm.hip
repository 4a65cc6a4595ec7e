// Prefill-sized quantized linear layer on gfx950, bound by the matrix cores.
//
// 1. The shared gather kernel writes the act-order-gathered activations into
//    the workspace, xq[m][32*blk + 2p + h] = x[m][perm[32*blk + row_h(p)]],
//    where (row_0(p), row_1(p)) are the two rows that pair p of block blk
//    unpacks to. Inside every 32-row block the K order is thus the unpacking
//    order, and the weights below are used in that same order, so the
//    contraction is unchanged.
// 2. gemm_kernel (one code width; several widths go to the kernel in
//    qgemm_lds.hip): a workgroup of 8 waves computes a 256 x 256 tile of y,
//    the waves as 2 x 4 tiles of 128 x 64, each as 8 x 4 fragments of
//    v_mfma_f32_16x16x32_f16 (one 32-row block is one MFMA K step).
//      - B (weights): no LDS. The B operand of a 16 x 16 x 32 MFMA gives
//        lane l column l % 16 of the fragment and rows 8 (l / 16) .. + 7 of
//        the block, i.e. pairs 4g .. 4g + 3 (g = l / 16); for 4-bit codes
//        those are exactly packed word g of the column. A lane's 4 fragments
//        take 4 adjacent columns, so one 16-byte load brings word g of all
//        four. Each wave dequantizes its fragments exactly to float16 in
//        registers (w = RNE(s * (q - z)), one rounding); each fragment feeds
//        8 MFMAs. The packed words run two blocks ahead in a register ring.
//        For widths whose k-group sits in one or two words (2, 4, 8) block
//        kb + 1 is dequantized while block kb's MFMAs run, so the unpacking
//        interleaves with the matrix core inside every wave; the other widths
//        (which read all b words per column) dequantize block kb in its own
//        step, which keeps them within 256 registers.
//      - A (activations): two LDS stages of 64-byte rows, 16-byte chunks
//        XOR-swizzled so that tile stores and fragment reads are free of bank
//        conflicts; block kb + 2's tile is loaded into registers during block
//        kb and stored one step later; one barrier per block.
//    Buffer loads take their per-block offsets in scalars; offsets are 32-bit,
//    so the host runs M in row chunks whose activations stay below 2 GiB.
//    Two waves per SIMD (256 registers per lane). Tiles are dealt to the 8
//    XCDs in contiguous ranges. Accumulation is float32; the epilogue rounds
//    to float16.
#include <algorithm>

#include "mfma_frag.hpp"

namespace qlinear {

namespace {

using namespace frag;

constexpr int kThreads = 512;
constexpr int BM = 256, BN = 256;
constexpr int WM = 128, WN = 64;             // wave tile: 2 x 4 waves
constexpr int FM = WM / 16, FN = WN / 16;    // 8 x 4 fragments per wave
constexpr int kLdsRow = kBlockRows;          // 32 halves = 64 bytes, four 16-byte chunks
constexpr int kAPieces = BM * kBlockRows / 8 / kThreads;  // 16-byte pieces of an A block per thread

// Partial sums of a layout with several code widths, run by one launch per
// run into float32 [M][N] in the workspace.
enum PartMode : int {
  kWhole = 0,   // the launch covers all of K: float16 output
  kFirst = 1,   // first run: write the partial sums
  kMiddle = 2,  // add into the partial sums
  kLast = 3,    // partial sums + this run: float16 output
};

struct GemmArgs {
  const uint16_t* xq;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint8_t* zeros;
  uint16_t* y;
  float* part;                 // partial sums (part_mode != kWhole)
  int M, K, N;
  int xq_bytes, qweight_bytes, scale_bytes;
  int kb_first, kb_end, run_row;   // the blocks of this launch: one run of one width
  int part_mode;
  Runs runs;
  Epilogue epi;
};

constexpr int kRing = 2;   // blocks of B loads in flight; also LDS stages of the A tile

// Register ring of the global loads of D blocks. A lane's 4 column
// fragments take 4 adjacent columns (its column quad), so each packed-word
// row, the 4 scales and the 4 zero points are one load each.
template <int kW, int D>
struct Ring {
  u32x4 w[D][kW];         // packed-word rows t of the quad's 4 columns
  u32x2 s[D];             // 4 float16 scales
  uint32_t z[D];          // 4 uint8 zero points
  int bits[D];
};

// Per-lane byte offsets that do not change along K.
struct LaneOffsets {
  uint32_t a[kAPieces];   // A piece (row, 16-byte chunk) at K = 0
  uint32_t w;             // packed row 0 of the quad's first column
  uint32_t col;           // the quad's first column
};

// The launch's blocks [first, end): one run of one width, starting at packed
// row `row`.
struct RunRef {
  int first, end, row;
};

template <unsigned BS, int kW, int D, int S>
__device__ __forceinline__ void load_block(const GemmArgs& a, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                                           __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rz, int g,
                                           const LaneOffsets& off, const RunRef& run, int blk, Ring<kW, D>& R) {
  static_assert((BS & (BS - 1)) == 0, "a launch streams one code width");
  const int bits = __builtin_ctz(BS);
  blk = min(blk, run.end - 1);   // loads past the run repeat its last block
  const int row = run.row + (blk - run.first) * bits;
  R.bits[S] = bits;
  with_width<BS>(bits, [&](auto BB) {
    constexpr int B = decltype(BB)::value;
    const uint32_t v = off.w + (uint32_t)frag_first_word<B>(g) * kPanel * 4;   // g differs between lanes
#pragma unroll
    for (int t = 0; t < frag_words<B>(); ++t)
      R.w[S][t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, v, (row + t) * kPanel * 4, 0));
  });
  const int grp = blk / a.runs.blocks_per_group;
  R.s[S] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off.col * 2, grp * a.N * 2, 0));
  R.z[S] = __builtin_amdgcn_raw_buffer_load_b32(rz, off.col, a.zeros ? grp * a.N : 0, 0);
}

// A tile rows are 64 bytes without padding; 16-byte chunk c of row r sits at
// chunk position c ^ ((r >> 1) & 3). Both the 16-lane groups of the tile
// stores (4 rows x 4 chunks) and of the fragment reads (16 rows, one chunk)
// then cover all 64 banks once.
__device__ __forceinline__ int lds_chunk(int r, int c) { return c ^ ((r >> 1) & 3); }

__device__ __forceinline__ void store_a(uint16_t* stage, int tid, const u32x4 (&pieces)[kAPieces]) {
#pragma unroll
  for (int i = 0; i < kAPieces; ++i) {
    const int lin = tid + i * kThreads;
    const int r = lin / 4, ch = lin % 4;
    *reinterpret_cast<u32x4*>(&stage[r * kLdsRow + lds_chunk(r, ch) * 8]) = pieces[i];
  }
}

// The B fragments of the block in ring slot S, exactly dequantized.
// Zero point and scale come as float16 bit patterns: -(1024 + z) is 0xE400 | z
// (z < 1024), and the scale is splatted into both halves with a byte permute.
template <unsigned BS, int kW, int D, int S>
__device__ __forceinline__ void dequant_block(const GemmArgs& a, const Ring<kW, D>& R, int g, uint32_t magic,
                                              half8_t (&bf)[FN]) {
  with_width<BS>(R.bits[S], [&](auto BB) {
    constexpr int B = decltype(BB)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      // byte j of the zero points into the low byte of both halves
      const uint32_t zsel = 0x0C000C00u | ((uint32_t)j << 16) | (uint32_t)j;
      const uint32_t zz = a.zeros ? __builtin_amdgcn_perm(0u, R.z[S], zsel) : (uint32_t)(1 << (B - 1)) * 0x10001u;
      const uint32_t nb = zz | 0xE400E400u;
      const uint32_t ssel = (j % 2) ? 0x03020302u : 0x01000100u;
      const uint32_t sv = __builtin_amdgcn_perm(R.s[S][j / 2], R.s[S][j / 2], ssel);
      uint32_t w[kW];
#pragma unroll
      for (int t = 0; t < kW; ++t) w[t] = R.w[S][t][j];
      bf[j] = dequant_frag<B, kW>(w, g, as_half2(nb), as_half2(sv), magic);
    }
  });
}

__device__ __forceinline__ void read_a(const uint16_t* stage, int lane, int g, int wr, half8_t (&af)[FM]) {
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = wr * WM + i * 16 + (lane & 15);
    af[i] = *reinterpret_cast<const half8_t*>(&stage[row * kLdsRow + lds_chunk(row, g) * 8]);
  }
}

// Whether block kb + 1's B fragments are dequantized during block kb's MFMAs
// (one or two words per k-group: widths 2, 4, 8).
template <int kW>
constexpr bool pipelined() {
  return kW <= 2;
}

// Block kb = kb0 + S; its A tile is in LDS stage S, block kb + 1's A pieces
// in an[S ^ 1]. The step loads block kb + 2's A pieces into an[S], runs block
// kb's MFMAs and stores block kb + 1's A pieces into stage S ^ 1.
//   pipelined: block kb's fragments are in bf[S] and block kb + 1's words in
//     slot S ^ 1; the step dequantizes block kb + 1 into bf[S ^ 1] and then
//     loads block kb + 3's words into slot S ^ 1.
//   otherwise: block kb's words are in slot S; the step dequantizes them into
//     bf[0] and then loads block kb + 2's words into slot S.
// A loads are clamped to the last block of K, B loads to the last of the run.
template <unsigned BS, int kW, int S>
__device__ __forceinline__ void block_step(const GemmArgs& a, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                                           __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rz, int tid, int lane,
                                           int g, int wr, uint32_t magic, const LaneOffsets& off, const RunRef& run,
                                           int kb, int nblk, uint16_t* As, Ring<kW, kRing>& R,
                                           u32x4 (&an)[2][kAPieces], half8_t (&bf)[2][FN], float4_t (&acc)[FM][FN]) {
  constexpr int kStage = BM * kLdsRow;
  constexpr int T = S ^ 1;
  constexpr bool kPipe = pipelined<kW>();
  constexpr int kUse = kPipe ? S : 0;   // fragments that this step's MFMAs use
  const int nb2 = min(kb + 2, nblk - 1);
#pragma unroll
  for (int i = 0; i < kAPieces; ++i)
    an[S][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off.a[i], nb2 * kBlockRows * 2, 0));
  half8_t af[FM];
  if constexpr (kPipe) {
    read_a(As + S * kStage, lane, g, wr, af);
    dequant_block<BS, kW, kRing, T>(a, R, g, magic, bf[T]);
    load_block<BS, kW, kRing, T>(a, rx, rw, rs, rz, g, off, run, kb + 3, R);
  } else {
    dequant_block<BS, kW, kRing, S>(a, R, g, magic, bf[0]);
    load_block<BS, kW, kRing, S>(a, rx, rw, rs, rz, g, off, run, kb + 2, R);
    read_a(As + S * kStage, lane, g, wr, af);
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[kUse][j], acc[i][j], 0, 0, 0);
  store_a(As + T * kStage, tid, an[T]);
  __syncthreads();
}

// kRange: the launch covers one run [kb_first, kb_end) of a layout computed
// run by run (partial sums per part_mode); otherwise all of K, one width.
template <unsigned BS, bool kRange>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs a) {
  constexpr int kW = max_frag_words<BS>();
  constexpr int D = kRing;
  __shared__ __align__(16) uint16_t As[kRing * BM * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 2, wc = wave & 3;
  // Tiles are taken XCD by XCD: workgroups are dispatched round-robin over
  // the 8 XCDs, so workgroup i works on tile (i % 8) * ceil(T / 8) + i / 8 of
  // the row-major tile order: an XCD's tiles share rows of A in its L2.
  const int gx = (a.N + BN - 1) / BN;
  const int ntiles = gx * ((a.M + BM - 1) / BM);
  const int bid = blockIdx.x;
  const int tile = (bid % 8) * ((ntiles + 7) / 8) + bid / 8;
  if (tile >= ntiles) return;   // the whole workgroup leaves together
  const int n0 = (tile % gx) * BN;
  const int m0 = (tile / gx) * BM;
  const int nblk = a.K / kBlockRows;
  const RunRef run = kRange ? RunRef{a.kb_first, a.kb_end, a.run_row} : RunRef{0, nblk, 0};
  const int g = lane >> 4;   // k-group of the lane's B fragments

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, 0, a.xq_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.qweight, 0, a.qweight_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)a.scales, 0, a.scale_bytes, kRsrcWord3);
  // Without zero points the zero loads read the scale buffer (not used).
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      a.zeros ? (void*)a.zeros : (void*)a.scales, 0, a.zeros ? a.scale_bytes / 2 : a.scale_bytes, kRsrcWord3);

  LaneOffsets off;
#pragma unroll
  for (int i = 0; i < kAPieces; ++i) {
    const int lin = tid + i * kThreads;
    const int m = min(m0 + lin / 4, a.M - 1);   // rows past M repeat row M - 1 (not stored)
    off.a[i] = ((uint32_t)m * (uint32_t)a.K + (uint32_t)(lin % 4) * 8) * 2;
  }
  // The lane's column quad; N is a multiple of 8, so a quad is in or out as a
  // whole. A quad past N reads at offsets beyond every buffer: the buffer
  // loads return zeros (zero scales), and it is not stored.
  const int nq = n0 + wc * WN + (lane & 15) * 4;
  const bool nok = nq < a.N;
  off.w = nok ? ((uint32_t)(nq / kPanel) * (uint32_t)a.runs.packed_rows * kPanel + nq % kPanel) * 4 : 0x80000000u;
  off.col = nok ? (uint32_t)nq : 0x40000000u;

  Ring<kW, D> R;
  const uint32_t magic = vgpr_magic();
  float4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = {0.f, 0.f, 0.f, 0.f};

  // Prologue: packed words of the launch's blocks f and f + 1 in slots 0 and
  // 1, their A pieces loaded, block f's A tile in stage 0. Pipelined: block
  // f's fragments in bf[0] and block f + 2's words in flight in slot 0.
  const int f = run.first;
  static_for<0, D>([&](auto SS) {
    constexpr int S = decltype(SS)::value;
    load_block<BS, kW, D, S>(a, rx, rw, rs, rz, g, off, run, f + S, R);
  });
  u32x4 an[2][kAPieces];
#pragma unroll
  for (int i = 0; i < kAPieces; ++i) {
    an[0][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off.a[i], f * kBlockRows * 2, 0));
    an[1][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
        rx, off.a[i], min(f + 1, nblk - 1) * kBlockRows * 2, 0));
  }
  half8_t bf[2][FN];
  if constexpr (pipelined<kW>()) {
    dequant_block<BS, kW, D, 0>(a, R, g, magic, bf[0]);
    load_block<BS, kW, D, 0>(a, rx, rw, rs, rz, g, off, run, f + 2, R);
  }
  store_a(As, tid, an[0]);
  __syncthreads();

  // Whole rounds of D blocks without conditions (static ring slots, exact
  // load counts), then the remaining blocks.
  const int nfull = f + (run.end - f) / D * D;
  for (int kb0 = f; kb0 < nfull; kb0 += D) {
    static_for<0, D>([&](auto SS) {
      constexpr int S = decltype(SS)::value;
      block_step<BS, kW, S>(a, rx, rw, rs, rz, tid, lane, g, wr, magic, off, run, kb0 + S, nblk, As, R, an, bf, acc);
    });
  }
  static_for<0, D - 1>([&](auto SS) {
    constexpr int S = decltype(SS)::value;
    if (nfull + S < run.end)
      block_step<BS, kW, S>(a, rx, rw, rs, rz, tid, lane, g, wr, magic, off, run, nfull + S, nblk, As, R, an, bf, acc);
  });

  // Epilogue: lane holds C[4*(lane/16) + r][lane % 16] of each 16 x 16 tile;
  // fragment j's column c is column 4c + j of the wave's 64, so a lane's 4
  // fragments give 4 adjacent columns of a row: one 8-byte store.
  if (nok) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wr * WM + i * 16 + 4 * (lane >> 4) + r;
        if (m < a.M) {
          float v4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = acc[i][j][r];
          if (kRange && a.part_mode != kWhole) {
            float4_t* pp = reinterpret_cast<float4_t*>(a.part + (size_t)m * a.N + nq);
            if (a.part_mode != kFirst) {
              const float4_t p = *pp;
#pragma unroll
              for (int j = 0; j < 4; ++j) v4[j] += p[j];
            }
            if (a.part_mode != kLast) {
              *pp = float4_t{v4[0], v4[1], v4[2], v4[3]};
              continue;
            }
          }
          uint16_t h[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            h[j] = __builtin_bit_cast(uint16_t, (_Float16)apply_epilogue(a.epi, v4[j], m, nq + j, a.N));
          u32x2 v;
          v[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
          v[1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
          *reinterpret_cast<u32x2*>(a.y + (size_t)m * a.N + nq) = v;
        }
      }
    }
  }
}

template <unsigned BS>
void launch_set(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  if (a.part_mode == kWhole)
    hipLaunchKernelGGL((gemm_kernel<BS, false>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<BS, true>), grid, dim3(kThreads), 0, stream, a);
}

}  // namespace

// Layouts with several code widths are computed one launch per run
// (register dequantization of that run's width), the runs adding up in
// float32 partial sums in the workspace, when K holds at least 16384 rows per
// run boundary (each boundary writes and reads the [M][N] partial sums, about
// 700 / K of the GEMM's own time) and the launch fills at least one round of
// 256 x 256 tiles on the 256 CUs. Otherwise the kernel that dequantizes into
// LDS block by block, whose 128 x 128 tiles fill the chip at smaller grids.
// Measured on MI355X (us, run by run vs LDS kernel, M = 512 / 1024 / 2048):
//   70B 2.5 bpw 28672 -> 8192, two runs:  888 / 970 / 1277 vs 632 / 786 / 1327
//   70B 2.5 bpw 8192 -> 28672, two runs:  358 / 693 / 1333 vs 349 / 641 / 1192
//   EXL2 4.0 bpw 4096 -> 11008, four runs: the LDS kernel at every M.
bool qgemm_split_runs(const qlinear_layout& L, int M) {
  unsigned set = 0;
  for (int r = 0; r < L.nruns; ++r) set |= 1u << L.run_bits[r];
  const int64_t tiles = (int64_t)((L.N + BN - 1) / BN) * ((M + BM - 1) / BM);
  return (set & (set - 1)) != 0 && (int64_t)(L.nruns - 1) * 16384 <= L.K && tiles >= 256;
}

// Slices of K for a call on the LDS-dequant kernel: a grid of few 128 x 128
// tiles leaves most of the about 1024 workgroup slots (four per CU) empty
// while each tile walks all of K, so K is cut into up to 16 slices of at
// least 16 blocks, whose float32 partial sums a second kernel adds. Not for
// calls run in row chunks (activations of 2^31 bytes or more).
int qgemm_k_slices(const qlinear_layout& L, int M) {
  if (M <= 0 || (int64_t)M * L.K * 2 >= ((int64_t)1 << 31)) return 1;
  const int64_t tiles = (int64_t)((L.N + 127) / 128) * ((M + 127) / 128);
  int64_t s = std::min<int64_t>(16, 1024 / tiles);
  s = std::min<int64_t>(s, (L.K / kBlockRows) / 16);
  return (int)std::max<int64_t>(s, 1);
}

// Whether a call without two-level scales takes the LDS-dequant kernel:
// several widths not computed run by run, or one width on a grid of at most
// half a round of 256 x 256 tiles, where the 128 x 128 tiles fill the chip
// better. Measured on MI355X (GPTQ 4-bit g128, us, register-dequant vs LDS
// kernel, both without split K): 4096 -> 4096 at M = 128 / 1024 / 2048 (16 /
// 64 / 128 tiles): 112.9 / 120.7 / 131.4 vs 95.2 / 105.2 / 126.5; 4096 ->
// 11008 at M = 1024 (172 tiles): 137.0 vs 148.0; 5120 -> 13824 at M = 1024 /
// 2048 (216 / 432 tiles): 182.1 / 355.4 vs 223.5 / 400.1.
bool qgemm_lds_path(const qlinear_layout& L, int M) {
  unsigned set = 0;
  for (int r = 0; r < L.nruns; ++r) set |= 1u << L.run_bits[r];
  if ((set & (set - 1)) != 0) return !qgemm_split_runs(L, M);
  const int64_t tiles = (int64_t)((L.N + BN - 1) / BN) * ((M + BM - 1) / BM);
  return tiles <= 128;
}

size_t qgemm_workspace_bytes(const qlinear_layout& L, int M) {
  const size_t xq = ((size_t)M * L.K * 2 + 255) / 256 * 256;
  // Float32 partial sums after the activations: [M][N] for a layout computed
  // run by run, [slices][M][N] for split K (two-level-scale calls take the
  // LDS kernel whatever the layout, so the slices count whenever there are
  // several).
  const size_t runs = qgemm_split_runs(L, M) ? (size_t)M * L.N * 4 : 0;
  const int slices = qgemm_k_slices(L, M);
  const size_t split = slices > 1 ? (size_t)slices * M * L.N * 4 : 0;
  const size_t bytes = xq + std::max(runs, split);
  // Calls run as decode launches use the decode workspace.
  return qgemm_as_decode(L, M) ? std::max(bytes, qgemv_workspace_bytes(L.K)) : bytes;
}

// 17..32 rows: two decode launches of at most 16 rows each (the matrix-core
// decode kernel) take less time than the prefill kernels there, whose tiles
// are 128 rows. Measured on MI355X (GPTQ 4-bit g128 act-order, us): one
// 16-row decode launch 10.2 / 15.1 / 16.5 on 4096 -> 4096 / 4096 -> 11008 /
// 11008 -> 4096, against 39 / 45 / 52 for the prefill path at M = 128.
bool qgemm_as_decode(const qlinear_layout& L, int M) {
  return M > QLINEAR_GEMV_MAX_M && M <= 2 * QLINEAR_GEMV_MAX_M && qgemv_mx_supported(L);
}

bool qgemm_supported(const qlinear_layout& L) {
  // Buffer offsets and sizes are 32-bit: the packed words and the scales must
  // stay below 2^31 bytes (the activations are run in row chunks that do).
  const size_t lim = (size_t)1 << 31;
  return (size_t)L.packed_words * 4 < lim && (size_t)L.groups * L.N * 2 < lim;
}

hipError_t launch_qgemm(const qlinear_layout& L, const Runs& runs, const uint16_t* x, int M,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        const int32_t* perm, uint16_t* y, void* ws, const Epilogue& epi, hipStream_t stream) {
  if (qgemm_as_decode(L, M)) {
    for (int m0 = 0; m0 < M; m0 += QLINEAR_GEMV_MAX_M) {
      const int mc = std::min(QLINEAR_GEMV_MAX_M, M - m0);
      Epilogue ec = epi;   // the chunk's rows of the residual and the addend
      if (ec.residual) ec.residual += (size_t)m0 * L.N;
      if (ec.addend) ec.addend += (size_t)m0 * L.N;
      uint16_t* yc = y + (size_t)m0 * L.N;
      const hipError_t e = launch_qgemv(L, runs, x + (size_t)m0 * L.K, mc, perm, 1, &qweight, &scales,
                                        zeros ? &zeros : nullptr, &yc, ws, ec, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // Row chunks whose gathered activations stay below 2^31 bytes (32-bit
  // buffer offsets); a chunk is a whole number of 256-row tiles.
  const int64_t rows_fit = (((int64_t)1 << 31) - 1) / ((int64_t)L.K * 2);
  const int chunk = (int)std::min<int64_t>(M, std::max<int64_t>(BM, rows_fit / BM * BM));
  for (int m0 = 0; m0 < M; m0 += chunk) {
    const int mc = std::min(chunk, M - m0);
    uint32_t* xq = reinterpret_cast<uint32_t*>(ws);
    // Several code widths not run by run, one width on a small grid, or
    // two-level scales (whose codes only that kernel reads): the kernel that
    // dequantizes into LDS, with split K on small grids. MFMA pair order for
    // the register-dequant kernel; natural order for the other.
    const bool lds = qgemm_lds_path(L, M) || epi.scale_max != nullptr;
    hipError_t e = launch_gather_rows(runs, x + (size_t)m0 * L.K, perm, mc, L.K, xq, !lds, stream);
    if (e != hipSuccess) return e;
    uint16_t* yc = y + (size_t)m0 * L.N;
    Epilogue ec = epi;   // the chunk's rows of the residual and the addend
    if (ec.residual) ec.residual += (size_t)m0 * L.N;
    if (ec.addend) ec.addend += (size_t)m0 * L.N;
    if (lds) {
      float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (((size_t)M * L.K * 2 + 255) / 256 * 256));
      e = launch_qgemm_lds(L, runs, reinterpret_cast<const uint16_t*>(xq), mc, qweight, scales, zeros, yc, ec,
                           qgemm_k_slices(L, M), part, stream);
      if (e != hipSuccess) return e;
      continue;
    }
    GemmArgs a;
    a.xq = reinterpret_cast<const uint16_t*>(xq);
    a.qweight = qweight;
    a.scales = scales;
    a.zeros = zeros;
    a.y = yc;
    a.M = mc;
    a.K = L.K;
    a.N = L.N;
    a.xq_bytes = (int)((size_t)mc * L.K * 2);
    a.qweight_bytes = (int)((size_t)L.packed_words * 4);
    a.scale_bytes = (int)((size_t)L.groups * L.N * 2);
    a.runs = runs;
    a.epi = ec;
    // The float32 partial sums of the chunk's rows follow the activations.
    a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (((size_t)M * L.K * 2 + 255) / 256 * 256));
    const int ntiles = ((L.N + BN - 1) / BN) * ((mc + BM - 1) / BM);
    const dim3 grid(8 * ((ntiles + 7) / 8), 1, 1);
    // One launch per run (a single one for one code width).
    for (int r = 0; r < L.nruns; ++r) {
      a.kb_first = runs.run_block[r];
      a.kb_end = runs.run_block[r + 1];
      a.run_row = runs.run_row[r];
      a.part_mode = L.nruns == 1 ? kWhole : r == 0 ? kFirst : r + 1 == L.nruns ? kLast : kMiddle;
      switch (runs.run_bits[r]) {
        case 2: launch_set<1u << 2>(a, grid, stream); break;
        case 3: launch_set<1u << 3>(a, grid, stream); break;
        case 4: launch_set<1u << 4>(a, grid, stream); break;
        case 5: launch_set<1u << 5>(a, grid, stream); break;
        case 6: launch_set<1u << 6>(a, grid, stream); break;
        default: launch_set<1u << 8>(a, grid, stream); break;
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace qlinear
