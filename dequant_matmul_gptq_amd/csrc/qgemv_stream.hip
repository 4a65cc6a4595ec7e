// Host side of the decode path: one launch for 1-4 rows of one width (the
// single-row kernel) and for 1-2 rows of several widths (its several-width
// form), the matrix-core kernel from 3 rows on (see below), otherwise the
// act-order gather into the workspace, then the multi-row VALU kernel
// instantiated for the smallest set of code widths covering the layout.
#include "qgemv_rowmix.hpp"

namespace qlinear {

namespace {
size_t align256(size_t v) { return (v + 255) / 256 * 256; }
}  // namespace

size_t qgemv_workspace_bytes(int K) {
  return align256((size_t)QLINEAR_GEMV_MAX_M * K * sizeof(uint16_t)) +
         align256((size_t)QLINEAR_GEMV_MAX_M * (K / kBlockRows) * sizeof(float2));
}

GemvWorkspace qgemv_workspace(void* ws, int K) {
  GemvWorkspace w;
  w.xq = reinterpret_cast<uint32_t*>(ws);
  w.xsum = reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) +
                                    align256((size_t)QLINEAR_GEMV_MAX_M * K * sizeof(uint16_t)));
  return w;
}

hipError_t launch_qgemv(const qlinear_layout& L, const Runs& runs, const uint16_t* x, int M, const int32_t* perm,
                        int mats, const uint32_t* const* qweights, const uint16_t* const* scales,
                        const uint8_t* const* zeros, uint16_t* const* ys, void* ws, const Epilogue& epi,
                        hipStream_t stream) {
  stream::StreamArgs a;
  a.x = x;
  a.perm = perm;
  a.xq = nullptr;
  a.xsum = nullptr;
  a.mats = mats;
  a.has_zeros = zeros != nullptr && zeros[0] != nullptr;
  for (int i = 0; i < stream::kMaxMats; ++i) {
    const int j = i < mats ? i : 0;   // unused entries repeat matrix 0
    a.mat[i].qweight = qweights[j];
    a.mat[i].scales = scales[j];
    a.mat[i].zeros = a.has_zeros ? zeros[j] : nullptr;
    a.mat[i].y = ys[j];
  }
  a.M = M;
  a.K = L.K;
  a.N = L.N;
  a.nstrips = 0;
  a.strips_per_xcd = 0;
  a.chunk = 1;
  a.xrow_words = 0;
  a.bpg_shift = L.group_size == 128 ? 2 : L.group_size == 64 ? 1 : 0;
  a.runs = runs;
  a.epi = epi;
  unsigned set = 0;
  for (int r = 0; r < L.nruns; ++r) set |= 1u << L.run_bits[r];
  // Measured on MI355X (graph-timed, weights from HBM, 4096^2 to 28672x8192
  // layers): at 1-2 rows the VALU kernels below are 1.1-1.7x faster than the
  // matrix-core kernel; at 3-4 rows the single-row kernel still wins on
  // layers of up to 2 * 4096 * 4096 weights and the matrix-core kernel on
  // larger ones (1.1-1.4x); from 5 rows on the matrix-core kernel wins (up
  // to 1.4x; within 8% on 8-bit layouts). 3-, 4- and 8-bit layers at 3-4
  // rows take the matrix-core kernel above 4096^2 weights, since its
  // one-launch mode widens strips (eager, us at M = 3 / 4, matrix-core vs
  // single-row: 4-bit 5120^2 9.96 / 10.10 vs 13.02 / 12.75, 4096 -> 8192
  // 9.33 / 9.35 vs 10.35 / 9.96; 3-bit 5120^2 13.37 / 13.53 vs 16.03 / 15.76,
  // 4096 -> 8192 equal; 8-bit 5120^2 15.79 / 15.70 vs 19.39 / 19.01, 4096 ->
  // 8192 14.15 / 14.31 vs 16.88 / 16.50; at 4096^2 the single-row kernel is
  // equal or faster). 2-, 5- and 6-bit layers measured equal or faster on
  // the single-row kernel up to 2 * 4096^2.
  // Two-level scales run the kernels that read scale codes: the matrix-core
  // kernel, and the multi-row kernel's several-width instances.
  const bool tl = epi.scale_max != nullptr;
  const bool row = !tl && stream::single_row(M, L.K, set);
  const bool mx_early = set == (1u << 3) || set == (1u << 4) || set == (1u << 8);
  const int64_t row_max = mx_early ? (int64_t)4096 * 4096 : (int64_t)2 * 4096 * 4096;
  // 2 rows of a 4-bit layer with K above 4096 and N of 8192 or more also run
  // the matrix-core kernel (eager, us, matrix-core vs single-row: 5120 ->
  // 13824 13.17 vs 16.35, 5120 -> 15360 13.84 vs 17.12, 8192^2 13.09 vs
  // 14.59, 8192 -> 28672 equal; the K = 4096 layers, 11008 -> 4096 and
  // 5120^2 stay faster on the single-row kernel).
  const bool mx2 = M == 2 && row && set == (1u << 4) && L.K > 4096 && L.N >= 8192 && !epi.addend &&
                   qgemv_mx_supported(L);
  if (mx2 || (M >= 3 && !(row && (int64_t)L.K * L.N <= row_max)))
    return launch_qgemv_mx(L, runs, x, M, perm, mats, qweights, scales, zeros, ys, ws, epi, stream);
  // A float32 addend (a LoRA update) runs instances of their own: reading one
  // more kernel argument in the prologue cost 3% on the 7B decode step
  // (measured on MI355X), so the plain instances do not.
  if (row) return epi.addend ? stream::launch_row_set_addend(set, a, stream) : stream::launch_row_set(set, a, stream);
  // One or two rows, several widths (or two-level scales): the one-launch
  // kernel that runs the single-row scheme run segment by segment.
  if (!epi.addend && stream::mixed_row(M, L.K, L.N, mats, set, tl)) {
    if ((set & ~stream::kLowBits) == 0)
      return tl ? stream::launch_rowmix_low_tl(a, stream) : stream::launch_rowmix_low(a, stream);
    if ((set & ~stream::kMidBits) == 0)
      return tl ? stream::launch_rowmix_mid_tl(a, stream) : stream::launch_rowmix_mid(a, stream);
    return tl ? stream::launch_rowmix_all_tl(a, stream) : stream::launch_rowmix_all(a, stream);
  }
  // 1-2 rows: the activations are gathered into the workspace (with the
  // per-block sums of the factored form) by a kernel of their own.
  const GemvWorkspace w = qgemv_workspace(ws, L.K);
  const hipError_t e = launch_gather_pairs(runs, x, perm, M, L.K, w.xq, w.xsum, true, false, stream);
  if (e != hipSuccess) return e;
  a.xq = w.xq;
  a.xsum = w.xsum;
  if (!tl && (set & (set - 1)) == 0) return stream::launch_uniform(set, a, stream);
  return stream::launch_mixed(set, a, stream);
}

}  // namespace qlinear
