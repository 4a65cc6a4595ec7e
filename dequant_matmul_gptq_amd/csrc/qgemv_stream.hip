// Host side of the decode path: the single-row kernel for M = 1, otherwise
// the act-order gather into the workspace, then for M <= 4 the multi-row
// VALU kernel instantiated for the smallest set of code widths covering the
// layout, and for 5 <= M <= 16 the MFMA kernel.
#include "qgemv_m1.hpp"

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
                        const uint8_t* const* zeros, uint16_t* const* ys, void* ws, hipStream_t stream) {
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
  unsigned set = 0;
  for (int r = 0; r < L.nruns; ++r) set |= 1u << L.run_bits[r];
  if (stream::single_row(M, L.K, set)) return stream::launch_row_set(set, a, stream);
  // The activations are gathered into the workspace by a kernel of their own.
  const GemvWorkspace w = qgemv_workspace(ws, L.K);
  if (M > 4 && qgemv_mfma_supported(L)) {
    // 5 to 16 rows: one MFMA row tile, unscaled activations. (Measured on
    // MI355X: up to 4 rows the factored VALU kernel below is as fast or
    // faster; from 8 rows on, the MFMA kernel is 3-7x faster.)
    const hipError_t e = launch_gather_pairs(runs, x, perm, M, L.K, w.xq, nullptr, false, stream);
    if (e != hipSuccess) return e;
    return launch_qgemv_mfma(L, runs, w.xq, M, mats, qweights, scales, zeros, ys, stream);
  }
  const hipError_t e = launch_gather_pairs(runs, x, perm, M, L.K, w.xq, w.xsum, true, stream);
  if (e != hipSuccess) return e;
  a.xq = w.xq;
  a.xsum = w.xsum;
  if (M > 4) return stream::launch_wide(a, stream);
  if ((set & (set - 1)) == 0) return stream::launch_uniform(set, a, stream);
  return stream::launch_mixed(set, a, stream);
}

}  // namespace qlinear
