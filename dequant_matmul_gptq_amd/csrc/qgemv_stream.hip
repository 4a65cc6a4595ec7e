// Host side of the decode path: the single-row kernel for M = 1, otherwise
// the act-order gather into the workspace, then the MFMA kernel (M >= 3, see
// below) or the multi-row VALU kernel instantiated for the smallest set of
// code widths covering the layout.
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
  // The single-launch kernel takes no float32 addend: reading one more kernel
  // argument in its prologue cost 3% on the 7B decode step (measured on
  // MI355X), so calls with an addend (a LoRA update) run the kernels below.
  if (!epi.addend && stream::single_row(M, L.K, set)) return stream::launch_row_set(set, a, stream);
  // The activations are gathered into the workspace by a kernel of their own.
  const GemvWorkspace w = qgemv_workspace(ws, L.K);
  // 3 to 16 rows: one MFMA row tile, unscaled activations in MFMA pair order.
  // Measured on MI355X: the factored VALU kernel below is faster at 2 rows,
  // and at 3-4 rows for single-width 3, 5 and 6-bit layouts (whose k-groups
  // spread over several words); the MFMA kernel wins at 3-4 rows on every
  // other shape measured (up to 1.7x) and from 5 rows on everywhere (3-7x at
  // 8-16 rows).
  const bool spread = set == (1u << 3) || set == (1u << 5) || set == (1u << 6);
  if (M > 4 || (M > 2 && !spread)) {
    const hipError_t e = launch_gather_pairs(runs, x, perm, M, L.K, w.xq, nullptr, false, true, stream);
    if (e != hipSuccess) return e;
    return launch_qgemv_mfma(L, runs, w.xq, M, mats, qweights, scales, zeros, ys, epi, stream);
  }
  const hipError_t e = launch_gather_pairs(runs, x, perm, M, L.K, w.xq, w.xsum, true, false, stream);
  if (e != hipSuccess) return e;
  a.xq = w.xq;
  a.xsum = w.xsum;
  if ((set & (set - 1)) == 0) return stream::launch_uniform(set, a, stream);
  return stream::launch_mixed(set, a, stream);
}

}  // namespace qlinear
