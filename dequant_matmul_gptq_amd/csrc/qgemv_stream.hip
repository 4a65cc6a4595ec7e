// Host side of the decode path: workspace layout, the act-order gather, and
// the choice of the streaming kernel instantiated for the smallest set of code
// widths covering the layout.
#include "qgemv_stream.hpp"

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

hipError_t launch_qgemv_gather(const qlinear_layout& L, const Runs& runs, const uint16_t* x, int M,
                               const int32_t* perm, void* ws, hipStream_t stream) {
  const GemvWorkspace w = qgemv_workspace(ws, L.K);
  return launch_gather_pairs(runs, x, perm, M, L.K, w.xq, w.xsum, true, stream);
}

hipError_t launch_qgemv_apply(const qlinear_layout& L, const Runs& runs, int M, const uint32_t* qweight,
                              const uint16_t* scales, const uint8_t* zeros, uint16_t* y, void* ws,
                              hipStream_t stream) {
  const GemvWorkspace w = qgemv_workspace(ws, L.K);
  stream::StreamArgs a;
  a.xq = w.xq;
  a.xsum = w.xsum;
  a.qweight = qweight;
  a.scales = scales;
  a.zeros = zeros;
  a.y = y;
  a.M = M;
  a.K = L.K;
  a.N = L.N;
  a.nstrips = 0;
  a.strips_per_xcd = 0;
  a.chunk = 1;
  a.bpg_shift = L.group_size == 128 ? 2 : L.group_size == 64 ? 1 : 0;
  a.runs = runs;
  if (M > 4) return stream::launch_wide(a, stream);
  unsigned set = 0;
  for (int r = 0; r < L.nruns; ++r) set |= 1u << L.run_bits[r];
  if ((set & (set - 1)) == 0) return stream::launch_uniform(set, a, stream);
  return stream::launch_mixed(set, a, stream);
}

}  // namespace qlinear
