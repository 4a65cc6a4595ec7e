// Matrix-core decode kernel instances: 4-bit codes (GPTQ): scale units of 4 blocks (128-row groups) or 1.
#include "qgemv_mx.hpp"

namespace qlinear {
namespace mxk {

hipError_t launch_set4_ub4(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream) {
  return launch_set<kSet4, 4>(a, fn, mode, lds, stream);
}
hipError_t launch_set4_ub1(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream) {
  return launch_set<kSet4, 1>(a, fn, mode, lds, stream);
}

}  // namespace mxk
}  // namespace qlinear
