// Matrix-core decode kernel instances: widths 2-3.
#include "qgemv_mx.hpp"

namespace qlinear {
namespace mxk {

hipError_t launch_low(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream) {
  return launch_set<stream::kLowBits, 1>(a, fn, mode, lds, stream);
}

}  // namespace mxk
}  // namespace qlinear
