// Matrix-core decode kernel instances: widths 3-6, one-launch modes.
#include "qgemv_mx.hpp"

namespace qlinear {
namespace mxk {

hipError_t launch_mid_few(const MxArgs& a, int fn, int mode, size_t lds, hipStream_t stream) {
  if (exact_mode(mode)) return launch_mode<stream::kMidBits, 1, kFewRows | kExact>(a, fn, lds, stream);
  return launch_mode<stream::kMidBits, 1, kFewRows>(a, fn, lds, stream);
}

}  // namespace mxk
}  // namespace qlinear
