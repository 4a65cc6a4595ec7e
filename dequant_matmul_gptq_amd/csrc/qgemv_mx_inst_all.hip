// Matrix-core decode kernel instances: any widths (two-launch mode only).
#include "qgemv_mx.hpp"

namespace qlinear {
namespace mxk {

hipError_t launch_all(const MxArgs& a, int fn, bool exact, size_t lds, hipStream_t stream) {
  if (exact) return launch_mode<stream::kAllBits, 1, kGathered | kExact>(a, fn, lds, stream);
  return launch_mode<stream::kAllBits, 1, kGathered>(a, fn, lds, stream);
}

}  // namespace mxk
}  // namespace qlinear
