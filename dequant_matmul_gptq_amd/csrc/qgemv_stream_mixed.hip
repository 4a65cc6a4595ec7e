// Multi-row (2 <= M <= 4) decode kernels for mixed-width (EXL2) matrices.
#include "qgemv_stream.hpp"

namespace qlinear {
namespace stream {


hipError_t launch_mixed(unsigned set, const StreamArgs& a, hipStream_t stream) {
  if (a.epi.scale_max) {   // two-level scales (any layout, one width included)
    if ((set & ~kLowBits) == 0) return launch_set_small_m<kLowBits | kTwoLevelBit>(a, stream);
    if ((set & ~kMidBits) == 0) return launch_set_small_m<kMidBits | kTwoLevelBit>(a, stream);
    return launch_set_small_m<kAllBits | kTwoLevelBit>(a, stream);
  }
  if ((set & ~kLowBits) == 0) return launch_set_small_m<kLowBits>(a, stream);
  if ((set & ~kMidBits) == 0) return launch_set_small_m<kMidBits>(a, stream);
  return launch_set_small_m<kAllBits>(a, stream);
}

}  // namespace stream
}  // namespace qlinear
