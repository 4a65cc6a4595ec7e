// One-launch M = 1-2 decode kernels with two-level scales (4-bit scale codes
// and a float16 maximum per output), widths any of 2, 3, 4, 5, 6 and 8 bits.
#include "qgemv_rowmix.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_rowmix_all_tl(const StreamArgs& a, hipStream_t stream) {
  return launch_rowmix_set<kAllBits | kTwoLevelBit>(a, stream);
}

}  // namespace stream
}  // namespace qlinear
