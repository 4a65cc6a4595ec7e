// One-launch M = 1-2 decode kernels with two-level scales (4-bit scale codes
// and a float16 maximum per output), widths 2-3 bits (EXL2 at about 2-3 bpw).
#include "qgemv_rowmix.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_rowmix_low_tl(const StreamArgs& a, hipStream_t stream) {
  return launch_rowmix_set<kLowBits | kTwoLevelBit>(a, stream);
}

}  // namespace stream
}  // namespace qlinear
