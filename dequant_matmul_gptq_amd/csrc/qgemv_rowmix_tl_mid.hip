// One-launch M = 1-2 decode kernels with two-level scales (4-bit scale codes
// and a float16 maximum per output), widths 3-6 bits (EXL2 at about 3.5-5 bpw).
#include "qgemv_rowmix.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_rowmix_mid_tl(const StreamArgs& a, hipStream_t stream) {
  return launch_rowmix_set<kMidBits | kTwoLevelBit>(a, stream);
}

}  // namespace stream
}  // namespace qlinear
