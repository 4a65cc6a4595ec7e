// One-launch M = 1-2 decode kernels for layouts of several code widths,
// widths any of 2, 3, 4, 5, 6 and 8 bits.
#include "qgemv_rowmix.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_rowmix_all(const StreamArgs& a, hipStream_t stream) { return launch_rowmix_set<kAllBits>(a, stream); }

}  // namespace stream
}  // namespace qlinear
