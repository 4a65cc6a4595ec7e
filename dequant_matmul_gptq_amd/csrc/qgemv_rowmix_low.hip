// One-launch M = 1-2 decode kernels for layouts of several code widths,
// widths 2-3 bits (EXL2 at about 2-3 bpw).
#include "qgemv_rowmix.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_rowmix_low(const StreamArgs& a, hipStream_t stream) { return launch_rowmix_set<kLowBits>(a, stream); }

}  // namespace stream
}  // namespace qlinear
