// One-launch M = 1-2 decode kernels for layouts of several code widths,
// widths 3-6 bits (EXL2 at about 3.5-5 bpw).
#include "qgemv_rowmix.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_rowmix_mid(const StreamArgs& a, hipStream_t stream) { return launch_rowmix_set<kMidBits>(a, stream); }

}  // namespace stream
}  // namespace qlinear
