// Streaming decode kernels for 4 < M <= 16 (any code widths).
#include "qgemv_stream.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_wide(const StreamArgs& a, hipStream_t stream) {
  if (a.M <= 8) return launch_set<8, kAllBits, 4>(a, stream);
  return launch_set<16, kAllBits, 4>(a, stream);
}

}  // namespace stream
}  // namespace qlinear
