// Multi-row (2 <= M <= 4) decode kernels for matrices with a single code width.
#include "qgemv_stream.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_uniform(unsigned set, const StreamArgs& a, hipStream_t stream) {
  switch (set) {
    case 1u << 2: return launch_set_small_m<1u << 2>(a, stream);
    case 1u << 3: return launch_set_small_m<1u << 3>(a, stream);
    case 1u << 4: return launch_set_small_m<1u << 4>(a, stream);
    case 1u << 5: return launch_set_small_m<1u << 5>(a, stream);
    case 1u << 6: return launch_set_small_m<1u << 6>(a, stream);
    default: return launch_set_small_m<1u << 8>(a, stream);
  }
}

}  // namespace stream
}  // namespace qlinear
