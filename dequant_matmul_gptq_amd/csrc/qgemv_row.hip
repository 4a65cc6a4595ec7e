// Single-row decode kernels, one per code width (no addend).
#include "qgemv_m1.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_row_set(unsigned set, const StreamArgs& a, hipStream_t stream) {
  switch (set) {
    case 1u << 2: return launch_row_width<2, false>(a, stream);
    case 1u << 3: return launch_row_width<3, false>(a, stream);
    case 1u << 4: return launch_row_width<4, false>(a, stream);
    case 1u << 5: return launch_row_width<5, false>(a, stream);
    case 1u << 6: return launch_row_width<6, false>(a, stream);
    case 1u << 8: return launch_row_width<8, false>(a, stream);
    default: return hipErrorInvalidValue;   // single_row() admits one width only
  }
}

}  // namespace stream
}  // namespace qlinear
