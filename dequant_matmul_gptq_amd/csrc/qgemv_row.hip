// Single-row decode kernels, one per set of code widths.
#include "qgemv_m1.hpp"

namespace qlinear {
namespace stream {


hipError_t launch_row_set(unsigned set, const StreamArgs& a, hipStream_t stream) {
  switch (set) {
    case 1u << 2: return launch_row_any<1u << 2, 8>(a, stream);
    case 1u << 3: return launch_row_any<1u << 3, 8>(a, stream);
    case 1u << 4: return launch_row_any<1u << 4, 8>(a, stream);
    case 1u << 5: return launch_row_any<1u << 5, 8>(a, stream);
    case 1u << 6: return launch_row_any<1u << 6, 8>(a, stream);
    case 1u << 8: return launch_row_any<1u << 8, 8>(a, stream);
    default: break;
  }
  if ((set & ~kLowBits) == 0) return launch_row_any<kLowBits, 8>(a, stream);
  if ((set & ~kMidBits) == 0) return launch_row_any<kMidBits, 8>(a, stream);
  return launch_row_any<kAllBits, 8>(a, stream);
}

}  // namespace stream
}  // namespace qlinear
