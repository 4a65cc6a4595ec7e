// Single-row decode kernels with a float32 addend in the epilogue (e.g. an
// on-the-fly LoRA update), one per code width.
#include "qgemv_m1.hpp"

namespace qlinear {
namespace stream {

hipError_t launch_row_set_addend(unsigned set, const StreamArgs& a, hipStream_t stream) {
  switch (set) {
    case 1u << 2: return launch_row_width<2, true>(a, stream);
    case 1u << 3: return launch_row_width<3, true>(a, stream);
    case 1u << 4: return launch_row_width<4, true>(a, stream);
    case 1u << 5: return launch_row_width<5, true>(a, stream);
    case 1u << 6: return launch_row_width<6, true>(a, stream);
    case 1u << 8: return launch_row_width<8, true>(a, stream);
    default: return hipErrorInvalidValue;   // single_row() admits one width only
  }
}

}  // namespace stream
}  // namespace qlinear
