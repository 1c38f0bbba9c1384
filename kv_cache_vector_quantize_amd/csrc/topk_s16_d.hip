// Instantiations of the fp16 top-k score kernel for 7- and
// 8-group rotated dimensions (d padded to 224 and 256).
#include "topk_common.hpp"

namespace tq {

void launch_score16_14(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  launch_score16_fixed<14>(a, narrow, grid, st);
}

void launch_score16_16(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  launch_score16_fixed<16>(a, narrow, grid, st);
}

}  // namespace tq
