// Instantiations of the fp16 top-k score kernel for 3- and
// 4-group rotated dimensions (d padded to 96 and 128).
#include "topk_common.hpp"

namespace tq {

void launch_score16_6(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  launch_score16_fixed<6>(a, narrow, grid, st);
}

void launch_score16_8(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  launch_score16_fixed<8>(a, narrow, grid, st);
}

}  // namespace tq
