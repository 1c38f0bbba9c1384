// Instantiations of the fp16 top-k score kernel for 1- and
// 2-group rotated dimensions (d padded to 32 and 64).
#include "topk_common.hpp"

namespace tq {

void launch_score16_2(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  launch_score16_fixed<2>(a, narrow, grid, st);
}

void launch_score16_4(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  launch_score16_fixed<4>(a, narrow, grid, st);
}

}  // namespace tq
