// Instantiations of the fp16 top-k score kernel for 5- and
// 6-group rotated dimensions (d padded to 160 and 192).
#include "topk_common.hpp"

namespace tq {

void launch_score16_10(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  launch_score16_fixed<10>(a, narrow, grid, st);
}

void launch_score16_12(const IS2Args& a, bool narrow, dim3 grid, hipStream_t st) {
  launch_score16_fixed<12>(a, narrow, grid, st);
}

}  // namespace tq
