// Grouped small-M instances (segments of few rows) for fp16 activations
// (64-row scale units, 2 per 128-row chunk).
#include "wq_small_kernel.h"

namespace wq {

hipError_t launch_seg_g2(const GroupedProblem& p, int rows, const SmallPlan& plan,
                         hipStream_t stream) {
  return launch_seg_gpc<2, false>(p, rows, plan, stream);
}

}  // namespace wq
