// Grouped small-M instances (segments of few rows) for bf16 activations
// (32-row scale units, 4 per 128-row chunk).
#include "wq_small_kernel.h"

namespace wq {

hipError_t launch_seg_bf16_g4(const GroupedProblem& p, int rows, const SmallPlan& plan,
                              hipStream_t stream) {
  return launch_seg_gpc<4, true>(p, rows, plan, stream);
}

}  // namespace wq
