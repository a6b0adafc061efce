// Grouped small-M instances (segments of few rows) for bf16 activations
// (128-row scale units, 1 per 128-row chunk).
#include "wq_small_kernel.h"

namespace wq {

hipError_t launch_seg_bf16_g1(const GroupedProblem& p, int rows, const SmallPlan& plan,
                              hipStream_t stream) {
  return launch_seg_gpc<1, true>(p, rows, plan, stream);
}

}  // namespace wq
