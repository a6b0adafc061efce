// Small-M W4A16 GEMM instances for fp16 activations
// (16-row scale units, 8 per 128-row chunk).
#include "wq_small_kernel.h"

namespace wq {

hipError_t launch_small_g8(const uint16_t* a, int lda, int m, const uint32_t* b,
                           const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                           const SmallPlan& plan, float* partials, hipStream_t stream) {
  return launch_small_gpc<8, false>(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
}

}  // namespace wq
