// Small-M GEMM instances: E4M3 weights, bf16 activations, 128-row scale units.
#include "wq_small_kernel.h"

namespace wq {

hipError_t launch_small_fp8_bf16(const uint16_t* a, int lda, int m, const uint32_t* b,
                                 const uint16_t* s, uint16_t* c, int n, int k,
                                 const SmallPlan& plan, float* partials, hipStream_t stream) {
  return launch_small_w8<true>(a, lda, m, b, s, c, n, k, plan, partials, stream);
}

}  // namespace wq
