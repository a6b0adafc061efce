// Tiled GEMM instances for E4M3 weights, fp16 or bf16 activations (the kernel is in
// wq_tile_kernel.h).
#include "wq_tile_kernel.h"

namespace wq {

hipError_t launch_tile_fp8(const TileArgs& p, bool grouped, bool swiglu, bool bf16,
                           hipStream_t stream) {
  return bf16 ? launch_tile_fp8_type<true>(p, grouped, swiglu, stream)
              : launch_tile_fp8_type<false>(p, grouped, swiglu, stream);
}

}  // namespace wq
