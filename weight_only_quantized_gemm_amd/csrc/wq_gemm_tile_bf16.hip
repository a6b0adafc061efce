// Tiled W4A16 GEMM instances for bf16 activations (the kernel is in wq_tile_kernel.h).
#include "wq_tile_kernel.h"

namespace wq {

hipError_t launch_tile_bf16(const TileArgs& p, bool grouped, bool swiglu, bool zp, int gpc,
                            bool tall, hipStream_t stream) {
  return launch_tile_type<true>(p, grouped, swiglu, zp, gpc, tall, stream);
}

}  // namespace wq
