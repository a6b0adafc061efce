// Tiled W8A16 GEMM instances: E4M3 weights, fp16 activations (the kernel is in
// wq_tile_kernel.h).
#include "wq_tile_kernel.h"

namespace wq {

hipError_t launch_tile_fp8(const TileArgs& p, bool grouped, hipStream_t stream) {
  return launch_tile_fp8_any(p, grouped, stream);
}

}  // namespace wq
