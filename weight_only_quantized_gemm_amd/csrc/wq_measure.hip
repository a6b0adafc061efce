// Measurement helpers, not steps of the method:
//  - a plain streaming read of a device buffer, the practical HBM read ceiling that the
//    weight-streaming GEMM is compared against.  It reads every byte once with the same
//    16-byte non-temporal loads (eight per lane, all issued before any use) and work-group
//    shape (four waves) as the small-M GEMM, and keeps the data live through a
//    data-dependent store that practically never happens;
//  - a register-only loop of the tiled GEMM's fp16 MFMAs on every CU, the practical matrix
//    rate (the chip lowers its clock with the operands' switching activity, so the rate
//    depends on the data the caller supplies).
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int kPerLane = 8;  // 16-byte loads per lane

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          long granules,
                                                          uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long base = wave * kPerLane * 64;
  u32x4 v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const long g = base + i * 64 + lane;
    v[i] = __builtin_nontemporal_load(src + (g < granules ? g : granules - 1));
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  if (x == 0x9E3779B9u) sink[wave] = x;
}

// One work-group per CU (the dynamic LDS the launch requests keeps a second one away), two
// waves per SIMD: each wave holds the A operands of four 32-row blocks and the B operands of
// two 32-column blocks, the tiled GEMM's 128 x 64 wave tile, and runs `iters` steps of the
// eight 32x32x16 products into eight fp32 accumulators.  Every thread stores its sum.
__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(const f16x8* __restrict__ ops,
                                                                 int iters,
                                                                 float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f16x8 a[4], b[2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) a[rb] = ops[rb * 64 + lane];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) b[cb] = ops[(4 + cb) * 64 + lane];
  f32x16 acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma32x32x16(a[rb], b[cb], acc[rb][cb]);
  }
  float x = 0.f;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x += acc[rb][cb][r];
  sink[(long)blockIdx.x * kMfmaThreads + threadIdx.x] = x;
}

}  // namespace

hipError_t launch_mfma_loop(const void* ops, int iters, float* sink, hipStream_t stream) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_loop_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kMfmaLds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(kMfmaBlocks), dim3(kMfmaThreads), kMfmaLds, stream,
                     static_cast<const f16x8*>(ops), iters, sink);
  return hipGetLastError();
}

long stream_read_sink_words(size_t bytes) {
  const long granules = (long)(bytes / 16);
  const long per_wave = kPerLane * 64;
  const long waves = (granules + per_wave - 1) / per_wave;
  return (waves + 3) / 4 * 4;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink,
                              hipStream_t stream) {
  const long granules = (long)(bytes / 16);
  const long blocks = stream_read_sink_words(bytes) / 4;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), granules, sink);
  return hipGetLastError();
}

}  // namespace wq
