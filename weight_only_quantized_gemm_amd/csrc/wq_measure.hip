// Measurement helper: a plain streaming read of a device buffer, the practical HBM read
// ceiling that the weight-streaming GEMM is compared against.  It reads every byte once
// with the same 16-byte non-temporal loads (eight per lane, all issued before any use) and
// work-group shape (four waves) as the small-M GEMM, and keeps the data live through a
// data-dependent store that practically never happens.
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

}  // namespace

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
