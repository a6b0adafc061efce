// Small-M W4A16 GEMM (m <= 16): decode and small batches, bound by the weight stream.
//
// One 16x16x32 fp16 MFMA block covers all m rows (rows >= m read as zero), so the packed
// weights are read exactly once.  A work-group owns `NB` 16-column blocks and a range of
// K; its four waves split that range, each streaming one 1 KiB layout chunk per 128-row
// group and 16-column block with a single 16-byte load per lane.  Codes become exact
// fp16 integers (q - z) in registers; each group's MFMA partial is scaled by the fp16
// group scale in fp32 and accumulated in fp32.
//
// Split-K (`splits` > 1 work-groups per column block) follows the pages' fp32 reduce
// (ferrum-kernels marlin.rs, `ferrum_vllm_marlin_moe_f16`: `use_fp32_reduce` with an fp32
// `c_tmp`): each split stores its fp32 partial tile, and the last work-group to arrive on
// the column block's counter adds the partials in split order 0..S-1 (a fixed order, so
// results do not depend on arrival order or device size: memra mmq_ffi.rs records that
// fold-order changes flipped outputs), writes fp16 C and resets the counter to zero.
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

template <bool ZP, int NB, int DEPTH>
__global__ __launch_bounds__(256) void gemm_small_kernel(
    const f16* __restrict__ a, int lda, int m, const u32x4* __restrict__ b,
    const f16* __restrict__ s, const u32x2* __restrict__ z, f16* __restrict__ c, int n,
    int groups, int splits, float* __restrict__ partials, int32_t* __restrict__ counters) {
  __shared__ f32x4 red[4][NB][64];
  __shared__ int is_last;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // column inside a 16-column block; also the A row of the lane
  const int qd = lane >> 4;   // which 8 rows of each 32-row MFMA step the lane carries
  const int nb0 = blockIdx.x * NB;
  const int split = blockIdx.y;

  const int gs0 = (int)((long)groups * split / splits);
  const int gs1 = (int)((long)groups * (split + 1) / splits);
  const int span = gs1 - gs0;
  const int g0 = gs0 + span * wave / 4;
  const int g1 = gs0 + span * (wave + 1) / 4;

  const bool row_ok = col < m;
  const f16* arow = a + (long)(row_ok ? col : 0) * lda + 8 * qd;

  f32x4 acc[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) acc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int gb = g0; gb < g1; gb += DEPTH) {
    const int cnt = min(DEPTH, g1 - gb);
    u32x4 bw[DEPTH][NB];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        if (i < cnt) bw[i][bb] = b[((long)(nb0 + bb) * groups + gb + i) * 64 + lane];

#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      if (i < cnt) {
        const int g = gb + i;
        f16x8 av[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          av[j] = row_ok ? *reinterpret_cast<const f16x8*>(arow + (long)g * kGroup + 32 * j)
                         : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const long blk = (long)(nb0 + bb) * groups + g;
          const float sc = (float)s[blk * 16 + col];
          const ZeroOffsets zo = zero_offsets(ZP ? zero_code(z[blk], col) : 8);
          f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) p = mfma16x16x32(av[j], dequant8(bw[i][bb][j], zo), p);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[bb][r] = __builtin_fmaf(sc, p[r], acc[bb][r]);
        }
      }
    }
  }

  // Work-group reduce over the four waves, in wave order.
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) red[wave][bb][lane] = acc[bb];
  __syncthreads();

  f32x4 tot[NB];
  if (wave == 0) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      f32x4 t = red[0][bb][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) t += red[w][bb][lane];
      tot[bb] = t;
    }
  }

  // Output layout of the 16x16 block: lane holds rows 4*qd + r of column `col`.
  if (splits == 1) {
    if (wave == 0) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * qd + r;
          if (row < m) c[(long)row * n + (nb0 + bb) * 16 + col] = (f16)tot[bb][r];
        }
    }
    return;
  }

  if (wave == 0) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * qd + r;
        if (row < m) partials[((long)split * m + row) * n + (nb0 + bb) * 16 + col] = tot[bb][r];
      }
    __threadfence();  // release this split's partials at device scope
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&counters[blockIdx.x], 1);
    const int last = prev == splits - 1;
    if (last) __hip_atomic_store(&counters[blockIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = last;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();  // acquire the other splits' partials

  if (wave == 0) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * qd + r;
        if (row >= m) continue;
        const long colx = (long)(nb0 + bb) * 16 + col;
        float sum = 0.f;
        for (int sp = 0; sp < splits; ++sp) {
          const float v = sp == split ? tot[bb][r] : partials[((long)sp * m + row) * n + colx];
          sum = sp == 0 ? v : sum + v;
        }
        c[(long)row * n + colx] = (f16)sum;
      }
  }
}

template <bool ZP, int NB, int DEPTH>
hipError_t launch_small_t(const uint16_t* a, int lda, int m, const uint32_t* b,
                          const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                          int splits, float* partials, int32_t* counters, hipStream_t stream) {
  const dim3 grid(n / (16 * NB), splits);
  hipLaunchKernelGGL((gemm_small_kernel<ZP, NB, DEPTH>), grid, dim3(256), 0, stream,
                     reinterpret_cast<const f16*>(a), lda, m,
                     reinterpret_cast<const u32x4*>(b), reinterpret_cast<const f16*>(s),
                     reinterpret_cast<const u32x2*>(z), reinterpret_cast<f16*>(c), n,
                     k / kGroup, splits, partials, counters);
  return hipGetLastError();
}

template <bool ZP, int NB>
hipError_t launch_small_depth(const uint16_t* a, int lda, int m, const uint32_t* b,
                              const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                              const SmallPlan& plan, float* partials, int32_t* counters,
                              hipStream_t stream) {
  switch (plan.depth) {
    case 1: return launch_small_t<ZP, NB, 1>(a, lda, m, b, s, z, c, n, k, plan.splits, partials, counters, stream);
    case 2: return launch_small_t<ZP, NB, 2>(a, lda, m, b, s, z, c, n, k, plan.splits, partials, counters, stream);
    case 4: return launch_small_t<ZP, NB, 4>(a, lda, m, b, s, z, c, n, k, plan.splits, partials, counters, stream);
    default: return launch_small_t<ZP, NB, 8>(a, lda, m, b, s, z, c, n, k, plan.splits, partials, counters, stream);
  }
}

template <bool ZP>
hipError_t launch_small_nb(const uint16_t* a, int lda, int m, const uint32_t* b,
                           const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                           const SmallPlan& plan, float* partials, int32_t* counters,
                           hipStream_t stream) {
  switch (plan.nb) {
    case 1: return launch_small_depth<ZP, 1>(a, lda, m, b, s, z, c, n, k, plan, partials, counters, stream);
    case 2: return launch_small_depth<ZP, 2>(a, lda, m, b, s, z, c, n, k, plan, partials, counters, stream);
    default: return launch_small_depth<ZP, 4>(a, lda, m, b, s, z, c, n, k, plan, partials, counters, stream);
  }
}

}  // namespace

hipError_t launch_gemm_small(const uint16_t* a, int lda, int m, const uint32_t* b,
                             const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                             const SmallPlan& plan, float* partials, int32_t* counters,
                             hipStream_t stream) {
  if (z != nullptr)
    return launch_small_nb<true>(a, lda, m, b, s, z, c, n, k, plan, partials, counters, stream);
  return launch_small_nb<false>(a, lda, m, b, s, z, c, n, k, plan, partials, counters, stream);
}

}  // namespace wq
