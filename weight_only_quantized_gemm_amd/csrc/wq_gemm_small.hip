// Small-M W4A16 GEMM: the split-K reduce, the plan check and the dispatch over scale
// groups per 128-row chunk; the kernel itself and its 1-group instances come from
// wq_small_kernel.h (2- and 4-group instances live in their own translation units).
//
// Split-K (`splits` > 1 work-groups per column block) follows the pages' fp32 reduce
// (ferrum-kernels marlin.rs, `ferrum_vllm_marlin_moe_f16`: `use_fp32_reduce` with an fp32
// `c_tmp`): each split stores its fp32 partial tile to the workspace and a second kernel
// adds the partials in split order 0..S-1 and rounds once to fp16.  The order is fixed, so
// results do not depend on scheduling or device size (memra mmq_ffi.rs records that
// fold-order changes flipped outputs).  The kernel boundary orders the partial stores
// before the reduce's loads; a device-scope fence inside the GEMM would instead write back
// and invalidate a whole L2 per work-group on this multi-L2 part.
#include "wq_small_kernel.h"

namespace wq {
namespace {

constexpr int kReduceSplits = 16;  // most splits the reduce adds (every caller's limit)

// c[row][col] = round(sum over splits 0..S-1 of partials[split][row][col]) to fp16 or bf16,
// eight columns per thread, added in split order.  PRELOAD issues every split's loads
// before the sums, for reduces too small to fill the CUs (latency-bound: M=1, N=256 or
// 512 with 8 splits, 5.8 -> 4.6 and 5.3 -> 4.5 us per product on MI355X); the plain loop
// streams larger ones (1% faster at M=64 and 256, N=14336).
template <bool BF16, bool PRELOAD>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ partials,
                                                            uint16_t* __restrict__ c, int m,
                                                            int n, int splits) {
  const long per_split = (long)m * n;
  const long total = per_split / 8;
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (long)gridDim.x * blockDim.x) {
    const long e = t * 8;
    f32x4 lo, hi;
    if constexpr (PRELOAD) {
      f32x4 vlo[kReduceSplits], vhi[kReduceSplits];
#pragma unroll
      for (int sp = 0; sp < kReduceSplits; ++sp) {
        if (sp < splits) {
          vlo[sp] = *reinterpret_cast<const f32x4*>(partials + sp * per_split + e);
          vhi[sp] = *reinterpret_cast<const f32x4*>(partials + sp * per_split + e + 4);
        }
      }
      lo = vlo[0];
      hi = vhi[0];
#pragma unroll
      for (int sp = 1; sp < kReduceSplits; ++sp) {
        if (sp < splits) {
          lo += vlo[sp];
          hi += vhi[sp];
        }
      }
    } else {
      lo = *reinterpret_cast<const f32x4*>(partials + e);
      hi = *reinterpret_cast<const f32x4*>(partials + e + 4);
      for (int sp = 1; sp < splits; ++sp) {
        lo += *reinterpret_cast<const f32x4*>(partials + sp * per_split + e);
        hi += *reinterpret_cast<const f32x4*>(partials + sp * per_split + e + 4);
      }
    }
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = j < 2 ? lo[2 * j] : hi[2 * j - 4];
      const float x1 = j < 2 ? lo[2 * j + 1] : hi[2 * j - 3];
      out[j] = (uint32_t)Act<BF16>::round(x0) | ((uint32_t)Act<BF16>::round(x1) << 16);
    }
    *reinterpret_cast<u32x4*>(c + e) = out;
  }
}

}  // namespace

hipError_t launch_reduce_splits(const float* partials, uint16_t* c, int m, int n, int splits,
                                bool bf16, hipStream_t stream) {
  if (splits < 1 || splits > kReduceSplits) return hipErrorInvalidValue;
  long blocks = ((long)m * n / 8 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  const bool preload = blocks < 256;  // fewer blocks than CUs
  const dim3 grid((unsigned)blocks);
  if (bf16) {
    if (preload)
      hipLaunchKernelGGL((reduce_splits_kernel<true, true>), grid, dim3(256), 0, stream,
                         partials, c, m, n, splits);
    else
      hipLaunchKernelGGL((reduce_splits_kernel<true, false>), grid, dim3(256), 0, stream,
                         partials, c, m, n, splits);
  } else {
    if (preload)
      hipLaunchKernelGGL((reduce_splits_kernel<false, true>), grid, dim3(256), 0, stream,
                         partials, c, m, n, splits);
    else
      hipLaunchKernelGGL((reduce_splits_kernel<false, false>), grid, dim3(256), 0, stream,
                         partials, c, m, n, splits);
  }
  return hipGetLastError();
}

hipError_t launch_small_g1(const uint16_t* a, int lda, int m, const uint32_t* b,
                           const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                           const SmallPlan& plan, float* partials, hipStream_t stream) {
  return launch_small_gpc<1, false>(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
}

bool small_plan_fits(int m, int k, const SmallPlan& plan) {
  const int groups = k / kGroup;
  if (plan.gpc != 1 && plan.gpc != 2 && plan.gpc != 4 && plan.gpc != 8) return false;
  if (plan.splits < 1 || plan.splits > groups) return false;
  if (plan.pair && plan.splits != 1) return false;  // the SwiGLU epilogue needs whole sums
  const int span = (groups + plan.splits - 1) / plan.splits;
  const int min_span = groups / plan.splits;  // every split holds at least this many groups
  if (plan.pair ? (plan.waves != 8 && plan.waves != 16)
                : (plan.waves != 4 && plan.waves != 8 && plan.waves != 16))
    return false;
  // sixteen waves without the pair: staged activations and eight or sixteen groups per
  // wave only; sixteen groups per wave only there
  if (!plan.pair && plan.waves == 16 && (plan.direct || plan.depth < 8)) return false;
  if (plan.depth > (!plan.pair && plan.waves == 16 ? 16 : 8)) return false;
  const int kw = plan.pair ? plan.waves / 2 : plan.waves;  // waves along K per block
  if (span > small_max_span(plan.waves, plan.pair, plan.depth) || min_span < kw)
    return false;  // at most `depth` groups and at least one per wave
  if ((span + kw - 1) / kw > plan.depth) return false;
  if (plan.dual && !plan.direct) return false;
  if (plan.direct)  // per-wave LDS regions of `depth` activation tiles and scale words
    return !plan.pair &&
           small_static_lds(plan.waves, false, plan.depth, plan.gpc, false, plan.dual, true) +
                   small_direct_lds(plan.waves, plan.depth, plan.gpc, true, plan.dual) <=
               kLdsBytes;
  const int slots = stage_slots(m, span, plan.waves);
  const long dynamic = (long)round_slots(slots) * plan.waves * 64 * (long)sizeof(f16x8);
  return slots <= 16 &&
         dynamic + small_static_lds(plan.waves, plan.pair, plan.depth, plan.gpc, m == 1,
                                    false) <= kLdsBytes;
}

bool grouped_small_plan(const GroupedProblem& p, int rows, SmallPlan* plan) {
  if (p.fp8 || rows < 1 || rows > kSegRows) return false;
  if (p.n_active > 65535) return false;                     // segments along grid y
  if ((long long)p.n_tokens * p.k > 0x7fffffffLL) return false;  // 32-bit row offsets
  const int groups = p.k / kGroup;
  // waves along K per block: 4, 8 or 16 (twice that with the SwiGLU pair, half on each
  // block, at most 16 waves in all)
  for (int kw = 4; kw <= (p.swiglu ? 8 : 16); kw *= 2) {
    const int per_wave = (groups + kw - 1) / kw;
    if (per_wave > 8) continue;
    SmallPlan q{};
    q.waves = p.swiglu ? 2 * kw : kw;
    q.splits = 1;
    q.depth = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : per_wave <= 4 ? 4 : 8;
    q.pair = p.swiglu;
    q.gpc = p.gpc;
    if (kw >= 8 && q.depth != 8) continue;  // the instances of 8 or 16 waves per block
    if (small_plan_fits(rows, p.k, q)) {
      *plan = q;
      return true;
    }
  }
  return false;
}

hipError_t launch_grouped_small(const GroupedProblem& p, int rows, const SmallPlan& plan,
                                hipStream_t stream) {
  SmallPlan check{};
  if (!grouped_small_plan(p, rows, &check) || check.waves != plan.waves ||
      check.depth != plan.depth || check.pair != plan.pair)
    return hipErrorInvalidConfiguration;
  if (p.bf16) {
    switch (p.gpc) {
      case 2: return launch_seg_bf16_g2(p, rows, plan, stream);
      case 4: return launch_seg_bf16_g4(p, rows, plan, stream);
      case 8: return launch_seg_bf16_g8(p, rows, plan, stream);
      default: return launch_seg_bf16_g1(p, rows, plan, stream);
    }
  }
  switch (p.gpc) {
    case 2: return launch_seg_g2(p, rows, plan, stream);
    case 4: return launch_seg_g4(p, rows, plan, stream);
    case 8: return launch_seg_g8(p, rows, plan, stream);
    default: return launch_seg_g1(p, rows, plan, stream);
  }
}

hipError_t launch_gemm_small(const uint16_t* a, int lda, int m, const uint32_t* b,
                             const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                             const SmallPlan& plan, float* partials, bool bf16, bool fp8,
                             hipStream_t stream) {
  if (!small_plan_fits(plan.rows > 0 && plan.rows < m ? plan.rows : m, k, plan))
    return hipErrorInvalidConfiguration;
  if (fp8) {
    if (z != nullptr) return hipErrorInvalidValue;
    return bf16 ? launch_small_fp8_bf16(a, lda, m, b, s, c, n, k, plan, partials, stream)
                : launch_small_fp8(a, lda, m, b, s, c, n, k, plan, partials, stream);
  }
  if (bf16) {
    switch (plan.gpc) {
      case 2: return launch_small_bf16_g2(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
      case 4: return launch_small_bf16_g4(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
      case 8: return launch_small_bf16_g8(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
      default: return launch_small_bf16_g1(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
    }
  }
  switch (plan.gpc) {
    case 2: return launch_small_g2(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
    case 4: return launch_small_g4(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
    case 8: return launch_small_g8(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
    default: return launch_small_g1(a, lda, m, b, s, z, c, n, k, plan, partials, stream);
  }
}

}  // namespace wq
