// C ABI of libwq: argument validation, planning and launches (see include/wq.h).
//
// Validation mirrors the fail-closed launch checks of ferrum-kernels marlin.rs
// (`MarlinMoeRawLaunchArgs::validate`: non-null and aligned pointers, positive shapes,
// group size rules, zero-point flag/pointer agreement, fp32-reduce/scratch agreement)
// and returns the staged status of `marlin_moe_ffi_status` instead of aborting.
#include <stdio.h>
#include <string.h>

#include <limits>
#include <vector>

#include "wq.h"
#include "wq_internal.h"

namespace {

constexpr int kGroupSize = 128;
constexpr int kMaxSplits = 16;  // fp32 partial slots per output element

int fail(int stage, int code) { return WQ_STATUS(stage, code); }
int hip_fail(hipError_t e) { return fail(WQ_STAGE_LAUNCH, (int)e); }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_ptr(const void* p, size_t align) {
  if (p == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (!aligned(p, align)) return fail(WQ_STAGE_ARGS, WQ_ERR_ALIGN);
  return 0;
}

// Supported group sizes: -1 (one group over K, channelwise, as transformer.rs
// `marlin_num_groups` maps it to one group) and every positive multiple of 16 dividing K
// (the pages' rule).  Scales and zero points are stored per unit of gcd(group_size, 128)
// rows, so a group is repeated for each unit it covers.
bool chunk_group_size(int k, int group_size) {
  if (group_size == -1) return true;
  return group_size > 0 && group_size % 16 == 0 && k % group_size == 0;
}

// Scale units per 128 rows of K (units of gcd(group_size, 128) rows: 1, 2, 4 or 8).
int subgroups(int k, int group_size) { return kGroupSize / wq::scale_unit_rows(k, group_size); }

// WQ_FLAG_FP8 (E4M3 weights): group_size -1 or 128, no zero points, no act_order.
int check_fp8(uint32_t flags, int group_size) {
  if (!(flags & WQ_FLAG_FP8)) return 0;
  if (group_size != -1 && group_size != kGroupSize) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  if (flags & (WQ_FLAG_HAS_ZP | WQ_FLAG_ACT_ORDER)) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  return 0;
}

// k % 128 == 0, n % 256 == 0, a supported group_size, and byte extents that fit.
int check_kn(int k, int n, int group_size) {
  if (k <= 0 || n <= 0 || k % kGroupSize != 0 || n % 256 != 0)
    return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  if (!chunk_group_size(k, group_size)) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  if ((long long)k * n / 8 > (long long)std::numeric_limits<int32_t>::max() * 4LL)
    return fail(WQ_STAGE_SHAPE, WQ_ERR_OVERFLOW);
  return 0;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// --- planning of the small-M kernel ------------------------------------------------------

// Plan of the small-M kernel's SwiGLU (paired) form: no split, 8 or 16 waves (4 or 8 per
// block along K), or false when no plan fits (the tiled kernel then computes it).
bool plan_small_pair(int m, int k, int gpc, wq::SmallPlan* plan) {
  const int groups = k / kGroupSize;
  for (int waves = 8; waves <= 16; waves *= 2) {
    const int per_wave = (groups + waves / 2 - 1) / (waves / 2);
    if (per_wave > 8) continue;
    wq::SmallPlan p{};
    p.waves = waves;
    p.splits = 1;
    p.depth = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : per_wave <= 4 ? 4 : 8;
    p.pair = true;
    p.gpc = gpc;
    if (wq::small_plan_fits(m, k, p)) {
      *plan = p;
      return true;
    }
  }
  return false;
}

constexpr int kDirectRows = 9;
// Two column blocks per wave halve the activation reads of the direct form but halve its
// work-groups too.  Measured on MI355X at M=16, K=4096 with zero points (single blocks on
// 8 waves of 4 groups, paired blocks on 4 waves of 8): N=4096 (128 paired work-groups)
// 5.9 against 4.9 us; N=8192 (256) 7.0 against 8.8 us; N=14336 (448) 11.7 against 15.5 us.
constexpr int kDualMinGroups = 256;

// Own choice with the flag, 4-bit weights, 4 to 16 rows and K from 64 groups: when the grid
// holds more work-groups than the CUs, K is split into ranges of at most kDeepSplitGroups
// groups, in ceil(groups / kDeepSplitGroups) splits (so that the ranges come out even: 112
// groups in 7, not 8 ranges of 14, which leave waves idle).  Measured on MI355X (us, two
// rounds, the previous own choice -> the deep split): K=14336, N=4096, m=8 15.5-15.7 -> 12.4,
// m=12 24.0 -> 13.6; K=14336, N=14336, m=4 31.5 -> 23.6-23.7, m=8 41.3 -> 28.9-29.0;
// K=28672, N=8192, m=4 32.5-33.0 -> 25.9-26.2, m=8 46.6 -> 32.4-32.8, m=12 82.0 -> 37.2,
// m=16 40.8-41.0 -> 38.8-39.1; K=28672, N=4096, m=4 18.4 -> 16.5, m=16 24.3 -> 22.6;
// K=16384, N=8192, m=4 18.6 -> 17.0-17.4, m=8 26.1 -> 21.3-22.2; K=11008, N=4096, m=8 about
// 15 -> 11.5; K=12288, N=4096, m=16 13.9 -> 12.4; K=8192, N=14336, m=8 22.2-22.6 ->
// 19.1-19.4.  Where one round of work-groups
// covers the grid the unsplit plan stays (K=8192, N=4096, m=8 7.6 against 8.7 with two
// splits; K=14336, N=4096, m=4 9.6 against 11.3 with four), and so does four rows at 64
// groups (K=8192, N=8192 with zero points 10.7-11.0 against 11.5-11.7 with four).  One to
// three rows split only beyond 64 groups and two work-groups per CU, into ranges of at most
// 32 groups: K=14336, N=14336, m=1 22.2-24.4 -> 20.6-20.8, m=3 29.7 -> 25.0-25.3; K=28672,
// N=8192 (four splits before), m=1 24.2 -> 22.8-22.9, m=2 28.0 -> 23.6, m=3 31.6-31.9 ->
// 25.7-26.4; K=28672, N=4096, m=3 18.5-18.7 -> 15.8-16.1.  With fewer work-groups it was
// as often slower (K=8192, N=14336, m=1 12.0 against 14.1-14.8 with two; K=16384, N=8192,
// m=1 13.6-13.8 against 14.8-15.3 with four).
constexpr int kDeepSplitGroups = 16;
constexpr int kCus = 256;

int deep_split(int m, int n, int groups, uint32_t flags, int s) {
  if (flags & WQ_FLAG_FP8) return s;
  int range = kDeepSplitGroups;
  if (m < 4) {
    if (groups <= 64 || (n / 16) * s <= 2 * kCus) return s;
    range = 2 * kDeepSplitGroups;
  } else if (groups < 64 || (m == 4 && groups == 64) || (n / 16) * s <= kCus) {
    return s;
  }
  int want = (groups + range - 1) / range;
  if (want > kMaxSplits) want = kMaxSplits;
  return want > s ? want : s;
}

// Plan of the small-M kernel, or false when no plan fits its staging limits (the tiled
// kernel then computes the product).  Without WQ_FLAG_FP32_REDUCE the product is never
// split (every output is one work-group's fp32 sum, rounded once).  With it, a requested
// split count is honoured, raised if the activation slice would not fit in LDS; the
// library's own choice splits when the 16-column blocks alone give fewer than 128
// work-groups (half the CUs), since every split adds an fp32 partial round trip and a
// reduce launch (measured on MI355X: at N=4096..14336 one split is fastest), and beyond
// 128 groups into ranges of at most 64, and deeper from 4 rows (deep_split).  Each
// split's groups are shared by 4, 8 or 16 waves: at most 8 groups per wave, or 16 with
// sixteen staged waves.
bool plan_small(int m, int n, int k, uint32_t flags, int requested, int gpc,
                wq::SmallPlan* plan) {
  const int groups = k / kGroupSize;
  const bool fp32 = (flags & WQ_FLAG_FP32_REDUCE) != 0;
  int s = 1;
  if (fp32 && requested > 0) {
    s = requested;
  } else if (fp32) {
    const int col_blocks = n / 16;
    s = col_blocks >= 128 ? 1 : (256 + col_blocks - 1) / col_blocks;
    // Beyond 128 groups a single work-group per column block would need sixteen groups per
    // wave; splits of at most 64 groups were faster where the flag allows them (MI355X,
    // K=28672, N=8192: m=1 27.0 against 31.9 us unsplit, m=4 34.8 against 42.2).
    if (groups > 128 && s < (groups + 63) / 64) s = (groups + 63) / 64;
    const int max_s = groups / 4 > 0 ? groups / 4 : 1;  // keep a group per wave of a split
    if (s > max_s) s = max_s;
  }
  for (; s <= groups && s <= kMaxSplits; ++s) {
    if (s > 1 && !fp32) return false;
    const int span = (groups + s - 1) / s;
    // From kDirectRows rows on, the activation slice shared through LDS costs more than
    // each wave fetching its own groups' tiles, so direct plans come first.
    for (int pass = m >= kDirectRows ? 0 : 1; pass < 2; ++pass) {
      // Direct activations are read by every work-group in full; pairing two column blocks
      // per wave halves those reads while at least kDualMinGroups work-groups remain (E4M3
      // weights excepted).  Direct single blocks try 8 waves first, paired ones 4 (the
      // faster of the two on MI355X at M=16, K=4096); staged plans 4 waves first.
      const bool dual = pass == 0 && !(flags & WQ_FLAG_FP8) && (n / 32) * s >= kDualMinGroups;
      // staged 4-bit plans may take sixteen waves of eight or sixteen groups (K up to 256
      // groups)
      const int tries = pass == 1 && !(flags & WQ_FLAG_FP8) ? 3 : 2;
      for (int wi = 0; wi < tries; ++wi) {
        const int waves = wi == 2 ? 16 : (pass == 0 && !dual) == (wi == 0) ? 8 : 4;
        const int per_wave = (span + waves - 1) / waves;
        if (per_wave > (waves == 16 ? 16 : 8)) continue;
        wq::SmallPlan p{};
        p.waves = waves;
        p.splits = s;
        p.depth = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : per_wave <= 4 ? 4 : per_wave <= 8 ? 8 : 16;
        p.gpc = gpc;
        p.direct = pass == 0;
        p.dual = dual;
        if (wq::small_plan_fits(m, k, p)) {
          if (fp32 && requested <= 0) {
            const int deep = deep_split(m, n, groups, flags, s);
            if (deep > s) return plan_small(m, n, k, flags, deep, gpc, plan);
          }
          *plan = p;
          return true;
        }
      }
    }
  }
  return false;
}

// The small-M plan of a dense product, if it takes one: m <= 16, or, without the fp32
// reduce flag, row chunks along grid z, each reading the weights (at most sixteen).  The
// chunks' weight reads are held to a budget proportional to K, since the unsplit row tiles
// that would take the product otherwise are few and their time grows with K:
// kChunkDirectBytes per K for 16-row chunks on the direct form, kChunkStagedBytes per K for
// staged chunks of 8, 4, 2 or 1 rows (slower per weight byte).  Measured on MI355X without
// the flag (one run each; chunks against tiles): K=N=4096 M=80..256 21-49 against 61-64 us;
// K=4096, N=8192, M=128 42 against 64; K=2048, N=4096, M=256 22 against 37; K=14336,
// N=4096, M=16 39 against 115; K=28672, N=8192, M=8 120 against 225; beyond the budgets
// K=8192, N=28672, M=24 123 against 78, and K=11008, N=4096, M=64 about 180 against 101.
// With the flag the tiles may split K instead, which is faster from about 50 MB of chunk
// reads at K = 4096 (K=4096, N=14336: 16-row chunks 20.5-21.5 us for 17-32 rows against
// split tiles 19.4-20.4; N=4096: chunks 9.3-9.5 against 13.6-14.2 us for 24-32 rows, 16.6
// against 18.5 for 64): direct chunks then take a budget of kChunkSplitBytes per K.  A
// requested split or the SwiGLU epilogue keeps the tiles.
bool plan_small_any(int m, int n, int k, uint32_t flags, int requested, int gpc, bool swiglu,
                    wq::SmallPlan* plan) {
  if (m <= 16) {
    if (swiglu) return plan_small_pair(m, k, gpc, plan);
    if (plan_small(m, n, k, flags, requested, gpc, plan)) return true;
  }
  if (swiglu || requested > 1) return false;
  const bool fp32 = (flags & WQ_FLAG_FP32_REDUCE) != 0;
  const double weight_bytes = (double)k * n * ((flags & WQ_FLAG_FP8) ? 1.0 : 0.5);
  // 16 rows on the direct form, or, where K is too long for it (beyond 32 groups), a staged
  // slice of 8, 4, 2 or 1 rows
  for (int rows = 16; rows >= 1; rows /= 2) {
    const int chunks = (m + rows - 1) / rows;
    if (chunks > 16) break;
    if (rows >= m) continue;
    wq::SmallPlan q{};
    if (!plan_small(rows, n, k, flags & ~(uint32_t)WQ_FLAG_FP32_REDUCE, 0, gpc, &q) ||
        q.splits != 1 || (!q.direct && rows > 8) || (fp32 && !q.direct))
      continue;
    const double budget =
        (fp32 ? wq::kChunkSplitBytes
              : (q.direct ? wq::kChunkDirectBytes : wq::kChunkStagedBytes)) * k;
    if (chunks * weight_bytes > budget) return false;
    q.rows = rows;
    *plan = q;
    return true;
  }
  return false;
}

// Splits of a tiled product: none without the fp32 reduce flag; a requested count, within
// what its tiles allow; else the planner's.
int tile_split_count(int m, int n, int k, uint32_t flags, int requested, int gpc, bool fp8,
                     bool swiglu) {
  if (!(flags & WQ_FLAG_FP32_REDUCE)) return 1;
  if (requested > 0) {
    const int most = wq::tile_max_splits(m, n, k, gpc, fp8, swiglu);
    return requested < most ? requested : most;
  }
  return wq::tile_splits(m, n, k, gpc, fp8, swiglu);
}

// fp32 partials [splits][m][n] for the largest split the small-M path may use, or for
// m > 16 the split the tiled path chooses (the same for 128- and 64-row scale units; the
// smaller units never split).
size_t gemm_workspace_bytes(int m, int n, int k, uint32_t flags) {
  if (!(flags & WQ_FLAG_FP32_REDUCE)) return 0;
  if (m > 16) {
    const bool fp8 = (flags & WQ_FLAG_FP8) != 0, swiglu = (flags & WQ_FLAG_SWIGLU) != 0;
    const int s = wq::tile_splits(m, n, k, 1, fp8, swiglu);
    return s > 1 ? (size_t)s * m * n * sizeof(float) : 0;
  }
  int smax = k / kGroupSize;
  if (smax > kMaxSplits) smax = kMaxSplits;
  if (smax <= 1) return 0;
  return (size_t)smax * m * n * sizeof(float);
}

const char* stage_name(int stage) {
  switch (stage) {
    case WQ_STAGE_ARGS: return "args";
    case WQ_STAGE_SHAPE: return "shape";
    case WQ_STAGE_DEVICE: return "device-query";
    case WQ_STAGE_LAUNCH_CONFIG: return "launch-config";
    case WQ_STAGE_FUNC_ATTR: return "function-attribute";
    case WQ_STAGE_LAUNCH: return "kernel-launch";
    default: return "unknown";
  }
}

const char* error_name(int code) {
  switch (code) {
    case WQ_ERR_NULL: return "null pointer";
    case WQ_ERR_ALIGN: return "misaligned pointer";
    case WQ_ERR_SHAPE: return "unsupported shape";
    case WQ_ERR_FLAGS: return "unsupported or inconsistent flags";
    case WQ_ERR_WORKSPACE: return "workspace too small";
    case WQ_ERR_ABI: return "abi version or struct size mismatch";
    case WQ_ERR_OVERFLOW: return "size overflow";
    case WQ_ERR_CSR: return "invalid expert CSR";
    case WQ_ERR_ACT_ORDER: return "act_order groups are not group_size rows each";
    default: return "unknown error";
  }
}

}  // namespace

extern "C" {

uint32_t wq_abi_version(void) { return WQ_ABI_VERSION; }

const char* wq_status_str(int status) {
  static thread_local char buf[160];
  if (status == 0) return "ok";
  const int stage = (int)((unsigned)status >> 16);
  const int code = (int)((unsigned)status & 0xFFFFu);
  if (stage == WQ_STAGE_ARGS || stage == WQ_STAGE_SHAPE)
    snprintf(buf, sizeof buf, "%s: %s (%d)", stage_name(stage), error_name(code), code);
  else if (stage >= WQ_STAGE_DEVICE && stage <= WQ_STAGE_LAUNCH)
    snprintf(buf, sizeof buf, "%s: %s (%d)", stage_name(stage),
             hipGetErrorString((hipError_t)code), code);
  else
    snprintf(buf, sizeof buf, "unknown: %d", status);
  return buf;
}

int wq_repack_b(const uint32_t* qweight, const int32_t* perm, void* b_out, int k, int n,
                void* stream) {
  int st = check_kn(k, n, kGroupSize);
  if (st) return st;
  if ((st = check_ptr(qweight, 4))) return st;
  if ((st = check_ptr(b_out, 16))) return st;
  if (perm && !aligned(perm, 4)) return fail(WQ_STAGE_ARGS, WQ_ERR_ALIGN);
  const hipError_t e = wq::launch_repack_b(qweight, perm, static_cast<uint32_t*>(b_out), k, n,
                                           as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_repack_fp8(const uint32_t* words, void* b_out, int k, int n, void* stream) {
  int st = check_kn(k, n, kGroupSize);
  if (st) return st;
  if ((st = check_ptr(words, 4))) return st;
  if ((st = check_ptr(b_out, 16))) return st;
  const hipError_t e =
      wq::launch_repack_fp8(words, static_cast<uint32_t*>(b_out), k, n, as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_repack_fp8_rows(const void* w_nk, void* b_out, int k, int n, void* stream) {
  int st = check_kn(k, n, kGroupSize);
  if (st) return st;
  if ((st = check_ptr(w_nk, 4))) return st;
  if ((st = check_ptr(b_out, 16))) return st;
  const hipError_t e = wq::launch_repack_fp8_rows(static_cast<const uint8_t*>(w_nk),
                                                  static_cast<uint32_t*>(b_out), k, n,
                                                  as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_fp8_block_scales(const void* inv_scales, void* s_out, int k, int n, void* stream) {
  int st = check_kn(k, n, kGroupSize);
  if (st) return st;
  if ((st = check_ptr(inv_scales, 2))) return st;
  if ((st = check_ptr(s_out, 16))) return st;
  const hipError_t e = wq::launch_fp8_block_scales(static_cast<const uint16_t*>(inv_scales),
                                                   static_cast<uint16_t*>(s_out), k, n,
                                                   as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_repack_scales(const void* scales, void* s_out, int k, int n, int group_size,
                     void* stream) {
  int st = check_kn(k, n, group_size);
  if (st) return st;
  if ((st = check_ptr(scales, 2))) return st;
  if ((st = check_ptr(s_out, 16))) return st;
  const hipError_t e =
      wq::launch_repack_scales(static_cast<const uint16_t*>(scales), static_cast<uint16_t*>(s_out),
                               k, n, group_size, as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_repack_zeros(const uint32_t* zeros, void* z_out, int k, int n, int group_size,
                    void* stream) {
  int st = check_kn(k, n, group_size);
  if (st) return st;
  if ((st = check_ptr(zeros, 4))) return st;
  if ((st = check_ptr(z_out, 16))) return st;
  const hipError_t e = wq::launch_repack_zeros(zeros, static_cast<uint32_t*>(z_out), k, n,
                                               group_size, as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_act_order_perm(const int32_t* g_idx, int k, int group_size, int32_t* perm_out,
                      int32_t* sorted_gidx_out) {
  if (g_idx == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (k > 0 && group_size == -1) group_size = k;  // channelwise: one group of all K rows
  if (k <= 0 || group_size <= 0 || k % group_size != 0) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  const int groups = k / group_size;
  // Counting sort by group keeps equal groups in ascending row order (a stable argsort).
  std::vector<int> count(groups + 1, 0);
  for (int r = 0; r < k; ++r) {
    const int g = g_idx[r];
    if (g < 0 || g >= groups) return fail(WQ_STAGE_ARGS, WQ_ERR_ACT_ORDER);
    ++count[g + 1];
  }
  for (int g = 0; g < groups; ++g)
    if (count[g + 1] != group_size) return fail(WQ_STAGE_ARGS, WQ_ERR_ACT_ORDER);
  for (int g = 0; g < groups; ++g) count[g + 1] += count[g];
  for (int r = 0; r < k; ++r) {
    const int pos = count[g_idx[r]]++;
    if (perm_out) perm_out[pos] = r;
    if (sorted_gidx_out) sorted_gidx_out[pos] = g_idx[r];
  }
  return 0;
}

int wq_gemm_workspace_bytes(int m, int n, int k, uint32_t flags, size_t* bytes_out) {
  if (bytes_out == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (m <= 0) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  const int st = check_kn(k, n, kGroupSize);
  if (st) return st;
  *bytes_out = gemm_workspace_bytes(m, n, k, flags);
  return 0;
}

int wq_gemm(const wq_gemm_args* args) {
  if (args == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (args->abi_version != WQ_ABI_VERSION || args->struct_size != sizeof(wq_gemm_args) ||
      args->reserved != 0)
    return fail(WQ_STAGE_ARGS, WQ_ERR_ABI);
  const wq_gemm_args& p = *args;
  const uint32_t known = WQ_FLAG_ACT_ORDER | WQ_FLAG_IS_K_FULL | WQ_FLAG_HAS_ZP |
                         WQ_FLAG_ATOMIC_ADD | WQ_FLAG_FP32_REDUCE | WQ_FLAG_SWIGLU |
                         WQ_FLAG_BF16 | WQ_FLAG_FP8;
  if ((p.flags & ~known) || (p.flags & WQ_FLAG_ATOMIC_ADD))
    return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  int st = check_kn(p.k, p.n, p.group_size);
  if (st) return st;
  if ((st = check_fp8(p.flags, p.group_size))) return st;
  if (p.m <= 0 || p.lda < p.k || p.lda % 8 != 0) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  if ((long long)p.m * p.lda > (long long)std::numeric_limits<int64_t>::max() / 4 ||
      (long long)(p.m + 255) / 256 > 65535)
    return fail(WQ_STAGE_SHAPE, WQ_ERR_OVERFLOW);
  if ((st = check_ptr(p.a, 16)) || (st = check_ptr(p.b, 16)) || (st = check_ptr(p.c, 16)) ||
      (st = check_ptr(p.b_scales, 16)))
    return st;
  const bool has_zp = (p.flags & WQ_FLAG_HAS_ZP) != 0;
  if (has_zp != (p.zero_points != nullptr)) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  if (has_zp && (st = check_ptr(p.zero_points, 16))) return st;
  const bool act_order = (p.flags & WQ_FLAG_ACT_ORDER) != 0;
  if (act_order != (p.perm != nullptr)) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  if (act_order) {
    if ((st = check_ptr(p.perm, 16))) return st;
    if ((st = check_ptr(p.a_tmp, 16))) return st;
  }
  // group_index only checks the act_order layout's groups (include/wq.h).
  if (p.group_index != nullptr && !act_order) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  if (p.group_index != nullptr && !aligned(p.group_index, 4))
    return fail(WQ_STAGE_ARGS, WQ_ERR_ALIGN);
  if (p.split_k < 0) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  if (p.split_k > 1 && !(p.flags & WQ_FLAG_FP32_REDUCE)) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  const bool swiglu = (p.flags & WQ_FLAG_SWIGLU) != 0;
  const bool bf16 = (p.flags & WQ_FLAG_BF16) != 0;
  const bool fp8 = (p.flags & WQ_FLAG_FP8) != 0;

  // Plan, and check the workspace the plan needs, before anything is enqueued.
  const int gpc = subgroups(p.k, p.group_size);
  wq::SmallPlan plan{};
  const bool small = plan_small_any(p.m, p.n, p.k, p.flags, p.split_k, gpc, swiglu, &plan);
  // Without a small-M plan the tiled kernel computes the product, split along K (with the
  // fp32 reduce) when its output tiles would leave CUs idle.
  const int tile_split =
      small ? 1 : tile_split_count(p.m, p.n, p.k, p.flags, p.split_k, gpc, fp8, swiglu);
  float* partials = nullptr;
  if ((small && plan.splits > 1) || tile_split > 1) {
    const size_t need =
        (size_t)(small ? plan.splits : tile_split) * p.m * p.n * sizeof(float);
    if (p.workspace == nullptr || p.workspace_bytes < need)
      return fail(WQ_STAGE_ARGS, WQ_ERR_WORKSPACE);
    if (!aligned(p.workspace, 16)) return fail(WQ_STAGE_ARGS, WQ_ERR_ALIGN);
    partials = static_cast<float*>(p.workspace);
  }

  const hipStream_t stream = as_stream(p.stream);
  const uint16_t* a = static_cast<const uint16_t*>(p.a);
  int lda = p.lda;
  if (act_order) {
    const hipError_t e =
        wq::launch_gather_columns(a, lda, p.perm, p.group_index, p.group_size,
                                  static_cast<uint16_t*>(p.a_tmp), p.m, p.k, stream);
    if (e != hipSuccess) return hip_fail(e);
    a = static_cast<const uint16_t*>(p.a_tmp);
    lda = p.k;
  }
  const uint32_t* b = static_cast<const uint32_t*>(p.b);
  const uint16_t* s = static_cast<const uint16_t*>(p.b_scales);
  const uint32_t* z = static_cast<const uint32_t*>(p.zero_points);
  uint16_t* c = static_cast<uint16_t*>(p.c);

  if (small) {
    const hipError_t e =
        wq::launch_gemm_small(a, lda, p.m, b, s, z, c, p.n, p.k, plan, partials, bf16, fp8,
                              stream);
    return e == hipSuccess ? 0 : hip_fail(e);
  }
  const hipError_t e = wq::launch_gemm_tile(a, lda, p.m, b, s, z, c, p.n, p.k, swiglu, gpc, bf16,
                                             fp8, tile_split, partials, stream);
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_gemm_plan(int m, int n, int k, int group_size, uint32_t flags, int split_k,
                 int32_t* kernel_out, int32_t* splits_out) {
  if (kernel_out == nullptr || splits_out == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  int st = check_kn(k, n, group_size);
  if (st) return st;
  if ((st = check_fp8(flags, group_size))) return st;
  if (m <= 0 || split_k < 0) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  const bool swiglu = (flags & WQ_FLAG_SWIGLU) != 0, fp8 = (flags & WQ_FLAG_FP8) != 0;
  const int gpc = subgroups(k, group_size);
  wq::SmallPlan plan{};
  const bool small = plan_small_any(m, n, k, flags, split_k, gpc, swiglu, &plan);
  if (small) {
    *kernel_out = WQ_KERNEL_SMALL_M;
    *splits_out = plan.splits;
    return 0;
  }
  *kernel_out = wq::tile_is_tall(m, n, gpc, fp8) ? WQ_KERNEL_TILE_128 : WQ_KERNEL_TILE_256;
  *splits_out = tile_split_count(m, n, k, flags, split_k, gpc, fp8, swiglu);
  return 0;
}

int wq_dequant(const void* b, const void* b_scales, const void* zero_points, int k, int n,
               int group_size, uint32_t flags, void* w_out, void* stream) {
  int st = check_kn(k, n, group_size);
  if (st) return st;
  if ((st = check_ptr(b, 16)) || (st = check_ptr(b_scales, 16)) || (st = check_ptr(w_out, 16)))
    return st;
  if (flags & ~(uint32_t)(WQ_FLAG_HAS_ZP | WQ_FLAG_ACT_ORDER | WQ_FLAG_IS_K_FULL | WQ_FLAG_BF16 |
                          WQ_FLAG_FP8))
    return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  if ((st = check_fp8(flags & ~(uint32_t)WQ_FLAG_ACT_ORDER, group_size))) return st;
  if (flags & WQ_FLAG_FP8) {
    if (zero_points != nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
    const hipError_t e = wq::launch_dequant_fp8(
        static_cast<const uint32_t*>(b), static_cast<const uint16_t*>(b_scales), k, n,
        static_cast<uint16_t*>(w_out), as_stream(stream));
    return e == hipSuccess ? 0 : hip_fail(e);
  }
  const bool has_zp = (flags & WQ_FLAG_HAS_ZP) != 0;
  if (has_zp != (zero_points != nullptr)) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  if (has_zp && (st = check_ptr(zero_points, 16))) return st;
  const hipError_t e = wq::launch_dequant(
      static_cast<const uint32_t*>(b), static_cast<const uint16_t*>(b_scales),
      static_cast<const uint32_t*>(zero_points), k, n, wq::scale_unit_rows(k, group_size),
      (flags & WQ_FLAG_BF16) != 0, static_cast<uint16_t*>(w_out), as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_csr_from_routes(const int32_t* selected, int n_tokens, int top_k, int n_expert,
                       int32_t* ex_ids, int32_t* ex_off, int32_t* ex_pairs, int32_t* pair_tok,
                       int32_t* n_active_out) {
  if (!selected || !ex_ids || !ex_off || !ex_pairs || !pair_tok || !n_active_out)
    return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (n_tokens <= 0 || top_k <= 0 || n_expert <= 0) return fail(WQ_STAGE_ARGS, WQ_ERR_CSR);
  const long long pairs = (long long)n_tokens * top_k;
  if (pairs > std::numeric_limits<int32_t>::max()) return fail(WQ_STAGE_ARGS, WQ_ERR_OVERFLOW);
  const int n_pairs = (int)pairs;
  std::vector<int> count(n_expert + 1, 0);
  for (int p = 0; p < n_pairs; ++p) {
    const int e = selected[p];
    if (e < 0 || e >= n_expert) return fail(WQ_STAGE_ARGS, WQ_ERR_CSR);
    ++count[e + 1];
  }
  for (int e = 0; e < n_expert; ++e) count[e + 1] += count[e];
  int active = 0;
  for (int e = 0; e < n_expert; ++e) {
    if (count[e + 1] > count[e]) {
      ex_ids[active] = e;
      ex_off[active] = count[e];
      ++active;
    }
  }
  ex_off[active] = n_pairs;
  for (int p = 0; p < n_pairs; ++p) {
    ex_pairs[count[selected[p]]++] = p;
    pair_tok[p] = p / top_k;
  }
  *n_active_out = active;
  return 0;
}

int wq_grouped_workspace_bytes(int n_pairs, int n_active, int n, int k, uint32_t flags,
                               size_t* bytes_out) {
  (void)flags;
  if (bytes_out == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (n_pairs <= 0 || n_active <= 0) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  const int st = check_kn(k, n, kGroupSize);
  if (st) return st;
  *bytes_out = 0;
  return 0;
}

int wq_grouped_gemm(const wq_grouped_args* args) {
  if (args == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (args->abi_version != WQ_ABI_VERSION || args->struct_size != sizeof(wq_grouped_args) ||
      args->reserved != 0)
    return fail(WQ_STAGE_ARGS, WQ_ERR_ABI);
  const wq_grouped_args& p = *args;
  if (p.flags & ~(uint32_t)(WQ_FLAG_HAS_ZP | WQ_FLAG_IS_K_FULL | WQ_FLAG_MUL_TOPK_WEIGHTS |
                            WQ_FLAG_SWIGLU | WQ_FLAG_BF16 | WQ_FLAG_FP8))
    return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  // The routing weight scales an expert's output, i.e. the down projection; the SwiGLU
  // activation of the gate/up projection takes none.
  if ((p.flags & WQ_FLAG_SWIGLU) && (p.flags & WQ_FLAG_MUL_TOPK_WEIGHTS))
    return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  int st = check_kn(p.k, p.n, p.group_size);
  if (st) return st;
  if ((st = check_fp8(p.flags, p.group_size))) return st;
  const bool fp8 = (p.flags & WQ_FLAG_FP8) != 0;
  if (p.n_expert <= 0 || p.n_active <= 0 || p.n_active > p.n_expert || p.n_pairs <= 0 ||
      p.n_tokens <= 0 || p.n_active > p.n_pairs)
    return fail(WQ_STAGE_ARGS, WQ_ERR_CSR);
  if ((st = check_ptr(p.a, 16)) || (st = check_ptr(p.b_bank, 16)) ||
      (st = check_ptr(p.s_bank, 16)) || (st = check_ptr(p.y, 16)) ||
      (st = check_ptr(p.ex_off, 4)) || (st = check_ptr(p.ex_pairs, 4)) ||
      (st = check_ptr(p.pair_tok, 4)))
    return st;
  if (p.ex_ids && !aligned(p.ex_ids, 4)) return fail(WQ_STAGE_ARGS, WQ_ERR_ALIGN);
  const bool has_zp = (p.flags & WQ_FLAG_HAS_ZP) != 0;
  if (has_zp != (p.zp_bank != nullptr)) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  if (has_zp && (st = check_ptr(p.zp_bank, 16))) return st;
  const bool mul_w = (p.flags & WQ_FLAG_MUL_TOPK_WEIGHTS) != 0;
  if (mul_w != (p.topk_weights != nullptr)) return fail(WQ_STAGE_ARGS, WQ_ERR_FLAGS);
  if (mul_w && !aligned(p.topk_weights, 4)) return fail(WQ_STAGE_ARGS, WQ_ERR_ALIGN);
  const size_t groups = (size_t)(p.k / wq::scale_unit_rows(p.k, p.group_size));  // scale rows
  const size_t b_bytes = fp8 ? (size_t)p.k * p.n : (size_t)p.k * p.n / 2;
  const size_t s_bytes = groups * p.n * 2;
  const size_t z_bytes = groups * p.n / 2;
  if (p.b_stride_bytes < b_bytes || p.b_stride_bytes % 16 || p.s_stride_bytes < s_bytes ||
      p.s_stride_bytes % 16 || (has_zp && (p.zp_stride_bytes < z_bytes || p.zp_stride_bytes % 16)))
    return fail(WQ_STAGE_ARGS, WQ_ERR_SHAPE);
  // The launch's work-group count: per-XCD shares of at most n_pairs/128 + n_active row
  // tiles and n_active tail tiles, each times n/256 column tiles.
  const long long ntn = p.n / wq::kTileN;
  const long long tiles = ((long long)p.n_pairs / wq::kTileMinM + 2LL * p.n_active) * ntn + 16;
  if (tiles > std::numeric_limits<int32_t>::max()) return fail(WQ_STAGE_SHAPE, WQ_ERR_OVERFLOW);

  wq::GroupedProblem g{};
  g.a = static_cast<const uint16_t*>(p.a);
  g.b_bank = static_cast<const uint8_t*>(p.b_bank);
  g.b_stride = p.b_stride_bytes;
  g.s_bank = static_cast<const uint8_t*>(p.s_bank);
  g.s_stride = p.s_stride_bytes;
  g.z_bank = static_cast<const uint8_t*>(p.zp_bank);
  g.z_stride = p.zp_stride_bytes;
  g.ex_ids = p.ex_ids;
  g.ex_off = p.ex_off;
  g.ex_pairs = p.ex_pairs;
  g.pair_tok = p.pair_tok;
  g.topk_w = p.topk_weights;
  g.y = static_cast<uint16_t*>(p.y);
  g.n_expert = p.n_expert;
  g.n_active = p.n_active;
  g.n_pairs = p.n_pairs;
  g.n_tokens = p.n_tokens;
  g.k = p.k;
  g.n = p.n;
  g.swiglu = (p.flags & WQ_FLAG_SWIGLU) != 0;
  g.bf16 = (p.flags & WQ_FLAG_BF16) != 0;
  g.fp8 = fp8;
  g.gpc = subgroups(p.k, p.group_size);
  // Few rows in every segment (decode-sized batches): the small-M kernel, one work-group per
  // 16-column block and segment, streams each active expert's weights on far more
  // work-groups than its row tiles would give.  Non-empty segments hold at most
  // n_pairs - n_active + 1 rows each.
  const long long seg_rows = (long long)p.n_pairs - p.n_active + 1;
  wq::SmallPlan sp{};
  const hipError_t e =
      seg_rows <= wq::kSegRows && wq::grouped_small_plan(g, (int)seg_rows, &sp)
          ? wq::launch_grouped_small(g, (int)seg_rows, sp, as_stream(p.stream))
          : wq::launch_grouped_tile(g, as_stream(p.stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_interleave_gate_up(const void* gate, const void* up, void* out, int rows, int cols,
                          int bits_per_column, void* stream) {
  if (bits_per_column != 32 && bits_per_column != 16 && bits_per_column != 4)
    return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  if ((long long)rows * cols * bits_per_column / 8 * 2 > (1LL << 46))
    return fail(WQ_STAGE_SHAPE, WQ_ERR_OVERFLOW);
  int st;
  if ((st = check_ptr(gate, 4)) || (st = check_ptr(up, 4)) || (st = check_ptr(out, 4)))
    return st;
  const hipError_t e = wq::launch_interleave_gate_up(gate, up, out, rows, cols,
                                                     bits_per_column, as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_mfma_rate(const void* operands, int iters, float* sink, size_t sink_floats,
                 double* flops_out, void* stream) {
  if (operands == nullptr || sink == nullptr || flops_out == nullptr)
    return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (!aligned(operands, 16) || !aligned(sink, 4)) return fail(WQ_STAGE_ARGS, WQ_ERR_ALIGN);
  if (iters <= 0 || iters > (1 << 20)) return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  if (sink_floats < (size_t)wq::kMfmaBlocks * wq::kMfmaThreads)
    return fail(WQ_STAGE_ARGS, WQ_ERR_WORKSPACE);
  // waves x iterations x 8 products x 2 * 32 * 32 * 16 flops
  *flops_out = (double)wq::kMfmaBlocks * (wq::kMfmaThreads / 64) * iters * 8 * 32768.0;
  const hipError_t e = wq::launch_mfma_loop(operands, iters, sink, as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

int wq_stream_read_sink_words(size_t bytes, size_t* words_out) {
  if (words_out == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (bytes == 0 || bytes % 16 != 0 || bytes / 16 > (size_t)1 << 40)
    return fail(WQ_STAGE_SHAPE, WQ_ERR_SHAPE);
  *words_out = (size_t)wq::stream_read_sink_words(bytes);
  return 0;
}

int wq_stream_read(const void* src, size_t bytes, void* sink, size_t sink_words,
                   void* stream) {
  size_t need = 0;
  const int st = wq_stream_read_sink_words(bytes, &need);
  if (st != 0) return st;
  if (src == nullptr || sink == nullptr) return fail(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(WQ_STAGE_ARGS, WQ_ERR_ALIGN);
  if (sink_words < need) return fail(WQ_STAGE_ARGS, WQ_ERR_WORKSPACE);
  if (need / 4 > 0x7fffffffu) return fail(WQ_STAGE_SHAPE, WQ_ERR_OVERFLOW);
  const hipError_t e =
      wq::launch_stream_read(src, bytes, static_cast<uint32_t*>(sink), as_stream(stream));
  return e == hipSuccess ? 0 : hip_fail(e);
}

}  // extern "C"
