// Small-M W4A16 GEMM (m <= 16): decode and small batches, bound by the weight stream.
//
// One 16x16x32 fp16 MFMA block covers all m rows (rows >= m repeat row m - 1 and are
// never stored), so the packed weights are read exactly once.  A work-group owns one
// 16-column block and a range of K groups; its WAVES waves split that range, each
// streaming one 1 KiB layout chunk per 128-row group with a single non-temporal 16-byte
// load per lane.  All of a wave's weight loads are issued before any arithmetic and
// consumed in issue order, so the weight stream is never stalled behind compute.
// Activations, scales and zero points reach LDS one of two ways: staged once for the
// work-group's range (up to 8 rows; by all its threads, or, on the one-row path, on
// sixteen waves and on eight waves with at most four rows, each wave staging its own share
// with no barrier before its arithmetic),
// or fetched by each wave for its own groups with direct-to-LDS loads (9 rows and more;
// the "direct" form below).  On the staged form every wave's activation and scale loads
// are issued before any wave's weight loads (measured faster: the staging then waits less
// behind other waves' weights).  Codes become
// exact fp16 integers (q - z) in registers; each scale group's MFMA partial is scaled by
// its fp16 group scale in fp32 and accumulated in fp32; the waves' sums are added in wave
// order.
//
// GPC is the number of scale units per 128-row chunk: scales and zero points are stored
// per unit of gcd(group_size, 128) rows (128, 64, 32 or 16), so a chunk owns GPC = 1, 2, 4
// or 8 consecutive unit rows of its column block.  The chunk's four 32-row MFMA steps then
// form one partial per unit, each scaled before it is added.  A 16-row unit is half an
// MFMA step (lanes 0-31 carry its first 16 rows, lanes 32-63 the rest), so with GPC = 8
// each step runs twice, once with the other half's weight lanes set to zero.
//
// BF16 selects bf16 activations, scales and outputs (bf16 MFMAs and dequant); the
// arithmetic is otherwise the same.  W8 selects E4M3 weights (one scale unit per 128 rows,
// no zero points): a lane's group is then two 16-byte vectors (rows 0-63 and 64-127 of the
// group), converted to the activation type two bytes per instruction.
//
// R1 (one activation row, 4-bit weights) is a leaner loop for the decode case:
//  - 4x4x4 MFMAs (16 blocks): with one real row the 16x16x32 product wastes 15 of its 16
//    rows, and two 4x4x4 products carry the same 512 weights in less MFMA time.  Block b of
//    a lane pair (col, qd) holds columns 4(b % 4).. and the lane's eight rows of the step, so
//    each lane keeps its own column's sum over its row class qd (rows 8qd..8qd+7 of every
//    32-row step); two shuffles add the four classes at the end.  A 16-row unit then lies in
//    the lane's own rows, and the masked double product of GPC = 8 is not needed.
//  - Activation broadcast: one block's A operand serves the four blocks of a row class, so
//    a lane reads two 4-row activation pieces per chunk instead of sixteen rows.
//  - Only the real output row is scaled and accumulated.
//  - The zero point is applied once per scale unit, not per weight.  fp16 operands are the
//    raw nibble bits read as fp16 subnormals: masking a word with 0x000F000F gives the
//    pair (q * 2^-24, q' * 2^-24) and with 0x00F000F0 the pair (q * 2^-20, q' * 2^-20),
//    both exact, so a word costs one shift and four ANDs instead of the general path's
//    nine operations.  The two scales go to separate products (rows 0, 1, 4, 5 of the
//    lane's eight at 2^-24, rows 2, 3, 6, 7 at 2^-20; the staged activations are stored
//    with their middle dwords swapped to match), and a unit's exact-weight partial is
//    2^24 p24 + 2^20 p20 - z S, S the activations' sum over the lane's rows of the unit.
//    bf16, which has no packed add, takes 128 + q for every row as on its general path
//    and subtracts (128 + z) S.  The staging threads form S per unit and row class from
//    the slice while the weights are in flight.  The products are exact; only the fp32
//    sums round, at magnitudes a few times those of the exact-weight sums.
//
// This header holds the kernel template and its launch chain; each translation unit that
// includes it instantiates one GPC and activation type, so that the instances compile in
// parallel.
#pragma once
#include "wq_device.h"
#include "wq_internal.h"

#include <type_traits>

namespace wq {
namespace {

// LDS of one work-group: 160 KiB on gfx950, shared by the statically sized scale, zero-point
// and reduction buffers and the dynamically sized activation slice (fp16 [m][span*128],
// padded to a whole number of staging rounds).
constexpr int kLdsBytes = 160 * 1024;

// Groups of K a staged work-group covers: gw per wave along K (pair: half the waves on
// each block), sized for at least eight.
constexpr int small_max_span(int waves, bool pair, int gw) {
  return (gw > 8 ? gw : 8) * (pair ? waves / 2 : waves);
}

// Scale and zero-point staging: the work-group's nb blocks hold at most nb x
// small_max_span chunks of GPC units, 8 scale dwords and one zero-point pair per unit.
// Threads stage whole slots of T entries (T = waves x 64).
constexpr int small_scale_slots(int waves, bool pair, int gw, int nb, int gpc) {
  return nb * small_max_span(waves, pair, gw) * 8 * gpc / (waves * 64);
}
constexpr int small_zero_slots(int waves, bool pair, int gw, int nb, int gpc) {
  return nb * small_max_span(waves, pair, gw) * gpc > waves * 64
             ? nb * small_max_span(waves, pair, gw) * gpc / (waves * 64) : 1;
}
// Static LDS of an instance (see the kernel's __shared__ arrays), an upper bound over ZP.
// (pair: two column blocks split between the waves; dual: two column blocks per wave;
// direct: per-wave regions in the dynamic LDS instead, see small_direct_lds)
constexpr long small_static_lds(int waves, bool pair, int gw, int gpc, bool r1, bool dual,
                                bool direct = false) {
  if (direct) return 4 + 8 + 16 + 4;
  const int nb = pair || dual ? 2 : 1;
  return (long)small_scale_slots(waves, pair, gw, nb, gpc) * waves * 64 * 4    // s_lds
         + (long)small_zero_slots(waves, pair, gw, nb, gpc) * waves * 64 * 8   // z_lds
         + (long)(dual ? 2 : 1) * waves * 64 * 16                              // red
         + (r1 ? (long)small_max_span(waves, pair, gw) * 16 * 4 : 0);          // rsum_lds
}

// Direct activations: each wave owns an LDS region holding, for each of its GW groups, the
// 16-row activation tile of the group (16 x 128 fp16, 4 KiB), and after all waves' tiles,
// the scale (8 dwords per unit) and zero-point (2 per unit) words of its groups for each
// of its column blocks, fetched 64 dwords per direct load.
constexpr int kDirectTile = 16 * kGroup * 2;
constexpr int direct_sz_loads(int gw, int gpc, bool zp) {
  return (gw * gpc * (zp ? 10 : 8) + 63) / 64;
}
constexpr long small_direct_lds(int waves, int gw, int gpc, bool zp, bool dual) {
  return (long)waves *
         ((long)gw * kDirectTile + (dual ? 2 : 1) * direct_sz_loads(gw, gpc, zp) * 256L);
}

// The kernel body is branch-free up to the arithmetic: every load is issued
// unconditionally (addresses are clamped into the tensors) and ragged ends are masked by
// value, so the compiler's in-order load counting can let LDS writes wait for the
// activations alone and each group wait for its own weight chunk, while the rest of the
// weight stream stays in flight.
// PAIR (the SwiGLU epilogue): the work-group owns a gate/up pair of 16-column blocks
// (2t, 2t+1, as wq_interleave_gate_up pairs them); its first half of waves streams the gate
// block, the second half the up block, both over the same K range and staged activations,
// and the reduction writes fp16(silu(g) * u) to column 16t + c of the [m][n/2] activation.
// SEG (grouped products with few rows per expert): blockIdx.y is a segment of the
// expert-major CSR (ex_ids, ex_off, ex_pairs, pair_tok), whose rows, at most kSegRows of
// them (one on the one-row path), all use one expert's weights, scales and zero points (b,
// s and z plus the expert times b_stride, s_stride and z_stride elements).  Segment row j
// reads activation row pair_tok[p] (p = ex_pairs[ex_off[seg] + j]) and writes output row p,
// times topk_w[p] when given.  As on the tiled path, CSR entries out of range are never
// followed: a segment with an expert outside [0, n_expert) is skipped, its range is
// clamped into [0, n_pairs], and a row whose pair or token is out of range reads a clamped
// activation row and is not written.  The expert's weights for the first groups are
// requested before the row indices, so that the weight stream starts while the index loads
// resolve.
template <bool ZP, int WAVES, int GW, int STAGE, bool PAIR, int GPC, bool BF16, bool W8,
          bool R1, bool DUAL, bool SEG = false, bool PWR = false>
__global__ __launch_bounds__(WAVES * 64) void gemm_small_kernel(
    const f16* __restrict__ a, int lda, int m, const u32x4* __restrict__ b,
    const uint16_t* __restrict__ s, const u32x2* __restrict__ z, uint16_t* __restrict__ c,
    int n, int groups, int splits, float* __restrict__ partials,
    const int32_t* __restrict__ ex_ids, const int32_t* __restrict__ ex_off,
    const int32_t* __restrict__ ex_pairs, const int32_t* __restrict__ pair_tok,
    const float* __restrict__ topk_w, long b_stride, long s_stride, long z_stride,
    int n_expert, int n_pairs, int n_tokens, int chunk_rows) {
  using A = Act<BF16>;
  static_assert(!W8 || (!ZP && GPC == 1), "E4M3: 128-row scale units, no zero points");
  constexpr int NV = W8 ? 2 : 1;  // 16-byte weight vectors per lane and group
  // STAGE 0 (direct activations): no shared slice; each wave fetches the activation tiles
  // of its own groups, and the scales and zero points of its own groups and blocks, into
  // its own LDS region with direct-to-LDS loads, so no barrier stands between the loads and
  // the arithmetic.  An MFMA operand holds 16 rows of 16 bytes per 32-row step, so loading
  // it straight into registers reads 16 rows x 64 bytes per instruction; the direct loads
  // instead read four whole 256-byte row pieces per instruction (measured on MI355X at
  // M=16, K=N=4096: 4.9 against 6.4 us).  A tile's 16 granules of row r are stored in the
  // order (granule ^ r), so that the operand reads of 8 or 16 consecutive lanes (rows)
  // fall in distinct banks.
  constexpr bool DA = STAGE == 0;
  static_assert(!DA || (GW <= 8 && !PAIR), "direct activations: at most 8 groups, no pair");
  static_assert(!R1 || (!DA && !W8), "one-row path: staged activations, 4-bit weights");
  // DUAL: each wave applies its activation operands to two adjacent column blocks, so the
  // activations are read once per two blocks (direct activations, 4-bit weights).
  static_assert(!DUAL || (DA && !PAIR && !W8 && !R1), "dual blocks: direct activations");
  static_assert(!SEG || (!DA && !W8 && !DUAL), "segments: staged activations, 4-bit weights");
  constexpr int SR = R1 ? 1 : kSegRows;  // rows of a segment (SEG)
  constexpr int T = WAVES * 64;
  constexpr int NB = (PAIR || DUAL) ? 2 : 1;  // column blocks of the work-group
  constexpr int NBV = DUAL ? 2 : 1;           // column blocks of each wave
  constexpr int KW = PAIR ? WAVES / 2 : WAVES;  // waves splitting K for one block
  constexpr int MS = small_max_span(WAVES, PAIR, GW);  // groups the staged scales cover
  constexpr int SU = small_scale_slots(WAVES, PAIR, GW, NB, GPC);  // staged scale dwords
  constexpr int ZU = small_zero_slots(WAVES, PAIR, GW, NB, GPC);   // staged zero points
  constexpr int JQ = GPC <= 4 ? 4 / GPC : 1;  // 32-row MFMA steps per scale unit (GPC <= 4)
  static_assert(SU >= 1 && SU * T == NB * MS * 8 * GPC, "scale slots cover the range");
  static_assert(ZU * T >= NB * MS * GPC, "zero-point slots cover the range");
  extern __shared__ f16x8 a_lds[];            // [m][span*16] granules (+ padding), or direct
  __shared__ uint32_t s_lds[DA ? 1 : SU * T];          // scales, [block][chunk][unit][col]
  __shared__ u32x2 z_lds[ZP && !DA ? ZU * T : 1];      // zero points, [block][chunk][unit]
  __shared__ f32x4 red[DA ? 1 : NBV][DA ? 1 : WAVES][64];
  // R1: per scale unit of the slice and row class, the activations' sum (the zero-point
  // term of the unit's partial).
  constexpr int EX = GPC == 8 ? 2 : 4;  // activation sums per scale unit: one per row class
  constexpr bool R1B = R1;              // one row: activation sums staged
  // Per-wave staging (PW): each wave stages only its own groups' activation granules, scale
  // words and zero points, at their places in the shared slice, so that its arithmetic
  // waits for its own loads only and no work-group barrier precedes it.  It serves the one-
  // row path, and on sixteen waves dense products of up to eight rows and grouped segments
  // of up to four.  Under a full weight stream the activation loads arrive late (a median
  // 2.4 us after the wave starts at K=14336, N=4096), and the barrier waited for the slowest
  // of the waves.  Measured on MI355X (one run each, us): m=1, K=14336, N=4096 8.4 -> 7.2;
  // K=11008 7.7 -> 6.7; K=28672, N=8192 29 -> 24; K=14336, N=14336 26 -> 22; decode
  // unchanged; m=2/4/8 at K=14336, N=4096 9.8/11.4/20.7 -> 8.4/9.7/17.8; MoE down projection
  // (K=14336, N=4096) at two and three tokens 28 -> 25.4 and 42 -> 37.  With four waves and
  // several rows it was slower (K=N=4096, m=8: 4.3 -> 5.2), so those keep the shared slice.
  // Dense eight-wave plans of up to four rows per work-group launch separate instances
  // that take it (PWR; K=N=8192, m=2/3/4: 8.9-10.0/10.0-10.3/10.0-10.3 -> 8.6-8.7/9.4/
  // 9.7-10.0 us; K=N=5120, m=4: 8.6-8.9 -> 8.2-8.4), while more rows keep the shared slice
  // (m=6/8 measured 2-8% slower with it).  The stage slots cover a wave's share
  // (stage_slots).
  static_assert(!PWR || (WAVES == 8 && !SEG && !DA && !PAIR && !R1 && !W8),
                "per-wave staging on request: dense eight-wave staged plans");
  constexpr bool PW = !DA && !PAIR && (R1 || WAVES == 16 || PWR);
  __shared__ float rsum_lds[R1B ? MS * GPC * EX : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform: every per-wave index below is formed once, on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;  // column inside the 16-column block; also the A row of the lane
  const int qd = lane >> 4;   // which 8 rows of each 32-row MFMA step the lane carries
  const int half = PAIR ? wave / KW : 0;       // the wave's block of the pair
  const int kwave = wave - half * KW;          // the wave's index along K
  const int nb = NB * blockIdx.x + half;
  const int split = SEG ? 0 : blockIdx.y;
  // Row chunks (grid z, one split): the work-group's chunk_rows rows of a taller product.
  if (!SEG && gridDim.z > 1) {
    const int r0 = chunk_rows * blockIdx.z;
    a += (long)r0 * lda;
    c += (long)r0 * (PAIR ? n / 2 : n);
    m = m - r0 < chunk_rows ? m - r0 : chunk_rows;
  }

  // SEG: the segment's expert and rows (wave-uniform, scalar loads).
  int seg_p0 = 0;
  if constexpr (SEG) {
    const int sgi = blockIdx.y;
    const int ex = ex_ids != nullptr ? ex_ids[sgi] : sgi;
    if (ex < 0 || ex >= n_expert) return;
    int a0 = ex_off[sgi], a1 = ex_off[sgi + 1];
    a0 = a0 < 0 ? 0 : (a0 > n_pairs ? n_pairs : a0);
    a1 = a1 < a0 ? a0 : (a1 > n_pairs ? n_pairs : a1);
    seg_p0 = a0;
    const int rows = a1 - a0;  // at most SR by the launch's bound for a valid CSR
    if (rows <= 0) return;
    m = rows < SR ? rows : SR;
    b += (long)ex * b_stride;
    s += (long)ex * s_stride;
    if constexpr (ZP) z += (long)ex * z_stride;
  }
  // SEG: output row (pair, or -1: not written) and activation row offset of segment row j
  // (rows past the last repeat it); filled once the first weight loads are in flight.
  i32x4 seg_pair = {0, 0, 0, 0};
  i32x4 seg_aoff = {0, 0, 0, 0};
  f32x4 seg_w = {1.f, 1.f, 1.f, 1.f};  // routing weights of the rows (with topk_w)
  static_assert(SR <= 4, "segment rows held in one register vector");
  const auto seg_rows = [&] {
#pragma unroll
    for (int j = 0; j < SR; ++j) seg_pair[j] = ex_pairs[seg_p0 + (j < m ? j : m - 1)];
    __builtin_amdgcn_sched_barrier(0);  // all row loads in flight before the first use
    i32x4 tok;
#pragma unroll
    for (int j = 0; j < SR; ++j) tok[j] = pair_tok[max(0, min(seg_pair[j], n_pairs - 1))];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < SR; ++j) {
      // a row with a pair or token out of range reads a clamped row and is not written
      const int pr = seg_pair[j];
      seg_aoff[j] = max(0, min(tok[j], n_tokens - 1)) * lda;
      const bool ok = ((unsigned)pr < (unsigned)n_pairs) & ((unsigned)tok[j] < (unsigned)n_tokens);
      seg_pair[j] = ok ? pr : -1;
    }
  };
  const auto seg_weights = [&] {
    if (topk_w != nullptr) {
#pragma unroll
      for (int j = 0; j < SR; ++j) seg_w[j] = topk_w[max(0, seg_pair[j])];
    }
  };
  // segment row rr (per lane) -> its entry of v
  const auto seg_select = [&](i32x4 v, int rr) {
    int x = v[0];
#pragma unroll
    for (int j = 1; j < SR; ++j) x = rr == j ? v[j] : x;
    return x;
  };

  // The work-group's range of K groups (groups * splits stays far below 2^31); a single
  // split, the common case, needs no division.
  int gs0 = 0, gs1 = groups;
  if (splits > 1) {
    gs0 = (int)((unsigned)(groups * split) / (unsigned)splits);
    gs1 = (int)((unsigned)(groups * (split + 1)) / (unsigned)splits);
  }
  const int span = gs1 - gs0;
  const int g0 = gs0 + span * kwave / KW;
  const int g1 = gs0 + span * (kwave + 1) / KW;
  const int gw = g1 - g0;  // <= GW by the launch plan

  // 1. Activation granules: slot u of this thread is granule tid + u*T of the slice, at row
  //    r and granule column q; (r, q) advance by a fixed (dr, dq) per slot.
  const int per_row = span * (kGroup / 8);
  int dr = 0, r = 0;  // a row at least as long as a staging round needs no division
  if (per_row < T) {
    dr = T / per_row;
    r = tid / per_row;
  }
  const int dq = T - dr * per_row;
  int q = tid - r * per_row;
  const f16* a_base = a + (long)gs0 * kGroup;
  f16x8 stage[DA ? 1 : STAGE];
  int stage_q[R1B ? STAGE : 1];        // granule of each slot in the slice
  bool stage_real[R1B ? STAGE : 1];    // the slot lies inside the slice (and its share)
  // The wave's share of the slice (dense, more than one row): m rows of gw * 16 granules;
  // slot u of the lane holds element lane + 64u of it, at row wr and granule wq of the row's
  // share, stepped like the shared slice.  f(u, row (clamped), slice column, inside).
  const auto pw_walk = [&](auto f) {
    const int per_w = gw * 16;
    int wr = 0, ddr = 0;
    if (per_w < 64) {
      ddr = 64 / per_w;
      wr = lane / per_w;
    }
    const int ddq = 64 - ddr * per_w;
    int wq = lane - wr * per_w;
#pragma unroll
    for (int u = 0; u < STAGE; ++u) {
      f(u, wr < m ? wr : m - 1, (g0 - gs0) * 16 + wq, wr < m);
      wq += ddq;
      wr += ddr;
      const bool wrap = wq >= per_w;
      wq = wrap ? wq - per_w : wq;
      wr = wrap ? wr + 1 : wr;
    }
  };
  const auto load_stage = [&] {
    if constexpr (PW && !R1) {
      pw_walk([&](int u, int rr, int col_g, bool) {
        const long row_off = SEG ? (long)seg_select(seg_aoff, rr) : (long)rr * lda;
        stage[u] = *reinterpret_cast<const f16x8*>(a_base + row_off + 8 * col_g);
      });
      return;
    }
    if constexpr (PW) {
      // one row: slot u of the lane holds granule lane + 64u of the wave's groups
#pragma unroll
      for (int u = 0; u < STAGE; ++u) {
        const bool real = lane + 64 * u < gw * 16;
        const int qq = (g0 - gs0) * 16 + (real ? lane + 64 * u : 0);
        stage_q[u] = qq;
        stage_real[u] = real;
        const long row_off = SEG ? (long)seg_select(seg_aoff, 0) : 0;
        stage[u] = *reinterpret_cast<const f16x8*>(a_base + row_off + 8 * qq);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < STAGE; ++u) {
      const int rr = r < m ? r : m - 1;
      if constexpr (R1B) {
        stage_q[u] = q;
        stage_real[u] = r < m;
      }
      const long row_off = SEG ? (long)seg_select(seg_aoff, rr) : (long)rr * lda;
      stage[u] = *reinterpret_cast<const f16x8*>(a_base + row_off + 8 * q);
      q += dq;
      r += dr;
      const bool wrap = q >= per_row;
      q = wrap ? q - per_row : q;
      r = wrap ? r + 1 : r;
    }
  };
  if constexpr (!DA && !SEG) load_stage();
  // 2. Scales (8 dwords of fp16 pairs per unit row) and zero points of the range, for each
  //    of the work-group's blocks ([block][unit] in LDS).  A block holds groups*GPC units.
  const long units = (long)groups * GPC;
  const long pair0 = (long)NB * blockIdx.x * units + (long)gs0 * GPC;  // first block's range
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(s);
  const int s_words = span * GPC * 8;
  uint32_t s_stage[DA ? 1 : SU];
#pragma unroll
  for (int u = 0; u < (DA ? 0 : SU); ++u) {
    int i = tid + u * T;
    if constexpr (PW) {
      const int e = lane + 64 * u;
      i = (g0 - gs0) * GPC * 8 + (e < gw * GPC * 8 ? e : 0);
    }
    i = i < NB * s_words ? i : NB * s_words - 1;
    const int h = NB == 2 && i >= s_words ? 1 : 0;  // block of the pair holding dword i
    s_stage[u] = s32[(pair0 + h * units) * 8 + (i - h * s_words)];
  }
  u32x2 z_stage[DA ? 1 : ZU];
#pragma unroll
  for (int u = 0; u < (DA ? 0 : ZU); ++u) {
    z_stage[u] = u32x2{0u, 0u};
    if constexpr (ZP) {
      const int z_words = span * GPC;
      int i = tid + u * T;
      if constexpr (PW) {
        const int e = lane + 64 * u;
        i = (g0 - gs0) * GPC + (e < gw * GPC ? e : 0);
      }
      i = i < NB * z_words ? i : NB * z_words - 1;
      const int h = NB == 2 && i >= z_words ? 1 : 0;
      z_stage[u] = z[pair0 + h * units + (i - h * z_words)];
    }
  }

  // 3. The wave's weight chunks, all in flight before any arithmetic.
  u32x4 bw[GW][NV * NBV];  // E4M3: the group's two vectors; DUAL: the two blocks' chunks
  const auto load_b = [&](int i) {
    const int g = g0 + (i < gw ? i : gw - 1);
#pragma unroll
    for (int v = 0; v < NV * NBV; ++v)
      bw[i][v] = __builtin_nontemporal_load(
          &b[(DUAL ? (long)(nb + v) * groups + g : ((long)nb * groups + g) * NV + v) * 64 + lane]);
  };
  // Direct activations: the wave's region (tiles of its GW groups) and its scale words.
  constexpr int SZN = direct_sz_loads(GW, GPC, ZP);
  constexpr int SZS = GW * GPC * 8;  // scale dwords per block; the zero-point words follow
  f16x8* const a_own = a_lds + wave * GW * (kDirectTile / 16);
  uint32_t* const sz_own =
      reinterpret_cast<uint32_t*>(a_lds + WAVES * GW * (kDirectTile / 16)) + wave * NBV * SZN * 64;
  if constexpr (DA) {
    // Issue order: scale words, group 0's weights, every activation tile, the remaining
    // weights; the scheduling barriers keep it, so the single wait below (for all loads but
    // the trailing weights) covers the LDS data, and each group's weights are waited for
    // in order as they are consumed.
    const long unit0 = (long)g0 * GPC;
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      const long units0 = (long)(nb + v) * units + unit0;  // the block's first unit of the wave
#pragma unroll
      for (int u = 0; u < SZN; ++u) {
        // dword d: scale dword d (d < SZS), else zero-point word d - SZS, clamped into the
        // wave's gw groups (the trailing padding repeats the last word)
        const int d = lane + 64 * u;
        const uint32_t* src;
        if (!ZP || d < SZS) {
          const int e = d < gw * GPC * 8 ? d : gw * GPC * 8 - 1;
          src = reinterpret_cast<const uint32_t*>(s) + units0 * 8 + e;
        } else {
          const int e = d - SZS < gw * GPC * 2 ? d - SZS : gw * GPC * 2 - 1;
          src = reinterpret_cast<const uint32_t*>(z) + units0 * 2 + e;
        }
        __builtin_amdgcn_global_load_lds(src, sz_own + (v * SZN + u) * 64, 4, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_b(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      // tile load t: rows 4t .. 4t + 3 (clamped to m - 1), lane granule (lane & 15) ^ row
      const int g = g0 + (i < gw ? i : gw - 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 4 * t + (lane >> 4);
        const int rr = r < m ? r : m - 1;
        __builtin_amdgcn_global_load_lds(
            a + (long)rr * lda + (long)g * kGroup + 8 * ((lane & 15) ^ r),
            a_own + (i * 4 + t) * 64, 16, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 1; i < GW; ++i) load_b(i);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(GW - 1) * NV * NBV>();
    __builtin_amdgcn_sched_barrier(0);  // no LDS read of the region moves above the wait
  } else if constexpr (SEG) {
    // the first groups' weights, then the row indices and the activation slice, then the
    // rest of the weights: the slice's LDS writes wait for the first groups' weights only
    constexpr int EARLY = GW >= 4 ? 2 : 1;
#pragma unroll
    for (int i = 0; i < EARLY; ++i) load_b(i);
    __builtin_amdgcn_sched_barrier(0);
    seg_rows();
    load_stage();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PW) {
      // every wave's activations ahead of any wave's remaining weights (as below)
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    seg_weights();
#pragma unroll
    for (int i = EARLY; i < GW; ++i) load_b(i);
  } else {
    // A bare barrier (no wait) issues every wave's activation and scale loads ahead of any
    // wave's weight loads, so that the slice's LDS writes, and so the arithmetic, wait less
    // behind other waves' weights (MI355X, one run: K=8192, N=4096, m=1 5.74 ->
    // 5.27 us; K=14336, N=4096, m=4 11.9 -> 11.3; K=4096, N=14336, m=4 9.2 -> 8.9; decode
    // unchanged).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < GW; ++i) load_b(i);
  }

  // 4. Stage into LDS (waits for the activations and scales only), then sync.
  if constexpr (!DA) {
#pragma unroll
    for (int u = 0; u < STAGE; ++u) {
      // one row, fp16: rows 0, 1, 4, 5 of the granule first, then 2, 3, 6, 7 (the order of
      // the subnormal operands' two products)
      const u32x4 w = __builtin_bit_cast(u32x4, stage[u]);
      const f16x8 v = R1 && !BF16 ? __builtin_bit_cast(f16x8, u32x4{w[0], w[2], w[1], w[3]})
                                  : stage[u];
      if constexpr (PW && R1) {
        if (stage_real[u]) a_lds[stage_q[u]] = v;
      } else if constexpr (!PW) {
        a_lds[tid + u * T] = v;
      }
    }
    if constexpr (PW && !R1) {
      pw_walk([&](int u, int rr, int col_g, bool inside) {
        if (inside) a_lds[rr * per_row + col_g] = stage[u];
      });
    }
  }
  if constexpr (PW) {
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int e = lane + 64 * u;
      if (e < gw * GPC * 8) s_lds[(g0 - gs0) * GPC * 8 + e] = s_stage[u];
    }
    if constexpr (ZP) {
#pragma unroll
      for (int u = 0; u < ZU; ++u) {
        const int e = lane + 64 * u;
        if (e < gw * GPC) z_lds[(g0 - gs0) * GPC + e] = z_stage[u];
      }
    }
  } else if constexpr (!DA) {
#pragma unroll
    for (int u = 0; u < SU; ++u) s_lds[tid + u * T] = s_stage[u];
    if constexpr (ZP) {
#pragma unroll
      for (int u = 0; u < ZU; ++u) z_lds[tid + u * T] = z_stage[u];
    }
  }
  if constexpr (R1B) {
    // A unit of the slice is GR consecutive granules, held by GR consecutive lanes of one
    // slot (aligned, since T and the row length are multiples of 16); granule q of a chunk
    // is row class q % 4 of step q / 4.  Each lane adds its eight activations, a butterfly
    // adds the lanes of one class (none for 16-row units), and the first EX lanes of the
    // unit store per class (per granule) at unit * EX + class.
    constexpr int GR = 16 / GPC;
#pragma unroll
    for (int u = 0; u < STAGE; ++u) {
      // fp16: a dot product of each pair with ones (exact products, fp32 sums).  bf16: each
      // value is the upper half of a binary32 (words reinterpreted as bf16 pairs for the dot
      // builtin are miscompiled by this toolchain inside this loop: it reads word 0 four
      // times).
      const u32x4 w = __builtin_bit_cast(u32x4, stage[u]);
      float rs = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if constexpr (BF16) {
          rs += __builtin_bit_cast(float, w[h] << 16) + __builtin_bit_cast(float, w[h] & 0xFFFF0000u);
        } else {
          rs = __builtin_amdgcn_fdot2(f16x2{stage[u][2 * h], stage[u][2 * h + 1]},
                                      f16x2{(f16)1.f, (f16)1.f}, rs, false);
        }
      }
#pragma unroll
      for (int d = EX; d < GR; d *= 2) rs += __shfl_xor(rs, d);
      if (stage_real[u] && (tid & (GR - 1)) < EX)
        rsum_lds[stage_q[u] / GR * EX + stage_q[u] % EX] = rs;
    }
  }
  if constexpr (PW) {
    // the wave reads only what its own lanes wrote: order its LDS writes before its reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else if constexpr (!DA) {
    __syncthreads();
  }

  // 5. Arithmetic.  MFMA rows >= m are never stored, and a row of the product depends on
  //    its own A row only, so those lanes read row m - 1 instead of selecting zeros.  The
  //    group scales are read up front and each chunk's activation operands are read from
  //    LDS while the previous chunk's MFMAs run, so that no LDS round trip sits between a
  //    weight chunk's arrival and its products.
  // fp16: the magic-number registers of the exact dequant; bf16: the 128.0 pattern of the
  // biased one (see below).
  const auto mr = [] {
    if constexpr (BF16)
      return magic_reg_bf128();
    else
      return A::magic();
  }();
  const int arow = (col < m ? col : m - 1) * per_row;
  const uint16_t* s_half = reinterpret_cast<const uint16_t*>(s_lds);
  int gl[GW];  // chunk of step i inside the staged range (clamped for the masked steps)
  // Scale bits of unit t of step i for this lane's column, and the zero-point words of that
  // unit, for block hb of the work-group (staged) or of the wave (direct).
  const auto scale_bits = [&](int hb, int i, int t) -> uint16_t {
    if constexpr (DA)
      return reinterpret_cast<const uint16_t*>(sz_own + hb * SZN * 64)[(i * GPC + t) * 16 + col];
    else
      return s_half[((hb * span + gl[i]) * GPC + t) * 16 + col];
  };
  const auto zero_word = [&](int hb, int i, int t) -> u32x2 {
    if constexpr (DA) {
      const uint32_t* zw = sz_own + hb * SZN * 64 + SZS + 2 * (i * GPC + t);
      return u32x2{zw[0], zw[1]};
    } else {
      return z_lds[(hb * span + gl[i]) * GPC + t];
    }
  };
  // Scales hoisted per chunk, for up to four units and eight groups per wave (read in place
  // otherwise: the registers of sixteen groups would spill).
  constexpr bool HSC = GPC <= 4 && GW <= 8;
  constexpr int HS = GPC <= 4 ? GPC : 1;
  float scs[NBV][HSC ? GW : 1][HSC ? HS : 1];  // per column block of the wave
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    gl[i] = g0 - gs0 + (i < gw ? i : gw - 1);
    if constexpr (HSC) {
#pragma unroll
      for (int v = 0; v < NBV; ++v) {
        const int hv = DUAL ? v : half;
#pragma unroll
        for (int t = 0; t < GPC; ++t) {
          const float x = A::value(scale_bits(hv, i, t));
          scs[v][i][t] = i < gw ? x : 0.f;
        }
      }
    }
  }
  // unit t of step i: its zero point for this lane's column
  const auto zero_of = [&](int i, int t) {
    return ZP ? zero_code(zero_word(half, i, t), col) : 8;
  };
  // R1: the zero-point term of unit t of step i, for this lane's column and row class:
  // (bias + z) S, the bias 128 of the bf16 operands (none for the fp16 subnormals).
  const auto excess = [&](int i, int t) -> float {
    const int unit = gl[i] * GPC + t;
    const int slot = GPC == 8 ? unit * 2 + (qd & 1) : unit * 4 + qd;
    return ((BF16 ? 128.f : 0.f) + (float)zero_of(i, t)) * rsum_lds[slot];
  };
  // Hoisted with the scales for up to two units per chunk; with more, the registers would
  // cost a wave of occupancy, so the excess is read in place.
  constexpr bool HX = GPC <= 2 && GW <= 8;
  float ex[R1B && HX ? GW : 1][R1B && HX ? HS : 1];
  if constexpr (R1B && HX) {
#pragma unroll
    for (int i = 0; i < GW; ++i) {
#pragma unroll
      for (int t = 0; t < GPC; ++t) ex[i][t] = excess(i, t);
    }
  }
  // R1: the 4x4x4 products broadcast one block's activation operand to the four blocks of
  // a row class (lanes 16qd..16qd+15), from the block ABID names.  Product p = 0..7 of a
  // chunk (step p / 2, half p % 2) takes it from lane 16qd + 4(p % 4), register pair p / 4,
  // so a lane holds two 4-row activation pieces per chunk instead of the sixteen rows of
  // all four steps: a quarter of the LDS reads.
  const u32x2* a_lds2 = reinterpret_cast<const u32x2*>(a_lds);
  const auto r1_operands = [&](int chunk, u32x2* r) {
    const int x = col >> 2;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      r[h] = a_lds2[2 * (chunk * 16 + 4 * (2 * h + (x >> 1)) + qd) + (x & 1)];
  };
  f16x8 an[R1 ? 1 : 4];
  u32x2 an1[2];
  if constexpr (R1) {
    r1_operands(gl[0], an1);
  } else if constexpr (!DA) {
#pragma unroll
    for (int j = 0; j < 4; ++j) an[j] = a_lds[arow + gl[0] * 16 + 4 * j + qd];
  }
  f32x4 accs[NBV];
#pragma unroll
  for (int v = 0; v < NBV; ++v) accs[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int half0 = half;
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    f16x8 ac[R1 ? 1 : 4];
    u32x2 ar[2];
    if constexpr (R1) {
      ar[0] = an1[0];
      ar[1] = an1[1];
      if (i + 1 < GW) r1_operands(gl[i + 1], an1);
    } else {
      if constexpr (DA) {
        // lane (row col, class qd) of step j: granule 4j + qd of row col, in tile load col / 4
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ac[j] = a_own[(i * 4 + (col >> 2)) * 64 + 16 * (col & 3) + ((4 * j + qd) ^ col)];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) ac[j] = an[j];
      }
      if (!DA && i + 1 < GW) {
#pragma unroll
        for (int j = 0; j < 4; ++j) an[j] = a_lds[arow + gl[i + 1] * 16 + 4 * j + qd];
      }
    }
    // With eight groups per wave, pin the prefetch ahead of this group's work (measured
    // faster for the decode shape, slower for shallower pipelines).
    if constexpr (GW >= 8) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
    // the wave's block v: its place in the staged scales and zero points, its weights and sums
    const int half = DUAL ? v : half0;
    const int bv = DUAL ? v : 0;
    f32x4& acc = accs[v];
    // unit t's scale of this chunk (zero for a masked chunk)
    const auto scale_at = [&](int t) -> float {
      if constexpr (HSC) {
        return scs[v][i][t];
      } else {
        const float x = A::value(scale_bits(half, i, t));
        return i < gw ? x : 0.f;
      }
    };
    if constexpr (W8) {
      // 32-row step j: vector j / 2, words 2(j % 2) and 2(j % 2) + 1 (rows 0-3 and 4-7).
      f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p = A::mfma16(ac[j], A::fp8(bw[i][j >> 1][2 * (j & 1)], bw[i][j >> 1][2 * (j & 1) + 1]),
                      p);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(scale_at(0), p[e], acc[e]);
    } else if constexpr (R1) {
      // Only row 0 of the product is real.  Operands: the fp16 subnormal nibbles, or biased
      // 128 + q for bf16 (see the header comment).
      // the zero-point term to remove from unit t's product
      const auto unit_excess = [&](int t) -> float {
        if constexpr (HX)
          return ex[i][t];
        else
          return excess(i, t);
      };
      // one 4x4x4 product (16 blocks) on four rows; the operand broadcast ID is an immediate
      const auto mfma1 = [](u32x2 a2, u32x2 b2, f32x4 cc, auto abid) {
        constexpr int ID = decltype(abid)::value;
        if constexpr (BF16) {
          typedef short s4 __attribute__((ext_vector_type(4)));
          return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s4, a2),
                                                        __builtin_bit_cast(s4, b2), cc, 2, ID, 0);
        } else {
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4, a2),
                                                    __builtin_bit_cast(h4, b2), cc, 2, ID, 0);
        }
      };
      // Step j's two products, operands broadcast from products 2j and 2j + 1 of the chunk
      // (ABID 2j % 4 and 2j % 4 + 1).  bf16: rows 0-3 and 4-7 into one sum c24.  fp16:
      // rows 0, 1, 4, 5 (nibbles at 2^-24) into c24, rows 2, 3, 6, 7 (at 2^-20) into c20,
      // each against the matching half of the reordered activation granule.
      const auto step = [&](int j, uint32_t w, f32x4& c24, f32x4& c20) {
        u32x2 b0, b1;
        if constexpr (BF16) {
          const u32x4 b = __builtin_bit_cast(u32x4, dequant8_bf_biased(w, mr));
          b0 = u32x2{b[0], b[1]};
          b1 = u32x2{b[2], b[3]};
        } else {
          const uint32_t w8 = w >> 8;
          b0 = u32x2{w & 0x000F000Fu, w8 & 0x000F000Fu};
          b1 = u32x2{w & 0x00F000F0u, w8 & 0x00F000F0u};
        }
        f32x4& second = BF16 ? c24 : c20;
        if (j & 1) {
          c24 = mfma1(ar[j >> 1], b0, c24, std::integral_constant<int, 2>{});
          second = mfma1(ar[j >> 1], b1, second, std::integral_constant<int, 3>{});
        } else {
          c24 = mfma1(ar[j >> 1], b0, c24, std::integral_constant<int, 0>{});
          second = mfma1(ar[j >> 1], b1, second, std::integral_constant<int, 1>{});
        }
      };
      // a unit's exact-weight partial: 2^24 c24 + 2^20 c20 - z S (fp16), c24 - (128 + z) S
      // (bf16)
      const auto unit_sum = [](f32x4 c24, f32x4 c20, float exv) -> float {
        if constexpr (BF16)
          return c24[0] - exv;
        else
          return __builtin_fmaf(__builtin_fmaf(c20[0], 0x1p-4f, c24[0]), 0x1p24f, -exv);
      };
      const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (GPC <= 4) {
#pragma unroll
        for (int t = 0; t < GPC; ++t) {
          f32x4 c24 = zero4, c20 = zero4;
#pragma unroll
          for (int jj = 0; jj < JQ; ++jj) {
            const int j = t * JQ + jj;
            step(j, bw[i][bv][j], c24, c20);
          }
          acc[0] = __builtin_fmaf(scale_at(t), unit_sum(c24, c20, unit_excess(t)), acc[0]);
        }
      } else {
        // 16-row units: the lane's eight rows of step j lie in unit 2j + (qd >> 1).
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 2 * j + (qd >> 1);
          f32x4 c24 = zero4, c20 = zero4;
          step(j, bw[i][bv][j], c24, c20);
          const float v = A::value(scale_bits(half, i, t));
          acc[0] = __builtin_fmaf(i < gw ? v : 0.f, unit_sum(c24, c20, excess(i, t)), acc[0]);
        }
      }
    } else if constexpr (BF16) {
      // bf16 has no packed add, and the exact dequant costs 21 VALU per word, which this
      // weight-stream-bound kernel cannot hide.  The weights enter the MFMA biased, as
      // 128 + q (7 VALU per word), and the same activations meet an all-ones operand: r is
      // the activation sum of each row, and p - (128 + z) * r the exact-weight partial,
      // formed in fp32 by one fma (the cancellation costs about 2^-19 relative).
      const bf16x8 ones = __builtin_bit_cast(
          bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
      const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (GPC <= 4) {
#pragma unroll
        for (int t = 0; t < GPC; ++t) {
          const int zc = ZP ? zero_code(zero_word(half, i, t), col) : 8;
          const float off = (float)(128 + zc);
          f32x4 p = zero4, r = zero4;
#pragma unroll
          for (int jj = 0; jj < JQ; ++jj) {
            const int j = t * JQ + jj;
            p = A::mfma16(ac[j], dequant8_bf_biased(bw[i][bv][j], mr), p);
            r = A::mfma16(ac[j], ones, r);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[e] = __builtin_fmaf(scale_at(t), __builtin_fmaf(-off, r[e], p[e]), acc[e]);
        }
      } else {
        // 16-row units: as on the fp16 path, each MFMA sees one unit's half of the step.
        const int hi = qd >> 1;
        const bf16x8 zero8{};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 w = dequant8_bf_biased(bw[i][bv][j], mr);
          const f32x4 p0 = A::mfma16(ac[j], hi ? zero8 : w, zero4);
          const f32x4 p1 = A::mfma16(ac[j], hi ? w : zero8, zero4);
          const f32x4 r0 = A::mfma16(ac[j], hi ? zero8 : ones, zero4);
          const f32x4 r1 = A::mfma16(ac[j], hi ? ones : zero8, zero4);
          const int z0 = ZP ? zero_code(zero_word(half, i, 2 * j), col) : 8;
          const int z1 = ZP ? zero_code(zero_word(half, i, 2 * j + 1), col) : 8;
          const float v0 = A::value(scale_bits(half, i, 2 * j));
          const float v1 = A::value(scale_bits(half, i, 2 * j + 1));
          const float s0 = i < gw ? v0 : 0.f;
          const float s1 = i < gw ? v1 : 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[e] = __builtin_fmaf(s0, __builtin_fmaf(-(float)(128 + z0), r0[e], p0[e]), acc[e]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[e] = __builtin_fmaf(s1, __builtin_fmaf(-(float)(128 + z1), r1[e], p1[e]), acc[e]);
        }
      }
    } else if constexpr (GPC <= 4) {
#pragma unroll
      for (int t = 0; t < GPC; ++t) {
        const auto zo = A::zero(ZP ? zero_code(zero_word(half, i, t), col) : 8);
        f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < JQ; ++jj) {
          const int j = t * JQ + jj;
          p = A::mfma16(ac[j], A::dequant(bw[i][bv][j], zo, mr), p);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(scale_at(t), p[e], acc[e]);
      }
    } else {
      // 16-row units: the lane's 8 rows of step j lie in unit 2j + hi.  Its weights enter
      // the MFMA of that unit and zeros the other's, so each product sums one unit only.
      const int hi = qd >> 1;
      const typename A::W8 zero8{};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto zo = A::zero(ZP ? zero_code(zero_word(half, i, 2 * j + hi), col) : 8);
        const typename A::W8 w = A::dequant(bw[i][bv][j], zo, mr);
        const f32x4 p0 = A::mfma16(ac[j], hi ? zero8 : w, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 p1 = A::mfma16(ac[j], hi ? w : zero8, f32x4{0.f, 0.f, 0.f, 0.f});
        // (the reads are unconditional, in bounds through the clamped chunk; a masked step
        // selects zero scales)
        const float v0 = A::value(scale_bits(half, i, 2 * j));
        const float v1 = A::value(scale_bits(half, i, 2 * j + 1));
        const float s0 = i < gw ? v0 : 0.f;
        const float s1 = i < gw ? v1 : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(s0, p0[e], acc[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(s1, p1[e], acc[e]);
      }
    }
    }  // blocks of the wave
    if constexpr (GW >= 8) __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (R1) {
    // each lane holds its column's sum over one of the four row classes of every step
    accs[0][0] += __shfl_xor(accs[0][0], 16);
    accs[0][0] += __shfl_xor(accs[0][0], 32);
  }
  // Work-group reduce over the waves, in wave order.  Direct plans put each wave's sums at
  // the start of its own region (its operand reads precede the writes in the wave's LDS
  // order, and no other wave reads that region).
  const auto red_at = [&](int v, int w) -> f32x4* {
    if constexpr (DA)
      return reinterpret_cast<f32x4*>(a_lds + w * GW * (kDirectTile / 16)) + v * 64;
    else
      return red[v][w];
  };
  if constexpr (R1 && !PAIR) {
    // One row: after the shuffles every row class holds the column sums, so each wave hands
    // over only its 16 column sums, and the first 16 lanes of wave 0 add them in wave order.
    float* const redf = reinterpret_cast<float*>(&red[0][0][0]);
    if (lane < 16) redf[wave * 16 + lane] = accs[0][0];
    __syncthreads();
    if (wave != 0 || lane >= 16) return;
    float tot = redf[lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) tot += redf[w * 16 + lane];
    const long colx = (long)nb * 16 + lane;
    if constexpr (SEG) {
      if (seg_pair[0] >= 0)
        c[(long)seg_pair[0] * n + colx] = A::round(topk_w != nullptr ? tot * seg_w[0] : tot);
    } else if (splits == 1) {
      c[colx] = A::round(tot);
    } else {
      partials[(long)split * n + colx] = tot;
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < NBV; ++v) red_at(v, wave)[lane] = accs[v];
  __syncthreads();
  if constexpr (PAIR) {
    // wave e (e < 4) sums element e of the lane's gate and up sums, in wave order
    if (wave >= 4) return;
    const int e = wave;
    const int row = 4 * qd + e;
    float gs = reinterpret_cast<const float*>(red_at(0, 0) + lane)[e];
    float us = reinterpret_cast<const float*>(red_at(0, KW) + lane)[e];
#pragma unroll
    for (int w = 1; w < KW; ++w) {
      gs += reinterpret_cast<const float*>(red_at(0, w) + lane)[e];
      us += reinterpret_cast<const float*>(red_at(0, KW + w) + lane)[e];
    }
    const long colj = (long)blockIdx.x * 16 + col;  // column of the [m][n/2] activation
    if (row >= m) return;
    // SEG: the pair's row of the activation (not written for an out-of-range pair)
    const int pr = SEG ? seg_select(seg_pair, row) : row;
    if (pr >= 0) c[(long)pr * (n / 2) + colj] = A::round(silu_times(gs, us));
    return;
  }
  // The 4 x NBV output elements of a lane are summed by different waves (part = wave, wave
  // + WAVES, ...: block part / 4, element part % 4), each adding the waves' sums in wave
  // order, so the reduction's tail is spread over the waves.
#pragma unroll
  for (int part = wave; part < 4 * NBV; part += WAVES) {
    const int v = part / 4;
    const int e = part % 4;
    float tot = reinterpret_cast<const float*>(red_at(v, 0) + lane)[e];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) tot += reinterpret_cast<const float*>(red_at(v, w) + lane)[e];

    // Output layout of the 16x16 block: lane holds rows 4*qd + e of column `col`.
    const long colx = (long)(nb + v) * 16 + col;
    const int row = 4 * qd + e;
    if (row >= m) continue;
    if constexpr (SEG) {
      // the pair's output row, times its routing weight in fp32 before the rounding
      const int pr = seg_select(seg_pair, row);
      float wr = seg_w[0];
#pragma unroll
      for (int j = 1; j < SR; ++j) wr = row == j ? seg_w[j] : wr;
      if (pr >= 0) c[(long)pr * n + colx] = A::round(topk_w != nullptr ? tot * wr : tot);
    } else if (splits == 1) {
      c[(long)row * n + colx] = A::round(tot);
    } else {
      partials[((long)split * m + row) * n + colx] = tot;
    }
  }
}

// Staging slots per thread for an activation slice of m rows and `span` groups: enough for
// the slice shared by all threads, and where the waves stage their own groups (sixteen
// waves, or eight with at most four rows) for each wave's own share of it: m rows of its
// ceil(span / waves) groups, 64 granules per slot.  (For one row the two counts agree.)
inline int stage_slots(int m, int span, int waves) {
  const long granules = (long)m * span * (kGroup / 8);
  const long per_slot = (long)waves * 64;
  const long shared = (granules + per_slot - 1) / per_slot;
  const long own = ((long)m * ((span + waves - 1) / waves) * (kGroup / 8) + 63) / 64;
  const bool per_wave = waves == 16 || (waves == 8 && m <= 4);
  return (int)(per_wave && own > shared ? own : shared);
}

inline int round_slots(int slots) {
  return slots <= 1 ? 1 : slots <= 2 ? 2 : slots <= 4 ? 4 : slots <= 8 ? 8 : 16;
}

template <bool ZP, int WAVES, int GW, int STAGE, bool PAIR, int GPC, bool BF16, bool W8,
          bool R1, bool DUAL, bool PWR = false>
hipError_t launch_small_t(const uint16_t* a, int lda, int m, const uint32_t* b,
                          const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                          int splits, float* partials, int chunk_rows, hipStream_t stream) {
  const int groups = k / kGroup;
  // The activation slice of this instance (its size is fixed by STAGE and WAVES), or the
  // waves' direct regions.
  constexpr size_t lds = STAGE == 0 ? (size_t)small_direct_lds(WAVES, GW, GPC, ZP, DUAL)
                                    : (size_t)STAGE * WAVES * 64 * sizeof(f16x8);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(
          &gemm_small_kernel<ZP, WAVES, GW, STAGE, PAIR, GPC, BF16, W8, R1, DUAL, false, PWR>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  // more rows than a work-group takes: chunks of chunk_rows rows along grid z (one split)
  if (chunk_rows < 1) return hipErrorInvalidValue;
  const int chunks = (m + chunk_rows - 1) / chunk_rows;
  if (chunks > 1 && splits != 1) return hipErrorInvalidValue;
  const dim3 grid(n / (PAIR || DUAL ? 32 : 16), splits, chunks);
  hipLaunchKernelGGL((gemm_small_kernel<ZP, WAVES, GW, STAGE, PAIR, GPC, BF16, W8, R1, DUAL, false,
                                       PWR>), grid,
                     dim3(WAVES * 64), lds, stream, reinterpret_cast<const f16*>(a), lda, m,
                     reinterpret_cast<const u32x4*>(b), s, reinterpret_cast<const u32x2*>(z), c,
                     n, groups, splits, partials, nullptr, nullptr, nullptr, nullptr, nullptr,
                     0L, 0L, 0L, 0, 0, 0, chunk_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_reduce_splits(partials, c, m, n, splits, BF16, stream);
}

// Grouped products with few rows per segment: grid (n / 16, n_active), one split; with the
// SwiGLU pair, (n / 32, n_active).
template <bool ZP, int WAVES, int GW, int STAGE, bool PAIR, int GPC, bool BF16, bool R1>
hipError_t launch_seg_t(const GroupedProblem& p, int rows, hipStream_t stream) {
  constexpr size_t lds = (size_t)STAGE * WAVES * 64 * sizeof(f16x8);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(
          &gemm_small_kernel<ZP, WAVES, GW, STAGE, PAIR, GPC, BF16, false, R1, false, true>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const dim3 grid(p.n / (PAIR ? 32 : 16), p.n_active);
  hipLaunchKernelGGL(
      (gemm_small_kernel<ZP, WAVES, GW, STAGE, PAIR, GPC, BF16, false, R1, false, true>), grid,
      dim3(WAVES * 64), lds, stream, reinterpret_cast<const f16*>(p.a), p.k, rows,
      reinterpret_cast<const u32x4*>(p.b_bank), reinterpret_cast<const uint16_t*>(p.s_bank),
      reinterpret_cast<const u32x2*>(p.z_bank), p.y, p.n, p.k / kGroup, 1, nullptr, p.ex_ids,
      p.ex_off, p.ex_pairs, p.pair_tok, p.topk_w, (long)(p.b_stride / 16),
      (long)(p.s_stride / 2), (long)(p.z_stride / 8), p.n_expert, p.n_pairs, p.n_tokens, 0);
  return hipGetLastError();
}

template <bool ZP, int WAVES, int GW, bool PAIR, int GPC, bool BF16>
hipError_t launch_seg_stage(const GroupedProblem& p, int rows, hipStream_t stream) {
  const int slots = round_slots(stage_slots(rows, p.k / kGroup, WAVES));
  if (rows == 1) {
    switch (slots) {
      case 1: return launch_seg_t<ZP, WAVES, GW, 1, PAIR, GPC, BF16, true>(p, rows, stream);
      case 2: return launch_seg_t<ZP, WAVES, GW, 2, PAIR, GPC, BF16, true>(p, rows, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (slots) {
    case 1: return launch_seg_t<ZP, WAVES, GW, 1, PAIR, GPC, BF16, false>(p, rows, stream);
    case 2: return launch_seg_t<ZP, WAVES, GW, 2, PAIR, GPC, BF16, false>(p, rows, stream);
    case 4: return launch_seg_t<ZP, WAVES, GW, 4, PAIR, GPC, BF16, false>(p, rows, stream);
    case 8: return launch_seg_t<ZP, WAVES, GW, 8, PAIR, GPC, BF16, false>(p, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

// Four waves of 1, 2, 4 or 8 groups (K up to 32 groups), or eight or sixteen waves of 8 (up
// to 64 or 128); with the SwiGLU pair twice the waves (at most sixteen), half on each block.
template <bool ZP, int GPC, bool BF16>
hipError_t launch_seg_zp(const GroupedProblem& p, int rows, const SmallPlan& plan,
                         hipStream_t stream) {
  if (plan.pair) {
    if (plan.waves == 16)
      return plan.depth == 8 ? launch_seg_stage<ZP, 16, 8, true, GPC, BF16>(p, rows, stream)
                             : hipErrorInvalidValue;
    switch (plan.depth) {
      case 1: return launch_seg_stage<ZP, 8, 1, true, GPC, BF16>(p, rows, stream);
      case 2: return launch_seg_stage<ZP, 8, 2, true, GPC, BF16>(p, rows, stream);
      case 4: return launch_seg_stage<ZP, 8, 4, true, GPC, BF16>(p, rows, stream);
      case 8: return launch_seg_stage<ZP, 8, 8, true, GPC, BF16>(p, rows, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (plan.waves == 16)
    return plan.depth == 8 ? launch_seg_stage<ZP, 16, 8, false, GPC, BF16>(p, rows, stream)
                           : hipErrorInvalidValue;
  if (plan.waves == 8)
    return plan.depth == 8 ? launch_seg_stage<ZP, 8, 8, false, GPC, BF16>(p, rows, stream)
                           : hipErrorInvalidValue;
  switch (plan.depth) {
    case 1: return launch_seg_stage<ZP, 4, 1, false, GPC, BF16>(p, rows, stream);
    case 2: return launch_seg_stage<ZP, 4, 2, false, GPC, BF16>(p, rows, stream);
    case 4: return launch_seg_stage<ZP, 4, 4, false, GPC, BF16>(p, rows, stream);
    case 8: return launch_seg_stage<ZP, 4, 8, false, GPC, BF16>(p, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int GPC, bool BF16>
hipError_t launch_seg_gpc(const GroupedProblem& p, int rows, const SmallPlan& plan,
                          hipStream_t stream) {
  if (p.z_bank != nullptr) return launch_seg_zp<true, GPC, BF16>(p, rows, plan, stream);
  return launch_seg_zp<false, GPC, BF16>(p, rows, plan, stream);
}

template <bool ZP, int WAVES, int GW, bool PAIR, int GPC, bool BF16, bool W8>
hipError_t launch_small_stage(const uint16_t* a, int lda, int m, const uint32_t* b,
                              const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                              const SmallPlan& plan, float* partials, hipStream_t stream) {
  const int span = (k / kGroup + plan.splits - 1) / plan.splits;
  const int mw = plan.rows > 0 && plan.rows < m ? plan.rows : m;  // rows per work-group
  if (plan.direct) {
    if constexpr (!PAIR && WAVES <= 8) {
      if constexpr (!W8) {
        if (plan.dual)
          return launch_small_t<ZP, WAVES, GW, 0, PAIR, GPC, BF16, W8, false, true>(
              a, lda, m, b, s, z, c, n, k, plan.splits, partials, mw, stream);
      }
      return launch_small_t<ZP, WAVES, GW, 0, PAIR, GPC, BF16, W8, false, false>(
          a, lda, m, b, s, z, c, n, k, plan.splits, partials, mw, stream);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (!W8) {
    // One row (at most 256 groups: at most four slots per thread).
    if (mw == 1) {
#define WQ_SMALL1(ST)                                                                        \
  launch_small_t<ZP, WAVES, GW, ST, PAIR, GPC, BF16, W8, true, false>(                        \
      a, lda, m, b, s, z, c, n, k, plan.splits, partials, mw, stream)
      switch (round_slots(stage_slots(mw, span, WAVES))) {
        case 1: return WQ_SMALL1(1);
        case 2: return WQ_SMALL1(2);
        case 4: return WQ_SMALL1(4);
        default: return hipErrorInvalidValue;
      }
#undef WQ_SMALL1
    }
  }
  if constexpr (WAVES == 8 && !PAIR && !W8) {
    // up to four rows per work-group: the per-wave staging instances (at most 8 slots)
    if (mw <= 4) {
#define WQ_SMALLW(ST)                                                                        \
  launch_small_t<ZP, WAVES, GW, ST, PAIR, GPC, BF16, W8, false, false, true>(                 \
      a, lda, m, b, s, z, c, n, k, plan.splits, partials, mw, stream)
      switch (round_slots(stage_slots(mw, span, WAVES))) {
        case 1: return WQ_SMALLW(1);
        case 2: return WQ_SMALLW(2);
        case 4: return WQ_SMALLW(4);
        case 8: return WQ_SMALLW(8);
        default: return hipErrorInvalidValue;
      }
#undef WQ_SMALLW
    }
  }
#define WQ_SMALL(ST)                                                                         \
  launch_small_t<ZP, WAVES, GW, ST, PAIR, GPC, BF16, W8, false, false>(                       \
      a, lda, m, b, s, z, c, n, k, plan.splits, partials, mw, stream)
  switch (round_slots(stage_slots(mw, span, WAVES))) {
    case 1: return WQ_SMALL(1);
    case 2: return WQ_SMALL(2);
    case 4: return WQ_SMALL(4);
    case 8: return WQ_SMALL(8);
    default: return WQ_SMALL(16);
  }
#undef WQ_SMALL
}

template <bool ZP, int WAVES, bool PAIR, int GPC, bool BF16, bool W8>
hipError_t launch_small_gw(const uint16_t* a, int lda, int m, const uint32_t* b,
                           const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                           const SmallPlan& plan, float* partials, hipStream_t stream) {
#define WQ_SMALL(GWV)                                                                          \
  launch_small_stage<ZP, WAVES, GWV, PAIR, GPC, BF16, W8>(a, lda, m, b, s, z, c, n, k, plan, \
                                                          partials, stream)
  switch (plan.depth) {
    case 1: return WQ_SMALL(1);
    case 2: return WQ_SMALL(2);
    case 4: return WQ_SMALL(4);
    case 8: return WQ_SMALL(8);
    default: return hipErrorInvalidValue;  // deeper plans only on sixteen waves
  }
#undef WQ_SMALL
}

template <bool ZP, int GPC, bool BF16>
hipError_t launch_small_waves(const uint16_t* a, int lda, int m, const uint32_t* b,
                              const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                              const SmallPlan& plan, float* partials, hipStream_t stream) {
  if (plan.pair) {
    if (plan.waves == 16)
      return launch_small_gw<ZP, 16, true, GPC, BF16, false>(a, lda, m, b, s, z, c, n, k, plan, partials,
                                                stream);
    return launch_small_gw<ZP, 8, true, GPC, BF16, false>(a, lda, m, b, s, z, c, n, k, plan, partials,
                                             stream);
  }
  if (plan.waves == 16) {  // staged, eight or sixteen groups per wave (K beyond 64 groups)
    if (plan.depth == 16)
      return launch_small_stage<ZP, 16, 16, false, GPC, BF16, false>(
          a, lda, m, b, s, z, c, n, k, plan, partials, stream);
    return plan.depth == 8 ? launch_small_stage<ZP, 16, 8, false, GPC, BF16, false>(
                                 a, lda, m, b, s, z, c, n, k, plan, partials, stream)
                           : hipErrorInvalidValue;
  }
  if (plan.waves == 8)
    return launch_small_gw<ZP, 8, false, GPC, BF16, false>(a, lda, m, b, s, z, c, n, k, plan, partials,
                                              stream);
  return launch_small_gw<ZP, 4, false, GPC, BF16, false>(a, lda, m, b, s, z, c, n, k, plan, partials,
                                            stream);
}

// E4M3 weights (128-row scale units, no zero points), either activation type, with or
// without the SwiGLU pair.
template <bool BF16>
hipError_t launch_small_w8(const uint16_t* a, int lda, int m, const uint32_t* b,
                           const uint16_t* s, uint16_t* c, int n, int k, const SmallPlan& plan,
                           float* partials, hipStream_t stream) {
  if (plan.gpc != 1) return hipErrorInvalidValue;
  if (plan.pair) {
    if (plan.waves == 16)
      return launch_small_gw<false, 16, true, 1, BF16, true>(a, lda, m, b, s, nullptr, c, n, k,
                                                             plan, partials, stream);
    return launch_small_gw<false, 8, true, 1, BF16, true>(a, lda, m, b, s, nullptr, c, n, k,
                                                          plan, partials, stream);
  }
  if (plan.waves == 8)
    return launch_small_gw<false, 8, false, 1, BF16, true>(a, lda, m, b, s, nullptr, c, n, k,
                                                           plan, partials, stream);
  return launch_small_gw<false, 4, false, 1, BF16, true>(a, lda, m, b, s, nullptr, c, n, k,
                                                         plan, partials, stream);
}

// Entry of one GPC and activation type: the plan has been checked by small_plan_fits.
template <int GPC, bool BF16>
hipError_t launch_small_gpc(const uint16_t* a, int lda, int m, const uint32_t* b,
                            const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                            const SmallPlan& plan, float* partials, hipStream_t stream) {
  if (z != nullptr)
    return launch_small_waves<true, GPC, BF16>(a, lda, m, b, s, z, c, n, k, plan, partials,
                                               stream);
  return launch_small_waves<false, GPC, BF16>(a, lda, m, b, s, z, c, n, k, plan, partials,
                                              stream);
}

}  // namespace
}  // namespace wq
