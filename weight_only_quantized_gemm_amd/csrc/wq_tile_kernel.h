// Tiled W4A16 GEMM for larger M (prefill) and the expert-major grouped (MoE) variant.
//
// Each wave computes 128 x 64 of C, a 4 x 2 grid of 32x32x16 fp16 MFMA blocks with fp32
// accumulators held in VGPRs.  A work-group is a 256 x 256 tile on eight waves (2 x 4), one
// per CU, or a 128 x 256 tile on four waves (1 x 4), two per CU (the TALL geometry below).
// Two waves share each SIMD, so one wave's MFMAs cover the other's LDS waits and barrier.
//
// Data movement is all direct-to-LDS loads (global_load_lds), issued at a fixed count per
// wave so that the in-order load counter tells exactly when a stage has landed:
//  * A (16-bit) in 256 x 64 chunks through a 3-stage ring (96 KiB), two chunks ahead (TALL:
//    128 x 64 chunks, a 2-stage ring, one chunk ahead);
//    each wave load writes 8 rows x 128 B, and the source granule of every lane is chosen
//    so that the ring holds the 16-byte granules of a row XOR-swizzled by ((row >> 1) & 7):
//    reads of one granule column by 32 consecutive rows are then free of bank conflicts.
//  * packed B (16 KiB per 128-row group for the tile's 16 column blocks) into one of two
//    group slots, issued with the odd chunk two groups ahead of its use;
//  * the group's scales / zero points into one of two small slots, two groups ahead.
// Every chunk waits for its own loads, meets the other waves at a barrier (after which
// the stage about to be refilled is no longer read by anyone), issues the next loads and
// computes.  Loads past the end re-read the last chunk / group into the free stage, so the
// counts never change; nothing is read outside the tensors.
//
// Inside a chunk each 16-row step reads the next step's A operands from LDS and
// dequantizes its weights while the current step's eight MFMAs run; the order is pinned
// with scheduling-group hints, as the default schedule waits on every LDS read right
// before its MFMA.
//
// Weights are dequantized in registers to exact integers (q - z) in the activation type:
// fp16 (magic-number halves) or bf16 (fp32 magic, then packed to bf16).  Group scales are
// applied in fp32 without a second accumulator set: after the last MFMAs of group g the
// running sums are multiplied by sigma_g / sigma_{g+1} (interleaved with those MFMAs), and
// the result is multiplied by sigma_last at the end, so C = sum_g sigma_g * P_g with P_g
// the exact-integer-weight partial of group g.  sigma is the 16-bit scale widened to fp32,
// with an exact zero replaced by 2^-60 so that the ratios stay finite: a zero-scale group
// then adds 2^-60-relative noise to the other groups' sum, which no output rounding keeps.
// A column whose every scale (in the work-group's range of K) is zero is written as
// exactly zero: a flag per column records whether any nonzero scale was read.
//
// Tiles are assigned XCD-aware: work-groups are dealt to the 8 XCDs round-robin, so tile
// ids are remapped to give each XCD a contiguous range (for a 2048-row problem, one
// 256-row A panel per XCD, which then stays in that XCD's L2).
//
// Dense split-K (fp32 reduce, few output tiles): the splits of a tile are consecutive work-
// groups, each over its own range of K groups; they store fp32 sums and a second kernel adds
// them in split order.
//
// Grouped variant (memra-engine mmq_ffi.rs, `ExpertCsr` and the grouped projection call):
// a tile's rows are CSR positions of one expert, A rows come from pair_tok[ex_pairs[j]]
// and outputs go to pair-major row ex_pairs[j].  Tiles are dispatched longest first:
// full row tiles before the short partial tiles that ragged expert sizes leave.
//
// This header holds the kernel template and its launch chain; wq_gemm_tile.hip (fp16) and
// wq_gemm_tile_bf16.hip (bf16) each instantiate one activation type.
#pragma once
#include <type_traits>

#include "wq_device.h"
#include "wq_internal.h"

namespace wq {

// Arguments of one tiled launch (dense or grouped); identical in every unit that includes
// this header.
struct TileArgs {
  const uint16_t* a;
  int lda;
  int m;
  const uint32_t* b;
  const uint16_t* s;
  const uint32_t* z;
  uint16_t* c;
  int n;
  int k;
  int ldc;    // output row stride: n, or n / 2 for the SwiGLU epilogue
  int tiles;  // work-groups launched (dense: output tiles x splits)
  int splits;        // dense: work-groups along K per output tile (1: c written directly)
  float* partials;   // dense, splits > 1: fp32 partial sums [splits][m][n]
  // grouped
  const uint8_t* b_bank;
  size_t b_stride;
  const uint8_t* s_bank;
  size_t s_stride;
  const uint8_t* z_bank;
  size_t z_stride;
  const int32_t* ex_ids;
  const int32_t* ex_off;
  const int32_t* ex_pairs;
  const int32_t* pair_tok;
  const float* topk_w;  // may be null
  int n_expert, n_active, n_pairs, n_tokens;
};

namespace {

constexpr int TN = kTileN;   // 256
constexpr int KC = 64;       // K rows per A chunk (half a group)
constexpr int kBlocks = TN / 16;  // 16-column blocks per tile
constexpr int kXcds = 8;

// Two tile geometries share the kernel.  Both give each wave 128 rows x 64 columns.
//  * 256 x 256 on eight waves (2 x 4), one work-group per CU: a 3-stage A ring (96 KiB).
//  * TALL: 128 x 256 on four waves (1 x 4), two work-groups per CU: a 2-stage A ring
//    (32 KiB), about 70 KiB of LDS per work-group.  The two waves sharing a SIMD then come
//    from different work-groups, and ragged row counts (expert segments, m % 256) leave
//    less padding.  It serves 128- and 64-row scale units of 4-bit weights.
//
// Direct-to-LDS loads each wave issues: 4 per A chunk, kDmaB (2 or 4) per B group, kDmaS
// per scale / zero-point group ("SZ").  Issue order (one group = 128 rows = chunks 2g, 2g+1):
//   256 x 256:  prologue SZ(0) B(0) SZ(1) A(0) A(1) B(1); chunk 2g: SZ(g+2) A(2g+2);
//               chunk 2g+1: A(2g+3) B(g+2).
//     Chunk 2g needs A(2g) (followed by A(2g+1), B(g+1)); chunk 2g+1 needs A(2g+1) and,
//     for the next group's weights read in its last step, B(g+1) (followed by SZ(g+2),
//     A(2g+2)).
//   TALL:       prologue SZ(0) B(0) A(0) SZ(1) B(1); chunk 2g: A(2g+1) SZ(g+2);
//               chunk 2g+1: A(2g+2) B(g+2).
//     With two ring stages a chunk can only be loaded once every wave has left the chunk
//     before it, one chunk ahead: chunk 2g needs A(2g) (followed by B(g+1)); chunk 2g+1
//     needs A(2g+1) (followed by SZ(g+2)), B(g+1) and SZ(g+1).  B(g+2) goes to the slot
//     of B(g), whose LDS reads (the last step of chunk 2g-1) lie two barriers back; a
//     barrier does not wait for a wave's LDS reads still in flight.
template <bool TALL>
struct Geo {
  static constexpr int TM = TALL ? 128 : 256;  // tile rows
  static constexpr int NS = TALL ? 2 : 3;      // A ring stages
  static constexpr int kWaves = TALL ? 4 : 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kTailRows = TM / 2;     // grouped tiles of at most this many rows are "small"
  static constexpr int kDmaA = TM * KC / 8 / kThreads;
  static constexpr int kDmaB = kBlocks / kWaves;
  static_assert(kDmaA == 4 && kDmaB * kWaves == kBlocks, "load split");
};

// Scale units smaller than 128 rows: scales and zero points are stored per unit of
// gcd(group_size, 128) rows, GPC = 1, 2, 4 or 8 sub-groups per 128-row group.  A group's SZ
// data is GPC x 128 dwords of scales (16 blocks x 16 fp16 per sub-group) then GPC x 32
// words of zero points, loaded 4 bytes per lane (kDmaS loads per wave).  With one sub-group its scales are read once, a group ahead, so two LDS slots
// suffice; with several, a group reads its own slot while the scales of two groups ahead
// arrive, hence three.
template <int GPC, bool TALL>
struct SzPlan {
  using G = Geo<TALL>;
  static constexpr int kDmaS = (160 * GPC + G::kThreads - 1) / G::kThreads;
  static constexpr int kSlots = GPC == 1 ? 2 : 3;
  static constexpr int kSlotWords = kDmaS * G::kThreads;
  static constexpr int kScaleWords = 128 * GPC;
  static constexpr int kWaitOdd = kDmaS + G::kDmaA;
  static constexpr int kWaitPrologue = kDmaS + 2 * G::kDmaA + G::kDmaB;  // SZ(0), B(0) landed
  static_assert(kWaitPrologue < 64, "vmcnt holds 6 bits");
  static_assert(160 * GPC <= kDmaS * G::kThreads, "SZ data fits the loads");
};

// Scheduling-group masks (instruction classes of the AMDGPU scheduler hints).
constexpr int kSchedVALU = 0x002;
constexpr int kSchedMFMA = 0x008;
constexpr int kSchedDSRead = 0x100;

// All of this wave's LDS reads have returned (vmcnt and expcnt not waited for).
__device__ __forceinline__ void wait_lds_reads() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}


template <bool BF16>
__device__ __forceinline__ float sigma_of(uint16_t bits) {
  const float f = Act<BF16>::value(bits);
  return f == 0.f ? 0x1p-60f : f;
}

// FP8: E4M3 weights are twice the bytes of a 4-bit group, so B is staged per 64-row chunk
// in a ring beside A's (3 x 16 KiB), and with one scale unit per 128 rows two SZ slots of
// one load per wave suffice: 96 + 48 + 4 KiB (256 x 256 only).
template <bool FP8, int GPC, bool TALL>
struct Smem {
  using G = Geo<TALL>;
  using SZ = SzPlan<GPC, TALL>;
  f16x8 a[G::NS][G::TM * KC / 8];             // 3 x 32 KiB, or TALL 2 x 16 KiB
  u32x4 b[FP8 ? G::NS : 2][kBlocks * 64];     // 16 column blocks x 64 lanes x 16 B per slot
  // scale / zero-point slots: TALL sized to its unit count; 256 x 256 room for three loads
  // per wave whatever the unit count
  uint32_t sz[TALL ? SZ::kSlots : FP8 ? 2 : 3][TALL ? SZ::kSlotWords : FP8 ? 512 : 1536];
  int row_a[G::TM];
  int row_c[G::TM];
  float row_w[G::TM];  // grouped: routing weight of each output row (1 without the multiply)
  int info[5];
  int wsum[2][16];  // grouped tile lookup: per-wave sums of the big and small tile counts
};

// The SwiGLU epilogue: B holds a gate and an up projection with their 16-column blocks
// paired (block 2t = gate columns 16t.., block 2t+1 = up columns 16t..), so in every 32x32
// output block lane c (c < 16) holds gate column j and lane c + 16 up column j of the same
// row.  The two lanes exchange their scaled sums (a lane swizzle, xor 16) and the gate lane
// writes fp16(silu(g) * u) to column j of the [rows][n/2] activation: the gate and up
// products never leave the registers.
template <bool ZP, bool GROUPED, bool SWIGLU, int GPC, bool BF16, bool FP8, bool TALL>
__device__ __forceinline__ void gemm_tile_body(TileArgs p) {
  using A = Act<BF16>;
  using Zo = typename A::Zo;
  using W8 = typename A::W8;
  using G = Geo<TALL>;  // geometry constants are used as G:: members throughout
  static_assert(!FP8 || (!ZP && GPC == 1), "E4M3: 128-row scale units, no zero points");
  static_assert(!TALL || (!FP8 && GPC <= 2), "TALL: 4-bit weights, 128- or 64-row units");
  __shared__ Smem<FP8, GPC, TALL> sm;
  using SZ = SzPlan<GPC, TALL>;
  constexpr int kDmaS = SZ::kDmaS;
  constexpr int kWaitOdd = SZ::kWaitOdd;
  constexpr int kWaitPrologue = SZ::kWaitPrologue;
  constexpr int kStepsPerSub = 8 / GPC;  // 16-row MFMA steps per scale sub-group
  // With four sub-groups the extra scale and zero-point registers leave no room for
  // reading the next step's A operands a step ahead; they are read at the step instead.
  constexpr bool kPrefetchA = GPC < 4;
  auto slot_of = [](int g) { return SZ::kSlots == 2 ? (g & 1) : g % 3; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int wm = TALL ? 0 : wave >> 2;    // wave's 128-row half of the tile
  const int wn = TALL ? wave : wave & 3;  // wave's 64-column quarter of the tile
  const int groups_all = p.k / kGroup;  // groups of K in the weights
  const int ntiles_n = p.n / TN;

  // XCD-aware tile id: work-group i runs on XCD i % 8; give each XCD a contiguous range.
  int t = blockIdx.x;
  if (!GROUPED && p.tiles % kXcds == 0) t = (t % kXcds) * (p.tiles / kXcds) + t / kXcds;
  // Dense split-K (128-row tiles with 128- or 64-row scale units: the planner only splits
  // products whose 256 x 256 tiles would be fewer than the CUs, and those take 128-row
  // tiles): the splits of one tile are consecutive, and split s covers groups
  // [groups_all * s / S, groups_all * (s + 1) / S) of K.
  constexpr bool kSplitK = !GROUPED && TALL && GPC <= 2;
  const int split = kSplitK ? t % p.splits : 0;
  if (kSplitK) t /= p.splits;
  const int gs0 = kSplitK ? (int)((long)groups_all * split / p.splits) : 0;
  const int groups =
      kSplitK ? (int)((long)groups_all * (split + 1) / p.splits) - gs0 : groups_all;

  int n0, valid_rows;
  const uint32_t* bptr;
  const uint16_t* sptr;
  const uint32_t* zptr;

  if constexpr (GROUPED) {
    // Tiles in longest-first order.  A segment's row tiles are its full TM-row tiles plus a
    // partial last one; a partial tile of at most G::kTailRows rows only busies the first
    // half of the waves and is "small", every other tile is "big".  Each XCD takes a
    // contiguous share of the big tiles (column tile fastest, so consecutive tiles reuse the
    // same activation rows) followed by a share of the small ones, and work-groups are
    // dispatched in order, so the small tiles fill the CUs that the last round of big tiles
    // leaves idle.  The lookup is parallel over segments (one per thread, in rounds of
    // kThreads): a block-wide sum of the tile counts, then a block-wide prefix sum that the
    // thread owning the work-group's tile index reads its tile from.
    const int wv = tid >> 6;
    // this thread's segment of round `base`: its big and small tile counts, and the segment
    auto seg_tiles = [&](int base, int* big, int* small, int* lo, int* rows) {
      const int i = base + tid;
      int a0 = 0, a1 = 0;
      if (i < p.n_active) {
        a0 = p.ex_off[i];
        a1 = p.ex_off[i + 1];
        a0 = a0 < 0 ? 0 : (a0 > p.n_pairs ? p.n_pairs : a0);
        a1 = a1 < a0 ? a0 : (a1 > p.n_pairs ? p.n_pairs : a1);
      }
      const int r = a1 - a0, full = r / G::TM, rem = r - full * G::TM;
      *big = (full + (rem > G::kTailRows ? 1 : 0)) * ntiles_n;
      *small = (rem > 0 && rem <= G::kTailRows) ? ntiles_n : 0;
      *lo = a0;
      *rows = r;
    };
    // block-wide inclusive prefix sums of (x, y) over the threads, and their totals
    auto block_scan = [&](int* x, int* y, int* tx, int* ty) {
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int ux = __shfl_up(*x, d), uy = __shfl_up(*y, d);
        if (lane >= d) {
          *x += ux;
          *y += uy;
        }
      }
      __syncthreads();  // the previous round's readers of wsum are done
      if (lane == 63) {
        sm.wsum[0][wv] = *x;
        sm.wsum[1][wv] = *y;
      }
      __syncthreads();
      int px = 0, py = 0, sx = 0, sy = 0;
#pragma unroll
      for (int w = 0; w < G::kWaves; ++w) {
        const int vx = sm.wsum[0][w], vy = sm.wsum[1][w];
        px += w < wv ? vx : 0;
        py += w < wv ? vy : 0;
        sx += vx;
        sy += vy;
      }
      *x += px;
      *y += py;
      *tx = sx;
      *ty = sy;
    };
    int nbig = 0, nsmall = 0;
    for (int base = 0; base < p.n_active; base += G::kThreads) {
      int b, sml, lo, rows, tb, ts;
      seg_tiles(base, &b, &sml, &lo, &rows);
      block_scan(&b, &sml, &tb, &ts);
      nbig += tb;
      nsmall += ts;
    }
    const int b8 = (nbig + kXcds - 1) / kXcds, s8 = (nsmall + kXcds - 1) / kXcds;
    const int x = (int)(blockIdx.x % kXcds), l = (int)(blockIdx.x / kXcds);
    int kind = -1, idx = 0;  // 0 big, 1 small
    if (l < b8) {
      idx = x * b8 + l;
      kind = idx < nbig ? 0 : -1;
    } else if (l < b8 + s8) {
      idx = x * s8 + (l - b8);
      kind = idx < nsmall ? 1 : -1;
    }
    if (tid == 0) sm.info[0] = -1;  // no tile unless a thread finds one below
    int done_b = 0, done_s = 0;     // tiles of the earlier rounds
    for (int base = 0; kind >= 0 && base < p.n_active; base += G::kThreads) {
      int b, sml, lo, rows, tb, ts;
      seg_tiles(base, &b, &sml, &lo, &rows);
      const int cnt = kind == 1 ? sml : b;
      int ib = b, is = sml;
      block_scan(&ib, &is, &tb, &ts);
      const int end = done_b * (kind == 0) + done_s * (kind == 1) + (kind == 1 ? is : ib);
      const int start = end - cnt;
      if (cnt > 0 && idx >= start && idx < end) {  // exactly one thread of the block
        const int seg = base + tid, j = idx - start;
        const int full = rows / G::TM;
        const int mt = kind == 1 ? full : j / ntiles_n;
        int e = seg;
        if (p.ex_ids != nullptr) e = p.ex_ids[seg];
        sm.info[0] = (e < 0 || e >= p.n_expert) ? -1 : seg;
        sm.info[1] = e;
        sm.info[2] = lo + mt * G::TM;    // first CSR position of the tile
        sm.info[3] = rows - mt * G::TM;  // CSR positions left in the segment from there
        sm.info[4] = kind == 1 ? j : j - (j / ntiles_n) * ntiles_n;
      }
      done_b += tb;
      done_s += ts;
    }
    __syncthreads();
    const int seg = sm.info[0];
    if (seg < 0) return;
    const int e = sm.info[1];
    const int pos0 = sm.info[2];
    const int left = sm.info[3];
    const int nt = sm.info[4];
    valid_rows = left < G::TM ? left : G::TM;
    n0 = nt * TN;
    // Row maps: CSR position -> (activation row, output row); rows without a valid pair
    // read activation row 0 (finite data, never stored) and are not written.
    int ra = 0, rc = -1;
    float rw = 1.f;
    if (tid < valid_rows) {
      const int pair = p.ex_pairs[pos0 + tid];
      if (pair >= 0 && pair < p.n_pairs) {
        const int tok = p.pair_tok[pair];
        if (tok >= 0 && tok < p.n_tokens) {
          ra = tok;
          rc = pair;
          if (p.topk_w != nullptr) rw = p.topk_w[pair];
        }
      }
    }
    if (tid < G::TM) {
      sm.row_a[tid] = ra;
      sm.row_c[tid] = rc;
      sm.row_w[tid] = rw;
    }
    bptr = reinterpret_cast<const uint32_t*>(p.b_bank + (size_t)e * p.b_stride);
    sptr = reinterpret_cast<const uint16_t*>(p.s_bank + (size_t)e * p.s_stride);
    zptr = ZP ? reinterpret_cast<const uint32_t*>(p.z_bank + (size_t)e * p.z_stride) : nullptr;
  } else {
    const int mt = t / ntiles_n;
    const int nt = t - mt * ntiles_n;
    n0 = nt * TN;
    const int m0 = mt * G::TM;
    valid_rows = p.m - m0 < G::TM ? p.m - m0 : G::TM;
    // Rows past m read the last row (finite, never stored).
    const int r = m0 + tid;
    if (tid < G::TM) {
      sm.row_a[tid] = r < p.m ? r : p.m - 1;
      sm.row_c[tid] = r < p.m ? r : -1;
    }
    bptr = p.b;
    sptr = p.s;
    zptr = p.z;
  }
  __syncthreads();

  // Row blocks of this wave that hold at least one valid row (wave-uniform).
  int nrb = (valid_rows - 128 * wm + 31) / 32;
  nrb = __builtin_amdgcn_readfirstlane(nrb < 0 ? 0 : (nrb > 4 ? 4 : nrb));

  // ---- load sources -------------------------------------------------------------------
  // A: slot u of this lane fills ring granule (u*8 + wave)*64 + lane = row 8*(u*8+wave) +
  // lane/8, physical granule lane%8, i.e. logical granule (lane%8) ^ ((row >> 1) & 7).
  const f16* asrc[G::kDmaA];
#pragma unroll
  for (int u = 0; u < G::kDmaA; ++u) {
    const int row = 8 * (u * G::kWaves + wave) + (lane >> 3);
    const int gi = (lane & 7) ^ ((row >> 1) & 7);
    asrc[u] = reinterpret_cast<const f16*>(p.a) + (long)sm.row_a[row] * p.lda +
              (long)gs0 * kGroup + 8 * gi;
  }
  // B: wave w fills column blocks kDmaB * w .. kDmaB * w + kDmaB - 1 of the tile (1 KiB each
  // per group), from the work-group's first group on.
  const int nb0 = n0 / 16;
  const u32x4* bsrc0 = reinterpret_cast<const u32x4*>(bptr) +
                       ((long)(nb0 + G::kDmaB * wave) * groups_all + gs0) * 64 + lane;
  // FP8 layout: 64-row chunk c of block nb is the 64 lanes' vectors at (nb * groups * 2 + c).
  const u32x4* b8src0 = reinterpret_cast<const u32x4*>(bptr) +
                        ((long)(nb0 + 2 * wave) * groups_all * 2 + 2 * gs0) * 64 + lane;
  const u32x4* b8src1 = b8src0 + (long)groups_all * 2 * 64;
  // SZ: load u of this lane fills slot dword d = u*512 + wave*64 + lane.  Dwords below
  // 128*GPC are scales (block d / (8 GPC), dword d % (8 GPC) of that block's GPC sub-groups),
  // the next 32*GPC zero-point words (block e / (2 GPC), word e % (2 GPC)); the rest re-read
  // the first scale dword.  Scales and zero points are stored [block][sub-group] with
  // groups*GPC sub-groups per block.
  const uint32_t* szsrc[kDmaS];
  long szstride[kDmaS];  // dwords per 128-row group
#pragma unroll
  for (int u = 0; u < kDmaS; ++u) {
    const int d = u * G::kThreads + wave * 64 + lane;
    const long sub_rows = (long)groups_all * GPC;
    if (d < SZ::kScaleWords) {
      szsrc[u] = reinterpret_cast<const uint32_t*>(sptr) +
                 ((long)(nb0 + d / (8 * GPC)) * sub_rows) * 8 + d % (8 * GPC);
      szstride[u] = 8 * GPC;
    } else if (ZP && d < SZ::kScaleWords + 32 * GPC) {
      const int e = d - SZ::kScaleWords;
      szsrc[u] = zptr + ((long)(nb0 + e / (2 * GPC)) * sub_rows) * 2 + e % (2 * GPC);
      szstride[u] = 2 * GPC;
    } else {
      szsrc[u] = reinterpret_cast<const uint32_t*>(sptr) + (long)nb0 * sub_rows * 8;
      szstride[u] = 8 * GPC;
    }
    szsrc[u] += gs0 * szstride[u];  // the work-group's first group
  }

  const int nchunks = 2 * groups;
  auto issue_a = [&](int c) {
    const int cc = c < nchunks ? c : nchunks - 1;
    f16x8* dst = &sm.a[c % G::NS][wave * 64];
#pragma unroll
    for (int u = 0; u < G::kDmaA; ++u)
      __builtin_amdgcn_global_load_lds(asrc[u] + (long)cc * KC, dst + u * G::kThreads, 16, 0, 0);
  };
  auto issue_b = [&](int g) {
    const int gg = g < groups ? g : groups - 1;
    u32x4* bdst = &sm.b[g & 1][G::kDmaB * wave * 64];
#pragma unroll
    for (int j = 0; j < G::kDmaB; ++j)
      __builtin_amdgcn_global_load_lds(bsrc0 + ((long)j * groups_all + gg) * 64, bdst + j * 64,
                                       16, 0, 0);
  };
  auto issue_b8 = [&](int c) {
    const int cc = c < nchunks ? c : nchunks - 1;
    u32x4* bdst = &sm.b[c % G::NS][2 * wave * 64];
    __builtin_amdgcn_global_load_lds(b8src0 + (long)cc * 64, bdst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(b8src1 + (long)cc * 64, bdst + 64, 16, 0, 0);
  };
  auto issue_sz = [&](int g) {
    const int gg = g < groups ? g : groups - 1;
#pragma unroll
    for (int u = 0; u < kDmaS; ++u)
      __builtin_amdgcn_global_load_lds(szsrc[u] + (long)gg * szstride[u],
                                       &sm.sz[slot_of(g)][u * G::kThreads + wave * 64], 4, 0, 0);
  };

  // ---- per-lane compute geometry ---------------------------------------------------------
  const int c32 = lane & 31;
  const int hh = lane >> 5;
  int bblk[2];  // tile column block holding the lane's column in each 32-column block
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) bblk[cb] = 4 * wn + 2 * cb + (c32 >> 4);
  const int c16 = c32 & 15;
  int aswz[4];  // granule of step s inside the lane's A row: (2s + h) ^ swizzle
#pragma unroll
  for (int st = 0; st < 4; ++st) aswz[st] = (2 * st + hh) ^ ((c32 >> 1) & 7);

  f32x16 acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;
  float sigma[2];
  bool scaled[2] = {false, false};  // a nonzero scale of the lane's column has been read
  u32x4 bw[2][2];  // [cb][r]: vector r of the lane's column, rows 16*r + 8*h + ... per step
  Zo zo[2];
  const auto mr = A::magic();

  // Scale and zero-point offsets of sub-group q of group g for the lane's two columns.
  auto read_sz = [&](int g, int q, float* sg, Zo* zg) {
    const uint32_t* slot = sm.sz[slot_of(g)];
    const uint16_t* sl = reinterpret_cast<const uint16_t*>(slot);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const uint16_t bits = sl[bblk[cb] * 16 * GPC + 16 * q + c16];
      sg[cb] = sigma_of<BF16>(bits);
      scaled[cb] = scaled[cb] || (bits & 0x7FFF) != 0;
      int zc = 8;
      if constexpr (ZP) {
        const uint32_t* zl = slot + SZ::kScaleWords + bblk[cb] * 2 * GPC + 2 * q;
        zc = zero_code(u32x2{zl[0], zl[1]}, c16);
      }
      zg[cb] = A::zero(zc);
    }
  };
  // The lane's weight vectors of group g (slot g & 1), or for FP8 of chunk g (slot g % G::NS).
  auto read_b = [&](int g) {
    const u32x4* bslot = sm.b[FP8 ? g % G::NS : g & 1];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int base = bblk[cb] * 64 + c16 + 16 * hh;
      bw[cb][0] = bslot[base];
      bw[cb][1] = bslot[base + 32];
    }
  };

  // Prologue (see the issue order above), then group 0's scales and weights.  FP8 issues
  //   prologue: SZ(0) SZ(1) A(0) B8(0) A(1) B8(1); chunk 2g: SZ(g+2) A(c+2) B8(c+2);
  //   chunk 2g+1: A(c+2) B8(c+2)
  // so that chunk c waits for A(c) and B8(c): 6 loads (A, B8 of chunk c+1) may stay in
  // flight at an even chunk, 7 (also SZ(g+2)) at an odd one.
  constexpr int kWait8Even = G::kDmaA + 2;
  constexpr int kWait8Odd = kDmaS + G::kDmaA + 2;
  if constexpr (FP8) {
    issue_sz(0);
    issue_sz(1);
    issue_a(0);
    issue_b8(0);
    issue_a(1);
    issue_b8(1);
    wait_vmcnt<kWait8Even>();
    __builtin_amdgcn_s_barrier();
    read_sz(0, 0, sigma, zo);
  } else if constexpr (TALL) {
    issue_sz(0);
    issue_b(0);
    issue_a(0);
    issue_sz(1);
    issue_b(1);
    wait_vmcnt<SZ::kDmaS + G::kDmaB>();  // SZ(0), B(0) and A(0) landed
    __builtin_amdgcn_s_barrier();
    read_sz(0, 0, sigma, zo);
    read_b(0);
  } else {
    issue_sz(0);
    issue_b(0);
    issue_sz(1);
    issue_a(0);
    issue_a(1);
    issue_b(1);
    wait_vmcnt<kWaitPrologue>();
    __builtin_amdgcn_s_barrier();
    read_sz(0, 0, sigma, zo);
    read_b(0);
  }
  // Group 0's scales are first used after chunk 0's barrier, behind which SZ(2) refills
  // their slot (one group ahead of two slots): their reads must have returned before it.
  wait_lds_reads();

  // One iteration per group: its even chunk and its odd chunk, so that the chunk parity,
  // and with it the weight dwords each step reads, is static.  NRB is the number of the
  // wave's 32-row blocks that hold valid rows (rounded up to 1, 2 or 4; 0 for none): the
  // loads and barriers are the same for every NRB, only the arithmetic shrinks.
  auto chunk = [&](auto h2c, auto nrbc, int c) {
    constexpr int h2 = decltype(h2c)::value;
    constexpr int NRB = decltype(nrbc)::value;
    const int g = c >> 1;
    if constexpr (FP8)
      wait_vmcnt<h2 == 0 ? kWait8Even : kWait8Odd>();
    else if constexpr (TALL)
      wait_vmcnt<h2 == 0 ? G::kDmaB : SZ::kDmaS>();
    else
      wait_vmcnt<h2 == 0 ? (G::kDmaA + G::kDmaB) : kWaitOdd>();
    __builtin_amdgcn_s_barrier();
    if constexpr (TALL) {
      // the stage chunk c + 1 refills was last read in chunk c - 1
      issue_a(c + 1);
      if (h2 == 0)
        issue_sz(g + 2);
      else
        issue_b(g + 2);
    } else if (h2 == 0) {
      issue_sz(g + 2);
      issue_a(c + 2);
      if constexpr (FP8) issue_b8(c + 2);
    } else {
      issue_a(c + 2);
      if constexpr (FP8)
        issue_b8(c + 2);
      else
        issue_b(g + 2);
    }
    if constexpr (FP8) read_b(c);  // this chunk's weights: step s in vector s % 2

    // Odd chunk: the next group's first scales, for the factor sigma / sigma_next applied
    // to the running sums after this group's last MFMAs (1 after the last group).  The
    // hardware reciprocal is about 1 ulp: a relative error near 1e-7 per boundary.
    float snext[2] = {1.f, 1.f}, gfactor[2] = {1.f, 1.f};
    Zo znext[2] = {zo[0], zo[1]};
    // With at most two sub-groups the running scale at the odd chunk's start is already the
    // group's last, so the factor is formed here, off the rescaling step's path.
    auto group_factor = [&](float* f) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        f[cb] = g + 1 < groups ? sigma[cb] * __builtin_amdgcn_rcpf(snext[cb]) : 1.f;
    };
    if (h2 == 1) {
      read_sz(g + 1, 0, snext, znext);
      if (GPC <= 2) group_factor(gfactor);
    }

    if constexpr (NRB > 0) {
      // Row 128*wm + 32*rb + c32 of the stage; its swizzle (row >> 1) & 7 = (c32 >> 1) & 7
      // does not depend on rb, so a step's reads share one address plus offsets.
      const f16x8* arow = sm.a[c % G::NS] + (128 * wm + c32) * 8;
      f16x8 aop[NRB];
      W8 bop[2];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) aop[rb] = arow[rb * 256 + aswz[0]];
      // Weights of 16-row step (4*h2 + s) of the group: dword (2*h2 + s/2) of vector s%2.
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if constexpr (FP8)
          bop[cb] = A::fp8(bw[cb][0][0], bw[cb][0][1]);
        else
          bop[cb] = A::dequant(bw[cb][0][2 * h2], zo[cb], mr);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // Step t of the group ends a sub-group when (t + 1) is a multiple of its steps;
        // an inner boundary switches to the group's next sub-group scale and zero point.
        const int t = 4 * h2 + s;
        const bool end_sub = ((t + 1) % kStepsPerSub) == 0;
        const bool end_group = t == 7;
        const bool inner = end_sub && !end_group;
        float sn[2] = {1.f, 1.f}, factor[2] = {1.f, 1.f};
        Zo zn[2] = {zo[0], zo[1]};
        if (inner) {
          read_sz(g, (t + 1) / kStepsPerSub, sn, zn);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) factor[cb] = sigma[cb] * __builtin_amdgcn_rcpf(sn[cb]);
        } else if (end_group) {
          if (GPC <= 2) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) factor[cb] = gfactor[cb];
          } else {
            group_factor(factor);
          }
        }
        f16x8 anext[NRB];
        W8 bnext[2];
        if (!kPrefetchA && s > 0) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) aop[rb] = arow[rb * 256 + aswz[s]];
        }
        if (s < 3) {
          if (kPrefetchA) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) anext[rb] = arow[rb * 256 + aswz[s + 1]];
          }
          if constexpr (FP8) {
            // FP8 step s: vector s % 2, words 2(s / 2) and 2(s / 2) + 1
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
              bnext[cb] = A::fp8(bw[cb][(s + 1) & 1][2 * ((s + 1) >> 1)],
                                 bw[cb][(s + 1) & 1][2 * ((s + 1) >> 1) + 1]);
          } else {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
              bnext[cb] = A::dequant(bw[cb][(s + 1) & 1][2 * h2 + ((s + 1) >> 1)],
                                     inner ? zn[cb] : zo[cb], mr);
          }
        } else if (!FP8 && h2 == 1) {
          read_b(g + 1);  // the current weights are dead after step 2's dequant
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = A::mfma32(aop[rb], bop[cb], acc[rb][cb]);
        if (end_sub) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[rb][cb][r] *= factor[cb];
        }
        // Schedule: LDS reads of the next step first, dequant between the MFMAs; in the
        // group's last step the products of the blocks follow the MFMAs.  (Steps at inner
        // sub-group boundaries are left to the compiler.)
        constexpr int nm = 2 * NRB;  // MFMAs per step
        if (s < 3 && !inner && kPrefetchA) {
          constexpr int per = (20 + nm - 1) / nm;
#pragma unroll
          for (int i = 0; i < nm; ++i) {
            if (i < NRB) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVALU, per, 0);
          }
        } else if (end_group) {
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
#pragma unroll
          for (int i = 2; i < nm; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedVALU, 16, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedVALU, 32, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (inner) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            sigma[cb] = sn[cb];
            zo[cb] = zn[cb];
          }
        }
        if (s < 3) {
          if (kPrefetchA) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) aop[rb] = anext[rb];
          }
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) bop[cb] = bnext[cb];
        }
      }
    }
    // After the last group the running sums stay in units of its last sub-group's scale,
    // which the epilogue applies.
    if (h2 == 1 && g + 1 < groups) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        sigma[cb] = snext[cb];
        zo[cb] = znext[cb];
      }
    }
  };
  auto run = [&](auto nrbc) {
    for (int g = 0; g < groups; ++g) {
      chunk(std::integral_constant<int, 0>{}, nrbc, 2 * g);
      chunk(std::integral_constant<int, 1>{}, nrbc, 2 * g + 1);
    }
  };
  if (nrb >= 3)
    run(std::integral_constant<int, 4>{});
  else if (nrb == 2)
    run(std::integral_constant<int, 2>{});
  else if (nrb == 1)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 0>{});
  wait_vmcnt<0>();  // the trailing re-reads have landed before the work-group ends

  // Epilogue: lane holds rows 8*(r/4) + 4*h + (r%4) of column c32 in each 32x32 block.
  if constexpr (SWIGLU) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (rb >= nrb) continue;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const long j = (n0 + 64 * wn + 32 * cb) / 2 + (c32 & 15);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 128 * wm + 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
          const float mine = scaled[cb] ? acc[rb][cb][r] * sigma[cb] : 0.f;
          // ds_swizzle bit mode: and 0x1f, or 0, xor 0x10 (lanes l and l ^ 16 swap)
          const float other = __builtin_bit_cast(
              float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, mine), 0x401F));
          const int orow = sm.row_c[row];
          if (c32 < 16 && orow >= 0)
            p.c[(long)orow * p.ldc + j] = A::round(silu_times(mine, other));
        }
      }
    }
    return;
  }
  if (kSplitK && p.splits > 1) {
    // Split K: this split's fp32 sums; a second kernel adds the splits in order and rounds.
    // (A loop of its own, so that the rounding below stays one rounding of the exact
    // product rather than of its fp32 value.)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (rb >= nrb) continue;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const long col = n0 + 64 * wn + 32 * cb + c32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 128 * wm + 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
          const int orow = sm.row_c[row];
          if (orow >= 0)
            p.partials[((long)split * p.m + orow) * p.n + col] =
                scaled[cb] ? acc[rb][cb][r] * sigma[cb] : 0.f;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb >= nrb) continue;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const long col = n0 + 64 * wn + 32 * cb + c32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 128 * wm + 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int orow = sm.row_c[row];
        // The routing weight (1 without the multiply) joins the scale, so that the output
        // is one rounding of acc * factor, as on the dense path.
        const float sig = scaled[cb] ? sigma[cb] : 0.f;
        const float factor = GROUPED ? sig * sm.row_w[row] : sig;
        if (orow >= 0)
          p.c[(long)orow * p.ldc + col] = A::round(acc[rb][cb][r] * factor);
      }
    }
  }
}

// The kernels of each instance, one per geometry.  (The body is a device function: with
// the geometry as a template parameter, this toolchain's host pass dropped the launch stubs
// of a kernel that held the body itself.)  Both run two waves per SIMD, at most 256 VGPRs
// per wave: eight-wave work-groups one per CU, four-wave work-groups two per CU.
template <bool ZP, bool GROUPED, bool SWIGLU, int GPC, bool BF16, bool FP8>
__global__ __launch_bounds__(512) void gemm_tile_kernel(TileArgs p) {
  gemm_tile_body<ZP, GROUPED, SWIGLU, GPC, BF16, FP8, false>(p);
}

template <bool ZP, bool GROUPED, bool SWIGLU, int GPC, bool BF16>
__global__ __launch_bounds__(256, 2) void gemm_tile_kernel_tall(TileArgs p) {
  gemm_tile_body<ZP, GROUPED, SWIGLU, GPC, BF16, false, true>(p);
}

template <bool GROUPED, bool SWIGLU, int GPC, bool BF16, bool TALL>
hipError_t launch_tile_g(const TileArgs& p, bool zp, hipStream_t stream) {
  const dim3 grid((unsigned)p.tiles), block(Geo<TALL>::kThreads);
  if constexpr (TALL) {
    if (zp)
      hipLaunchKernelGGL((gemm_tile_kernel_tall<true, GROUPED, SWIGLU, GPC, BF16>), grid, block,
                         0, stream, p);
    else
      hipLaunchKernelGGL((gemm_tile_kernel_tall<false, GROUPED, SWIGLU, GPC, BF16>), grid, block,
                         0, stream, p);
  } else {
    if (zp)
      hipLaunchKernelGGL((gemm_tile_kernel<true, GROUPED, SWIGLU, GPC, BF16, false>), grid, block,
                         0, stream, p);
    else
      hipLaunchKernelGGL((gemm_tile_kernel<false, GROUPED, SWIGLU, GPC, BF16, false>), grid,
                         block, 0, stream, p);
  }
  return hipGetLastError();
}

// gpc: scale units per 128 rows of K (1, 2, 4 or 8); tall: the 128 x 256 geometry (gpc 1
// or 2).
template <bool GROUPED, bool SWIGLU, bool BF16>
hipError_t launch_tile_t(const TileArgs& p, bool zp, int gpc, bool tall, hipStream_t stream) {
  switch (gpc) {
    case 1:
      return tall ? launch_tile_g<GROUPED, SWIGLU, 1, BF16, true>(p, zp, stream)
                  : launch_tile_g<GROUPED, SWIGLU, 1, BF16, false>(p, zp, stream);
    case 2:
      return tall ? launch_tile_g<GROUPED, SWIGLU, 2, BF16, true>(p, zp, stream)
                  : launch_tile_g<GROUPED, SWIGLU, 2, BF16, false>(p, zp, stream);
    case 4:
      return tall ? hipErrorInvalidValue : launch_tile_g<GROUPED, SWIGLU, 4, BF16, false>(p, zp, stream);
    case 8:
      return tall ? hipErrorInvalidValue : launch_tile_g<GROUPED, SWIGLU, 8, BF16, false>(p, zp, stream);
    default: return hipErrorInvalidValue;
  }
}

// Every instance of one activation type.
template <bool BF16>
hipError_t launch_tile_type(const TileArgs& p, bool grouped, bool swiglu, bool zp, int gpc,
                            bool tall, hipStream_t stream) {
  if (grouped)
    return swiglu ? launch_tile_t<true, true, BF16>(p, zp, gpc, tall, stream)
                  : launch_tile_t<true, false, BF16>(p, zp, gpc, tall, stream);
  return swiglu ? launch_tile_t<false, true, BF16>(p, zp, gpc, tall, stream)
                : launch_tile_t<false, false, BF16>(p, zp, gpc, tall, stream);
}

// E4M3 weights: 128-row scale units, no zero points, the 256 x 256 geometry; every layout
// of one activation type.
template <bool BF16>
hipError_t launch_tile_fp8_type(const TileArgs& p, bool grouped, bool swiglu,
                                hipStream_t stream) {
#define WQ_TILE_FP8(G, S)                                                                  \
  hipLaunchKernelGGL((gemm_tile_kernel<false, G, S, 1, BF16, true>),                      \
                     dim3((unsigned)p.tiles), dim3(Geo<false>::kThreads), 0, stream, p)
  if (grouped) {
    if (swiglu)
      WQ_TILE_FP8(true, true);
    else
      WQ_TILE_FP8(true, false);
  } else {
    if (swiglu)
      WQ_TILE_FP8(false, true);
    else
      WQ_TILE_FP8(false, false);
  }
#undef WQ_TILE_FP8
  return hipGetLastError();
}

// Geometry of a tiled product: 128-row tiles for grouped products (expert segments leave
// partial tiles), for dense ones that 128-row tiles cover with fewer padding rows, and for
// dense ones whose 256 x 256 tiles would be fewer than the CUs (n columns); 4-bit weights
// with 128- or 64-row scale units only.  256 x 256 otherwise.
inline bool tile_tall(bool grouped, int m, int gpc, bool fp8, int n) {
  if (fp8 || gpc > 2) return false;
  return grouped || (m + 127) / 128 * 128 < (m + 255) / 256 * 256 ||
         (long)(n / TN) * ((m + 255) / 256) < 256;
}

inline int tile_rows(bool tall) { return tall ? Geo<true>::TM : Geo<false>::TM; }

}  // namespace

// The instances of each type (wq_gemm_tile.hip: fp16; wq_gemm_tile_bf16.hip: bf16;
// wq_gemm_tile_fp8.hip: E4M3 weights).
hipError_t launch_tile_f16(const TileArgs& p, bool grouped, bool swiglu, bool zp, int gpc,
                           bool tall, hipStream_t stream);
hipError_t launch_tile_bf16(const TileArgs& p, bool grouped, bool swiglu, bool zp, int gpc,
                            bool tall, hipStream_t stream);
hipError_t launch_tile_fp8(const TileArgs& p, bool grouped, bool swiglu, bool bf16,
                           hipStream_t stream);

}  // namespace wq

