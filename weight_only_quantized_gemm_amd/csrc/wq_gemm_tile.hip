// Tiled W4A16 GEMM for larger M (prefill) and the expert-major grouped (MoE) variant.
//
// A work-group computes a 256 x 128 tile of C with four waves of 128 x 64, each a 4 x 2
// grid of 32x32x16 fp16 MFMA blocks with fp32 accumulators.  A (fp16) goes through LDS
// in 256 x 64 chunks, double-buffered and XOR-swizzled by 16-byte granule so that both
// the row-per-lane reads and the coalesced writes are free of bank conflicts.  Packed
// weights go straight from HBM into registers (two 16-byte loads per lane and 32-column
// block per 128-row group), one group ahead of use, and are dequantized in registers to
// exact fp16 integers (q - z).
//
// Group scales are applied in fp32 without a second accumulator set: before the MFMAs of
// group g accumulate, the running sums are multiplied by sigma_{g-1} / sigma_g, and the
// result is multiplied by sigma_last at the end, so C = sum_g sigma_g * P_g with P_g the
// exact-integer-weight partial of group g.  sigma is the fp16 scale widened to fp32, with
// an exact zero replaced by 2^-60 (its contribution then vanishes after rounding to fp16).
//
// Grouped variant (memra-engine mmq_ffi.rs, `ExpertCsr` and the grouped projection call):
// tiles are enumerated over (active expert segment, column tile, row tile); a tile's rows
// are CSR positions of one expert, A rows come from pair_tok[ex_pairs[j]] and outputs go
// to pair-major row ex_pairs[j].
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int TM = kTileM;   // 256
constexpr int TN = kTileN;   // 128
constexpr int KC = 64;       // K rows per LDS chunk (half a group)

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
  int n_expert, n_active, n_pairs, n_tokens;
};

__device__ __forceinline__ float sigma_of(f16 v) {
  const float f = (float)v;
  return f == 0.f ? 0x1p-60f : f;
}

template <bool ZP, bool GROUPED>
__global__ __launch_bounds__(256) void gemm_tile_kernel(TileArgs p) {
  __shared__ f16x8 lds_a[2][TM * (KC / 8)];
  __shared__ int row_a[TM];
  __shared__ int row_c[TM];
  __shared__ int tile_info[5];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;   // wave's 128-row half of the tile
  const int wn = wave & 1;    // wave's 64-column half of the tile
  const int groups = p.k / kGroup;
  const int ntiles_n = p.n / TN;

  int n0, valid_rows;
  const uint32_t* bptr;
  const uint16_t* sptr;
  const uint32_t* zptr;

  if constexpr (GROUPED) {
    if (tid == 0) {
      int t = blockIdx.x;
      int seg = -1, lo = 0, rows = 0, mt = 0, nt = 0;
      for (int i = 0; i < p.n_active; ++i) {
        int a0 = p.ex_off[i], a1 = p.ex_off[i + 1];
        a0 = a0 < 0 ? 0 : (a0 > p.n_pairs ? p.n_pairs : a0);
        a1 = a1 < a0 ? a0 : (a1 > p.n_pairs ? p.n_pairs : a1);
        const int r = a1 - a0;
        const int mtiles = (r + TM - 1) / TM;
        const int tiles = mtiles * ntiles_n;
        if (t < tiles) {
          seg = i;
          lo = a0;
          rows = r;
          mt = t % mtiles;
          nt = t / mtiles;
          break;
        }
        t -= tiles;
      }
      int e = seg;
      if (seg >= 0 && p.ex_ids != nullptr) e = p.ex_ids[seg];
      if (e < 0 || e >= p.n_expert) seg = -1;
      tile_info[0] = seg;
      tile_info[1] = e;
      tile_info[2] = lo + mt * TM;   // first CSR position of the tile
      tile_info[3] = rows - mt * TM; // CSR positions left in the segment from there
      tile_info[4] = nt;
    }
    __syncthreads();
    const int seg = tile_info[0];
    if (seg < 0) return;
    const int e = tile_info[1];
    const int pos0 = tile_info[2];
    const int left = tile_info[3];
    const int nt = tile_info[4];
    valid_rows = left < TM ? left : TM;
    n0 = nt * TN;
    // Row maps: CSR position -> (activation row, output row); invalid entries -> -1.
    {
      int ra = -1, rc = -1;
      if (tid < valid_rows) {
        const int pair = p.ex_pairs[pos0 + tid];
        if (pair >= 0 && pair < p.n_pairs) {
          const int tok = p.pair_tok[pair];
          if (tok >= 0 && tok < p.n_tokens) {
            ra = tok;
            rc = pair;
          }
        }
      }
      row_a[tid] = ra;
      row_c[tid] = rc;
    }
    bptr = reinterpret_cast<const uint32_t*>(p.b_bank + (size_t)e * p.b_stride);
    sptr = reinterpret_cast<const uint16_t*>(p.s_bank + (size_t)e * p.s_stride);
    zptr = ZP ? reinterpret_cast<const uint32_t*>(p.z_bank + (size_t)e * p.z_stride) : nullptr;
    __syncthreads();
  } else {
    const int mt = blockIdx.y;
    n0 = blockIdx.x * TN;
    const int m0 = mt * TM;
    valid_rows = p.m - m0 < TM ? p.m - m0 : TM;
    {
      const int r = m0 + tid;
      row_a[tid] = tid < valid_rows ? r : -1;
      row_c[tid] = tid < valid_rows ? r : -1;
    }
    bptr = p.b;
    sptr = p.s;
    zptr = p.z;
    __syncthreads();
  }

  // Row blocks of this wave that hold at least one valid row (wave-uniform).
  int nrb = (valid_rows - 128 * wm + 31) / 32;
  nrb = nrb < 0 ? 0 : (nrb > 4 ? 4 : nrb);

  // ---- A staging: thread owns granule gi of rows (tid >> 3) + 32 * i --------------------
  const int gi = tid & 7;
  const f16* arows[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = row_a[(tid >> 3) + 32 * i];
    arows[i] = r >= 0 ? reinterpret_cast<const f16*>(p.a) + (long)r * p.lda + 8 * gi : nullptr;
  }
  auto load_a = [&](int chunk, f16x8 (&st)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      st[i] = arows[i] ? *reinterpret_cast<const f16x8*>(arows[i] + (long)chunk * KC)
                       : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
  };
  auto store_a = [&](int stage, const f16x8 (&st)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i;
      lds_a[stage][row * 8 + (gi ^ (row & 7))] = st[i];
    }
  };

  // ---- B: lane (c = lane & 31, h = lane >> 5) of 32-column block cb ----------------------
  const int c32 = lane & 31;
  const int hh = lane >> 5;
  long bbase[2];   // index (in 16-byte units) of the lane's first vector, group 0
  long sbase[2];   // scale index of the lane's column, group 0
  long zbase[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = n0 + 64 * wn + 32 * cb + c32;
    const long nb = col >> 4;
    bbase[cb] = nb * groups * 64 + (col & 15) + 16 * hh;
    sbase[cb] = nb * groups * 16 + (col & 15);
    zbase[cb] = nb * groups;
  }
  const u32x4* bvec = reinterpret_cast<const u32x4*>(bptr);
  const f16* svec = reinterpret_cast<const f16*>(sptr);
  const u32x2* zvec = reinterpret_cast<const u32x2*>(zptr);

  u32x4 bcur[2][2], bnext[2][2];   // [cb][r]: r = 0 rows 8h.., r = 1 rows 16 + 8h..
  f16 scur[2], snext[2];
  u32x2 zcur[2], znext[2];
  auto load_b = [&](int g, u32x4 (&bw)[2][2], f16 (&sv)[2], u32x2 (&zv)[2]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const long base = bbase[cb] + (long)g * 64;
      bw[cb][0] = bvec[base];
      bw[cb][1] = bvec[base + 32];
      sv[cb] = svec[sbase[cb] + (long)g * 16];
      if (ZP) zv[cb] = zvec[zbase[cb] + g];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;
  float sigma[2] = {1.f, 1.f};

  // Prologue: chunk 0 into LDS stage 0, weights of group 0 into registers.
  {
    f16x8 st[8];
    load_a(0, st);
    store_a(0, st);
  }
  load_b(0, bcur, scur, zcur);
  __syncthreads();

  const MagicRegs mr = magic_regs();
  const int nchunks = p.k / KC;
  for (int ch = 0; ch < nchunks; ++ch) {
    const int g = ch >> 1;
    const int h2 = ch & 1;
    ZeroOffsets zo[2];
    if (h2 == 0) {
      // New group: rescale running sums to this group's scale, fetch next group's weights.
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const float sn = sigma_of(scur[cb]);
        if (g > 0) {
          const float ratio = sigma[cb] / sn;
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rb][cb][r] *= ratio;
        }
        sigma[cb] = sn;
      }
      if (g + 1 < groups) load_b(g + 1, bnext, snext, znext);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) zo[cb] = zero_offsets(ZP ? zero_code(zcur[cb], c32 & 15) : 8);

    f16x8 st[8];
    const bool more = ch + 1 < nchunks;
    if (more) load_a(ch + 1, st);

    const f16x8* lds = lds_a[ch & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // Weights of 16-row step (4*h2 + s) of the group: dword (2*h2 + s/2) of vector s%2.
      f16x8 bop[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        bop[cb] = dequant8(bcur[cb][s & 1][2 * h2 + (s >> 1)], zo[cb], mr);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (rb < nrb) {
          const int row = 128 * wm + 32 * rb + c32;
          const f16x8 aop = lds[row * 8 + ((2 * s + hh) ^ (row & 7))];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma32x32x16(aop, bop[cb], acc[rb][cb]);
        }
      }
    }

    if (more) store_a((ch + 1) & 1, st);
    __syncthreads();
    if (h2 == 1 && g + 1 < groups) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        bcur[cb][0] = bnext[cb][0];
        bcur[cb][1] = bnext[cb][1];
        scur[cb] = snext[cb];
        zcur[cb] = znext[cb];
      }
    }
  }

  // Epilogue: lane holds rows 8*(r/4) + 4*h + (r%4) of column c32 in each 32x32 block.
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb >= nrb) continue;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const long col = n0 + 64 * wn + 32 * cb + c32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 128 * wm + 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int orow = row_c[row];
        if (orow >= 0)
          p.c[(long)orow * p.n + col] =
              __builtin_bit_cast(uint16_t, (f16)(acc[rb][cb][r] * sigma[cb]));
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_tile(const uint16_t* a, int lda, int m, const uint32_t* b,
                            const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                            hipStream_t stream) {
  TileArgs p{};
  p.a = a;
  p.lda = lda;
  p.m = m;
  p.b = b;
  p.s = s;
  p.z = z;
  p.c = c;
  p.n = n;
  p.k = k;
  const dim3 grid(n / TN, (m + TM - 1) / TM);
  if (z != nullptr)
    hipLaunchKernelGGL((gemm_tile_kernel<true, false>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<false, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_grouped_tile(const GroupedProblem& g, hipStream_t stream) {
  TileArgs p{};
  p.a = g.a;
  p.lda = g.k;
  p.m = 0;
  p.c = g.y;
  p.n = g.n;
  p.k = g.k;
  p.b_bank = g.b_bank;
  p.b_stride = g.b_stride;
  p.s_bank = g.s_bank;
  p.s_stride = g.s_stride;
  p.z_bank = g.z_bank;
  p.z_stride = g.z_stride;
  p.ex_ids = g.ex_ids;
  p.ex_off = g.ex_off;
  p.ex_pairs = g.ex_pairs;
  p.pair_tok = g.pair_tok;
  p.n_expert = g.n_expert;
  p.n_active = g.n_active;
  p.n_pairs = g.n_pairs;
  p.n_tokens = g.n_tokens;
  // Upper bound on tiles: every segment adds at most one partial row tile.
  const long tiles = ((long)(g.n_pairs + TM - 1) / TM + g.n_active) * (g.n / TN);
  if (tiles <= 0) return hipSuccess;
  if (g.z_bank != nullptr)
    hipLaunchKernelGGL((gemm_tile_kernel<true, true>), dim3((unsigned)tiles), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<false, true>), dim3((unsigned)tiles), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace wq
