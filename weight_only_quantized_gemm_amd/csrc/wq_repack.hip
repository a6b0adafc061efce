// Offline repack of plain GPTQ weights, scales and zero points into the library layout,
// the dequant export used by bit-exact tests, and the act_order column gather.
//
// The repack is a pure permutation of the 4-bit codes with an optional row permutation
// (ferrum-kernels vllm_marlin.rs, `ferrum_vllm_gptq_marlin_repack` doc: same byte count;
// marlin.rs, `MarlinWeight.perm` doc: weight rows stored in argsort(g_idx) order).  The
// target order is this library's own (see include/wq.h), built here by a direct index
// formula per output word.
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

// Row offset i of a layout word lives in nibble slot (i even ? i/2 : 4 + i/2).
__device__ __forceinline__ uint32_t place_codes(const uint32_t codes[8]) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= codes[i] << (4 * ((i & 1) ? 4 + (i >> 1) : (i >> 1)));
  return w;
}

__global__ __launch_bounds__(256) void repack_b_kernel(const uint32_t* __restrict__ qweight,
                                                       const int32_t* __restrict__ perm,
                                                       uint32_t* __restrict__ out, int k, int n) {
  const long total = (long)k * n / 8;
  const int groups = k / kGroup;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int j = (int)(o & 3);
    const int lane = (int)((o >> 2) & 63);
    const long rest = o >> 8;
    const int g = (int)(rest % groups);
    const long nb = rest / groups;
    const int col = (int)(nb * 16 + (lane & 15));
    const int row0 = g * kGroup + 32 * j + 8 * (lane >> 4);
    uint32_t codes[8];
    if (perm == nullptr) {
      const uint32_t src = qweight[(long)(row0 >> 3) * n + col];
#pragma unroll
      for (int i = 0; i < 8; ++i) codes[i] = (src >> (4 * i)) & 0xFu;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int r = perm[row0 + i];
        r = r < 0 ? 0 : (r >= k ? k - 1 : r);
        codes[i] = (qweight[(long)(r >> 3) * n + col] >> (4 * (r & 7))) & 0xFu;
      }
    }
    out[o] = place_codes(codes);
  }
}

// Scales and zero points are stored per unit of min(group_size, 128) rows of K.  Unit u
// takes the group holding its rows, u * unit / group_size (a group larger than 128 rows is
// repeated for each chunk it covers); group_size -1 is one group over all of K.
__device__ __forceinline__ long source_group(int u, int unit, int group_size) {
  return group_size > 0 ? (long)u * unit / group_size : 0;
}

__global__ __launch_bounds__(256) void repack_scales_kernel(const uint16_t* __restrict__ s,
                                                            uint16_t* __restrict__ out, int k,
                                                            int n, int unit, int group_size) {
  const int units = k / unit;
  const long total = (long)units * n;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int c = (int)(o & 15);
    const long rest = o >> 4;
    const int g = (int)(rest % units);
    const long nb = rest / units;
    out[o] = s[source_group(g, unit, group_size) * n + nb * 16 + c];
  }
}

__global__ __launch_bounds__(256) void repack_zeros_kernel(const uint32_t* __restrict__ z,
                                                           uint32_t* __restrict__ out, int k,
                                                           int n, int unit, int group_size) {
  const int units = k / unit;
  const long total = (long)units * (n / 8);
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int h = (int)(o & 1);
    const long rest = o >> 1;
    const int g = (int)(rest % units);
    const long nb = rest / units;
    out[o] = z[source_group(g, unit, group_size) * (n / 8) + nb * 2 + h];
  }
}

// E4M3 weights: words [k/4][n] (byte i of word (r, col) is row 4r + i) -> the FP8 layout.
// Word d of lane l = c + 16*qd in (block nb, group g, half h) covers rows
// 128g + 32(2h + d/2) + 8qd + 4(d%2) .. +3 of column 16nb + c: one input word, moved whole.
__global__ __launch_bounds__(256) void repack_fp8_kernel(const uint32_t* __restrict__ words,
                                                         uint32_t* __restrict__ out, int k,
                                                         int n) {
  const long total = (long)k * n / 4;
  const int groups = k / kGroup;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int d = (int)(o & 3);
    const int lane = (int)((o >> 2) & 63);
    const int h = (int)((o >> 8) & 1);
    const long rest = o >> 9;
    const int g = (int)(rest % groups);
    const long nb = rest / groups;
    const int col = (int)(nb * 16 + (lane & 15));
    const int row0 = g * kGroup + 32 * (2 * h + (d >> 1)) + 8 * (lane >> 4) + 4 * (d & 1);
    out[o] = words[(long)(row0 >> 2) * n + col];
  }
}

// Block-FP8 checkpoint weights, E4M3 bytes row-major [n][k], -> the FP8 layout: a layout
// word's four rows are K-consecutive bytes of one checkpoint row, one aligned 32-bit read.
__global__ __launch_bounds__(256) void repack_fp8_rows_kernel(const uint8_t* __restrict__ w_nk,
                                                              uint32_t* __restrict__ out, int k,
                                                              int n) {
  const long total = (long)k * n / 4;
  const int groups = k / kGroup;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int d = (int)(o & 3);
    const int lane = (int)((o >> 2) & 63);
    const int h = (int)((o >> 8) & 1);
    const long rest = o >> 9;
    const int g = (int)(rest % groups);
    const long nb = rest / groups;
    const long col = nb * 16 + (lane & 15);
    const int row0 = g * kGroup + 32 * (2 * h + (d >> 1)) + 8 * (lane >> 4) + 4 * (d & 1);
    out[o] = *reinterpret_cast<const uint32_t*>(w_nk + col * k + row0);
  }
}

// Block-FP8 inverse scales, bf16 [n/128][k/128], -> fp16 scales in the library layout
// [n/16][k/128][16]: column col of group g takes block (col / 128, g), rounded to fp16.
__global__ __launch_bounds__(256) void fp8_block_scales_kernel(const uint16_t* __restrict__ inv,
                                                               uint16_t* __restrict__ out, int k,
                                                               int n) {
  const int groups = k / kGroup;
  const long total = (long)groups * n;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int c = (int)(o & 15);
    const long rest = o >> 4;
    const int g = (int)(rest % groups);
    const long col = (rest / groups) * 16 + c;
    out[o] = Act<false>::round(Act<true>::value(inv[(col / kGroup) * groups + g]));
  }
}

// E4M3 dequant export: w[row][col] = fp16_rne(e4m3 * s), the product exact in fp32.
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const u32x4* __restrict__ b,
                                                          const uint16_t* __restrict__ s,
                                                          int k, int n,
                                                          uint16_t* __restrict__ w) {
  const long total = (long)k * n / 16;  // one u32x4 (16 weights) per item
  const int groups = k / kGroup;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int lane = (int)(o & 63);
    const int h = (int)((o >> 6) & 1);
    const long rest = o >> 7;
    const int g = (int)(rest % groups);
    const long nb = rest / groups;
    const int c = lane & 15;
    const long col = nb * 16 + c;
    const float scale = Act<false>::value(s[(nb * groups + g) * 16 + c]);
    const u32x4 v = b[o];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const f16x8 x = dequant8_fp8(v[2 * jj], v[2 * jj + 1]);
      const int row0 = g * kGroup + 32 * (2 * h + jj) + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[(long)(row0 + i) * n + col] = Act<false>::round((float)x[i] * scale);
    }
  }
}

// w[row][col] = rne((q - z) * s) in the scale's type (fp16, or bf16): the product is exact
// in fp32 (a 5-bit integer times a 16-bit float), so the one conversion is the only rounding.
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ b,
                                                      const uint16_t* __restrict__ s,
                                                      const uint32_t* __restrict__ z, int k,
                                                      int n, int unit,
                                                      uint16_t* __restrict__ w) {
  const long total = (long)k * n / 8;
  const int groups = k / kGroup;
  const int units = k / unit;  // scale rows per column block
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int j = (int)(o & 3);
    const int lane = (int)((o >> 2) & 63);
    const long rest = o >> 8;
    const int g = (int)(rest % groups);
    const long nb = rest / groups;
    const int c = lane & 15;
    const long col = nb * 16 + c;
    const int row0 = g * kGroup + 32 * j + 8 * (lane >> 4);
    const long blk = nb * units + row0 / unit;  // the 8 rows share one scale unit
    const float scale = Act<BF16>::value(s[blk * 16 + c]);
    int zc = 8;
    if (z != nullptr) zc = zero_code(u32x2{z[blk * 2], z[blk * 2 + 1]}, c);
    const uint32_t word = b[o];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = (i & 1) ? 4 + (i >> 1) : (i >> 1);
      const int q = (int)((word >> (4 * slot)) & 0xFu);
      w[(long)(row0 + i) * n + col] = Act<BF16>::round((float)(q - zc) * scale);
    }
  }
}

// The act_order gather also checks an optional group_index against the layout's groups
// (sorted position i in group i / gsz; CHECK instances): a column whose entry differs is
// written as NaN (0xFFFF is a NaN in both fp16 and bf16), so that every output of the
// product is NaN.  Positions 8g .. 8g + 7 lie in group q = 8g / gsz, or q + 1 from the
// position where 8g - q gsz + e reaches gsz (gsz >= 16: at most two groups).
constexpr uint16_t kNaN16 = 0xFFFF;

// out[r][i] = a[r][perm[i]] for the act_order gather (eight columns per thread).
template <bool CHECK>
__global__ __launch_bounds__(256) void gather_columns_kernel(const uint16_t* __restrict__ a,
                                                             int lda,
                                                             const int32_t* __restrict__ perm,
                                                             const int32_t* __restrict__ gidx,
                                                             int gsz,
                                                             uint16_t* __restrict__ out, int m,
                                                             int k) {
  const int per_row = k / 8;
  const long total = (long)m * per_row;
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (long)gridDim.x * blockDim.x) {
    const long r = t / per_row;
    const int i0 = (int)(t % per_row) * 8;
    const i32x4 p0 = *reinterpret_cast<const i32x4*>(perm + i0);
    const i32x4 p1 = *reinterpret_cast<const i32x4*>(perm + i0 + 4);
    const uint16_t* row = a + r * lda;
    int q = 0, rem = 0;
    if constexpr (CHECK) {
      q = i0 / gsz;
      rem = i0 - q * gsz;
    }
    uint16_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int c = j < 4 ? p0[j] : p1[j - 4];
      c = c < 0 ? 0 : (c >= k ? k - 1 : c);
      v[j] = row[c];
      if constexpr (CHECK) v[j] = gidx[i0 + j] != q + (rem + j >= gsz ? 1 : 0) ? kNaN16 : v[j];
    }
    u32x4 packed;
#pragma unroll
    for (int j = 0; j < 4; ++j) packed[j] = (uint32_t)v[2 * j] | ((uint32_t)v[2 * j + 1] << 16);
    *reinterpret_cast<u32x4*>(out + r * k + i0) = packed;
  }
}

// Row-staged gather for K up to 8 * 256 * G: a work-group copies whole activation rows into
// LDS with coalesced 16-byte loads (the next row's loads issued before the current row is
// gathered), then each thread assembles its G output granules of 8 columns from LDS through
// the permutation it holds in registers.  Reading permuted columns straight from global
// memory touches a different cache line per lane and element.  CHECK: a column that fails
// the group_index check gathers from a NaN slot past the row's end instead, so the gather
// itself carries no per-element test.  The check is a template parameter so that both
// prologues are straight-line code: a branch per element would end a basic block after
// every load and serialize the loads (measured 2-3x slower at M=2048, K=4096).
template <int G, bool CHECK>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ a,
                                                          int lda,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ gidx,
                                                          int gsz,
                                                          uint16_t* __restrict__ out, int m,
                                                          int k) {
  extern __shared__ u32x4 row_lds[];  // one row, k / 8 granules, then one granule of NaNs
  const uint16_t* row16 = reinterpret_cast<const uint16_t*>(row_lds);
  const int t = threadIdx.x;
  const int granules = k / 8;
  if (t == 0) row_lds[granules] = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  // Permuted source column of each output column (clamped into the row), or k (the NaN
  // slot) where group_index disagrees with the layout's group of the sorted position.
  int src[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int g = t + 256 * j;
    const int gg = g < granules ? g : granules - 1;
    // sorted position 8gg + e lies in group q, or q + 1 once rem + e reaches gsz (gsz >= 16,
    // so a granule's eight positions span at most two groups)
    int q = 0, rem = 0;
    if constexpr (CHECK) {
      q = 8 * gg / gsz;
      rem = 8 * gg - q * gsz;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = perm[8 * gg + e];
      int sc = c < 0 ? 0 : (c >= k ? k - 1 : c);
      if constexpr (CHECK) sc = gidx[8 * gg + e] != q + (rem + e >= gsz ? 1 : 0) ? k : sc;
      src[j][e] = sc;
    }
  }
  int r = blockIdx.x;
  u32x4 next[G];
  auto load_row = [&](int rr) {
    const u32x4* rp = reinterpret_cast<const u32x4*>(a + (long)rr * lda);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int g = t + 256 * j;
      next[j] = rp[g < granules ? g : granules - 1];
    }
  };
  if (r < m) load_row(r);
  for (; r < m; r += gridDim.x) {
    __syncthreads();  // the previous row's gather is done with the buffer
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int g = t + 256 * j;
      if (g < granules) row_lds[g] = next[j];
    }
    __syncthreads();
    const int rn = r + (int)gridDim.x;
    if (rn < m) load_row(rn);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int g = t + 256 * j;
      if (g >= granules) break;
      u32x4 packed;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        packed[e] = (uint32_t)row16[src[j][2 * e]] | ((uint32_t)row16[src[j][2 * e + 1]] << 16);
      *reinterpret_cast<u32x4*>(out + (long)r * k + 8 * g) = packed;
    }
  }
}

// Pair two row-major tensors' columns in 16-column blocks (gate block t, then up block t)
// for the fused gate/up projection.  Words of 4 bytes; `block_words` words per 16 columns.
__global__ __launch_bounds__(256) void interleave_gate_up_kernel(
    const uint32_t* __restrict__ gate, const uint32_t* __restrict__ up,
    uint32_t* __restrict__ out, long rows, long row_words, int block_words) {
  const long total = rows * 2 * row_words;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const long r = o / (2 * row_words);
    const long w = o - r * 2 * row_words;
    const long blk = w / block_words;
    const long src = (blk >> 1) * block_words + (w - blk * block_words);
    out[o] = ((blk & 1) ? up : gate)[r * row_words + src];
  }
}

int grid_for(long work) {
  long blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return (int)(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_repack_b(const uint32_t* qweight, const int32_t* perm, uint32_t* out, int k,
                           int n, hipStream_t stream) {
  hipLaunchKernelGGL(repack_b_kernel, dim3(grid_for((long)k * n / 8)), dim3(256), 0, stream,
                     qweight, perm, out, k, n);
  return hipGetLastError();
}

hipError_t launch_repack_fp8(const uint32_t* words, uint32_t* out, int k, int n,
                             hipStream_t stream) {
  hipLaunchKernelGGL(repack_fp8_kernel, dim3(grid_for((long)k * n / 4)), dim3(256), 0, stream,
                     words, out, k, n);
  return hipGetLastError();
}

hipError_t launch_repack_fp8_rows(const uint8_t* w_nk, uint32_t* out, int k, int n,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(repack_fp8_rows_kernel, dim3(grid_for((long)k * n / 4)), dim3(256), 0,
                     stream, w_nk, out, k, n);
  return hipGetLastError();
}

hipError_t launch_fp8_block_scales(const uint16_t* inv, uint16_t* out, int k, int n,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(fp8_block_scales_kernel, dim3(grid_for((long)(k / kGroup) * n)), dim3(256),
                     0, stream, inv, out, k, n);
  return hipGetLastError();
}

hipError_t launch_dequant_fp8(const uint32_t* b, const uint16_t* s, int k, int n, uint16_t* w,
                              hipStream_t stream) {
  hipLaunchKernelGGL(dequant_fp8_kernel, dim3(grid_for((long)k * n / 16)), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(b), s, k, n, w);
  return hipGetLastError();
}

int scale_unit_rows(int k, int group_size) {
  (void)k;
  if (group_size <= 0) return kGroup;  // channelwise: one unit per 128-row chunk
  int a = group_size, b = kGroup;      // gcd(group_size, 128): 16, 32, 64 or 128
  while (b != 0) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

hipError_t launch_repack_scales(const uint16_t* s, uint16_t* out, int k, int n,
                                int group_size, hipStream_t stream) {
  const int unit = scale_unit_rows(k, group_size);
  hipLaunchKernelGGL(repack_scales_kernel, dim3(grid_for((long)(k / unit) * n)), dim3(256), 0,
                     stream, s, out, k, n, unit, group_size);
  return hipGetLastError();
}

hipError_t launch_repack_zeros(const uint32_t* z, uint32_t* out, int k, int n, int group_size,
                               hipStream_t stream) {
  const int unit = scale_unit_rows(k, group_size);
  hipLaunchKernelGGL(repack_zeros_kernel, dim3(grid_for((long)(k / unit) * (n / 8))),
                     dim3(256), 0, stream, z, out, k, n, unit, group_size);
  return hipGetLastError();
}

hipError_t launch_interleave_gate_up(const void* gate, const void* up, void* out, int rows,
                                     int cols, int bits_per_column, hipStream_t stream) {
  const long row_words = (long)cols * bits_per_column / 32;
  const int block_words = 16 * bits_per_column / 32;
  hipLaunchKernelGGL(interleave_gate_up_kernel, dim3(grid_for((long)rows * 2 * row_words)),
                     dim3(256), 0, stream, static_cast<const uint32_t*>(gate),
                     static_cast<const uint32_t*>(up), static_cast<uint32_t*>(out), (long)rows,
                     row_words, block_words);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* b, const uint16_t* s, const uint32_t* z, int k, int n,
                          int unit, bool bf16, uint16_t* w, hipStream_t stream) {
  const dim3 grid(grid_for((long)k * n / 8));
  if (bf16)
    hipLaunchKernelGGL(dequant_kernel<true>, grid, dim3(256), 0, stream, b, s, z, k, n, unit, w);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, grid, dim3(256), 0, stream, b, s, z, k, n, unit, w);
  return hipGetLastError();
}

template <int G>
hipError_t launch_gather_rows(const uint16_t* a, int lda, const int32_t* perm,
                              const int32_t* gidx, int gsz, uint16_t* out, int m, int k,
                              hipStream_t stream) {
  // Up to 1024 work-groups (four per CU); larger m loops, amortizing the permutation loads.
  const int blocks = m < 1024 ? m : 1024;
  if (gidx != nullptr)
    hipLaunchKernelGGL((gather_rows_kernel<G, true>), dim3(blocks), dim3(256), (size_t)k * 2 + 16,
                       stream, a, lda, perm, gidx, gsz, out, m, k);
  else
    hipLaunchKernelGGL((gather_rows_kernel<G, false>), dim3(blocks), dim3(256),
                       (size_t)k * 2 + 16, stream, a, lda, perm, gidx, gsz, out, m, k);
  return hipGetLastError();
}

hipError_t launch_gather_columns(const uint16_t* a, int lda, const int32_t* perm,
                                 const int32_t* group_index, int group_size, uint16_t* out,
                                 int m, int k, hipStream_t stream) {
  const int gsz = group_size == -1 ? k : group_size;
  const int granules = k / 8;
  if (granules <= 256) return launch_gather_rows<1>(a, lda, perm, group_index, gsz, out, m, k, stream);
  if (granules <= 512) return launch_gather_rows<2>(a, lda, perm, group_index, gsz, out, m, k, stream);
  if (granules <= 1024) return launch_gather_rows<4>(a, lda, perm, group_index, gsz, out, m, k, stream);
  if (granules <= 2048) return launch_gather_rows<8>(a, lda, perm, group_index, gsz, out, m, k, stream);
  if (group_index != nullptr)
    hipLaunchKernelGGL(gather_columns_kernel<true>, dim3(grid_for((long)m * (k / 8))), dim3(256),
                       0, stream, a, lda, perm, group_index, gsz, out, m, k);
  else
    hipLaunchKernelGGL(gather_columns_kernel<false>, dim3(grid_for((long)m * (k / 8))),
                       dim3(256), 0, stream, a, lda, perm, group_index, gsz, out, m, k);
  return hipGetLastError();
}

}  // namespace wq
