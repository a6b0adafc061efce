// Host-side launchers of the kernels, shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

// Repack / export / gather kernels (wq_repack.hip).
hipError_t launch_repack_b(const uint32_t* qweight, const int32_t* perm, uint32_t* out, int k,
                           int n, hipStream_t stream);
// group_size: -1 (channelwise) or a multiple of 16 dividing k.  The output holds one entry
// per unit of gcd(group_size, 128) rows of K (128 for -1): a group is repeated for each
// unit it covers.
int scale_unit_rows(int k, int group_size);
hipError_t launch_repack_scales(const uint16_t* s, uint16_t* out, int k, int n,
                                int group_size, hipStream_t stream);
hipError_t launch_repack_zeros(const uint32_t* z, uint32_t* out, int k, int n, int group_size,
                               hipStream_t stream);
// Gate/up column pairing for the SwiGLU epilogue (bits_per_column 32, 16 or 4).
hipError_t launch_interleave_gate_up(const void* gate, const void* up, void* out, int rows,
                                     int cols, int bits_per_column, hipStream_t stream);
// E4M3 weights: K-major words [k/4][n] -> the FP8 layout (k % 128 == 0, n % 16 == 0), and
// the dequant export of that layout with fp16 scales (one unit per 128 rows).
hipError_t launch_repack_fp8(const uint32_t* words, uint32_t* out, int k, int n,
                             hipStream_t stream);
hipError_t launch_dequant_fp8(const uint32_t* b, const uint16_t* s, int k, int n, uint16_t* w,
                              hipStream_t stream);
// Block-FP8 checkpoints: E4M3 bytes row-major [n][k] -> the FP8 layout; bf16 inverse scales
// [n/128][k/128] -> fp16 scales in the library layout.
hipError_t launch_repack_fp8_rows(const uint8_t* w_nk, uint32_t* out, int k, int n,
                                  hipStream_t stream);
hipError_t launch_fp8_block_scales(const uint16_t* inv, uint16_t* out, int k, int n,
                                   hipStream_t stream);
// bf16: s and w hold bf16 values (else fp16).
hipError_t launch_dequant(const uint32_t* b, const uint16_t* s, const uint32_t* z, int k, int n,
                          int unit, bool bf16, uint16_t* w, hipStream_t stream);
// out[r][i] = a[r][perm[i]]; with group_index, columns whose entry is not i / group_size
// (k for -1) are written as NaN.
hipError_t launch_gather_columns(const uint16_t* a, int lda, const int32_t* perm,
                                 const int32_t* group_index, int group_size, uint16_t* out,
                                 int m, int k, hipStream_t stream);

// Small-M kernel (wq_gemm_small.hip): m <= 16, one 16-row MFMA block; with `splits` > 1
// work-groups per column block, fp32 partials go to `partials` [splits][m][n] and a second
// kernel reduces them in split order.
struct SmallPlan {
  int waves;       // waves per work-group splitting K: 4 or 8, or 16 on the staged form
                   // (8 or 16 when pair)
  int splits;      // work-groups along K per column block
  int depth;       // groups of K per wave, all loaded before arithmetic: 1, 2, 4 or 8, or
                   // 16 with sixteen staged waves
  bool pair;       // SwiGLU epilogue: a gate/up pair of blocks per work-group, half the
                   // waves on each (n counts both; c is [m][n/2]; splits must be 1)
  int gpc;         // scale units per 128-row chunk: 1, 2, 4 or 8 (units of 128/gpc rows)
  bool direct;     // each wave fetches its own groups' activation tiles, scales and zero
                   // points into its own LDS region (no shared slice; not with pair)
  bool dual;       // direct only: each wave covers two adjacent column blocks, reading the
                   // activations once for both (4-bit weights)
  int rows;        // rows per work-group when the product is split into row chunks along
                   // grid z (one split), else 0 (every work-group takes all m rows)
};
bool small_plan_fits(int m, int k, const SmallPlan& plan);
// Dense products without the fp32 reduce flag that one small-M work-group cannot take (more
// than 16 rows, or a staged slice too long for LDS) run on it in row chunks along grid z
// (SmallPlan::rows), one split: at most sixteen chunks, while their weight reads stay within
// K x kChunkDirectBytes (16-row chunks on the direct form) or K x kChunkStagedBytes (staged
// chunks of at most 8 rows).
constexpr double kChunkDirectBytes = 38e3;
constexpr double kChunkStagedBytes = 20e3;
// With the fp32 reduce flag (the tiles may split K): direct chunks only, K x kChunkSplitBytes.
constexpr double kChunkSplitBytes = 12e3;
// bf16: A, s and c hold bf16 values (else fp16).  fp8: b holds E4M3 weights in the FP8
// layout (no zero points, 128-row scale units).
hipError_t launch_gemm_small(const uint16_t* a, int lda, int m, const uint32_t* b,
                             const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                             const SmallPlan& plan, float* partials, bool bf16, bool fp8,
                             hipStream_t stream);
// The E4M3 instances (wq_gemm_small_fp8.hip: fp16; wq_gemm_small_fp8_bf16.hip: bf16).
hipError_t launch_small_fp8(const uint16_t* a, int lda, int m, const uint32_t* b,
                            const uint16_t* s, uint16_t* c, int n, int k, const SmallPlan& plan,
                            float* partials, hipStream_t stream);
hipError_t launch_small_fp8_bf16(const uint16_t* a, int lda, int m, const uint32_t* b,
                                 const uint16_t* s, uint16_t* c, int n, int k,
                                 const SmallPlan& plan, float* partials, hipStream_t stream);
// The instances of each scale-unit count and activation type (wq_gemm_small.hip, _g2.hip,
// _g4.hip, _g8.hip; wq_gemm_small_bf16.hip, _bf16_g2.hip, _bf16_g4.hip, _bf16_g8.hip).
#define WQ_SMALL_GPC_DECL(NAME)                                                             \
  hipError_t NAME(const uint16_t* a, int lda, int m, const uint32_t* b, const uint16_t* s,  \
                  const uint32_t* z, uint16_t* c, int n, int k, const SmallPlan& plan,      \
                  float* partials, hipStream_t stream);
WQ_SMALL_GPC_DECL(launch_small_g1)
WQ_SMALL_GPC_DECL(launch_small_g2)
WQ_SMALL_GPC_DECL(launch_small_g4)
WQ_SMALL_GPC_DECL(launch_small_g8)
WQ_SMALL_GPC_DECL(launch_small_bf16_g1)
WQ_SMALL_GPC_DECL(launch_small_bf16_g2)
WQ_SMALL_GPC_DECL(launch_small_bf16_g4)
WQ_SMALL_GPC_DECL(launch_small_bf16_g8)
#undef WQ_SMALL_GPC_DECL
// c = round(sum of the fp32 partials [splits][m][n] in split order) to fp16, or bf16.
hipError_t launch_reduce_splits(const float* partials, uint16_t* c, int m, int n, int splits,
                                bool bf16, hipStream_t stream);

// Tiled kernel (wq_tile_kernel.h, wq_gemm_tile*.hip): 256 x 256 output tiles on 8 waves
// of 128 x 64, or 128 x 256 tiles on 4 waves (kTileMinM rows: grouped products and ragged
// row counts).
constexpr int kTileMinM = 128;
constexpr int kTileN = 256;
// swiglu: B pairs gate/up 16-column blocks and c is the [m][n/2] activation.  gpc: scale
// units per 128 rows of K (1, 2, 4 or 8).  bf16: A, s and c hold bf16 values (else fp16).
// fp8: b holds E4M3 weights in the FP8 layout (gpc 1, no zero points).
// splits > 1 (from tile_splits): work-groups along K per output tile, fp32 partials
// [splits][m][n] in `partials`, added in split order by launch_reduce_splits.
hipError_t launch_gemm_tile(const uint16_t* a, int lda, int m, const uint32_t* b,
                            const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                            bool swiglu, int gpc, bool bf16, bool fp8, int splits,
                            float* partials, hipStream_t stream);
// Splits along K of a dense tiled product with the fp32 reduce: about one work-group per CU
// (two from K = 8192 with 128 tiles or more) when the 128-row tiles are fewer (at least two groups of K each, at
// most 16); 1 for SwiGLU, E4M3 weights, 32- or 16-row scale units (gpc > 2), 256-row tiles
// or enough tiles.  tile_max_splits: the most a requested split may take (1: none).
int tile_splits(int m, int n, int k, int gpc, bool fp8, bool swiglu);
int tile_max_splits(int m, int n, int k, int gpc, bool fp8, bool swiglu);
// Whether a dense tiled product takes 128 x 256 tiles (else 256 x 256).
bool tile_is_tall(int m, int n, int gpc, bool fp8);

struct GroupedProblem {
  const uint16_t* a;
  const uint8_t* b_bank;
  size_t b_stride;
  const uint8_t* s_bank;
  size_t s_stride;
  const uint8_t* z_bank;  // may be null
  size_t z_stride;
  const int32_t* ex_ids;  // may be null
  const int32_t* ex_off;
  const int32_t* ex_pairs;
  const int32_t* pair_tok;
  const float* topk_w;    // may be null: no routing-weight multiply
  uint16_t* y;
  int n_expert, n_active, n_pairs, n_tokens, k, n;
  bool swiglu;            // SwiGLU epilogue: y is [n_pairs][n/2]
  int gpc;                // scale units per 128 rows of K (1, 2, 4 or 8)
  bool bf16;              // a, scales and y hold bf16 values (else fp16)
  bool fp8;               // the banks hold E4M3 weights in the FP8 layout
};
hipError_t launch_grouped_tile(const GroupedProblem& p, hipStream_t stream);
// Grouped products whose segments all hold few rows run on the small-M kernel instead (4-bit
// weights): one work-group per 16-column block (a gate/up pair of blocks with the SwiGLU
// epilogue) and segment, its activation rows gathered through pair_tok and its outputs
// scattered to the pair rows.  `rows` bounds every segment's row count (n_pairs - n_active
// + 1 for a CSR of non-empty segments) and is 1 or at most kSegRows; `plan` is a
// single-split staged plan for m = rows (four waves per block, or eight or sixteen with
// GW 8).
constexpr int kSegRows = 4;
bool grouped_small_plan(const GroupedProblem& p, int rows, SmallPlan* plan);
hipError_t launch_grouped_small(const GroupedProblem& p, int rows, const SmallPlan& plan,
                                hipStream_t stream);
#define WQ_SEG_GPC_DECL(NAME)                                                               \
  hipError_t NAME(const GroupedProblem& p, int rows, const SmallPlan& plan, hipStream_t stream);
WQ_SEG_GPC_DECL(launch_seg_g1)
WQ_SEG_GPC_DECL(launch_seg_g2)
WQ_SEG_GPC_DECL(launch_seg_g4)
WQ_SEG_GPC_DECL(launch_seg_g8)
WQ_SEG_GPC_DECL(launch_seg_bf16_g1)
WQ_SEG_GPC_DECL(launch_seg_bf16_g2)
WQ_SEG_GPC_DECL(launch_seg_bf16_g4)
WQ_SEG_GPC_DECL(launch_seg_bf16_g8)
#undef WQ_SEG_GPC_DECL

// Register-only MFMA measurement helper (wq_measure.hip): kMfmaBlocks work-groups of
// kMfmaThreads threads, each thread running `iters` steps of eight 32x32x16 fp16 MFMAs on
// operands ops[6][64] (f16x8: four A operands, then two B operands) and storing one float.
constexpr int kMfmaBlocks = 256;
constexpr int kMfmaThreads = 512;
constexpr int kMfmaLds = 96 * 1024;  // two work-groups never share a CU
hipError_t launch_mfma_loop(const void* ops, int iters, float* sink, hipStream_t stream);

// Streaming-read measurement helper (wq_measure.hip).
long stream_read_sink_words(size_t bytes);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink,
                              hipStream_t stream);

}  // namespace wq
