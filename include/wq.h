/*
 * wq.h -- C ABI of the MI355X (gfx950) W4A16 weight-only quantized GEMM library (libwq.so).
 *
 * Operation: C[m][n] = sum_k A[m][k] * W[k][n], W[k][n] = (q[k][n] - z) * s[g(k)][n],
 * fp16 activations, output and group scales s (bf16 with WQ_FLAG_BF16), fp32 accumulation,
 * 4-bit codes q, zero point z = 8 (symmetric "u4b8") or a per-group 4-bit code ("u4").
 * Sources: ferrum-kernels marlin.rs (module doc: Marlin INT4 x FP16 GEMM, K % 128 == 0,
 * N % 256 == 0; `marlin_gemm` doc: C = A @ dequant(B)); ferrum-kernels vllm_marlin.rs
 * (`FerrumMarlinLaunch`, the versioned launch problem this ABI is trimmed from; the scalar
 * ids and flag bits; `ferrum_vllm_gptq_marlin_repack`); memra-engine mmq_ffi.rs
 * (`ExpertCsr`, `memra_mmq_fp8_blk_grouped`: the expert-major grouped call).
 *
 * Conventions for every call:
 *  - Device pointers are caller-owned and must stay valid until the work enqueued on
 *    `stream` (a hipStream_t, NULL = the null stream) has completed.  Calls enqueue and
 *    return: they never allocate, free or synchronize, and never abort the process.
 *  - Return value: 0 on success, else (stage << 16) | code.  Stages: WQ_STAGE_ARGS and
 *    WQ_STAGE_SHAPE carry a wq_error code; WQ_STAGE_DEVICE (device query),
 *    WQ_STAGE_LAUNCH_CONFIG, WQ_STAGE_FUNC_ATTR and WQ_STAGE_LAUNCH carry the hipError_t.
 *    This is the staged native status of ferrum-kernels marlin.rs (`marlin_moe_ffi_status`).
 *  - Validation happens before any launch (fail closed); nothing is enqueued on error.
 *  - Shapes: k % 128 == 0, n % 256 == 0.  group_size (rows of K per scale / zero point) is
 *    -1 (channelwise: one group over all of K, as transformer.rs `marlin_num_groups` maps
 *    it) or a positive multiple of 16 dividing k (the pages' rule); anything else fails
 *    with WQ_ERR_SHAPE.  The library stores scales and zero points per unit of
 *    U = gcd(group_size, 128) rows (U = 128 for -1; so 16, 32, 64 or 128): a group is
 *    repeated for each unit it covers.  Both kernels (small-M and tiled) take every
 *    supported group size.
 *
 * Library weight layout (produced by the wq_repack_* calls; G = k / 128):
 *  - B: k*n/8 uint32 words (k*n/2 bytes, the plain format's byte count).  For 16-column
 *    block nb (columns 16*nb + c), 128-row chunk g, lane l = c + 16*qd (qd = 0..3) and
 *    dword j = 0..3, word ((nb*G + g)*64 + l)*4 + j holds rows 128*g + 32*j + 8*qd + i
 *    (i = 0..7) of column 16*nb + c; row offset i sits in nibble slot {0,4,1,5,2,6,3,7}[i].
 *    One 16-byte load per lane then feeds four 16x16x32 fp16 MFMA B operands of a wave.
 *  - scales: fp16 [n/16][k/U][16]; zero points: uint32 [n/16][k/U][2] (16 codes per pair,
 *    column c of the block in bits 4*(c%8) of word c/8).
 *  - act_order: B rows are stored in sorted order (row position i holds original row
 *    perm[i]); sorted position i belongs to group i / group_size (see wq_act_order_perm).
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQ_ABI_VERSION 3u

/* Flag bits: the bit positions of the vllm_marlin.rs launch flags. */
#define WQ_FLAG_ACT_ORDER   (1u << 1) /* gather A by perm before the product              */
#define WQ_FLAG_IS_K_FULL   (1u << 2) /* accepted, no effect: one GPU always holds all of K */
#define WQ_FLAG_HAS_ZP      (1u << 3) /* u4 with per-group zero points (else u4b8)         */
#define WQ_FLAG_ATOMIC_ADD  (1u << 4) /* not supported: rejected (non-deterministic sums)  */
#define WQ_FLAG_FP32_REDUCE (1u << 5) /* allow split-K with an fp32 workspace reduce        */
/* Grouped call only: scale each output row by its pair's fp32 routing weight (vllm_marlin.rs
 * MoE launch, `mul_topk_weights` with `topk_weights`). */
#define WQ_FLAG_MUL_TOPK_WEIGHTS (1u << 6)
/* SwiGLU epilogue (the transformer.rs dense SwiGLU chain's gate and up projections with its
 * planar silu*mul, fused): B, scales and zero points hold a gate and an up projection of
 * n/2 columns each, paired by wq_interleave_gate_up before the repack (16-column block 2t
 * is gate block t, block 2t+1 up block t); the output is the [rows][n/2] activation
 * round(silu(A Wg) * (A Wu)), silu(x) = x / (1 + exp(-x)), from the fp32 sums.  Not with
 * WQ_FLAG_MUL_TOPK_WEIGHTS. */
#define WQ_FLAG_SWIGLU (1u << 7)
/* bf16 activations (the element type of the pages' vllm_marlin.rs MXFP4 MoE entry point,
 * `ferrum_vllm_marlin_moe_mxfp4_bf16`, here with the same 4-bit integer weights): a, the
 * scales, c (y of the grouped call, w of wq_dequant) and a_tmp hold bf16 values instead of
 * fp16; codes and zero points are unchanged.  Products are accumulated in fp32 and rounded
 * once to bf16 (round to nearest even).  Scales are repacked bit for bit either way. */
#define WQ_FLAG_BF16 (1u << 8)
/* W8A16: B holds FP8 E4M3 weights (the "fn" variant: bias 7, no infinities, 0x7F/0xFF NaN)
 * in the FP8 library layout (wq_repack_fp8), one byte per weight: the pages' E4M3 weight
 * type (vllm_marlin.rs `ferrum_vllm_marlin_moe_fp8_f16`).  W[k][n] = e4m3(code) * s.
 * As the pages require: group_size -1 or 128, no zero points; here also no act_order
 * (WQ_ERR_FLAGS / WQ_ERR_SHAPE otherwise).  fp16 activations as on the pages, or bf16
 * (WQ_FLAG_BF16: the weights are converted to bf16 instead); the SwiGLU epilogue works as
 * for 4-bit weights. */
#define WQ_FLAG_FP8 (1u << 9)

enum wq_stage {
  WQ_STAGE_ARGS = 1,
  WQ_STAGE_SHAPE = 2,
  WQ_STAGE_DEVICE = 3,
  WQ_STAGE_LAUNCH_CONFIG = 4,
  WQ_STAGE_FUNC_ATTR = 5,
  WQ_STAGE_LAUNCH = 6
};

enum wq_error {
  WQ_ERR_NULL = 1,        /* a required pointer is NULL                                 */
  WQ_ERR_ALIGN = 2,       /* a pointer is misaligned (16 B for fp16/packed, 4 B for ints) */
  WQ_ERR_SHAPE = 3,       /* m/n/k/lda/group_size outside the supported set             */
  WQ_ERR_FLAGS = 4,       /* unknown or unsupported flag, or flag/pointer mismatch      */
  WQ_ERR_WORKSPACE = 5,   /* workspace missing or smaller than wq_*_workspace_bytes     */
  WQ_ERR_ABI = 6,         /* abi_version / struct_size mismatch                         */
  WQ_ERR_OVERFLOW = 7,    /* a byte extent overflows                                    */
  WQ_ERR_CSR = 8,         /* expert-major CSR invariant violated                        */
  WQ_ERR_ACT_ORDER = 9    /* g_idx does not give every group exactly group_size rows    */
};

#define WQ_STATUS(stage, code) ((int)(((unsigned)(stage) << 16) | ((unsigned)(code) & 0xFFFFu)))

/* ABI version of the loaded library (WQ_ABI_VERSION). */
uint32_t wq_abi_version(void);

/* Static text naming a status: "ok", or "<stage>: <code>" (never NULL, never freed). */
const char* wq_status_str(int status);

/*
 * Repack plain GPTQ words into the library's B layout (vllm_marlin.rs,
 * `ferrum_vllm_gptq_marlin_repack`: same byte count, a pure permutation of the codes,
 * optional row permutation for act_order).
 *   qweight: device uint32 [k/8][n]; rows 8r..8r+7 of column c in word (r, c), row 8r+i
 *            in bits 4i (low nibble first).
 *   perm:    device int32 [k] or NULL; when given, row position i of the output is input
 *            row perm[i] (perm must be a permutation of 0..k-1; entries are clamped into
 *            range, so a bad perm gives wrong codes, never an out-of-bounds read).
 *   b_out:   device, k*n/2 bytes, 16-byte aligned; must not overlap qweight.
 */
int wq_repack_b(const uint32_t* qweight, const int32_t* perm, void* b_out, int k, int n,
                void* stream);

/*
 * Scales fp16 or bf16 [k/group_size][n] row-major ([1][n] for group_size -1), moved as
 * 16-bit values -> library layout [n/16][k/U][16]: unit u takes the scales of the group
 * holding its rows.
 */
int wq_repack_scales(const void* scales, void* s_out, int k, int n, int group_size,
                     void* stream);

/*
 * E4M3 weights for WQ_FLAG_FP8: K-major words [k/4][n] uint32, byte i (bits 8i..8i+7) of
 * word (r, col) holding row 4r + i of column col (vllm_marlin.rs
 * `vllm_fp8_marlin_repack_raw_bits`; a row-major [n][k] checkpoint must be transposed and
 * packed this way first) -> FP8 library layout, k*n bytes: for 16-column block nb,
 * 128-row group g and half h (rows 64h..64h+63), lane l = c + 16*qd holds 16 bytes whose
 * word d covers rows 128g + 32(2h + d/2) + 8qd + 4(d%2) .. +3 of column 16nb + c, at word
 * (((nb * k/128 + g) * 2 + h) * 64 + l) * 4 + d.  A word permutation, nothing decoded.
 *   words: device, 4-byte aligned; b_out: device, k*n bytes, 16-byte aligned, no overlap.
 */
int wq_repack_fp8(const uint32_t* words, void* b_out, int k, int n, void* stream);

/*
 * Block-FP8 checkpoints (vllm_marlin.rs `launch_block_fp8_group128_repack` and
 * `launch_block_fp8_group128_scales`: E4M3 weights row-major [n][k] with one bf16 inverse
 * scale per 128 x 128 block), load time:
 *  - wq_repack_fp8_rows: E4M3 bytes [n][k] (row per output channel, 4-byte aligned) ->
 *    the FP8 layout of wq_repack_fp8 (k*n bytes, 16-byte aligned, no overlap);
 *  - wq_fp8_block_scales: bf16 [n/128][k/128] -> fp16 scales in the library scale layout
 *    for group_size 128 ([n/16][k/128][16], 16-byte aligned): column c of group g takes
 *    block (c/128, g), rounded to nearest even (exact for values in fp16's normal range).
 * k % 128 == 0, n % 256 == 0; device pointers; enqueued on `stream`.
 */
int wq_repack_fp8_rows(const void* w_nk, void* b_out, int k, int n, void* stream);
int wq_fp8_block_scales(const void* inv_scales, void* s_out, int k, int n, void* stream);

/*
 * Zero points uint32 [k/group_size][n/8] (actual codes 0..15, column 8j+i in bits 4i of
 * word j: vllm_marlin.rs `repack_gptq_qzeros_to_marlin`; [1][n/8] for group_size -1) ->
 * library layout [n/16][k/U][2], unit u taking the codes of the group holding its rows.
 */
int wq_repack_zeros(const uint32_t* zeros, void* z_out, int k, int n, int group_size,
                    void* stream);

/*
 * Load-time helper for WQ_FLAG_SWIGLU: pairs the columns of a gate and an up tensor in
 * 16-column blocks, out[r] = [gate block 0, up block 0, gate block 1, up block 1, ...].
 * gate and up are row-major [rows][cols] with bits_per_column bits per column: 32 for
 * GPTQ qweight words ([k/8][cols] uint32), 16 for scales, 4 for packed zero points
 * ([groups][cols/8] uint32); out has 2*cols columns.  cols % 16 == 0; device pointers,
 * 4-byte aligned; enqueued on `stream`.
 */
int wq_interleave_gate_up(const void* gate, const void* up, void* out, int rows, int cols,
                          int bits_per_column, void* stream);

/*
 * act_order helper (host memory, synchronous): perm_out[i] = stable argsort(g_idx)[i]
 * (marlin.rs `MarlinWeight.perm` doc: perm = argsort(g_idx)), sorted_gidx_out[i] =
 * g_idx[perm[i]] (either output may be NULL).  Fails with WQ_ERR_ACT_ORDER unless every
 * group 0..k/group_size-1 holds exactly group_size rows, the GPTQ construction, which
 * makes sorted position i belong to group i / group_size (group_size -1: one group of k
 * rows).
 */
int wq_act_order_perm(const int32_t* g_idx, int k, int group_size, int32_t* perm_out,
                      int32_t* sorted_gidx_out);

/* Workspace bytes wq_gemm needs for (m, n, k, flags): room for the fp32 split-K partials
 * [splits][m][n] of the largest split the library may choose (0 when it never splits: no
 * WQ_FLAG_FP32_REDUCE, or m > 16 with enough output tiles to occupy every CU).  For
 * m > 16 the tiled kernel splits K when its 256-column tiles are fewer than the CUs, the
 * pages' fp32 global reduce (marlin.rs MoE entry point: use_fp32_reduce with c_tmp).
 * Contents need no initialization; calls that share one workspace must not run
 * concurrently. */
int wq_gemm_workspace_bytes(int m, int n, int k, uint32_t flags, size_t* bytes_out);

/* Which kernel wq_gemm runs for a problem, and how many splits along K it uses (host,
 * no device access): the planner's own choice for (m, n, k, group_size, flags, split_k),
 * the same arguments as in wq_gemm_args.  kernel_out: WQ_KERNEL_SMALL_M (16-column blocks:
 * m <= 16, weights streamed once; or, without SwiGLU or a requested split, up to sixteen
 * row chunks of 16 rows, or of 8, 4, 2 or 1 where K is long, each streaming the weights
 * with K not split, while the chunks' weight reads stay within K x 38 kB (16-row chunks)
 * or K x 20 kB (shorter chunks); with WQ_FLAG_FP32_REDUCE, 16-row chunks within K x
 * 12 kB, since the tiles may then split K), WQ_KERNEL_TILE_256 or
 * WQ_KERNEL_TILE_128 (MFMA tiles of 256 or 128 rows by 256 columns); splits_out: 1 = K not
 * split, s > 1 = s fp32 partials added by a second kernel in split order.  Shape errors as
 * in wq_gemm. */
#define WQ_KERNEL_SMALL_M 1
#define WQ_KERNEL_TILE_256 2
#define WQ_KERNEL_TILE_128 3
int wq_gemm_plan(int m, int n, int k, int group_size, uint32_t flags, int split_k,
                 int32_t* kernel_out, int32_t* splits_out);

typedef struct wq_gemm_args {
  uint32_t abi_version;     /* WQ_ABI_VERSION                                          */
  uint32_t struct_size;     /* sizeof(wq_gemm_args)                                   */
  const void* a;            /* device fp16 (bf16) [m][lda], 16-byte aligned rows        */
  const void* b;            /* device, library B layout (wq_repack_b)                   */
  void* c;                  /* device fp16 (bf16) [m][n], output                        */
  const void* b_scales;     /* device, library scale layout (wq_repack_scales)          */
  const void* zero_points;  /* device, library zero-point layout, or NULL (u4b8)        */
  const int32_t* perm;      /* device int32 [k] with WQ_FLAG_ACT_ORDER, else NULL       */
  const int32_t* group_index; /* device int32 [k] or NULL (act_order only): the group of
                               each sorted row position, g_idx[perm[i]] (the sorted_gidx_out
                               of wq_act_order_perm).  The library layout puts sorted
                               position i in group i / group_size (k for -1), so this is a
                               check, not an input: positions whose entry differs make the
                               act_order gather write NaN into that activation column, and
                               every output of the call is then NaN                      */
  void* a_tmp;              /* device [m][k] 16-bit gather scratch with act_order, or NULL */
  void* workspace;          /* device scratch (wq_gemm_workspace_bytes), may be NULL if 0 */
  size_t workspace_bytes;
  void* stream;             /* hipStream_t                                              */
  int32_t m, n, k;          /* m >= 1, n % 256 == 0, k % 128 == 0                        */
  int32_t lda;              /* row stride of a in elements, >= k, multiple of 8         */
  int32_t group_size;       /* as repacked: -1 or a multiple of 16 dividing k           */
  uint32_t flags;           /* WQ_FLAG_*; HAS_ZP iff zero_points != NULL; ACT_ORDER iff perm */
  int32_t split_k;          /* 0 = library's choice; 1 = no split; s > 1 requests s splits
                               along K (needs WQ_FLAG_FP32_REDUCE; clamped to k/128 and 16
                               for m <= 16, and for m > 16 to what the tiles allow: none
                               on 256-row tiles, SwiGLU, E4M3 or 32/16-row units, else
                               k/256 and 16); partials are added in split order.  A split
                               above the library's choice needs split*m*n*4 workspace bytes */
  int32_t reserved;         /* must be 0                                                */
} wq_gemm_args;

/*
 * C = A @ dequant(B) (all of it enqueued on args->stream).  (ferrum-kernels vllm_marlin.rs,
 * `FerrumMarlinLaunch`: a, b, c, scales, zero points, group_index and permutation, the
 * scratch buffers, the sizes, the group size and the flag word.)  A group_index without
 * WQ_FLAG_ACT_ORDER fails with WQ_ERR_FLAGS, a misaligned one with WQ_ERR_ALIGN.  With WQ_FLAG_SWIGLU, c is the
 * [m][n/2] activation silu(A Wg) * (A Wu) of paired gate/up weights (any m; for m <= 16
 * and k <= 8192 the small-M kernel computes both sums of a pair in one work-group, with
 * no split along K).
 */
int wq_gemm(const wq_gemm_args* args);

/*
 * wq_gemm without caller scratch, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments and result as wq_gemm, except that workspace, workspace_bytes and a_tmp must be
 * NULL / 0 (else WQ_ERR_WORKSPACE): the act_order gather buffer (m*k 16-bit values, rounded
 * up to 256 bytes) and the split-K fp32 partials (splits*m*n floats, splits as
 * wq_gemm_plan reports) come from one static device array of WQ_NOALLOC_SCRATCH_BYTES per
 * GPU, reserved when the library is first used on that GPU and held until the process
 * ends.  When the library's own split (split_k 0) would not fit beside the gather buffer,
 * the call takes the largest split that does (none if even two do not), and its result is
 * then that of wq_gemm with that split_k.  A problem whose scratch still exceeds the array
 * fails with WQ_ERR_WORKSPACE before anything is enqueued.  It allocates and frees nothing.  All calls on one GPU share that array: calls
 * that may overlap on one GPU (other streams, other threads) race and must be serialized by
 * the caller.  The calling thread's current device must be the device of args->stream.
 */
#define WQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int wq_gemm_noalloc(const wq_gemm_args* args);

/*
 * Dequant export for bit-exact tests: reads library-layout B, scales and optional zero
 * points and writes w[k][n] = rne((q - z) * s) (fp16, or bf16 with WQ_FLAG_BF16; row-major,
 * rows in the stored order, i.e. sorted order for act_order weights).  flags: HAS_ZP, BF16
 * and FP8 are read (FP8: b in the FP8 layout, w = fp16_rne(e4m3 * s)), ACT_ORDER and
 * IS_K_FULL accepted; any other bit fails with WQ_ERR_FLAGS.
 */
int wq_dequant(const void* b, const void* b_scales, const void* zero_points, int k, int n,
               int group_size, uint32_t flags, void* w_out, void* stream);

/*
 * Expert-major CSR from token-major top-k routes (host memory, synchronous), as
 * mmq_ffi.rs `ExpertCsr::from_token_routes`: count pairs per expert, list non-empty
 * experts ascending (ex_ids, n_active of them) with segment starts ex_off (n_active + 1
 * entries, last = n_pairs), place pairs into segments in ascending pair order (ex_pairs),
 * pair_tok[p] = p / top_k.  Capacities: ex_ids and ex_off hold n_expert (+1) entries,
 * ex_pairs and pair_tok n_tokens*top_k.  Fails with WQ_ERR_CSR on an out-of-range expert.
 */
int wq_csr_from_routes(const int32_t* selected, int n_tokens, int top_k, int n_expert,
                       int32_t* ex_ids, int32_t* ex_off, int32_t* ex_pairs, int32_t* pair_tok,
                       int32_t* n_active_out);

typedef struct wq_grouped_args {
  uint32_t abi_version;
  uint32_t struct_size;     /* sizeof(wq_grouped_args)                                  */
  const void* a;            /* device fp16 (bf16) [n_tokens][k]                          */
  const void* b_bank;       /* expert e's library-layout B at b_bank + e*b_stride_bytes  */
  size_t b_stride_bytes;    /* >= k*n/2, multiple of 16                                  */
  const void* s_bank;       /* expert e's scales at s_bank + e*s_stride_bytes            */
  size_t s_stride_bytes;    /* >= (k/128)*n*2, multiple of 16                            */
  const void* zp_bank;      /* expert e's zero points at zp_bank + e*zp_stride_bytes, or NULL */
  size_t zp_stride_bytes;
  const int32_t* ex_ids;    /* device [n_active] expert of each segment, or NULL = identity */
  const int32_t* ex_off;    /* device [n_active + 1] segment starts into ex_pairs        */
  const int32_t* ex_pairs;  /* device [n_pairs] pair ids grouped by expert               */
  const int32_t* pair_tok;  /* device [n_pairs] activation row of each pair              */
  const float* topk_weights; /* device fp32 [n_pairs], pair-major routing weights, with
                                WQ_FLAG_MUL_TOPK_WEIGHTS; else NULL                      */
  void* y;                  /* device fp16 (bf16) [n_pairs][n], pair-major output        */
  void* workspace;          /* reserved for the grouped schedule; may be NULL            */
  size_t workspace_bytes;
  void* stream;
  int32_t n_expert, n_active, n_pairs, n_tokens;
  int32_t k, n, group_size;
  uint32_t flags;           /* WQ_FLAG_HAS_ZP iff zp_bank != NULL; WQ_FLAG_MUL_TOPK_WEIGHTS
                               iff topk_weights != NULL                                   */
  int32_t reserved;
} wq_grouped_args;

/* Workspace bytes wq_grouped_gemm needs (currently 0 for every shape). */
int wq_grouped_workspace_bytes(int n_pairs, int n_active, int n, int k, uint32_t flags,
                               size_t* bytes_out);

/*
 * Grouped W4A16 product over an expert-major CSR (mmq_ffi.rs grouped projection call):
 * for active segment i with expert e = ex_ids[i] (i when ex_ids is NULL) and each pair p
 * in ex_pairs[ex_off[i] .. ex_off[i+1]), y[p][:] = A[pair_tok[p]][:] @ dequant(B_e).
 * With WQ_FLAG_MUL_TOPK_WEIGHTS the row is also multiplied by topk_weights[p], on the fp32
 * result before its one rounding to the output type (the vllm_marlin.rs MoE launch's
 * `mul_topk_weights` with its fp32 `topk_weights`, one per routed pair).  The device CSR is
 * not re-validated (that would need a host sync): build it with wq_csr_from_routes;
 * entries out of range are skipped by the kernel (never read or written out of bounds),
 * leaving those output rows unwritten.  Segments must be non-empty: when n_pairs -
 * n_active + 1 <= 4 (every segment then holds at most four rows; decode-sized batches)
 * products with 4-bit weights (K up to 128 groups of 128 rows, 64 with WQ_FLAG_SWIGLU) run
 * on the small-M kernel, one work-group per 16-column block (a gate/up pair of blocks with
 * the SwiGLU epilogue) and segment, which computes at most that many rows of a segment;
 * E4M3 weights and longer K take the tiled kernel.
 */
int wq_grouped_gemm(const wq_grouped_args* args);

/*
 * Measurement helper, not a step of the method: reads the `bytes` bytes at device address
 * `src` (16-byte aligned, bytes a positive multiple of 16) once, with the 16-byte
 * non-temporal loads the small-M GEMM streams its weights with, as the practical HBM read
 * ceiling to report that GEMM against.  `sink` is device memory of at least
 * wq_stream_read_sink_words(bytes) uint32 words; a word is written only when the data
 * XOR of a wave's reads equals a fixed constant (its content is meaningless).  Enqueues on
 * `stream`; fails with WQ_ERR_NULL / WQ_ERR_ALIGN / WQ_ERR_SHAPE / WQ_ERR_WORKSPACE.
 */
int wq_stream_read_sink_words(size_t bytes, size_t* words_out);
int wq_stream_read(const void* src, size_t bytes, void* sink, size_t sink_words,
                   void* stream);

/*
 * Measurement helper, not a step of the method: the practical fp16 matrix rate.  One work-
 * group per CU (256), two waves per SIMD; every wave keeps the tiled GEMM's 128 x 64 wave
 * tile in registers (four A operands, two B operands: `operands` is device f16 [6][64][8],
 * 16-byte aligned, A first) and runs `iters` (1 .. 2^20) steps of its eight
 * v_mfma_f32_32x32x16_f16 products.  No memory is touched between the operand loads and
 * one fp32 store per thread into `sink` (device, at least 256 * 512 floats).  The chip's
 * clock falls with the operands' switching activity, so the rate depends on the data.
 * *flops_out receives the launch's floating-point operation count.  Enqueues on `stream`.
 */
int wq_mfma_rate(const void* operands, int iters, float* sink, size_t sink_floats,
                 double* flops_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
