"""CPU oracle for the W4A16 weight-only quantized GEMM: the plain definition, computed slowly.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
module; only the tests, the smoke check of the build entry point and the bench's CPU
baseline leg use it.  It shares no code, tables or constants with the HIP library.

What it computes (the pages give the operation only through interfaces, doc comments and
tests; this is the plain definition they describe):

  C[m, n] = sum_k A[m, k] * W[k, n],   W[k, n] = (q[k, n] - z(k, n)) * s[g(k), n]

* ferrum-kernels marlin.rs, module doc and `marlin_gemm` doc: C = A @ dequant(B), INT4
  weights, FP16 activations, constraints K % 128 == 0 and N % 256 == 0.
* ferrum-kernels marlin.rs, `ferrum_vllm_marlin_moe_f16` declaration (`has_zp`): symmetric
  kU4B8 (zero point fixed at 8) or asymmetric kU4 with per-group zero points.
* ferrum-kernels marlin.rs, `MarlinWeight.qzeros` doc and vllm_marlin.rs
  `repack_gptq_qzeros_to_marlin`: zero points are the actual codes (0..15).
* ferrum-kernels marlin.rs, `MarlinWeight.perm` doc: act_order; each row k belongs to group
  g_idx[k]; the permutation is argsort(g_idx).
* ferrum-kernels vllm_marlin.rs, `ferrum_vllm_marlin_moe_fp8_f16` and
  `vllm_fp8_marlin_repack_raw_bits`: W8A16 with E4M3 weights (K-major words of four bytes),
  fp16 scales channelwise or per 128 rows, no zero points.
* ferrum-kernels vllm_marlin.rs, `ferrum_vllm_marlin_moe_mxfp4_bf16`: the pages' bf16
  activation and output type.  Read here with the same 4-bit integer weights: with bf16,
  activations and scales arrive as bf16 bit patterns (the upper half of a binary32).

Precision: codes, zero points and scales are exact; W = (q - z) * s is formed exactly
(a 5-bit integer times an fp16 value fits in fp64, and in fp32 too); the product is
accumulated in fp64 and left unrounded.  Only `dequantize_fp16` and `round_bf16` round
(once, to nearest even), for the bit-exact check of the library's dequant export and for
the 16-bit activation handed on in the SwiGLU chain.
"""

from __future__ import annotations

import numpy as np

U4B8_ZERO = 8  # kU4B8: stored code q means q - 8


# ---------------------------------------------------------------------------------------
# Unpacking the plain input formats
# ---------------------------------------------------------------------------------------

def unpack_qweight(qweight: np.ndarray) -> np.ndarray:
    """GPTQ words uint32 [K/8][N] -> codes uint8 [K][N]; row 8r+i sits in bits 4i of word r.

    Reading of the pages: 4-bit codes are packed low nibble first (the zero-point words of
    vllm_marlin.rs's qzeros tests and the low-nibble-first source decode of marlin.rs's
    MXFP4 quality test use that order; GPTQ's [K/8, N] qweight shape is named on
    vllm_marlin.rs, `load_stacked_gptq_vllm_marlin` doc).
    """
    qweight = np.asarray(qweight, dtype=np.uint32)
    k8, n = qweight.shape
    q = np.empty((k8 * 8, n), dtype=np.uint8)
    for i in range(8):
        q[i::8] = (qweight >> np.uint32(4 * i)) & np.uint32(0xF)
    return q


def unpack_zero_points(zeros: np.ndarray) -> np.ndarray:
    """Zero-point words uint32 [G][N/8] -> codes uint8 [G][N]; column 8j+i in bits 4i of word j.

    vllm_marlin.rs, `repack_gptq_qzeros_to_marlin` and its test
    `qzeros_repack_preserves_kernel_layout` (codes 1..8 pack to 0x87654321).
    """
    zeros = np.asarray(zeros, dtype=np.uint32)
    g, n8 = zeros.shape
    z = np.empty((g, n8 * 8), dtype=np.uint8)
    for i in range(8):
        z[:, i::8] = (zeros >> np.uint32(4 * i)) & np.uint32(0xF)
    return z


def num_groups(k: int, group_size: int) -> int:
    """Group count along K, as transformer.rs `marlin_num_groups` defines it: -1 means one
    channelwise group; any other size must be positive and divide K."""
    if k <= 0:
        raise ValueError(f"input width {k} must be positive")
    if group_size == -1:
        return 1
    if group_size <= 0:
        raise ValueError(f"group size {group_size} must be -1 for channelwise weights or positive")
    if k % group_size:
        raise ValueError(f"input width {k} is not divisible by group size {group_size}")
    return k // group_size


def group_of_rows(k: int, group_size: int, g_idx: np.ndarray | None = None) -> np.ndarray:
    """Group of every original row: g_idx[k] with act_order, else k // group_size (0 for
    every row when channelwise, group_size -1)."""
    if g_idx is not None:
        g = np.asarray(g_idx, dtype=np.int64)
        if g.shape != (k,):
            raise ValueError("g_idx must have one entry per row of K")
        return g
    if group_size == -1:
        return np.zeros(k, dtype=np.int64)
    return np.arange(k, dtype=np.int64) // group_size


# ---------------------------------------------------------------------------------------
# Dequantization and the product
# ---------------------------------------------------------------------------------------

def bf16_value(bits) -> np.ndarray:
    """fp64 values of bf16 bit patterns (uint16): bfloat16 is the upper half of an IEEE
    binary32 (sign, 8-bit exponent, 7 stored mantissa bits), so the value is that of the
    binary32 word bits << 16."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even, as fp64.

    bf16 is the upper half of a binary32, so it keeps 8 significant bits down to 2^-126
    and below that a fixed spacing of 2^-133 (its subnormals).  No overflow handling is
    needed here (|x| stays far below 2^127)."""
    x = np.asarray(x, dtype=np.float64)
    _, exp = np.frexp(x)                    # x = mant * 2**exp, 0.5 <= |mant| < 1
    quantum = np.ldexp(1.0, np.maximum(exp, -125) - 8)
    return np.round(x / quantum) * quantum  # np.round: half to even


def values16(x, bf16: bool = False) -> np.ndarray:
    """fp64 values of 16-bit operands: fp16 numbers, or bf16 bit patterns when bf16."""
    return bf16_value(x) if bf16 else np.asarray(x, dtype=np.float16).astype(np.float64)


def dequantize(q: np.ndarray, scales: np.ndarray, group: np.ndarray,
               zero_codes: np.ndarray | None = None, bf16: bool = False) -> np.ndarray:
    """W[k, n] = (q[k, n] - z) * s[group[k], n] in fp64 (exact).

    z = 8 without zero points (kU4B8), else the code zero_codes[group[k], n] (kU4).  Scales
    are fp16, or bf16 bit patterns with bf16.
    """
    s = values16(scales, bf16)
    qi = q.astype(np.int64)
    zi = U4B8_ZERO if zero_codes is None else np.asarray(zero_codes).astype(np.int64)[group, :]
    return (qi - zi).astype(np.float64) * s[group, :]


def dequantize_fp16(w: np.ndarray) -> np.ndarray:
    """fp16 round-to-nearest-even of the exact dequantized weights (one rounding)."""
    return np.asarray(w, dtype=np.float64).astype(np.float16)


def matmul_fp64(a: np.ndarray, w: np.ndarray, bf16: bool = False) -> np.ndarray:
    """fp64 product A @ W of 16-bit activations (fp16, or bf16 bit patterns with bf16) and
    exact weights (unrounded result)."""
    return values16(a, bf16) @ w


def w4a16_weights(qweight, scales, *, zeros=None, g_idx=None, group_size=128,
                  columns=None, bf16=False) -> np.ndarray:
    """Exact fp64 weights W [K][N] (or [K][len(columns)] for a column subset)."""
    qweight = np.asarray(qweight, dtype=np.uint32)
    scales = np.asarray(scales)
    k = qweight.shape[0] * 8
    num_groups(k, group_size)
    zero_codes = None if zeros is None else unpack_zero_points(zeros)
    if columns is not None:
        cols = np.asarray(columns, dtype=np.int64)
        qweight, scales = qweight[:, cols], scales[:, cols]
        zero_codes = None if zero_codes is None else zero_codes[:, cols]
    group = group_of_rows(k, group_size, g_idx)
    return dequantize(unpack_qweight(qweight), scales, group, zero_codes, bf16)


def w4a16_gemm(a, qweight, scales, *, zeros=None, g_idx=None, group_size=128,
               columns=None, bf16=False) -> np.ndarray:
    """Reference C = A @ dequant(B) in fp64, [M][N] (or [M][len(columns)]); with bf16 the
    activations and scales are bf16 bit patterns."""
    w = w4a16_weights(qweight, scales, zeros=zeros, g_idx=g_idx, group_size=group_size,
                      columns=columns, bf16=bf16)
    return matmul_fp64(a, w, bf16)


# ---------------------------------------------------------------------------------------
# W8A16: FP8 E4M3 weights (vllm_marlin.rs `ferrum_vllm_marlin_moe_fp8_f16`, the E4M3 weight
# type: fp16 activations and scales, scales channelwise (group_size -1) or per 128 rows of
# K, no zero points; weights arrive as K-major words of four E4M3 bytes per output channel,
# `vllm_fp8_marlin_repack_raw_bits`)
# ---------------------------------------------------------------------------------------

FP8_GROUP_SIZES = (-1, 128)


def e4m3_value(codes) -> np.ndarray:
    """fp64 values of E4M3 (the "fn" variant the pages name, FE4M3FN) bytes: sign bit, 4
    exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal (2^-6 * m/8);
    0x7F and 0xFF are NaN; there are no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def unpack_fp8_words(words: np.ndarray) -> np.ndarray:
    """uint32 [K/4][N] -> uint8 codes [K][N]: byte i (bits 8i..8i+7) of word (r, n) is row
    4r + i of column n (little-endian, K-major)."""
    w = np.asarray(words, dtype=np.uint32)
    r, n = w.shape
    out = np.empty((4 * r, n), dtype=np.uint8)
    for i in range(4):
        out[i::4, :] = (w >> np.uint32(8 * i)) & np.uint32(0xFF)
    return out


def w8a16_weights(words, scales, *, group_size=128, columns=None, bf16=False) -> np.ndarray:
    """Exact fp64 weights W[k, n] = e4m3(code[k, n]) * s[g(k), n]."""
    if group_size not in FP8_GROUP_SIZES:
        raise ValueError(f"E4M3 group size must be -1 or 128, got {group_size}")
    words = np.asarray(words, dtype=np.uint32)
    scales = np.asarray(scales)
    k = words.shape[0] * 4
    num_groups(k, group_size)
    if columns is not None:
        cols = np.asarray(columns, dtype=np.int64)
        words, scales = words[:, cols], scales[:, cols]
    group = group_of_rows(k, group_size)
    return e4m3_value(unpack_fp8_words(words)) * values16(scales, bf16)[group, :]


def fp8_rows_to_words(w_nk: np.ndarray) -> np.ndarray:
    """Block-FP8 checkpoint weights, E4M3 bytes row-major [N][K] (one row per output
    channel), -> the K-major input words [K/4][N] (vllm_marlin.rs block-FP8 repack: the
    checkpoint matrix transposed and packed four K-consecutive bytes per word)."""
    w = np.asarray(w_nk, dtype=np.uint8)
    n, k = w.shape
    b = w.T.astype(np.uint32).reshape(k // 4, 4, n)
    return b[:, 0] | (b[:, 1] << np.uint32(8)) | (b[:, 2] << np.uint32(16)) | (b[:, 3] << np.uint32(24))


def fp8_block_scales(inv_scales_bf16: np.ndarray) -> np.ndarray:
    """Block-FP8 inverse scales, bf16 bit patterns [N/128][K/128] (one per 128 x 128 block of
    the [N][K] weight), -> per-group fp16 scales [K/128][N]: column n of group g takes the
    scale of block (n // 128, g), rounded to fp16 (nearest even; exact for bf16 values in
    fp16's normal range)."""
    v = bf16_value(inv_scales_bf16)                 # [N/128][G]
    return np.repeat(v, 128, axis=0).T.astype(np.float16)


def w8a16_gemm(a, words, scales, *, group_size=128, columns=None, bf16=False) -> np.ndarray:
    """Reference C = A @ W for E4M3 weights, fp64 and unrounded."""
    return matmul_fp64(a, w8a16_weights(words, scales, group_size=group_size, columns=columns,
                                        bf16=bf16), bf16)


# ---------------------------------------------------------------------------------------
# act_order
# ---------------------------------------------------------------------------------------

def act_order_perm(g_idx: np.ndarray, group_size: int) -> tuple[np.ndarray, np.ndarray]:
    """perm = stable argsort(g_idx) and the group of each sorted position, g_idx[perm].

    marlin.rs, `MarlinWeight.perm` doc: perm[i] is the original row placed at position i,
    computed as argsort of g_idx; weight rows are stored in that order and activations are
    gathered by it, which leaves the product unchanged.  Reading: ties keep ascending row
    order (stable sort), and the layout requires every group to hold exactly group_size
    rows (GPTQ's construction), so that sorted position i belongs to group i // group_size.
    """
    g = np.asarray(g_idx, dtype=np.int64)
    perm = np.argsort(g, kind="stable")
    sorted_g = g[perm]
    k = g.size
    if group_size == -1:
        group_size = k
    if k % group_size or not np.array_equal(sorted_g, np.arange(k) // group_size):
        raise ValueError("act_order groups must each hold exactly group_size rows, "
                         "numbered 0..K/group_size-1")
    return perm.astype(np.int32), sorted_g.astype(np.int32)


# ---------------------------------------------------------------------------------------
# Expert-major CSR (mmq_ffi.rs, `ExpertCsr`) and the grouped product
# ---------------------------------------------------------------------------------------

class CsrError(ValueError):
    pass


def csr_from_pair_rows(n_expert: int, n_tokens: int, selected, pair_tok) -> dict:
    """Expert-major CSR of routed pairs, from each pair's expert and activation row.

    mmq_ffi.rs, `ExpertCsr` (the grouped projection's contract): the pair ids listed in
    order of their expert, experts ascending and pair ids ascending within an expert
    (ex_pairs); the experts that own at least one pair, ascending (ex_ids); where each
    expert's run starts in that list, followed by the pair count (ex_off); and the
    activation row of every pair, indexed by pair id (pair_tok).  Written here as a stable
    sort of the pairs by expert.
    """
    sel = np.asarray(selected, dtype=np.int64).reshape(-1)
    tok = np.asarray(pair_tok, dtype=np.int64).reshape(-1)
    if n_expert <= 0 or n_tokens <= 0 or sel.size == 0:
        raise CsrError("an expert CSR needs at least one expert, one token and one pair")
    if tok.size != sel.size:
        raise CsrError(f"{sel.size} expert choices but {tok.size} activation rows")
    if sel.min() < 0 or sel.max() >= n_expert:
        raise CsrError(f"an expert choice lies outside 0..{n_expert - 1}")
    if tok.min() < 0 or tok.max() >= n_tokens:
        raise CsrError(f"an activation row lies outside 0..{n_tokens - 1}")
    order = np.argsort(sel, kind="stable")            # by expert; pair order kept within one
    experts, first = np.unique(sel[order], return_index=True)
    csr = dict(ex_ids=experts.tolist(), ex_off=first.tolist() + [int(sel.size)],
               ex_pairs=order.tolist(), pair_tok=tok.tolist(), n_expert=n_expert,
               n_tokens=n_tokens)
    validate_csr(csr)
    return csr


def csr_from_token_routes(n_expert: int, n_tokens: int, top_k: int, selected) -> dict:
    """CSR from token-major top-k routes: route j of token t is pair t * top_k + j, which
    reads activation row t (mmq_ffi.rs, `ExpertCsr::from_token_routes`)."""
    if top_k <= 0:
        raise CsrError("each token needs at least one route")
    sel = np.asarray(selected, dtype=np.int64).reshape(-1)
    if sel.size != n_tokens * top_k:
        raise CsrError(f"{sel.size} routes for {n_tokens} tokens of {top_k} routes each")
    return csr_from_pair_rows(n_expert, n_tokens, sel, np.arange(sel.size) // top_k)


def validate_csr(csr: dict) -> None:
    """Raise CsrError unless `csr` is a well-formed expert-major CSR (the invariants the
    mmq_ffi.rs grouped call relies on): non-empty; ex_off starts at 0, ends at the pair
    count and rises strictly (no empty segment); expert ids rise strictly inside
    0..n_expert-1; ex_pairs lists every pair id once; every activation row is in range."""
    ids = np.asarray(csr["ex_ids"], dtype=np.int64)
    off = np.asarray(csr["ex_off"], dtype=np.int64)
    pairs = np.asarray(csr["ex_pairs"], dtype=np.int64)
    tok = np.asarray(csr["pair_tok"], dtype=np.int64)
    n_expert, n_tokens = csr["n_expert"], csr["n_tokens"]
    if n_expert <= 0 or n_tokens <= 0 or ids.size == 0 or pairs.size == 0:
        raise CsrError("an expert CSR needs at least one expert, one token and one pair")
    if off.size != ids.size + 1 or off[0] != 0 or off[-1] != pairs.size:
        raise CsrError("ex_off must hold one start per listed expert plus the pair count")
    if np.any(np.diff(off) <= 0):
        raise CsrError("every listed expert must own at least one pair")
    if np.any(np.diff(ids) <= 0) or ids.min() < 0 or ids.max() >= n_expert:
        raise CsrError(f"expert ids must rise strictly inside 0..{n_expert - 1}")
    if tok.size != pairs.size:
        raise CsrError("pair_tok must hold one activation row per pair")
    if not np.array_equal(np.sort(pairs), np.arange(pairs.size)):
        raise CsrError("ex_pairs must list every pair id exactly once")
    if tok.min() < 0 or tok.max() >= n_tokens:
        raise CsrError(f"an activation row lies outside 0..{n_tokens - 1}")


def grouped_w4a16_gemm(a, experts, csr, *, group_size=128, columns=None,
                       pairs=None, topk_weights=None, bf16=False, fp8=False) -> np.ndarray:
    """Pair-major reference y[p] = A[pair_tok[p]] @ dequant(B_e) for the expert e owning p.

    Walks the expert-major CSR: segment i covers positions ex_off[i]..ex_off[i+1] of
    ex_pairs and uses expert ex_ids[i] (mmq_ffi.rs grouped projection contract).
    `experts[e]` holds that expert's qweight, scales and optional zeros.  `pairs` restricts
    the rows computed (others stay NaN).

    With `topk_weights` (one fp32 routing weight per pair, pair-major: the vllm_marlin.rs
    MoE launch's `topk_weights` under `mul_topk_weights`), row p is multiplied by
    topk_weights[p], in fp64.  With bf16, A and the scales are bf16 bit patterns; with fp8,
    each expert's qweight holds E4M3 words ([K/4][N]) instead of 4-bit codes.
    """
    a = np.asarray(a)
    n_pairs = len(csr["ex_pairs"])
    ncols = experts[0]["qweight"].shape[1] if columns is None else len(columns)
    y = np.full((n_pairs, ncols), np.nan)
    want = None if pairs is None else set(int(p) for p in pairs)
    for i, e in enumerate(csr["ex_ids"]):
        rows = [csr["ex_pairs"][j] for j in range(csr["ex_off"][i], csr["ex_off"][i + 1])]
        if want is not None:
            rows = [p for p in rows if p in want]
        if not rows:
            continue
        ex = experts[e]
        if fp8:
            w = w8a16_weights(ex["qweight"], ex["scales"], group_size=group_size,
                              columns=columns, bf16=bf16)
        else:
            w = w4a16_weights(ex["qweight"], ex["scales"], zeros=ex.get("zeros"),
                              group_size=group_size, columns=columns, bf16=bf16)
        toks = [csr["pair_tok"][p] for p in rows]
        y[rows, :] = matmul_fp64(a[toks, :], w, bf16)
        if topk_weights is not None:
            scale = np.asarray(topk_weights, dtype=np.float32)[rows].astype(np.float64)
            y[rows, :] *= scale[:, None]
    return y


# ---------------------------------------------------------------------------------------
# SwiGLU MLP chain (ferrum-kernels transformer.rs, the dense SwiGLU encode with W4
# projections: gate and up projections of the same activations, the planar silu*mul of the
# two, then the down projection of its fp16 result)
# ---------------------------------------------------------------------------------------

def silu(x: np.ndarray) -> np.ndarray:
    """silu(x) = x * sigmoid(x) = x / (1 + exp(-x)), fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu_activation(a, gate: dict, up: dict, *, group_size=128, columns=None,
                      bf16=False, fp8=False) -> np.ndarray:
    """act = silu(A @ W_gate) * (A @ W_up), fp64 and unrounded ([M][I], or a column subset).

    `gate` and `up` hold qweight, scales and optional zeros of the two projections (E4M3
    words and scales with fp8).
    """
    if fp8:
        g = w8a16_gemm(a, gate["qweight"], gate["scales"], group_size=group_size,
                       columns=columns, bf16=bf16)
        u = w8a16_gemm(a, up["qweight"], up["scales"], group_size=group_size,
                       columns=columns, bf16=bf16)
        return silu(g) * u
    g = w4a16_gemm(a, gate["qweight"], gate["scales"], zeros=gate.get("zeros"),
                   group_size=group_size, columns=columns, bf16=bf16)
    u = w4a16_gemm(a, up["qweight"], up["scales"], zeros=up.get("zeros"),
                   group_size=group_size, columns=columns, bf16=bf16)
    return silu(g) * u


def swiglu_mlp(a, gate: dict, up: dict, down: dict, *, group_size=128) -> tuple:
    """The chain: act16 = fp16_rne(swiglu_activation) (the activation handed to the down
    projection is fp16, as every W4A16 operand A is), out = act16 @ W_down in fp64.
    Returns (act16, out)."""
    act16 = dequantize_fp16(swiglu_activation(a, gate, up, group_size=group_size))
    out = w4a16_gemm(act16, down["qweight"], down["scales"], zeros=down.get("zeros"),
                     group_size=group_size)
    return act16, out


def swiglu_mlp_bf16(a, gate: dict, up: dict, down: dict, *, group_size=128) -> tuple:
    """The chain with bf16 activations: act = bf16_rne(swiglu_activation), out = act @
    W_down in fp64 (A and every scale as bf16 bit patterns).  Returns (act values, out)."""
    act = round_bf16(swiglu_activation(a, gate, up, group_size=group_size, bf16=True))
    w = w4a16_weights(down["qweight"], down["scales"], zeros=down.get("zeros"),
                      group_size=group_size, bf16=True)
    return act, act @ w


# ---------------------------------------------------------------------------------------
# Checker
# ---------------------------------------------------------------------------------------

def check(c: np.ndarray, ref: np.ndarray, *, rel_max: float = 2e-3, abs_max: float = 1e-3,
          rel_frob: float = 1e-3, rel_elem: float = 0.0) -> dict:
    """Tolerance test of an fp16 result against the fp64 reference.

    Pass iff no non-finite output, |C - ref| <= rel_elem * |ref| + rel_max * rms(ref) +
    abs_max for every element (rel_elem is 0 for the GEMM outputs), and
    ||C - ref||_F / ||ref||_F <= rel_frob (rms over every compared element).
    """
    c64 = np.asarray(c).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if c64.shape != ref.shape:
        raise ValueError(f"shape mismatch {c64.shape} vs {ref.shape}")
    nonfinite = int(np.count_nonzero(~np.isfinite(c64)))
    diff = np.abs(c64 - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    tol = rel_max * rms + abs_max
    if rel_elem:
        diff = diff - rel_elem * np.abs(ref)  # the element's own rounding allowance
    max_err = float(np.max(diff)) if diff.size else 0.0
    ref_norm = float(np.linalg.norm(ref))
    relf = float(np.linalg.norm(c64 - ref) / ref_norm) if ref_norm > 0 else float(
        np.linalg.norm(c64 - ref))
    ok = nonfinite == 0 and max_err <= tol and relf <= rel_frob
    return dict(ok=bool(ok), max_err=max_err, tol=tol, rms=rms, rel_frob=relf,
                nonfinite=nonfinite, violations=int(np.count_nonzero(diff > tol)))
