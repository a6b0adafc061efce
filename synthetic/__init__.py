"""Seeded synthetic inputs for the W4A16 GEMM (shared by the tests, the bench and the oracle).

This module only draws random numbers and lays them out in the input formats the
library accepts; it holds none of the method's arithmetic (no unpacking, no dequant,
no products, no routing tables).

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; Vigna's reference splitmix64.c), used counter-style: draw i of
stream s is mix64(s + (i + 1) * 0x9E3779B97F4A7C15).  Each tensor gets its own stream,
derived from a root seed and a per-tensor tag, in the spirit of the seeded-LCG test
vectors of the ferrum-kernels marlin.rs page (GPT-OSS MXFP4 Marlin-MoE quality test:
root seed XOR a per-tensor stream constant).

Input formats (the boundary's plain formats, before the library repacks them):
  * activations A: fp16 [M][K], row-major;
  * qweight: uint32 [K/8][N]; word (r, n) carries the 4-bit codes of rows 8r..8r+7 of
    column n, row 8r+i in bits 4i..4i+3 (GPTQ on-disk order, low nibble first);
  * scales: fp16 [K/group][N];
  * zero points: uint32 [K/group][N/8]; column 8j+i of group g in bits 4i of word (g, j)
    (the zero-point word layout pinned by the vllm_marlin.rs page's
    qzeros_repack_preserves_kernel_layout test);
  * act_order: g_idx int32 [K] (group of each original row);
  * MoE routes: int32 [tokens][top_k] expert choices, token-major.

Uniform nibbles are uniform 32-bit words, so codes are drawn as whole words.
"""

from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Per-tensor stream tags (ASCII mnemonics, like the pages' per-tensor XOR constants).
TAG_ACT = 0x4143544956415445      # "ACTIVATE"
TAG_WEIGHT = 0x5745494748545F31   # "WEIGHT_1"
TAG_SCALE = 0x5343414C455F5F31    # "SCALE__1"
TAG_ZERO = 0x5A45524F5F5F5F31     # "ZERO___1"
TAG_PERM = 0x5045524D5F5F5F31     # "PERM___1"
TAG_ROUTE = 0x524F5554455F5F31    # "ROUTE__1"

ROOT_SEED = 0x5745514D0000000C


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_seed(root: int, tag: int, index: int = 0) -> int:
    """Seed of the stream for one tensor: mix64(root ^ tag ^ index * gamma)."""
    with np.errstate(over="ignore"):
        x = np.uint64(root & 0xFFFFFFFFFFFFFFFF) ^ np.uint64(tag) ^ (np.uint64(index) * GAMMA)
        return int(_mix64(np.array([x], dtype=np.uint64))[0])


def draws_u64(seed: int, count: int, offset: int = 0) -> np.ndarray:
    """`count` 64-bit SplitMix64 outputs of stream `seed`, starting at draw `offset`."""
    ctr = np.arange(offset + 1, offset + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(np.uint64(seed) + ctr * GAMMA)


def uniform01(seed: int, count: int) -> np.ndarray:
    """Doubles in [0, 1): the top 53 bits of each draw times 2**-53."""
    return (draws_u64(seed, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, count: int) -> np.ndarray:
    """Standard normal doubles by the Box-Muller transform on pairs of uniforms."""
    pairs = (count + 1) // 2
    u = uniform01(seed, 2 * pairs)
    u1 = 1.0 - u[0::2]             # (0, 1]: log is finite
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * pairs, dtype=np.float64)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:count]


def words_u32(seed: int, count: int) -> np.ndarray:
    """`count` uniform 32-bit words (two per 64-bit draw: low half, then high half)."""
    d = draws_u64(seed, (count + 1) // 2)
    out = np.empty(2 * d.size, dtype=np.uint32)
    out[0::2] = (d & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    out[1::2] = (d >> np.uint64(32)).astype(np.uint32)
    return out[:count]


def below(seed: int, count: int, bound: int) -> np.ndarray:
    """Integers in [0, bound) by multiply-shift of the top 32 bits (bias < 2**-32 * bound)."""
    hi = (draws_u64(seed, count) >> np.uint64(32)).astype(np.uint64)
    return ((hi * np.uint64(bound)) >> np.uint64(32)).astype(np.int64)


# ---------------------------------------------------------------------------------------
# Tensors in the boundary's input formats
# ---------------------------------------------------------------------------------------

def activations(seed: int, m: int, k: int) -> np.ndarray:
    """A ~ N(0, 1), rounded to fp16 (round to nearest even), shape [m][k]."""
    return normal(seed, m * k).astype(np.float16).reshape(m, k)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Inputs for the bf16 path: fp64 draws -> binary32 -> the nearest bf16 (ties to even on
    the binary32 bits), as uint16 bit patterns (numpy has no bf16 type)."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def activations_bf16(seed: int, m: int, k: int) -> np.ndarray:
    """A ~ N(0, 1) as bf16 bit patterns, shape [m][k] (the draws of `activations`)."""
    return bf16_bits(normal(seed, m * k)).reshape(m, k)


def scales_bf16(seed: int, groups: int, n: int, lo: float = 0.005,
                hi: float = 0.02) -> np.ndarray:
    """Group scales ~ U[lo, hi) as bf16 bit patterns: [groups][n] (the draws of `scales`)."""
    return bf16_bits(lo + (hi - lo) * uniform01(seed, groups * n)).reshape(groups, n)


def qweight_words(seed: int, k: int, n: int) -> np.ndarray:
    """Uniform 4-bit codes 0..15 packed GPTQ-style: uint32 [k/8][n]."""
    return words_u32(seed, (k // 8) * n).reshape(k // 8, n)


def scales(seed: int, groups: int, n: int, lo: float = 0.005, hi: float = 0.02) -> np.ndarray:
    """Group scales ~ U[lo, hi) drawn in fp64 and rounded to fp16: [groups][n]."""
    return (lo + (hi - lo) * uniform01(seed, groups * n)).astype(np.float16).reshape(groups, n)


FP8_CODES = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint32)  # no NaN


def fp8_words(seed: int, k: int, n: int) -> np.ndarray:
    """E4M3 weight codes, uniform over the 254 non-NaN bytes, packed K-major four to a
    word (byte i of word (r, n) is row 4r + i): uint32 [k/4][n]."""
    codes = FP8_CODES[below(seed, k * n, FP8_CODES.size)].reshape(k // 4, 4, n)
    words = np.zeros((k // 4, n), dtype=np.uint32)
    for i in range(4):
        words |= codes[:, i, :] << np.uint32(8 * i)
    return words


def zero_point_words(seed: int, groups: int, n: int) -> np.ndarray:
    """Uniform 4-bit zero-point codes 0..15 packed 8 per word: uint32 [groups][n/8]."""
    return words_u32(seed, groups * (n // 8)).reshape(groups, n // 8)


def permutation(seed: int, k: int) -> np.ndarray:
    """Seeded Fisher-Yates shuffle of 0..k-1 (int64)."""
    p = np.arange(k, dtype=np.int64)
    d = draws_u64(seed, k)
    for i in range(k - 1, 0, -1):
        r = int(d[i]) % (i + 1)
        p[i], p[r] = p[r], p[i]
    return p


def act_order_g_idx(seed: int, k: int, group_size: int) -> np.ndarray:
    """act_order group index: g_idx[k] = perm_gen[k] // group_size for a seeded shuffle."""
    return (permutation(seed, k) // group_size).astype(np.int32)


def routing_weights(seed: int, n_tokens: int, top_k: int) -> np.ndarray:
    """Routing weights, pair-major fp32 [n_tokens * top_k]: per token, top_k draws from
    U[0.05, 1) divided by their sum (a renormalised top-k selection)."""
    u = 0.05 + 0.95 * uniform01(seed, n_tokens * top_k).reshape(n_tokens, top_k)
    return (u / u.sum(axis=1, keepdims=True)).astype(np.float32).reshape(-1)


def top2_routes(seed: int, n_tokens: int, n_expert: int) -> np.ndarray:
    """Two distinct experts per token, uniform without replacement, in draw order.

    First choice e1 ~ U{0..E-1}; second e2 ~ U over the other E-1 experts (draw from E-1
    and skip e1).  Returns int32 [n_tokens][2], token-major.
    """
    d = below(seed, 2 * n_tokens, 1 << 30)
    e1 = d[0::2] % n_expert
    e2 = d[1::2] % (n_expert - 1)
    e2 = e2 + (e2 >= e1)
    return np.stack([e1, e2], axis=1).astype(np.int32)


# ---------------------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------------------

CONFIGS = {
    "tiny": dict(m=16, k=1024, n=256, zp=False, act_order=False, fp32_reduce=False),
    "decode": dict(m=1, k=4096, n=14336, zp=False, act_order=False, fp32_reduce=True),
    "batched": dict(m=16, k=4096, n=4096, zp=True, act_order=False, fp32_reduce=True),
    "prefill": dict(m=2048, k=4096, n=14336, zp=False, act_order=True, fp32_reduce=False),
}
MOE_CONFIG = dict(n_tokens=1024, n_expert=8, top_k=2, k=4096, n=14336, zp=False)
CONFIG_INDEX = {"tiny": 0, "decode": 1, "batched": 2, "prefill": 3, "moe": 4}
GROUP_SIZE = 128


def dense_case(m: int, k: int, n: int, *, zp: bool = False, act_order: bool = False,
               group_size: int = GROUP_SIZE, seed: int = ROOT_SEED, bf16: bool = False) -> dict:
    """One dense problem's inputs in the boundary's plain formats (group_size -1: one
    channelwise group; bf16: activations and scales as bf16 bit patterns)."""
    groups = 1 if group_size == -1 else k // group_size
    act, sc = (activations_bf16, scales_bf16) if bf16 else (activations, scales)
    case = dict(
        m=m, k=k, n=n, group_size=group_size, bf16=bf16,
        a=act(stream_seed(seed, TAG_ACT), m, k),
        qweight=qweight_words(stream_seed(seed, TAG_WEIGHT), k, n),
        scales=sc(stream_seed(seed, TAG_SCALE), groups, n),
        zeros=zero_point_words(stream_seed(seed, TAG_ZERO), groups, n) if zp else None,
        g_idx=(act_order_g_idx(stream_seed(seed, TAG_PERM), k,
                               k if group_size == -1 else group_size) if act_order else None),
    )
    return case


def fp8_case(m: int, k: int, n: int, *, group_size: int = GROUP_SIZE, seed: int = ROOT_SEED,
             bf16: bool = False) -> dict:
    """One dense W8A16 problem: A, E4M3 words [k/4][n] and scales (group_size -1 or 128)."""
    groups = 1 if group_size == -1 else k // group_size
    act, sc = (activations_bf16, scales_bf16) if bf16 else (activations, scales)
    return dict(m=m, k=k, n=n, group_size=group_size, bf16=bf16, fp8=True,
                a=act(stream_seed(seed, TAG_ACT), m, k),
                qweight=fp8_words(stream_seed(seed, TAG_WEIGHT), k, n),
                scales=sc(stream_seed(seed, TAG_SCALE), groups, n))


def config_case(name: str, seed: int | None = None) -> dict:
    """Inputs of a named dense workload (tiny, decode, batched, prefill)."""
    cfg = CONFIGS[name]
    root = (ROOT_SEED ^ CONFIG_INDEX[name]) if seed is None else seed
    case = dense_case(cfg["m"], cfg["k"], cfg["n"], zp=cfg["zp"], act_order=cfg["act_order"],
                      seed=root)
    case["fp32_reduce"] = cfg["fp32_reduce"]
    case["name"] = name
    return case


def moe_case(n_tokens: int = 1024, n_expert: int = 8, k: int = 4096, n: int = 14336,
             *, group_size: int = GROUP_SIZE, seed: int | None = None,
             bf16: bool = False) -> dict:
    """Grouped (MoE) problem: A [tokens][k], one weight bank per expert, top-2 routes
    (bf16: activations and scales as bf16 bit patterns)."""
    root = (ROOT_SEED ^ CONFIG_INDEX["moe"]) if seed is None else seed
    groups = k // group_size
    act, sc = (activations_bf16, scales_bf16) if bf16 else (activations, scales)
    experts = []
    for e in range(n_expert):
        experts.append(dict(
            qweight=qweight_words(stream_seed(root, TAG_WEIGHT, e + 1), k, n),
            scales=sc(stream_seed(root, TAG_SCALE, e + 1), groups, n),
        ))
    return dict(
        n_tokens=n_tokens, n_expert=n_expert, top_k=2, k=k, n=n, group_size=group_size,
        bf16=bf16, a=act(stream_seed(root, TAG_ACT), n_tokens, k),
        experts=experts,
        routes=(top2_routes(stream_seed(root, TAG_ROUTE), n_tokens, n_expert) if n_expert > 1
                else np.zeros((n_tokens, 2), dtype=np.int32)),
    )
