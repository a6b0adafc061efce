"""Reference construction of the library's weight layout (test infrastructure only).

The pages fix only that the repack is a pure permutation of the 4-bit codes into the
kernel's own tile order, with the same byte count, and that act_order stores weight rows
in the permuted order (vllm_marlin.rs, `ferrum_vllm_gptq_marlin_repack` doc; marlin.rs,
`MarlinWeight.perm` doc).  The order itself is this library's design; it is stated here
as nested loops (the slow, checkable form) so that the GPU repack kernel, which uses a
direct index formula, can be compared against it bit for bit.

Layout of repacked B (uint32 words, K*N/8 of them), with G = K/128:
  for each 16-column block nb (columns n = 16*nb + c), each 128-row chunk g, each lane
  l = c + 16*q (q = 0..3) and each dword j = 0..3, word ((nb*G + g)*64 + l)*4 + j holds
  the codes of rows k = 128*g + 32*j + 8*q + i (i = 0..7) of column n; the code of row
  offset i sits in nibble slot SLOT[i] (bits 4*SLOT[i]..+3), SLOT = [0, 4, 1, 5, 2, 6, 3, 7],
  i.e. even offsets in the low half-word and odd offsets in the high half-word.
  With act_order, row position k of the repacked matrix is original row perm[k].

Layout of repacked scales (fp16): [N/16][G][16], element (nb, g, c) = s[g][16*nb + c].
Layout of repacked zero points (uint32): [N/16][G][2], word (nb, g, h) = zeros[g][2*nb + h]
  (column 16*nb + 8*h + i in bits 4*i).
"""

from __future__ import annotations

import numpy as np

from .reference import unpack_qweight

SLOT = (0, 4, 1, 5, 2, 6, 3, 7)
CHUNK = 128  # rows of K per layout chunk (and per stored scale row)


def repack_b_loops(codes: np.ndarray, perm=None) -> np.ndarray:
    """Nested-loop construction from codes uint8 [K][N] (small shapes only)."""
    k_total, n_total = codes.shape
    groups = k_total // 128
    out = np.zeros(k_total * n_total // 8, dtype=np.uint32)
    for nb in range(n_total // 16):
        for g in range(groups):
            for lane in range(64):
                c, q = lane % 16, lane // 16
                for j in range(4):
                    word = 0
                    for i in range(8):
                        k = 128 * g + 32 * j + 8 * q + i
                        src = int(perm[k]) if perm is not None else k
                        word |= int(codes[src, 16 * nb + c]) << (4 * SLOT[i])
                    out[((nb * groups + g) * 64 + lane) * 4 + j] = word
    return out


def repack_b(qweight: np.ndarray, perm=None) -> np.ndarray:
    """Same layout as `repack_b_loops`, built with array reshapes (any size)."""
    codes = unpack_qweight(qweight)
    if perm is not None:
        codes = codes[np.asarray(perm, dtype=np.int64), :]
    k_total, n_total = codes.shape
    groups = k_total // 128
    # k = 128*g + 32*j + 8*q + i ; n = 16*nb + c
    t = codes.reshape(groups, 4, 4, 8, n_total // 16, 16)          # g, j, q, i, nb, c
    t = t.transpose(4, 0, 2, 5, 1, 3).astype(np.uint32)            # nb, g, q, c, j, i
    word = np.zeros(t.shape[:-1], dtype=np.uint32)
    for i in range(8):
        word |= t[..., i] << np.uint32(4 * SLOT[i])
    return word.reshape(-1)


def unrepack_b(words: np.ndarray, k_total: int, n_total: int) -> np.ndarray:
    """Inverse of `repack_b`: codes uint8 [K][N] in the repacked row order."""
    groups = k_total // 128
    w = np.asarray(words, dtype=np.uint32).reshape(n_total // 16, groups, 4, 16, 4)
    codes = np.empty((n_total // 16, groups, 4, 16, 4, 8), dtype=np.uint8)
    for i in range(8):
        codes[..., i] = (w >> np.uint32(4 * SLOT[i])) & np.uint32(0xF)
    # nb, g, q, c, j, i -> g, j, q, i, nb, c
    return codes.transpose(1, 4, 2, 5, 0, 3).reshape(k_total, n_total)


def repack_fp8_loops(codes: np.ndarray) -> np.ndarray:
    """Library layout of E4M3 weights from codes uint8 [K][N] (nested loops, small shapes).

    Per 16-column block nb, 128-row group g and half h (rows 64h..64h+63 of the group), each
    lane l = c + 16*qd (column 16*nb + c) holds four words; word d covers rows
    128g + 32(2h + d//2) + 8qd + 4(d%2) + i in byte i.  The lane's eight rows of each 32-row
    step are thus two words, the B operand of one 16x16x32 MFMA after conversion.
    Flat word index: (((nb * G + g) * 2 + h) * 64 + l) * 4 + d.
    """
    k_total, n_total = codes.shape
    groups = k_total // 128
    out = np.zeros(k_total * n_total // 4, dtype=np.uint32)
    for nb in range(n_total // 16):
        for g in range(groups):
            for h in range(2):
                for lane in range(64):
                    c, qd = lane % 16, lane // 16
                    for d in range(4):
                        word = 0
                        for i in range(4):
                            row = 128 * g + 32 * (2 * h + d // 2) + 8 * qd + 4 * (d % 2) + i
                            word |= int(codes[row, 16 * nb + c]) << (8 * i)
                        out[(((nb * groups + g) * 2 + h) * 64 + lane) * 4 + d] = word
    return out


def unrepack_fp8(words: np.ndarray, k_total: int, n_total: int) -> np.ndarray:
    """Inverse of repack_fp8_loops (vectorized): library words -> codes uint8 [K][N]."""
    groups = k_total // 128
    w = np.asarray(words, dtype=np.uint32).reshape(n_total // 16, groups, 2, 4, 16, 2, 2)
    # axes: nb, g, h, qd, c, jj (= d // 2), half (= d % 2)
    out = np.empty((k_total, n_total), dtype=np.uint8)
    for i in range(4):
        b = ((w >> np.uint32(8 * i)) & np.uint32(0xFF)).astype(np.uint8)
        # row = 128g + 64h + 32jj + 8qd + 4half + i; column = 16nb + c
        t = b.transpose(1, 2, 5, 3, 6, 0, 4)  # g, h, jj, qd, half, nb, c
        out[i::4, :] = t.reshape(k_total // 4, n_total)
    return out


def interleave_gate_up(gate: np.ndarray, up: np.ndarray, cols_per_elem: int = 1) -> np.ndarray:
    """Pair the columns of two row-major tensors in 16-column blocks: out column block 2t is
    block t of `gate`, block 2t+1 block t of `up` (a fused gate/up projection's weights).
    `cols_per_elem` columns share one element (8 for packed 4-bit zero points)."""
    g = np.asarray(gate)
    u = np.asarray(up)
    per = 16 // cols_per_elem  # elements per 16-column block
    rows, cols = g.shape
    out = np.empty((rows, 2 * cols), dtype=g.dtype)
    for t in range(cols // per):
        out[:, 2 * t * per:(2 * t + 1) * per] = g[:, t * per:(t + 1) * per]
        out[:, (2 * t + 1) * per:(2 * t + 2) * per] = u[:, t * per:(t + 1) * per]
    return out


def unit_rows(group_size: int) -> int:
    """Rows of K per stored scale / zero-point row: the largest power of two dividing both
    the group size and the 128-row chunk (16, 32, 64 or 128; 128 when channelwise), so that
    every unit lies inside one group and one chunk."""
    if group_size == -1:
        return CHUNK
    unit = CHUNK
    while group_size % unit:
        unit //= 2
    return unit


def chunk_rows(values: np.ndarray, k: int | None, group_size: int) -> np.ndarray:
    """Per-group rows [K/group_size][...] -> the library's stored rows, one per unit of
    unit_rows(group_size) rows of K: unit u takes the row of the group holding its rows
    (the single row when channelwise)."""
    v = np.asarray(values)
    unit = unit_rows(group_size)
    if k is None:
        if unit != group_size:
            raise ValueError(f"group size {group_size} needs k to lay out its units")
        return v  # one stored row per group
    first_row = np.arange(k // unit, dtype=np.int64) * unit
    src = np.zeros(k // unit, dtype=np.int64) if group_size == -1 else first_row // group_size
    return v[src]


def repack_scales(scales: np.ndarray, k: int | None = None, group_size: int = 128) -> np.ndarray:
    """fp16 [K/group_size][N] -> fp16 [N/16][K/U][16] (flattened), U = unit_rows(group_size)."""
    s = chunk_rows(np.asarray(scales, dtype=np.float16), k, group_size)
    groups, n_total = s.shape
    return s.reshape(groups, n_total // 16, 16).transpose(1, 0, 2).reshape(-1).copy()


def repack_zero_points(zeros: np.ndarray, k: int | None = None,
                       group_size: int = 128) -> np.ndarray:
    """uint32 [K/group_size][N/8] -> uint32 [N/16][K/U][2] (flattened)."""
    z = chunk_rows(np.asarray(zeros, dtype=np.uint32), k, group_size)
    groups, n8 = z.shape
    return z.reshape(groups, n8 // 2, 2).transpose(1, 0, 2).reshape(-1).copy()
