"""Python binding of libwq (include/wq.h): same names, argument marshalling only.

Every step of the W4A16 path runs in the HIP kernels of libwq.so; this module converts
tensors (torch device tensors, or raw integer addresses) into pointers, sizes and the
current HIP stream, and turns nonzero statuses into exceptions.  If the library has not
been built, the first call raises: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwq.so")

WQ_ABI_VERSION = 3
WQ_FLAG_ACT_ORDER = 1 << 1
WQ_FLAG_IS_K_FULL = 1 << 2
WQ_FLAG_HAS_ZP = 1 << 3
WQ_FLAG_ATOMIC_ADD = 1 << 4
WQ_FLAG_FP32_REDUCE = 1 << 5
WQ_FLAG_MUL_TOPK_WEIGHTS = 1 << 6
WQ_FLAG_SWIGLU = 1 << 7
WQ_FLAG_BF16 = 1 << 8
WQ_FLAG_FP8 = 1 << 9

WQ_STAGE_ARGS, WQ_STAGE_SHAPE, WQ_STAGE_DEVICE = 1, 2, 3
WQ_STAGE_LAUNCH_CONFIG, WQ_STAGE_FUNC_ATTR, WQ_STAGE_LAUNCH = 4, 5, 6
(WQ_ERR_NULL, WQ_ERR_ALIGN, WQ_ERR_SHAPE, WQ_ERR_FLAGS, WQ_ERR_WORKSPACE, WQ_ERR_ABI,
 WQ_ERR_OVERFLOW, WQ_ERR_CSR, WQ_ERR_ACT_ORDER) = range(1, 10)

EXPORTED = (
    "wq_abi_version", "wq_status_str", "wq_repack_b", "wq_repack_scales", "wq_repack_zeros",
    "wq_act_order_perm", "wq_gemm_workspace_bytes", "wq_gemm", "wq_dequant",
    "wq_csr_from_routes", "wq_grouped_workspace_bytes", "wq_grouped_gemm",
    "wq_stream_read_sink_words", "wq_stream_read", "wq_interleave_gate_up", "wq_repack_fp8",
    "wq_repack_fp8_rows", "wq_fp8_block_scales", "wq_mfma_rate", "wq_gemm_plan",
    "wq_gemm_noalloc",
)
WQ_NOALLOC_SCRATCH_BYTES = 32 << 20

WQ_KERNEL_SMALL_M, WQ_KERNEL_TILE_256, WQ_KERNEL_TILE_128 = 1, 2, 3
KERNEL_NAMES = {WQ_KERNEL_SMALL_M: "small-M (16-column blocks)",
                WQ_KERNEL_TILE_256: "tiled 256 x 256", WQ_KERNEL_TILE_128: "tiled 128 x 256"}


class WQError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"libwq status {status:#x}: {text}")
        self.status = status
        self.stage = status >> 16
        self.code = status & 0xFFFF


class wq_gemm_args(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("struct_size", ctypes.c_uint32),
        ("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("c", ctypes.c_void_p),
        ("b_scales", ctypes.c_void_p), ("zero_points", ctypes.c_void_p),
        ("perm", ctypes.c_void_p), ("group_index", ctypes.c_void_p),
        ("a_tmp", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("m", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
        ("lda", ctypes.c_int32), ("group_size", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("split_k", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class wq_grouped_args(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("struct_size", ctypes.c_uint32),
        ("a", ctypes.c_void_p),
        ("b_bank", ctypes.c_void_p), ("b_stride_bytes", ctypes.c_size_t),
        ("s_bank", ctypes.c_void_p), ("s_stride_bytes", ctypes.c_size_t),
        ("zp_bank", ctypes.c_void_p), ("zp_stride_bytes", ctypes.c_size_t),
        ("ex_ids", ctypes.c_void_p), ("ex_off", ctypes.c_void_p),
        ("ex_pairs", ctypes.c_void_p), ("pair_tok", ctypes.c_void_p),
        ("topk_weights", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("n_expert", ctypes.c_int32), ("n_active", ctypes.c_int32),
        ("n_pairs", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
        ("k", ctypes.c_int32), ("n", ctypes.c_int32), ("group_size", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("reserved", ctypes.c_int32),
    ]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libwq.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        sig = {
            "wq_abi_version": (u32, []),
            "wq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "wq_repack_b": (ctypes.c_int, [vp, vp, vp, i32, i32, vp]),
            "wq_repack_fp8": (ctypes.c_int, [vp, vp, i32, i32, vp]),
            "wq_repack_fp8_rows": (ctypes.c_int, [vp, vp, i32, i32, vp]),
            "wq_fp8_block_scales": (ctypes.c_int, [vp, vp, i32, i32, vp]),
            "wq_repack_scales": (ctypes.c_int, [vp, vp, i32, i32, i32, vp]),
            "wq_repack_zeros": (ctypes.c_int, [vp, vp, i32, i32, i32, vp]),
            "wq_act_order_perm": (ctypes.c_int, [vp, i32, i32, vp, vp]),
            "wq_gemm_workspace_bytes": (ctypes.c_int, [i32, i32, i32, u32, ctypes.POINTER(sz)]),
            "wq_gemm": (ctypes.c_int, [ctypes.POINTER(wq_gemm_args)]),
            "wq_gemm_noalloc": (ctypes.c_int, [ctypes.POINTER(wq_gemm_args)]),
            "wq_gemm_plan": (ctypes.c_int, [i32, i32, i32, i32, u32, i32, ctypes.POINTER(i32),
                                            ctypes.POINTER(i32)]),
            "wq_dequant": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, u32, vp, vp]),
            "wq_csr_from_routes": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp,
                                                  ctypes.POINTER(i32)]),
            "wq_grouped_workspace_bytes": (ctypes.c_int, [i32, i32, i32, i32, u32,
                                                          ctypes.POINTER(sz)]),
            "wq_grouped_gemm": (ctypes.c_int, [ctypes.POINTER(wq_grouped_args)]),
            "wq_stream_read_sink_words": (ctypes.c_int, [sz, ctypes.POINTER(sz)]),
            "wq_stream_read": (ctypes.c_int, [vp, sz, vp, sz, vp]),
            "wq_mfma_rate": (ctypes.c_int, [vp, i32, vp, sz, ctypes.POINTER(ctypes.c_double),
                                            vp]),
            "wq_interleave_gate_up": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _ptr(x) -> int | None:
    """Address of a tensor / numpy array / integer (None stays None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream, *tensors) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if t is not None and not isinstance(t, (int, np.ndarray)) and t.is_cuda:
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status: int) -> None:
    if status != 0:
        raise WQError(status, wq_status_str(status))


def wq_abi_version() -> int:
    return int(lib().wq_abi_version())


def wq_status_str(status: int) -> str:
    return lib().wq_status_str(int(status)).decode()


def wq_repack_b(qweight, b_out, k: int, n: int, perm=None, stream=None) -> None:
    _check(lib().wq_repack_b(_ptr(qweight), _ptr(perm), _ptr(b_out), k, n,
                             _stream(stream, b_out)))


def wq_repack_fp8(words, b_out, k: int, n: int, stream=None) -> None:
    """E4M3 words [k/4][n] (K-major, four bytes per word) -> the FP8 library layout."""
    _check(lib().wq_repack_fp8(_ptr(words), _ptr(b_out), k, n, _stream(stream, b_out)))


def wq_repack_fp8_rows(w_nk, b_out, k: int, n: int, stream=None) -> None:
    """Block-FP8 checkpoint weights, E4M3 bytes [n][k], -> the FP8 library layout."""
    _check(lib().wq_repack_fp8_rows(_ptr(w_nk), _ptr(b_out), k, n, _stream(stream, b_out)))


def wq_fp8_block_scales(inv_scales, s_out, k: int, n: int, stream=None) -> None:
    """Block-FP8 bf16 inverse scales [n/128][k/128] -> fp16 scales in the library layout."""
    _check(lib().wq_fp8_block_scales(_ptr(inv_scales), _ptr(s_out), k, n,
                                     _stream(stream, s_out)))


def wq_repack_scales(scales, s_out, k: int, n: int, group_size: int = 128, stream=None) -> None:
    _check(lib().wq_repack_scales(_ptr(scales), _ptr(s_out), k, n, group_size,
                                  _stream(stream, s_out)))


def wq_repack_zeros(zeros, z_out, k: int, n: int, group_size: int = 128, stream=None) -> None:
    _check(lib().wq_repack_zeros(_ptr(zeros), _ptr(z_out), k, n, group_size,
                                 _stream(stream, z_out)))


def wq_act_order_perm(g_idx, group_size: int = 128) -> tuple[np.ndarray, np.ndarray]:
    g = np.ascontiguousarray(np.asarray(g_idx, dtype=np.int32))
    perm = np.empty_like(g)
    sorted_g = np.empty_like(g)
    _check(lib().wq_act_order_perm(g.ctypes.data, g.size, group_size, perm.ctypes.data,
                                   sorted_g.ctypes.data))
    return perm, sorted_g


def wq_gemm_workspace_bytes(m: int, n: int, k: int, flags: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().wq_gemm_workspace_bytes(m, n, k, flags, ctypes.byref(out)))
    return int(out.value)


def wq_gemm(a, b, c, b_scales, *, m: int, n: int, k: int, zero_points=None, perm=None,
            group_index=None, a_tmp=None, workspace=None, workspace_bytes: int | None = None, flags: int = 0,
            split_k: int = 0, lda: int | None = None, group_size: int = 128,
            stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else (
            workspace.numel() * workspace.element_size())
    args = wq_gemm_args(
        abi_version=WQ_ABI_VERSION, struct_size=ctypes.sizeof(wq_gemm_args),
        a=_ptr(a), b=_ptr(b), c=_ptr(c), b_scales=_ptr(b_scales),
        zero_points=_ptr(zero_points), perm=_ptr(perm), group_index=_ptr(group_index),
        a_tmp=_ptr(a_tmp),
        workspace=_ptr(workspace), workspace_bytes=workspace_bytes,
        stream=_stream(stream, c), m=m, n=n, k=k, lda=k if lda is None else lda,
        group_size=group_size, flags=flags, split_k=split_k, reserved=0)
    _check(lib().wq_gemm(ctypes.byref(args)))


def wq_gemm_noalloc(a, b, c, b_scales, *, m: int, n: int, k: int, zero_points=None,
                    perm=None, group_index=None, flags: int = 0, split_k: int = 0,
                    lda: int | None = None, group_size: int = 128, stream=None) -> None:
    """wq_gemm with the library's own static scratch (no workspace or a_tmp argument)."""
    args = wq_gemm_args(
        abi_version=WQ_ABI_VERSION, struct_size=ctypes.sizeof(wq_gemm_args),
        a=_ptr(a), b=_ptr(b), c=_ptr(c), b_scales=_ptr(b_scales),
        zero_points=_ptr(zero_points), perm=_ptr(perm), group_index=_ptr(group_index),
        a_tmp=None, workspace=None, workspace_bytes=0,
        stream=_stream(stream, c), m=m, n=n, k=k, lda=k if lda is None else lda,
        group_size=group_size, flags=flags, split_k=split_k, reserved=0)
    _check(lib().wq_gemm_noalloc(ctypes.byref(args)))


def wq_gemm_plan(m: int, n: int, k: int, *, group_size: int = 128, flags: int = 0,
                 split_k: int = 0) -> tuple[int, int]:
    """(kernel, splits) the library picks for this problem (see include/wq.h)."""
    kernel, splits = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().wq_gemm_plan(m, n, k, group_size, flags, split_k, ctypes.byref(kernel),
                              ctypes.byref(splits)))
    return int(kernel.value), int(splits.value)


def wq_dequant(b, b_scales, zero_points, w_out, *, k: int, n: int, flags: int = 0,
               group_size: int = 128, stream=None) -> None:
    _check(lib().wq_dequant(_ptr(b), _ptr(b_scales), _ptr(zero_points), k, n, group_size,
                            flags, _ptr(w_out), _stream(stream, w_out)))


def wq_csr_from_routes(selected, n_tokens: int, top_k: int, n_expert: int) -> dict:
    sel = np.ascontiguousarray(np.asarray(selected, dtype=np.int32).reshape(-1))
    n_pairs = n_tokens * top_k
    if sel.size != n_pairs:
        raise WQError((WQ_STAGE_ARGS << 16) | WQ_ERR_CSR, "route count != tokens x top_k")
    ex_ids = np.zeros(n_expert, np.int32)
    ex_off = np.zeros(n_expert + 1, np.int32)
    ex_pairs = np.zeros(n_pairs, np.int32)
    pair_tok = np.zeros(n_pairs, np.int32)
    active = ctypes.c_int32(0)
    _check(lib().wq_csr_from_routes(sel.ctypes.data, n_tokens, top_k, n_expert,
                                    ex_ids.ctypes.data, ex_off.ctypes.data,
                                    ex_pairs.ctypes.data, pair_tok.ctypes.data,
                                    ctypes.byref(active)))
    na = int(active.value)
    return dict(ex_ids=ex_ids[:na], ex_off=ex_off[:na + 1], ex_pairs=ex_pairs,
                pair_tok=pair_tok, n_active=na, n_pairs=n_pairs, n_tokens=n_tokens,
                n_expert=n_expert)


def wq_grouped_workspace_bytes(n_pairs: int, n_active: int, n: int, k: int,
                               flags: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().wq_grouped_workspace_bytes(n_pairs, n_active, n, k, flags, ctypes.byref(out)))
    return int(out.value)


def wq_grouped_gemm(a, b_bank, b_stride_bytes: int, s_bank, s_stride_bytes: int, ex_ids,
                    ex_off, ex_pairs, pair_tok, y, *, n_expert: int, n_active: int,
                    n_pairs: int, n_tokens: int, k: int, n: int, zp_bank=None,
                    zp_stride_bytes: int = 0, topk_weights=None, flags: int = 0,
                    workspace=None, workspace_bytes: int = 0, group_size: int = 128,
                    stream=None) -> None:
    args = wq_grouped_args(
        abi_version=WQ_ABI_VERSION, struct_size=ctypes.sizeof(wq_grouped_args),
        a=_ptr(a), b_bank=_ptr(b_bank), b_stride_bytes=b_stride_bytes, s_bank=_ptr(s_bank),
        s_stride_bytes=s_stride_bytes, zp_bank=_ptr(zp_bank), zp_stride_bytes=zp_stride_bytes,
        ex_ids=_ptr(ex_ids), ex_off=_ptr(ex_off), ex_pairs=_ptr(ex_pairs),
        pair_tok=_ptr(pair_tok), topk_weights=_ptr(topk_weights), y=_ptr(y),
        workspace=_ptr(workspace),
        workspace_bytes=workspace_bytes, stream=_stream(stream, y), n_expert=n_expert,
        n_active=n_active, n_pairs=n_pairs, n_tokens=n_tokens, k=k, n=n,
        group_size=group_size, flags=flags, reserved=0)
    _check(lib().wq_grouped_gemm(ctypes.byref(args)))


def wq_stream_read_sink_words(nbytes: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().wq_stream_read_sink_words(nbytes, ctypes.byref(out)))
    return out.value


def wq_stream_read(src, nbytes: int, sink, sink_words: int, stream=None) -> None:
    """Measurement helper: one streaming read of `nbytes` at `src` (see include/wq.h)."""
    _check(lib().wq_stream_read(_ptr(src), nbytes, _ptr(sink), sink_words,
                                _stream(stream, src)))


def wq_mfma_rate(operands, iters: int, sink, sink_floats: int, stream=None) -> float:
    """Measurement helper: one register-only MFMA loop launch (see include/wq.h); returns
    the launch's floating-point operation count."""
    flops = ctypes.c_double(0.0)
    _check(lib().wq_mfma_rate(_ptr(operands), iters, _ptr(sink), sink_floats,
                              ctypes.byref(flops), _stream(stream, sink)))
    return float(flops.value)


def wq_interleave_gate_up(gate, up, out, rows: int, cols: int, bits_per_column: int,
                          stream=None) -> None:
    """Pair gate/up columns in 16-column blocks for WQ_FLAG_SWIGLU (see include/wq.h)."""
    _check(lib().wq_interleave_gate_up(_ptr(gate), _ptr(up), _ptr(out), rows, cols,
                                       bits_per_column, _stream(stream, out)))
