"""Device-memory plumbing around libwq with PyTorch tensors.

PyTorch only allocates device buffers and supplies the stream; every operation on the
data (repack, gather, GEMM, reduce) is a libwq kernel called through the binding.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from . import (WQ_FLAG_ACT_ORDER, WQ_FLAG_BF16, WQ_FLAG_FP8, WQ_FLAG_FP32_REDUCE,
               WQ_FLAG_HAS_ZP, WQ_FLAG_MUL_TOPK_WEIGHTS, WQ_FLAG_SWIGLU, wq_act_order_perm,
               wq_fp8_block_scales, wq_repack_fp8, wq_repack_fp8_rows, wq_interleave_gate_up,
               wq_gemm, wq_gemm_workspace_bytes, wq_grouped_gemm, wq_repack_b,
               wq_repack_scales, wq_repack_zeros)

GROUP = 128


def to_device(x: np.ndarray, device) -> torch.Tensor:
    """Upload a numpy array (a tensor is moved as it is); uint32 words travel as int32 and
    uint16 arrays, which hold bf16 bit patterns (numpy has no bf16), arrive as bfloat16."""
    if isinstance(x, torch.Tensor):
        return x.to(device)
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint32:
        x = x.view(np.int32)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def act_dtype(bf16: bool) -> torch.dtype:
    """Element type of activations, scales and outputs."""
    return torch.bfloat16 if bf16 else torch.float16


class PackedWeight:
    """One weight matrix in the library layout (B, scales, optional zero points, perm).
    bf16: the scales (numpy uint16 bit patterns or a bfloat16 tensor) and the activations
    and outputs of its products are bf16.  fp8: qweight holds E4M3 words [K/4][N] (four
    K-consecutive bytes per word), repacked with wq_repack_fp8."""

    def __init__(self, qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray | None = None,
                 g_idx: np.ndarray | None = None, device="cuda", group_size: int = GROUP,
                 bf16: bool = False, fp8: bool = False):
        self.k = qweight.shape[0] * (4 if fp8 else 8)
        self.n = qweight.shape[1]
        self.group_size = group_size
        self.bf16 = bf16
        self.fp8 = fp8
        self.swiglu = False
        self.device = torch.device(device)
        self.perm = None
        self.group_index = None  # sorted per-position groups, checked by every act_order call
        if g_idx is not None:
            perm, sorted_g = wq_act_order_perm(g_idx, group_size)
            self.perm = to_device(perm, self.device)
            self.group_index = to_device(sorted_g, self.device)
        qw = to_device(qweight, self.device)
        if fp8:
            self.b = torch.empty(self.k * self.n // 4, dtype=torch.int32, device=self.device)
            wq_repack_fp8(qw, self.b, self.k, self.n)
        else:
            self.b = torch.empty(self.k * self.n // 8, dtype=torch.int32, device=self.device)
            wq_repack_b(qw, self.b, self.k, self.n, perm=self.perm)
        sc = to_device(scales if isinstance(scales, torch.Tensor)
                       else np.asarray(scales, dtype=np.uint16 if bf16 else np.float16),
                       self.device)
        unit = math.gcd(group_size, GROUP) if group_size > 0 else GROUP  # rows per scale row
        self.s = torch.empty((self.k // unit) * self.n, dtype=act_dtype(bf16), device=self.device)
        wq_repack_scales(sc, self.s, self.k, self.n, group_size)
        self.z = None
        if zeros is not None:
            zw = to_device(zeros, self.device)
            self.z = torch.empty((self.k // unit) * self.n // 8, dtype=torch.int32,
                                 device=self.device)
            wq_repack_zeros(zw, self.z, self.k, self.n, group_size)
        torch.cuda.synchronize(self.device)

    @classmethod
    def gate_up(cls, gate: dict, up: dict, device="cuda", group_size: int = GROUP,
                g_idx: np.ndarray | None = None, bf16: bool = False,
                fp8: bool = False) -> "PackedWeight":
        """One weight of 2*I columns for the SwiGLU epilogue: the gate and up projections'
        qweight, scales and zero points paired in 16-column blocks on the device
        (wq_interleave_gate_up), then repacked like any weight."""
        dev = torch.device(device)
        i = gate["qweight"].shape[1]

        def pair(key, bits):
            g, u = to_device(gate[key], dev), to_device(up[key], dev)
            out = torch.empty((g.shape[0], 2 * g.shape[1]), dtype=g.dtype, device=dev)
            wq_interleave_gate_up(g, u, out, g.shape[0], i, bits)
            return out

        zeros = pair("zeros", 4) if gate.get("zeros") is not None else None
        w = cls(pair("qweight", 32), pair("scales", 16), zeros, g_idx, device=dev,
                group_size=group_size, bf16=bf16, fp8=fp8)
        w.swiglu = True
        return w

    @classmethod
    def from_fp8_blocks(cls, w_nk: np.ndarray, inv_scales: np.ndarray,
                        device="cuda") -> "PackedWeight":
        """A block-FP8 checkpoint weight: E4M3 bytes row-major [N][K] and bf16 inverse scales
        [N/128][K/128] (numpy uint16 bit patterns), converted on the device."""
        dev = torch.device(device)
        n, k = w_nk.shape
        w = object.__new__(cls)
        w.k, w.n, w.group_size, w.bf16, w.fp8, w.swiglu = k, n, GROUP, False, True, False
        w.device, w.perm, w.group_index, w.z = dev, None, None, None
        src = torch.from_numpy(np.ascontiguousarray(w_nk, dtype=np.uint8)).to(dev)
        w.b = torch.empty(k * n // 4, dtype=torch.int32, device=dev)
        wq_repack_fp8_rows(src, w.b, k, n)
        inv = to_device(np.ascontiguousarray(inv_scales, dtype=np.uint16), dev)
        w.s = torch.empty((k // GROUP) * n, dtype=torch.float16, device=dev)
        wq_fp8_block_scales(inv, w.s, k, n)
        torch.cuda.synchronize(dev)
        return w

    def clone(self) -> "PackedWeight":
        """A second copy of the device buffers (same values, new memory)."""
        other = object.__new__(PackedWeight)
        other.__dict__.update(self.__dict__)
        other.b = self.b.clone()
        other.s = self.s.clone()
        other.z = None if self.z is None else self.z.clone()
        return other

    def flags(self, fp32_reduce: bool = False) -> int:
        f = 0
        if self.z is not None:
            f |= WQ_FLAG_HAS_ZP
        if self.perm is not None:
            f |= WQ_FLAG_ACT_ORDER
        if fp32_reduce:
            f |= WQ_FLAG_FP32_REDUCE
        if self.swiglu:
            f |= WQ_FLAG_SWIGLU
        if self.bf16:
            f |= WQ_FLAG_BF16
        if self.fp8:
            f |= WQ_FLAG_FP8
        return f


class GemmBuffers:
    """Scratch a call needs: the act_order gather buffer and the split-K workspace."""

    def __init__(self, w: PackedWeight, m: int, fp32_reduce: bool):
        self.flags = w.flags(fp32_reduce)
        self.a_tmp = (torch.empty((m, w.k), dtype=act_dtype(w.bf16), device=w.device)
                      if w.perm is not None else None)
        nbytes = wq_gemm_workspace_bytes(m, w.n, w.k, self.flags)
        self.workspace = (torch.zeros(nbytes, dtype=torch.uint8, device=w.device)
                          if nbytes else None)


def gemm(a: torch.Tensor, w: PackedWeight, out: torch.Tensor | None = None, *,
         fp32_reduce: bool = False, split_k: int = 0, buffers: GemmBuffers | None = None,
         stream=None) -> torch.Tensor:
    """C = A @ dequant(B) through wq_gemm (A fp16 [m][k], row stride a.stride(0)); for a
    gate/up weight, the [m][n/2] SwiGLU activation."""
    m = a.shape[0]
    if a.dtype != act_dtype(w.bf16):
        raise TypeError(f"activations are {a.dtype}, the weight expects {act_dtype(w.bf16)}")
    if out is None:
        cols = w.n // 2 if w.swiglu else w.n
        out = torch.empty((m, cols), dtype=act_dtype(w.bf16), device=a.device)
    if buffers is None:
        buffers = GemmBuffers(w, m, fp32_reduce)
    wq_gemm(a, w.b, out, w.s, m=m, n=w.n, k=w.k, zero_points=w.z, perm=w.perm,
            group_index=w.group_index, a_tmp=buffers.a_tmp, workspace=buffers.workspace, flags=buffers.flags,
            split_k=split_k, lda=a.stride(0), group_size=w.group_size, stream=stream)
    return out


class ExpertBank:
    """Repacked weights of several experts stored back to back (one stride per tensor)."""

    def __init__(self, experts: list[dict], device="cuda", bf16: bool = False,
                 fp8: bool = False):
        """Each expert is a weight dict (qweight, scales, optional zeros and group_size), or
        {"gate": ..., "up": ...} for a fused gate/up projection with the SwiGLU epilogue."""
        def pack(e):
            gs = e.get("group_size", GROUP)
            if "gate" in e:
                return PackedWeight.gate_up(e["gate"], e["up"], device=device, group_size=gs,
                                            bf16=bf16, fp8=fp8)
            return PackedWeight(e["qweight"], e["scales"], e.get("zeros"), device=device,
                                group_size=gs, bf16=bf16, fp8=fp8)
        self.packed = [pack(e) for e in experts]
        p0 = self.packed[0]
        self.k, self.n, self.group_size, self.swiglu = p0.k, p0.n, p0.group_size, p0.swiglu
        self.bf16 = bf16
        self.fp8 = fp8
        self.b = torch.stack([p.b for p in self.packed])
        self.s = torch.stack([p.s for p in self.packed])
        self.z = torch.stack([p.z for p in self.packed]) if p0.z is not None else None
        self.packed = None  # the stacked copies are the bank
        self.b_stride = self.b.stride(0) * self.b.element_size()
        self.s_stride = self.s.stride(0) * self.s.element_size()
        self.z_stride = 0 if self.z is None else self.z.stride(0) * self.z.element_size()
        self.n_expert = self.b.shape[0]


def grouped_gemm(a: torch.Tensor, bank: ExpertBank, csr: dict, out: torch.Tensor | None = None,
                 device_csr: dict | None = None, topk_weights: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Pair-major y = grouped product over an expert-major CSR (host dict from the library),
    each row times its fp32 routing weight when `topk_weights` [n_pairs] is given."""
    if device_csr is None:
        device_csr = {key: to_device(np.asarray(csr[key], dtype=np.int32), a.device)
                      for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok")}
    n_pairs = len(csr["ex_pairs"])
    if out is None:
        cols = bank.n // 2 if bank.swiglu else bank.n
        out = torch.empty((n_pairs, cols), dtype=act_dtype(bank.bf16), device=a.device)
    wq_grouped_gemm(a, bank.b, bank.b_stride, bank.s, bank.s_stride, device_csr["ex_ids"],
                    device_csr["ex_off"], device_csr["ex_pairs"], device_csr["pair_tok"], out,
                    n_expert=bank.n_expert, n_active=len(csr["ex_ids"]), n_pairs=n_pairs,
                    n_tokens=a.shape[0], k=bank.k, n=bank.n, zp_bank=bank.z,
                    zp_stride_bytes=bank.z_stride, topk_weights=topk_weights,
                    group_size=bank.group_size,
                    flags=(WQ_FLAG_HAS_ZP if bank.z is not None else 0)
                    | (WQ_FLAG_MUL_TOPK_WEIGHTS if topk_weights is not None else 0)
                    | (WQ_FLAG_SWIGLU if bank.swiglu else 0)
                    | (WQ_FLAG_BF16 if bank.bf16 else 0)
                    | (WQ_FLAG_FP8 if bank.fp8 else 0),
                    stream=stream)
    return out
