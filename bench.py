"""Benchmark of the W4A16 GEMM on one MI355X; prints one JSON line.

Headline (value): packed-weight TB/s of the decode GEMM, M=1 K=4096 N=14336, u4b8, group
128, with the fp32-reduce flag set (the planner keeps K unsplit at this shape; the line's
workload text says what runs).  Each step is one wq_gemm call; steps rotate over enough
weight copies that the weights stream from HBM rather than from the 256 MB Infinity Cache.
The same line carries the prefill (M=2048, act_order) TFLOP/s with its MFMA roofline, the
batched-decode, tiny and grouped-MoE figures, the measured HBM-read and MFMA ceilings, and
the oracle timed on the host cores for every workload as the CPU baseline; `extended` adds
other group sizes, bf16, E4M3, SwiGLU, MoE variants, split-K batches and down projections.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weight TB/s at M=1 + TFLOP/s at M=2048 W4A16 g128; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published


TIMED_LOOPS = 5  # timed replays of each captured loop; the median is reported


def timed_loop(torch, fn, steps: int, warmup: int) -> float:
    """Seconds per step: the median over TIMED_LOOPS timed loops of `steps` calls, after
    `warmup` eager calls.

    The timed calls are captured once into a HIP graph and replayed, so that host-side
    launch overhead (Python, ctypes) does not hide the kernels' own time; each replay is
    bracketed by HIP events on the stream the kernels run on.
    """
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(warmup):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            fn(i)
    graph.replay()                      # one untimed replay
    torch.cuda.synchronize()
    times = []
    for _ in range(TIMED_LOOPS):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        graph.replay()
        stop.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(stop) / 1e3 / steps)
    return sorted(times)[len(times) // 2]


def dense_setup(torch, torch_ops, name: str, copies: int):
    import synthetic
    case = synthetic.config_case(name)
    w0 = torch_ops.PackedWeight(case["qweight"], case["scales"], case["zeros"], case["g_idx"],
                                device="cuda")
    weights = [w0] + [w0.clone() for _ in range(copies - 1)]
    a = torch_ops.to_device(case["a"], "cuda")
    out = torch.empty((case["m"], case["n"]), dtype=torch.float16, device="cuda")
    bufs = torch_ops.GemmBuffers(w0, case["m"], case["fp32_reduce"])
    torch.cuda.synchronize()
    return case, weights, a, out, bufs


def algorithmic_bytes(case) -> int:
    m, k, n = case["m"], case["k"], case["n"]
    b = k * n // 2 + (k // 128) * n * 2 + m * k * 2 + m * n * 2
    if case["zeros"] is not None:
        b += (k // 128) * n // 2
    return b


def bench_dense(torch, torch_ops, name, copies, steps, warmup):
    case, weights, a, out, bufs = dense_setup(torch, torch_ops, name, copies)
    fp32 = case["fp32_reduce"]

    def step(i):
        torch_ops.gemm(a, weights[i % len(weights)], out, fp32_reduce=fp32, buffers=bufs)

    sec = timed_loop(torch, step, steps, warmup)
    m, k, n = case["m"], case["k"], case["n"]
    return dict(case=case, sec=sec, weight_bytes=k * n // 2, alg_bytes=algorithmic_bytes(case),
                flops=2.0 * m * n * k, weights=weights)


def bench_stream_read(torch, weights, steps, warmup):
    """Practical HBM read ceiling: the library's plain streaming read (wq_stream_read)
    over the same rotating packed-weight buffers the GEMM reads, timed the same way."""
    import weight_only_quantized_gemm_amd as wq
    nbytes = weights[0].b.numel() * 4
    words = wq.wq_stream_read_sink_words(nbytes)
    sink = torch.zeros(words, dtype=torch.int32, device="cuda")

    def step(i):
        wq.wq_stream_read(weights[i % len(weights)].b, nbytes, sink, words)

    sec = timed_loop(torch, step, steps, warmup)
    return dict(sec=sec, bytes=nbytes)


def bench_moe(torch, torch_ops, steps, warmup):
    import synthetic
    import weight_only_quantized_gemm_amd as wq
    moe = synthetic.moe_case()
    bank = torch_ops.ExpertBank(moe["experts"], device="cuda")
    csr = wq.wq_csr_from_routes(moe["routes"], moe["n_tokens"], moe["top_k"], moe["n_expert"])
    dcsr = {key: torch_ops.to_device(np.asarray(csr[key], np.int32), "cuda")
            for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok")}
    a = torch_ops.to_device(moe["a"], "cuda")
    y = torch.empty((csr["n_pairs"], moe["n"]), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        torch_ops.grouped_gemm(a, bank, csr, y, device_csr=dcsr)

    sec = timed_loop(torch, step, steps, warmup)
    flops = 2.0 * csr["n_pairs"] * moe["n"] * moe["k"]
    return dict(sec=sec, flops=flops, weight_bytes=moe["n_expert"] * moe["k"] * moe["n"] // 2)


def bench_extended(torch, torch_ops, steps, warmup):
    """Timings of the widened features on the same workload shapes (one object per row):
    the SwiGLU gate/up projection with its fused activation at decode (M=1) and prefill
    (M=2048) shape, other scale-group sizes, bf16 activations, E4M3 weights, mid-size
    batches with the split-K fp32 reduce, a decode down projection (K=14336) at one and four
    rows, and MoE with routing weights."""
    import synthetic
    import weight_only_quantized_gemm_amd as wq
    out = {}
    k, inter = 4096, 14336

    def proj(seed):
        return dict(qweight=synthetic.qweight_words(seed, k, inter),
                    scales=synthetic.scales(seed + 1, k // 128, inter))
    gate, up = proj(11), proj(13)
    w0 = torch_ops.PackedWeight.gate_up(gate, up, device="cuda")
    for m, copies in ((1, 6), (2048, 1)):
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        a = torch_ops.to_device(synthetic.activations(15, m, k), "cuda")
        act = torch.empty((m, inter), dtype=torch.float16, device="cuda")
        bufs = torch_ops.GemmBuffers(w0, m, False)

        def step(i, ws=ws, a=a, act=act, bufs=bufs, copies=copies):
            torch_ops.gemm(a, ws[i % copies], act, buffers=bufs)
        sec = timed_loop(torch, step, steps if m == 1 else max(5, steps // 8), warmup)
        flops = 2.0 * m * 2 * inter * k
        out[f"swiglu_gate_up_m{m}"] = {
            "workload": f"gate+up M={m} K={k} I={inter} u4b8 g128, fused silu*mul epilogue",
            "us": round(sec * 1e6, 2), "tflops": round(flops / sec / 1e12, 2),
            "weight_tbs": round(k * 2 * inter / 2 / sec / 1e12, 4)}
        del ws
    # group 128 at decode shape is the control: the same kernel timed in the same context
    # (bf16 rows: bf16 activations, scales and outputs, with the headline's flags)
    for name, gs, bf16 in (("decode", 128, False), ("decode", -1, False), ("decode", 64, False),
                           ("decode", 32, False), ("decode", 16, False),
                           ("prefill", 32, False), ("prefill", 16, False),
                           ("decode", 128, True), ("prefill", 128, True)):
        cfg = synthetic.CONFIGS[name]
        act_order = bf16 and cfg["act_order"]
        case = synthetic.dense_case(cfg["m"], cfg["k"], cfg["n"], group_size=gs, seed=17,
                                    act_order=act_order, bf16=bf16)
        w = torch_ops.PackedWeight(case["qweight"], case["scales"], None, case["g_idx"],
                                   device="cuda", group_size=gs, bf16=bf16)
        copies = 12 if name == "decode" else 1
        ws = [w] + [w.clone() for _ in range(copies - 1)]
        a = torch_ops.to_device(case["a"], "cuda")
        c = torch.empty((cfg["m"], cfg["n"]), dtype=torch_ops.act_dtype(bf16), device="cuda")
        fp32 = cfg["fp32_reduce"]
        bufs = torch_ops.GemmBuffers(w, cfg["m"], fp32)

        def step(i, ws=ws, a=a, c=c, bufs=bufs, copies=copies, fp32=fp32):
            torch_ops.gemm(a, ws[i % copies], c, fp32_reduce=fp32, buffers=bufs)
        sec = timed_loop(torch, step, steps if name == "decode" else max(5, steps // 8), warmup)
        flops = 2.0 * cfg["m"] * cfg["n"] * cfg["k"]
        key = f"{name}_bf16" if bf16 else f"{name}_group{gs}"
        out[key] = {
            "workload": f"{name} shape M={cfg['m']} K={cfg['k']} N={cfg['n']} u4b8 "
                        f"group_size {gs}" + (" act_order" if act_order else "")
                        + (" bf16 activations" if bf16 else ""),
            "us": round(sec * 1e6, 2), "tflops": round(flops / sec / 1e12, 2),
            "weight_tbs": round(cfg["k"] * cfg["n"] / 2 / sec / 1e12, 4)}
        del ws
    # W8A16 (E4M3 weights, one byte each): decode and prefill shapes, group 128
    for name in ("decode", "prefill"):
        cfg = synthetic.CONFIGS[name]
        case = synthetic.fp8_case(cfg["m"], cfg["k"], cfg["n"], seed=19)
        w = torch_ops.PackedWeight(case["qweight"], case["scales"], device="cuda", fp8=True)
        copies = 12 if name == "decode" else 1
        ws = [w] + [w.clone() for _ in range(copies - 1)]
        a = torch_ops.to_device(case["a"], "cuda")
        c = torch.empty((cfg["m"], cfg["n"]), dtype=torch.float16, device="cuda")
        fp32 = cfg["fp32_reduce"]
        bufs = torch_ops.GemmBuffers(w, cfg["m"], fp32)

        def step(i, ws=ws, a=a, c=c, bufs=bufs, copies=copies, fp32=fp32):
            torch_ops.gemm(a, ws[i % copies], c, fp32_reduce=fp32, buffers=bufs)
        sec = timed_loop(torch, step, steps if name == "decode" else max(5, steps // 8), warmup)
        out[f"{name}_fp8"] = {
            "workload": f"{name} shape M={cfg['m']} K={cfg['k']} N={cfg['n']} E4M3 weights "
                        "group_size 128",
            "us": round(sec * 1e6, 2),
            "tflops": round(2.0 * cfg["m"] * cfg["n"] * cfg["k"] / sec / 1e12, 2),
            "weight_tbs": round(cfg["k"] * cfg["n"] / sec / 1e12, 4)}
        del ws
    # Mid-size batches on the decode weights with the fp32 reduce: the tiled kernel splits K
    # when its 256-column tiles would leave CUs idle.
    cfg = synthetic.CONFIGS["decode"]
    case = synthetic.dense_case(1, cfg["k"], cfg["n"], seed=21)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device="cuda")
    ws = [w] + [w.clone() for _ in range(11)]
    for m in (64, 256):
        a = torch_ops.to_device(synthetic.activations(23, m, cfg["k"]), "cuda")
        c = torch.empty((m, cfg["n"]), dtype=torch.float16, device="cuda")
        bufs = torch_ops.GemmBuffers(w, m, True)

        def step(i, a=a, c=c, bufs=bufs):
            torch_ops.gemm(a, ws[i % 12], c, fp32_reduce=True, buffers=bufs)
        sec = timed_loop(torch, step, max(5, steps // 4), warmup)
        out[f"batch_m{m}_fp32_reduce"] = {
            "workload": f"M={m} K={cfg['k']} N={cfg['n']} u4b8 g128, fp32 reduce (split K), "
                        "12 rotating weight copies",
            "us": round(sec * 1e6, 2),
            "tflops": round(2.0 * m * cfg["n"] * cfg["k"] / sec / 1e12, 2),
            "weight_tbs": round(cfg["k"] * cfg["n"] / 2 / sec / 1e12, 4)}
    del ws
    # A decode down projection (the MLP's second product, K = 14336, N = 4096): one row and a
    # four-row batch, no flags, on the small-M kernel's sixteen-wave plans.
    kd, nd = 14336, 4096
    case = synthetic.dense_case(1, kd, nd, seed=25)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device="cuda")
    ws = [w] + [w.clone() for _ in range(11)]
    for m in (1, 4):
        a = torch_ops.to_device(synthetic.activations(27, m, kd), "cuda")
        c = torch.empty((m, nd), dtype=torch.float16, device="cuda")
        bufs = torch_ops.GemmBuffers(w, m, False)

        def step(i, a=a, c=c, bufs=bufs):
            torch_ops.gemm(a, ws[i % 12], c, buffers=bufs)
        sec = timed_loop(torch, step, steps, warmup)
        out[f"down_proj_m{m}"] = {
            "workload": f"M={m} K={kd} N={nd} u4b8 g128 (a decode down projection), 12 rotating "
                        "weight copies",
            "us": round(sec * 1e6, 2),
            "weight_tbs": round(kd * nd / 2 / sec / 1e12, 4)}
    # The same down projection for 8- and 16-row batches with the fp32 reduce flag (K split
    # into seven even 16-group ranges), and a 70B-class one (K = 28672, N = 8192, 117 MB of
    # weights, four rotating copies) for a four-row batch (fourteen ranges).
    long_rows = [(m, kd, nd, ws, 12) for m in (8, 16)]
    case = synthetic.dense_case(1, 28672, 8192, seed=26)
    w70 = torch_ops.PackedWeight(case["qweight"], case["scales"], device="cuda")
    long_rows.append((4, 28672, 8192, [w70] + [w70.clone() for _ in range(3)], 4))
    for m, kl, nl, wl, copies in long_rows:
        a = torch_ops.to_device(synthetic.activations(28, m, kl), "cuda")
        c = torch.empty((m, nl), dtype=torch.float16, device="cuda")
        bufs = torch_ops.GemmBuffers(wl[0], m, True)

        def step(i, a=a, c=c, bufs=bufs, wl=wl, copies=copies):
            torch_ops.gemm(a, wl[i % copies], c, fp32_reduce=True, buffers=bufs)
        sec = timed_loop(torch, step, steps, warmup)
        splits = wq.wq_gemm_plan(m, nl, kl, flags=wq.WQ_FLAG_FP32_REDUCE)[1]
        out[f"down_proj_{kl}x{nl}_m{m}_fp32_reduce"] = {
            "workload": f"M={m} K={kl} N={nl} u4b8 g128 (a down projection), fp32 reduce "
                        f"({splits} splits), {copies} rotating weight copies",
            "us": round(sec * 1e6, 2),
            "weight_tbs": round(kl * nl / 2 / sec / 1e12, 4)}
    del ws, w70, long_rows
    moe = synthetic.moe_case()
    bank = torch_ops.ExpertBank(moe["experts"], device="cuda")
    csr = wq.wq_csr_from_routes(moe["routes"], moe["n_tokens"], moe["top_k"], moe["n_expert"])
    dcsr = {key: torch_ops.to_device(np.asarray(csr[key], np.int32), "cuda")
            for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok")}
    a = torch_ops.to_device(moe["a"], "cuda")
    y = torch.empty((csr["n_pairs"], moe["n"]), dtype=torch.float16, device="cuda")
    wts = torch_ops.to_device(synthetic.routing_weights(19, moe["n_tokens"], 2), "cuda")

    def moe_step(i):
        torch_ops.grouped_gemm(a, bank, csr, y, device_csr=dcsr, topk_weights=wts)
    sec = timed_loop(torch, moe_step, max(5, steps // 8), warmup)
    out["moe_routing_weights"] = {
        "workload": "MoE config with a per-pair fp32 routing-weight multiply",
        "us": round(sec * 1e6, 2),
        "tflops": round(2.0 * csr["n_pairs"] * moe["n"] * moe["k"] / sec / 1e12, 2)}
    del bank
    # Many experts: 1024 tokens, top-2 of 64 experts (about 32 rows per expert), the same
    # K and N; every expert holds the same synthetic weights (the time does not depend on
    # the values), 64 x 29.4 MB of banks.
    one = synthetic.moe_case(1024, 1, seed=41)
    bank = torch_ops.ExpertBank(one["experts"] * 64, device="cuda")
    routes = synthetic.top2_routes(43, 1024, 64)
    csr = wq.wq_csr_from_routes(routes, 1024, 2, 64)
    dcsr = {key: torch_ops.to_device(np.asarray(csr[key], np.int32), "cuda")
            for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok")}
    a = torch_ops.to_device(one["a"], "cuda")

    def moe64_step(i):
        torch_ops.grouped_gemm(a, bank, csr, y, device_csr=dcsr)
    sec = timed_loop(torch, moe64_step, max(5, steps // 8), warmup)
    out["moe_64_experts"] = {
        "workload": "1024 tokens top-2 of 64 experts K=4096 N=14336 u4b8 group 128 "
                    f"({csr['n_active']} active experts)",
        "us": round(sec * 1e6, 2),
        "tflops": round(2.0 * csr["n_pairs"] * one["n"] * one["k"] / sec / 1e12, 2),
        "weight_tbs": round(csr["n_active"] * one["k"] * one["n"] / 2 / sec / 1e12, 4)}
    del bank
    # MoE decode: a few tokens, top-2 of 8 experts, the same K and N (segments of at most four
    # rows run on the small-M kernel).  Three banks of eight experts rotate with sixteen
    # routings, so that the experts read by one step are not those of the step before.
    one = synthetic.moe_case(4, 1, seed=45)
    banks = [torch_ops.ExpertBank(one["experts"] * 8, device="cuda") for _ in range(3)]
    for tokens in (1, 4):
        csrs, dcsrs = [], []
        for r in range(16):
            routes = synthetic.top2_routes(47 + 16 * tokens + r, tokens, 8)
            csr = wq.wq_csr_from_routes(routes, tokens, 2, 8)
            csrs.append(csr)
            dcsrs.append({key: torch_ops.to_device(np.asarray(csr[key], np.int32), "cuda")
                          for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok")})
        a = torch_ops.to_device(synthetic.activations(49, tokens, one["k"]), "cuda")
        y = torch.empty((2 * tokens, one["n"]), dtype=torch.float16, device="cuda")

        def decode_step(i, a=a, y=y, csrs=csrs, dcsrs=dcsrs):
            torch_ops.grouped_gemm(a, banks[i % 3], csrs[i % 16], y, device_csr=dcsrs[i % 16])
        sec = timed_loop(torch, decode_step, 48, warmup)
        active = float(np.mean([c["n_active"] for c in csrs]))
        out[f"moe_decode_{tokens}_tokens"] = {
            "workload": f"{tokens} token(s) top-2 of 8 experts K=4096 N=14336 u4b8 group 128 "
                        f"({active:.2f} active experts on average), 3 rotating banks",
            "us": round(sec * 1e6, 2),
            "weight_tbs": round(active * one["k"] * one["n"] / 2 / sec / 1e12, 4)}
    del banks
    # The matching down projection at one token: K=14336, N=4096 per expert.
    down = synthetic.moe_case(1, 1, 14336, 4096, seed=51)
    banks = [torch_ops.ExpertBank(down["experts"] * 8, device="cuda") for _ in range(3)]
    csrs, dcsrs = [], []
    for r in range(16):
        csr = wq.wq_csr_from_routes(synthetic.top2_routes(53 + r, 1, 8), 1, 2, 8)
        csrs.append(csr)
        dcsrs.append({key: torch_ops.to_device(np.asarray(csr[key], np.int32), "cuda")
                      for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok")})
    a = torch_ops.to_device(synthetic.activations(55, 2, 14336), "cuda")
    y = torch.empty((2, 4096), dtype=torch.float16, device="cuda")
    ident = [dict(c, pair_tok=[0, 1]) for c in csrs]
    dident = [dict(d, pair_tok=torch_ops.to_device(np.arange(2, dtype=np.int32), "cuda"))
              for d in dcsrs]

    def down_step(i):
        torch_ops.grouped_gemm(a, banks[i % 3], ident[i % 16], y, device_csr=dident[i % 16])
    sec = timed_loop(torch, down_step, 48, warmup)
    out["moe_decode_1_token_down"] = {
        "workload": "1 token top-2 of 8 experts, down projection K=14336 N=4096 u4b8 group 128 "
                    "over the pair rows (2 active experts), 3 rotating banks",
        "us": round(sec * 1e6, 2),
        "weight_tbs": round(2 * 14336 * 4096 / 2 / sec / 1e12, 4)}
    return out


MFMA_ITERS = 512  # K steps of the register-only MFMA loop per launch (about 0.1-0.2 ms)


def bench_mfma(torch, steps, warmup):
    """Practical fp16 matrix rate (wq_mfma_rate): the tiled GEMM's per-wave products from
    registers on every CU, with this method's operand data (A ~ N(0,1) in fp16, B integer
    codes q - 8 in -8..7) and with all-zero operands (the least switching activity)."""
    import synthetic
    import weight_only_quantized_gemm_amd as wq
    a = synthetic.activations(31, 4 * 64, 8).reshape(4, 64, 8)
    b = (synthetic.below(32, 2 * 64 * 8, 16).astype(np.float16) - 8).reshape(2, 64, 8)
    data = {"method_operands": np.concatenate([a, b]).astype(np.float16),
            "zeros": np.zeros((6, 64, 8), np.float16)}
    sink = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    out = {}
    for key, ops_h in data.items():
        ops = torch.from_numpy(ops_h).cuda()
        flops = [0.0]

        def step(i, ops=ops):
            flops[0] = wq.wq_mfma_rate(ops, MFMA_ITERS, sink, sink.numel())
        sec = timed_loop(torch, step, steps, warmup)
        out[key] = {"us": round(sec * 1e6, 2), "tflops": round(flops[0] / sec / 1e12, 1)}
    return out


COPY_BYTES = 1 << 30  # plain device copy used to calibrate the HBM byte counters


def bench_copy(torch, steps, warmup):
    """A plain 1 GiB device-to-device copy (reads and writes COPY_BYTES each)."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sec = timed_loop(torch, lambda i: dst.copy_(src), steps, warmup)
    return dict(sec=sec, bytes=COPY_BYTES)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_hbm_traffic.txt")
SMALL_SOURCE = os.path.join(ROOT, "weight_only_quantized_gemm_amd", "csrc", "wq_small_kernel.h")


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic() -> float | None:
    """HBM bytes per decode launch from the committed counter summary, or None.

    The summary records FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the decode kernel
    and of a plain copy of known size; each counter is scaled by the factor the copy gives.
    It only applies while the kernel source is the one that was profiled.
    """
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    try:
        if vals.get("kernel_source_sha256_16") != source_hash(SMALL_SOURCE):
            return None
        fetch = float(vals["decode_fetch_kib"]) * 1024 * float(vals["fetch_factor"])
        write = float(vals["decode_write_kib"]) * 1024 * float(vals["write_factor"])
        return fetch + write
    except (KeyError, ValueError):
        return None


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return 1


def _time_repeated(fn, budget_s: float) -> tuple[float, int]:
    """Seconds per call of fn, repeated until about budget_s has passed (at least once)."""
    runs, t0 = 0, time.perf_counter()
    while True:
        fn()
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return (time.perf_counter() - t0) / runs, runs


def cpu_baseline(budget_s: float, gpu_us: dict) -> dict:
    """The oracle (fp64 numpy: unpack, exact dequant, fp64 matmul) timed on the host cores
    for every workload, beside the GPU time of the same workload.  The headline fields are
    the decode workload's, in the line's unit; `configs` holds each workload's oracle time
    (the MoE workload on a sample of its columns, scaled to all of them)."""
    import synthetic
    from oracle import reference as ref
    blas = _blas_threads()
    per = {}
    share = budget_s / 6.0

    def dense(name, frac=1.0):
        case = synthetic.config_case(name)
        cols = None if frac >= 1.0 else np.arange(int(case["n"] * frac))
        sec, runs = _time_repeated(lambda: ref.w4a16_gemm(
            case["a"], case["qweight"], case["scales"], zeros=case["zeros"],
            g_idx=case["g_idx"], columns=cols), share)
        scale = case["n"] / (case["n"] if cols is None else len(cols))
        return case, sec * scale, runs, cols

    for name in ("tiny", "decode", "batched", "prefill"):
        case, sec, runs, _ = dense(name)
        per[name] = {"oracle_s": round(sec, 5), "runs": runs,
                     "sample": f"full problem M={case['m']} K={case['k']} N={case['n']}",
                     "gpu_us": gpu_us.get(name),
                     "gpu_speedup": round(sec / (gpu_us[name] * 1e-6), 1) if gpu_us.get(name)
                     else None}
    moe = synthetic.moe_case()
    csr = ref.csr_from_token_routes(moe["n_expert"], moe["n_tokens"], moe["top_k"],
                                    moe["routes"])
    cols = np.arange(moe["n"] // 7)             # 2048 of the 14336 columns
    sec, runs = _time_repeated(lambda: ref.grouped_w4a16_gemm(moe["a"], moe["experts"], csr,
                                                              columns=cols), share)
    sec *= moe["n"] / len(cols)
    per["moe"] = {"oracle_s": round(sec, 4), "runs": runs,
                  "sample": f"columns 0..{len(cols) - 1} of {moe['n']} (all 2048 pairs, all 8 "
                            "experts), time scaled by 7",
                  "gpu_us": gpu_us.get("moe"),
                  "gpu_speedup": round(sec / (gpu_us["moe"] * 1e-6), 1) if gpu_us.get("moe")
                  else None}
    dec = per["decode"]
    weight_bytes = 4096 * 14336 // 2
    return {"value": round(weight_bytes / dec["oracle_s"] / 1e12, 8), "unit": "TB/s",
            "cores": blas, "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": f"full decode problem M=1 K=4096 N=14336, {dec['runs']} runs, "
                      f"{dec['oracle_s'] * 1e3:.0f} ms per run; numpy elementwise work on 1 "
                      f"thread, BLAS (the fp64 matmul) on {blas} of {os.cpu_count()} host "
                      "cores; every workload under `configs`",
            "configs": per}


def plan_text(m, n, k, flags) -> str:
    """What the library runs for a problem, from its own planner (wq_gemm_plan)."""
    import weight_only_quantized_gemm_amd as wq
    kernel, splits = wq.wq_gemm_plan(m, n, k, flags=flags)
    split = "K not split" if splits == 1 else f"K split {splits} ways, fp32 partials reduced"
    return f"{wq.KERNEL_NAMES[kernel]} kernel, {split}"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extended", action="store_true",
                    help="skip the timings of the widened features")
    ap.add_argument("--only", choices=["decode", "batched", "prefill", "moe", "tiny", "copy",
                                       "ceiling", "mfma"],
                    default=None, help="time one workload (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        return 2

    import torch
    import weight_only_quantized_gemm_amd as wq
    from weight_only_quantized_gemm_amd import torch_ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.only:
        if args.only == "copy":
            r = bench_copy(torch, args.steps, args.warmup)
            print(json.dumps({"only": "copy", "bytes_read": r["bytes"], "bytes_written": r["bytes"],
                              "us": r["sec"] * 1e6,
                              "TBs_read_plus_write": 2 * r["bytes"] / r["sec"] / 1e12}), flush=True)
        elif args.only == "ceiling":
            r = bench_dense(torch, torch_ops, "decode", 12, 1, 1)
            c = bench_stream_read(torch, r["weights"], args.steps, args.warmup)
            print(json.dumps({"only": "ceiling", "bytes": c["bytes"], "us": c["sec"] * 1e6,
                              "TBs": c["bytes"] / c["sec"] / 1e12}), flush=True)
        elif args.only == "mfma":
            print(json.dumps({"only": "mfma", **bench_mfma(torch, args.steps, args.warmup)}),
                  flush=True)
        elif args.only == "moe":
            r = bench_moe(torch, torch_ops, args.steps, args.warmup)
            print(json.dumps({"only": "moe", "us": r["sec"] * 1e6,
                              "tflops": r["flops"] / r["sec"] / 1e12}), flush=True)
        else:
            copies = {"decode": 12, "batched": 40}.get(args.only, 1)
            r = bench_dense(torch, torch_ops, args.only, copies, args.steps, args.warmup)
            print(json.dumps({"only": args.only, "us": r["sec"] * 1e6,
                              "weight_tbs": r["weight_bytes"] / r["sec"] / 1e12,
                              "tflops": r["flops"] / r["sec"] / 1e12}), flush=True)
        return 0

    def log(text):
        print(text, file=sys.stderr, flush=True)

    dec = bench_dense(torch, torch_ops, "decode", 12, args.steps, args.warmup)
    log(f"decode: {dec['sec'] * 1e6:.2f} us/call")
    ceil = bench_stream_read(torch, dec.pop("weights"), args.steps, args.warmup)
    ceil_tbs = ceil["bytes"] / ceil["sec"] / 1e12
    log(f"streaming read of the decode weights: {ceil['sec'] * 1e6:.2f} us ({ceil_tbs:.3f} TB/s)")
    bat = bench_dense(torch, torch_ops, "batched", 40, args.steps, args.warmup)
    bceil = bench_stream_read(torch, bat.pop("weights"), args.steps, args.warmup)
    log(f"batched: {bat['sec'] * 1e6:.2f} us/call; streaming read of its weights: "
        f"{bceil['sec'] * 1e6:.2f} us")
    tiny = bench_dense(torch, torch_ops, "tiny", 1, args.steps, args.warmup)
    tiny.pop("weights")
    log(f"tiny: {tiny['sec'] * 1e6:.2f} us/call")
    pre_steps = max(10, args.steps // 4)
    pre = bench_dense(torch, torch_ops, "prefill", 1, pre_steps, max(3, args.warmup // 4))
    pre.pop("weights")
    log(f"prefill: {pre['sec'] * 1e6:.1f} us/call")
    moe = bench_moe(torch, torch_ops, pre_steps, max(3, args.warmup // 4))
    log(f"moe: {moe['sec'] * 1e6:.1f} us/call")
    mfma = bench_mfma(torch, max(10, args.steps // 10), 3)
    log("mfma register-only rate: " + ", ".join(f"{k} {v['tflops']} TFLOP/s"
                                                 for k, v in mfma.items()))

    fp32 = wq.WQ_FLAG_FP32_REDUCE
    tbs = dec["weight_bytes"] / dec["sec"] / 1e12
    achieved = dec["weight_bytes"] / dec["sec"] / 1e9          # packed-weight bytes
    achieved_all = dec["alg_bytes"] / dec["sec"] / 1e9         # weights, scales, A and C
    pre_tflops = pre["flops"] / pre["sec"] / 1e12
    moe_tflops = moe["flops"] / moe["sec"] / 1e12
    bat_tbs = bat["weight_bytes"] / bat["sec"] / 1e12
    bceil_tbs = bceil["bytes"] / bceil["sec"] / 1e12
    real_mfma = mfma["method_operands"]["tflops"]
    line = {
        "metric": METRIC,
        "value": round(tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["sec"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "decode GEMM M=1 K=4096 N=14336 u4b8 group 128, fp32-reduce "
                               "flag set; " + plan_text(1, 14336, 4096, fp32)
                               + "; 12 rotating weight copies",
                   "m": 1, "k": 4096, "n": 14336, "weight_bytes": dec["weight_bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "basis": "packed-weight bytes K*N/2 per launch",
                     "achieved_all_operands": round(achieved_all, 1),
                     "frac_all_operands": round(achieved_all / HBM_PEAK_GBS, 4)},
        "hbm_read_ceiling": {"kernel": "wq_stream_read (plain 16-byte non-temporal streaming "
                                       "read of the same 12 rotating weight buffers)",
                             "bytes": ceil["bytes"], "us": round(ceil["sec"] * 1e6, 3),
                             "TBs": round(ceil_tbs, 4),
                             "frac_of_peak": round(ceil_tbs * 1e3 / HBM_PEAK_GBS, 4),
                             "decode_frac_of_ceiling": round(tbs / ceil_tbs, 4)},
        "prefill": {"workload": "M=2048 K=4096 N=14336 u4b8 group 128 act_order (gather + GEMM); "
                                + plan_text(2048, 14336, 4096, wq.WQ_FLAG_ACT_ORDER),
                    "tflops": round(pre_tflops, 2), "us": round(pre["sec"] * 1e6, 2),
                    "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2),
                                 "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(pre_tflops / MFMA_FP16_PEAK_TFLOPS, 4)},
                    "frac_of_mfma_ceiling": round(pre_tflops / real_mfma, 4)},
        "batched": {"workload": "M=16 K=4096 N=4096 u4 + zero points group 128, fp32-reduce "
                                "flag set; " + plan_text(16, 4096, 4096, fp32 | wq.WQ_FLAG_HAS_ZP)
                                + "; 40 rotating weight copies",
                    "us": round(bat["sec"] * 1e6, 3), "weight_tbs": round(bat_tbs, 4),
                    "hbm_frac": round(bat_tbs * 1e3 / HBM_PEAK_GBS, 4),
                    "hbm_frac_all_operands": round(
                        bat["alg_bytes"] / bat["sec"] / 1e9 / HBM_PEAK_GBS, 4),
                    "read_ceiling_us": round(bceil["sec"] * 1e6, 3),
                    "read_ceiling_tbs": round(bceil_tbs, 4),
                    "frac_of_read_ceiling": round(bat_tbs / bceil_tbs, 4)},
        "tiny": {"workload": "M=16 K=1024 N=256 u4b8 group 128 (one 131 KB weight, cache "
                             "resident); " + plan_text(16, 256, 1024, 0),
                 "us": round(tiny["sec"] * 1e6, 3)},
        "moe": {"workload": "1024 tokens top-2 of 8 experts K=4096 N=14336 u4b8 group 128, "
                            "grouped tiled kernel (128 x 256 tiles)",
                "us": round(moe["sec"] * 1e6, 2), "tflops": round(moe_tflops, 2),
                "mfma_frac": round(moe_tflops / MFMA_FP16_PEAK_TFLOPS, 4),
                "frac_of_mfma_ceiling": round(moe_tflops / real_mfma, 4)},
        "mfma_ceiling": {"kernel": "wq_mfma_rate (register-only v_mfma_f32_32x32x16_f16 loop, "
                                   "the tiled GEMM's 128 x 64 wave tile, 2 waves per SIMD on "
                                   "every CU)", **mfma,
                         "frac_of_peak": {k: round(v["tflops"] / MFMA_FP16_PEAK_TFLOPS, 4)
                                          for k, v in mfma.items()}},
    }
    if not args.no_extended:
        line["extended"] = bench_extended(torch, torch_ops, args.steps, max(3, args.warmup // 4))
        log("extended: " + ", ".join(f"{k} {v['us']} us" for k, v in line["extended"].items()))
    if not args.no_cpu_baseline:
        gpu_us = {"tiny": tiny["sec"] * 1e6, "decode": dec["sec"] * 1e6,
                  "batched": bat["sec"] * 1e6, "prefill": pre["sec"] * 1e6,
                  "moe": moe["sec"] * 1e6}
        line["cpu_baseline"] = cpu_baseline(args.cpu_budget, gpu_us)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
