"""Benchmark of the W4A16 GEMM on one MI355X; prints one JSON line.

Headline (value): packed-weight TB/s of the decode GEMM, M=1 K=4096 N=14336, u4b8, group
128, split-K with the fp32 workspace reduce.  Each step is one wq_gemm call; steps rotate
over enough weight copies that the weights stream from HBM rather than from the 256 MB
Infinity Cache.  The same line carries the prefill (M=2048, act_order) TFLOP/s with its
MFMA roofline, the batched-decode and grouped-MoE figures, and the oracle timed on the
host cores as the CPU baseline.
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
    batches with the split-K fp32 reduce, and MoE with routing weights."""
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


def cpu_baseline(budget_s: float) -> dict:
    """The oracle (fp64 numpy) on the decode workload, repeated for about `budget_s`."""
    import synthetic
    from oracle import reference as ref
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        blas = 1
    case = synthetic.config_case("decode")
    runs, t0 = 0, time.perf_counter()
    while True:
        ref.w4a16_gemm(case["a"], case["qweight"], case["scales"])
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    sec = (time.perf_counter() - t0) / runs
    weight_bytes = case["k"] * case["n"] // 2
    return {"value": weight_bytes / sec / 1e12, "unit": "TB/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"full decode problem M=1 K=4096 N=14336 (unpack, exact dequant, fp64 "
                      f"matmul), {runs} runs in {sec * runs:.1f} s; {sec * 1e3:.0f} ms per run; "
                      f"elementwise numpy on 1 thread, BLAS on {blas}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extended", action="store_true",
                    help="skip the timings of the widened features")
    ap.add_argument("--only", choices=["decode", "batched", "prefill", "moe", "tiny", "copy",
                                       "ceiling"],
                    default=None, help="time one workload (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        return 2

    import torch
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

    dec = bench_dense(torch, torch_ops, "decode", 12, args.steps, args.warmup)
    print(f"decode: {dec['sec'] * 1e6:.2f} us/call", file=sys.stderr, flush=True)
    ceil = bench_stream_read(torch, dec.pop("weights"), args.steps, args.warmup)
    ceil_tbs = ceil["bytes"] / ceil["sec"] / 1e12
    print(f"streaming read of the same bytes: {ceil['sec'] * 1e6:.2f} us ({ceil_tbs:.3f} TB/s)",
          file=sys.stderr, flush=True)
    bat = bench_dense(torch, torch_ops, "batched", 40, args.steps, args.warmup)
    bat.pop("weights")
    print(f"batched: {bat['sec'] * 1e6:.2f} us/call", file=sys.stderr, flush=True)
    pre_steps = max(10, args.steps // 4)
    pre = bench_dense(torch, torch_ops, "prefill", 1, pre_steps, max(3, args.warmup // 4))
    pre.pop("weights")
    print(f"prefill: {pre['sec'] * 1e6:.1f} us/call", file=sys.stderr, flush=True)
    moe = bench_moe(torch, torch_ops, pre_steps, max(3, args.warmup // 4))
    print(f"moe: {moe['sec'] * 1e6:.1f} us/call", file=sys.stderr, flush=True)

    tbs = dec["weight_bytes"] / dec["sec"] / 1e12
    achieved = dec["alg_bytes"] / dec["sec"] / 1e9
    pre_tflops = pre["flops"] / pre["sec"] / 1e12
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
        "config": {"workload": "decode GEMM M=1 K=4096 N=14336 u4b8 group128 split-K fp32 "
                               "reduce, 12 rotating weight copies",
                   "m": 1, "k": 4096, "n": 14336, "weight_bytes": dec["weight_bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic()},
        "hbm_read_ceiling": {"kernel": "wq_stream_read (plain 16-byte non-temporal streaming "
                                       "read of the same 12 rotating weight buffers)",
                             "bytes": ceil["bytes"], "us": round(ceil["sec"] * 1e6, 3),
                             "TBs": round(ceil_tbs, 4),
                             "frac_of_peak": round(ceil_tbs * 1e3 / HBM_PEAK_GBS, 4),
                             "decode_frac_of_ceiling": round(tbs / ceil_tbs, 4)},
        "prefill": {"workload": "M=2048 K=4096 N=14336 u4b8 group128 act_order (gather + GEMM)",
                    "tflops": round(pre_tflops, 2), "us": round(pre["sec"] * 1e6, 2),
                    "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2),
                                 "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(pre_tflops / MFMA_FP16_PEAK_TFLOPS, 4)}},
        "batched": {"workload": "M=16 K=4096 N=4096 u4+zp group128 fp32 reduce, 40 copies",
                    "us": round(bat["sec"] * 1e6, 3),
                    "weight_tbs": round(bat["weight_bytes"] / bat["sec"] / 1e12, 4),
                    "hbm_frac": round(bat["alg_bytes"] / bat["sec"] / 1e9 / HBM_PEAK_GBS, 4)},
        "moe": {"workload": "1024 tokens top-2 of 8 experts K=4096 N=14336 u4b8 group128",
                "us": round(moe["sec"] * 1e6, 2),
                "tflops": round(moe["flops"] / moe["sec"] / 1e12, 2),
                "mfma_frac": round(moe["flops"] / moe["sec"] / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4)},
    }
    if not args.no_extended:
        line["extended"] = bench_extended(torch, torch_ops, args.steps, max(3, args.warmup // 4))
        print("extended: " + ", ".join(f"{k} {v['us']} us" for k, v in line["extended"].items()),
              file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
