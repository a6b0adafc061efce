"""A seeded sweep of dense products over both kernels and every plan form (staged and
direct small-M, paired blocks, the one-row path, 128- and 256-row tiles, split K), every
activation and weight type, group sizes, zero points, act_order and strided activations,
and of grouped (MoE) products over token and expert counts, types, group sizes, zero
points and routing weights, each compared with the CPU oracle on every output.  Two more
sweeps take long K (8192 to 28672: sixteen-wave small-M plans with per-wave staging, row
chunks and split tiles, and grouped segments of a few rows).

The shapes come from a fixed-seed generator, so the sweep is the same on every run; each
case prints its parameters before it runs.
"""

import numpy as np
import pytest

import synthetic
from oracle import reference as ref

torch = pytest.importorskip("torch")
wq = pytest.importorskip("weight_only_quantized_gemm_amd")
from weight_only_quantized_gemm_amd import torch_ops  # noqa: E402

pytestmark = pytest.mark.gpu

# Tolerances: fp16 outputs use the GEMM criterion; bf16 outputs add their own rounding
# (2^-8 |ref| per element, Frobenius 4e-3); E4M3 weights add the fp16 output's rounding per
# element (their magnitudes span 2^-9 .. 448, far beyond the rms).
FP16_TOL = {}
BF16_TOL = dict(rel_elem=2.0 ** -8, rel_frob=4e-3)
FP8_TOL = dict(rel_elem=2.0 ** -11)

M_CHOICES = [1, 2, 3, 5, 8, 9, 12, 16, 17, 33, 64, 100, 129, 256, 300]
K_CHOICES = [128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096]
N_CHOICES = [256, 512, 768, 1024, 2048, 4096, 8192]
GS_CHOICES = [-1, 16, 32, 48, 64, 80, 96, 128, 256, 512, 1024]


def sweep_cases(count=160, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        kind = ["u4b8", "u4zp", "bf16", "fp8"][int(rng.integers(4))]
        m = int(rng.choice(M_CHOICES))
        k = int(rng.choice(K_CHOICES))
        n = int(rng.choice(N_CHOICES))
        if m * k * n > 1_500_000_000 or (m > 16 and n > 4096):
            continue  # keeps each oracle product well under a second
        if kind == "fp8":
            gs = int(rng.choice([-1, 128]))
        else:
            gs = int(rng.choice([g for g in GS_CHOICES if g == -1 or (g <= k and k % g == 0)]))
        zp = kind == "u4zp" or (kind == "bf16" and bool(rng.integers(2)))
        act_order = kind != "fp8" and rng.random() < 0.3
        fp32 = bool(rng.integers(2))
        split = int(rng.choice([0, 0, 2, 3, 5])) if fp32 else 0
        lda_pad = int(rng.choice([0, 0, 0, 8, 64]))
        bf16_act = kind == "bf16" or (kind == "fp8" and rng.random() < 0.25)
        cases.append((kind, m, k, n, gs, zp, act_order, fp32, split, lda_pad, bf16_act))
    return cases


CASES = sweep_cases()

LONG_M = [1, 2, 3, 4, 5, 6, 8, 9, 12, 16, 24]
LONG_K = [8192, 9216, 11008, 12288, 14336, 16384, 20480, 24576, 28672]


def long_k_cases(count=24, seed=20261205):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        kind = ["u4b8", "u4zp", "bf16", "fp8"][int(rng.choice(4, p=[0.35, 0.3, 0.25, 0.1]))]
        m = int(rng.choice(LONG_M))
        k = int(rng.choice(LONG_K))
        n = int(rng.choice([256, 512, 1024]))
        if m * k * n > 400_000_000:
            continue
        if kind == "fp8":
            gs = int(rng.choice([-1, 128]))
        else:
            gs = int(rng.choice([g for g in GS_CHOICES if g == -1 or (g <= k and k % g == 0)]))
        zp = kind == "u4zp" or (kind == "bf16" and bool(rng.integers(2)))
        act_order = kind != "fp8" and rng.random() < 0.25
        fp32 = bool(rng.integers(2))
        split = int(rng.choice([0, 0, 0, 2, 4])) if fp32 else 0
        lda_pad = int(rng.choice([0, 0, 8]))
        bf16_act = kind == "bf16"
        cases.append((kind, m, k, n, gs, zp, act_order, fp32, split, lda_pad, bf16_act))
    return cases


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def strided(a, pad, dev, bf16):
    """The activations on the device with row stride k + pad (pad columns hold NaNs that no
    product may read)."""
    m, k = a.shape
    dt = torch.bfloat16 if bf16 else torch.float16
    base = torch_ops.to_device(a, dev)
    if pad == 0:
        return base
    wide = torch.full((m, k + pad), float("nan"), dtype=dt, device=dev)
    wide[:, :k] = base
    return wide[:, :k]


@pytest.mark.parametrize("kind,m,k,n,gs,zp,act_order,fp32,split,lda_pad,bf16_act", CASES)
def test_sweep_matches_oracle(dev, kind, m, k, n, gs, zp, act_order, fp32, split, lda_pad,
                              bf16_act):
    run_dense(dev, "sweep", kind, m, k, n, gs, zp, act_order, fp32, split, lda_pad, bf16_act)


@pytest.mark.parametrize("kind,m,k,n,gs,zp,act_order,fp32,split,lda_pad,bf16_act",
                         long_k_cases())
def test_long_k_sweep_matches_oracle(dev, kind, m, k, n, gs, zp, act_order, fp32, split,
                                     lda_pad, bf16_act):
    run_dense(dev, "long-K sweep", kind, m, k, n, gs, zp, act_order, fp32, split, lda_pad,
              bf16_act)


def run_dense(dev, name, kind, m, k, n, gs, zp, act_order, fp32, split, lda_pad, bf16_act):
    label = (f"{name} {kind} m={m} k={k} n={n} group_size={gs} zp={zp} act_order={act_order} "
             f"fp32={fp32} split={split} lda=k+{lda_pad} bf16={bf16_act}")
    print(label, flush=True)
    seed = 7000 + m * 31 + k * 7 + n + gs
    if kind == "fp8":
        case = synthetic.fp8_case(m, k, n, group_size=gs, seed=seed, bf16=bf16_act)
        w = torch_ops.PackedWeight(case["qweight"], case["scales"], device=dev, group_size=gs,
                                   bf16=bf16_act, fp8=True)
        want = ref.w8a16_gemm(case["a"], case["qweight"], case["scales"], group_size=gs,
                              bf16=bf16_act)
        tol = BF16_TOL if bf16_act else FP8_TOL
    else:
        case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                    seed=seed, bf16=bf16_act)
        w = torch_ops.PackedWeight(case["qweight"], case["scales"], case["zeros"],
                                   case["g_idx"], device=dev, group_size=gs, bf16=bf16_act)
        want = ref.w4a16_gemm(case["a"], case["qweight"], case["scales"], zeros=case["zeros"],
                              g_idx=case["g_idx"], group_size=gs, bf16=bf16_act)
        tol = BF16_TOL if bf16_act else FP16_TOL
    a = strided(case["a"], lda_pad, dev, bf16_act)
    c = torch_ops.gemm(a, w, fp32_reduce=fp32, split_k=split)
    torch.cuda.synchronize()
    res = ref.check(to_host(c), want, **tol)
    print(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} "
          f"rel_frob={res['rel_frob']:.3e} nonfinite={res['nonfinite']}", flush=True)
    assert res["ok"], (label, res)


def grouped_cases(count=48, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        kind = ["fp16", "bf16", "fp8"][int(rng.integers(3))]
        tokens = int(rng.choice([1, 3, 40, 129, 300, 700]))
        experts = int(rng.choice([1, 2, 3, 8, 17]))
        k = int(rng.choice([128, 256, 512, 1024]))
        n = int(rng.choice([256, 512, 768]))
        gs = 128 if kind == "fp8" else int(rng.choice([g for g in (16, 32, 64, 128) if k % g == 0]))
        zp = kind != "fp8" and bool(rng.integers(2))
        weighted = bool(rng.integers(2))
        cases.append((kind, tokens, experts, k, n, gs, zp, weighted))
    return cases


def grouped_long_k_cases(count=16, seed=20261206):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        kind = ["fp16", "bf16", "fp8"][int(rng.choice(3, p=[0.55, 0.35, 0.1]))]
        tokens = int(rng.choice([1, 2, 3, 4]))
        experts = int(rng.choice([2, 3, 8]))
        k = int(rng.choice([8192, 11008, 14336, 16384]))
        n = int(rng.choice([256, 512]))
        gs = 128 if kind == "fp8" else int(rng.choice([g for g in (16, 32, 64, 128) if k % g == 0]))
        zp = kind != "fp8" and bool(rng.integers(2))
        weighted = bool(rng.integers(2))
        cases.append((kind, tokens, experts, k, n, gs, zp, weighted))
    return cases


@pytest.mark.parametrize("kind,tokens,experts,k,n,gs,zp,weighted", grouped_cases())
def test_grouped_sweep_matches_oracle(dev, kind, tokens, experts, k, n, gs, zp, weighted):
    run_grouped(dev, "grouped sweep", kind, tokens, experts, k, n, gs, zp, weighted)


@pytest.mark.parametrize("kind,tokens,experts,k,n,gs,zp,weighted", grouped_long_k_cases())
def test_grouped_long_k_sweep_matches_oracle(dev, kind, tokens, experts, k, n, gs, zp,
                                             weighted):
    run_grouped(dev, "grouped long-K sweep", kind, tokens, experts, k, n, gs, zp, weighted)


def run_grouped(dev, name, kind, tokens, experts, k, n, gs, zp, weighted):
    label = (f"{name} {kind} tokens={tokens} experts={experts} k={k} n={n} "
             f"group_size={gs} zp={zp} weighted={weighted}")
    print(label, flush=True)
    seed = 9000 + tokens * 13 + experts * 101 + k + n + gs
    bf16 = kind == "bf16"
    fp8 = kind == "fp8"
    moe = synthetic.moe_case(tokens, experts, k, n, group_size=gs, seed=seed, bf16=bf16)
    ex = []
    for i, e in enumerate(moe["experts"]):
        d = dict(e, group_size=gs)
        if fp8:
            d["qweight"] = synthetic.fp8_words(seed + 50 + i, k, n)
        if zp:
            d["zeros"] = synthetic.zero_point_words(seed + 100 + i, k // gs, n)
        ex.append(d)
    bank = torch_ops.ExpertBank(ex, device=dev, bf16=bf16, fp8=fp8)
    csr = wq.wq_csr_from_routes(moe["routes"], moe["n_tokens"], moe["top_k"], moe["n_expert"])
    wts = synthetic.routing_weights(seed + 200, tokens, 2) if weighted else None
    y = torch_ops.grouped_gemm(torch_ops.to_device(moe["a"], dev), bank, csr,
                               topk_weights=None if wts is None else torch_ops.to_device(wts, dev))
    torch.cuda.synchronize()
    ocsr = ref.csr_from_token_routes(moe["n_expert"], moe["n_tokens"], moe["top_k"],
                                     moe["routes"])
    want = ref.grouped_w4a16_gemm(moe["a"], ex, ocsr, group_size=gs, topk_weights=wts,
                                  bf16=bf16, fp8=fp8)
    # fp16 outputs with routing weights, and E4M3 weights, add the fp16 output's own
    # rounding per element (see the dense tolerances above)
    tol = BF16_TOL if bf16 else (FP8_TOL if fp8 or weighted else FP16_TOL)
    res = ref.check(to_host(y), want, **tol)
    print(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} "
          f"rel_frob={res['rel_frob']:.3e} nonfinite={res['nonfinite']}", flush=True)
    assert res["ok"], (label, res)
