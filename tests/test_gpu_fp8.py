"""Parity of the W8A16 path (WQ_FLAG_FP8: E4M3 weights) with the CPU oracle, on an MI355X.

The repack and the dequant export must match bit for bit; the export of every E4M3 code
with unit scales pins the hardware conversion (OCP E4M3 "fn": bias 7, 0x7F / 0xFF NaN).
GEMM outputs are fp16 and must satisfy |C - ref| <= 2^-11 * |ref| + 2e-3 * rms(ref) + 1e-3
per element (2^-11: the output's own rounding, as E4M3 magnitudes span 2^-9 .. 448 and
leave large elements far above the rms) and ||C - ref||_F / ||ref||_F <= 1e-3.
"""

import numpy as np
import pytest

import synthetic
from conftest import by_column_chunks
from oracle import layout
from oracle import reference as ref

torch = pytest.importorskip("torch")
wq = pytest.importorskip("weight_only_quantized_gemm_amd")
from weight_only_quantized_gemm_amd import torch_ops  # noqa: E402

pytestmark = pytest.mark.gpu

FP8_TOL = dict(rel_elem=2.0 ** -11)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def say(*args):
    print(*args, flush=True)


def host(t):
    return t.cpu().numpy()


def assert_parity(c, want, label):
    res = ref.check(c, want, **FP8_TOL)
    say(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} "
        f"rel_frob={res['rel_frob']:.3e} nonfinite={res['nonfinite']}")
    assert res["ok"], (label, res)


def words_of(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [K][N] -> K-major words [K/4][N], byte i = row 4r + i."""
    c = codes.astype(np.uint32).reshape(codes.shape[0] // 4, 4, codes.shape[1])
    return c[:, 0] | (c[:, 1] << 8) | (c[:, 2] << 16) | (c[:, 3] << 24)


def test_fp8_repack_matches_layout_bitwise(dev):
    k, n = 384, 256
    say(f"fp8 repack k={k} n={n}")
    codes = np.random.default_rng(6000).integers(0, 256, size=(k, n)).astype(np.uint8)
    out = torch.empty(k * n // 4, dtype=torch.int32, device=dev)
    wq.wq_repack_fp8(torch_ops.to_device(words_of(codes), dev), out, k, n)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), layout.repack_fp8_loops(codes))


@pytest.mark.parametrize("unit_scales,gs", [(True, 128), (False, 128), (False, -1)])
def test_fp8_dequant_of_every_code(dev, unit_scales, gs):
    """Every byte value appears (codes (row + 3 col) mod 256); with unit scales the export
    is the conversion itself, exact in fp16."""
    k, n = 512, 256
    say(f"fp8 dequant of every code unit_scales={unit_scales} group_size={gs}")
    rows, cols = np.meshgrid(np.arange(k), np.arange(n), indexing="ij")
    codes = ((rows + 3 * cols) % 256).astype(np.uint8)
    groups = 1 if gs == -1 else k // 128
    s = (np.ones((groups, n), np.float16) if unit_scales
         else synthetic.scales(6001, groups, n))
    w = torch_ops.PackedWeight(words_of(codes), s, device=dev, group_size=gs, fp8=True)
    out = torch.empty((k, n), dtype=torch.float16, device=dev)
    wq.wq_dequant(w.b, w.s, None, out, k=k, n=n, flags=wq.WQ_FLAG_FP8, group_size=gs)
    torch.cuda.synchronize()
    want = ref.dequantize_fp16(ref.w8a16_weights(words_of(codes), s, group_size=gs))
    got = host(out)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok].view(np.uint16), want[ok].view(np.uint16))


FP8_SHAPES = [
    # m, k, n, group_size, fp32_reduce, split_k
    (1, 4096, 512, 128, False, 0),
    (1, 2048, 256, -1, True, 3),
    (5, 1024, 512, 128, True, 0),
    (16, 2048, 256, -1, False, 0),
    (3, 8192, 256, 128, False, 0),
    (17, 1024, 256, 128, False, 0),
    (300, 1024, 512, 128, False, 0),
    (257, 384, 256, -1, False, 0),
    (513, 2048, 768, 128, False, 0),
    (11, 2048, 256, 128, False, 0),   # direct activation tiles
    (16, 4096, 4096, 128, False, 0),  # direct, 8 waves x 4 groups of two vectors each
    (14, 4096, 256, -1, True, 2),
]


@pytest.mark.parametrize("m,k,n,gs,fp32,split", FP8_SHAPES)
def test_fp8_gemm_matches_oracle(dev, m, k, n, gs, fp32, split):
    label = f"fp8 gemm m={m} k={k} n={n} group_size={gs} fp32={fp32} split={split}"
    say(label)
    case = synthetic.fp8_case(m, k, n, group_size=gs, seed=6100 + m + k)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device=dev, group_size=gs,
                               fp8=True)
    c = host(torch_ops.gemm(torch_ops.to_device(case["a"], dev), w, fp32_reduce=fp32,
                            split_k=split))
    torch.cuda.synchronize()
    want = ref.w8a16_gemm(case["a"], case["qweight"], case["scales"], group_size=gs)
    assert_parity(c, want, label)


def test_fp8_decode_config_in_full(dev):
    m, k, n = 1, 4096, 14336
    say("fp8 decode shape M=1 K=4096 N=14336 g128 (full)")
    case = synthetic.fp8_case(m, k, n, seed=6200)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device=dev, fp8=True)
    c = host(torch_ops.gemm(torch_ops.to_device(case["a"], dev), w, fp32_reduce=True))
    torch.cuda.synchronize()
    assert_parity(c, ref.w8a16_gemm(case["a"], case["qweight"], case["scales"]), "fp8 decode")


def test_fp8_prefill_shape_in_full(dev):
    m, k, n = 2048, 4096, 14336
    say("fp8 prefill shape M=2048 K=4096 N=14336 g128 (every output)")
    case = synthetic.fp8_case(m, k, n, seed=6300)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device=dev, fp8=True)
    c = host(torch_ops.gemm(torch_ops.to_device(case["a"], dev), w))
    torch.cuda.synchronize()
    want = by_column_chunks(
        lambda cols: ref.w8a16_gemm(case["a"], case["qweight"], case["scales"], columns=cols), n)
    assert_parity(c, want, "fp8 prefill")


@pytest.mark.parametrize("tokens,experts,k,n,weighted", [(40, 4, 256, 256, False),
                                                         (300, 3, 512, 512, True),
                                                         (700, 2, 256, 256, False)])
def test_fp8_grouped_matches_oracle(dev, tokens, experts, k, n, weighted):
    label = f"fp8 grouped tokens={tokens} experts={experts} k={k} n={n} weighted={weighted}"
    say(label)
    moe = synthetic.moe_case(tokens, experts, k, n, seed=6400 + tokens)
    ex = [dict(qweight=synthetic.fp8_words(6500 + e, k, n), scales=x["scales"])
          for e, x in enumerate(moe["experts"])]
    bank = torch_ops.ExpertBank(ex, device=dev, fp8=True)
    csr = wq.wq_csr_from_routes(moe["routes"], moe["n_tokens"], moe["top_k"], moe["n_expert"])
    wts = synthetic.routing_weights(6600 + tokens, tokens, 2) if weighted else None
    y = host(torch_ops.grouped_gemm(torch_ops.to_device(moe["a"], dev), bank, csr,
                                    topk_weights=None if wts is None
                                    else torch_ops.to_device(wts, dev)))
    torch.cuda.synchronize()
    ocsr = ref.csr_from_token_routes(moe["n_expert"], moe["n_tokens"], moe["top_k"],
                                     moe["routes"])
    want = ref.grouped_w4a16_gemm(moe["a"], ex, ocsr, topk_weights=wts, fp8=True)
    assert_parity(y, want, label)


@pytest.mark.parametrize("m", [5, 300])
def test_fp8_from_block_checkpoint(dev, m):
    """Row-major E4M3 weights with one bf16 inverse scale per 128 x 128 block (the pages'
    block-FP8 checkpoint): the device transforms match the layout and scale oracles bit for
    bit, and the product matches the oracle."""
    n, k = 512, 768
    say(f"fp8 block checkpoint m={m} n={n} k={k}")
    rng = np.random.default_rng(6700 + m)
    w_nk = synthetic.FP8_CODES[rng.integers(0, 254, size=(n, k))].astype(np.uint8)
    inv = (0x3B80 + 0x20 * rng.integers(0, 5, size=(n // 128, k // 128))).astype(np.uint16)
    w = torch_ops.PackedWeight.from_fp8_blocks(w_nk, inv, device=dev)
    assert np.array_equal(host(w.b).view(np.uint32), layout.repack_fp8_loops(w_nk.T.copy()))
    scales = ref.fp8_block_scales(inv)
    assert np.array_equal(host(w.s).view(np.uint16),
                          layout.repack_scales(scales).view(np.uint16))
    a = synthetic.activations(6800 + m, m, k)
    c = host(torch_ops.gemm(torch_ops.to_device(a, dev), w))
    torch.cuda.synchronize()
    assert_parity(c, ref.w8a16_gemm(a, ref.fp8_rows_to_words(w_nk), scales),
                  f"fp8 block checkpoint m={m}")


BF16_TOL = dict(rel_elem=2.0 ** -8, rel_frob=4e-3)  # bf16 outputs (see test_gpu_bf16.py)


@pytest.mark.parametrize("m,k,n,gs", [(1, 4096, 512, 128), (11, 2048, 256, -1),
                                      (300, 1024, 512, 128), (17, 768, 256, -1)])
def test_fp8_with_bf16_activations(dev, m, k, n, gs):
    label = f"fp8 bf16 gemm m={m} k={k} n={n} group_size={gs}"
    say(label)
    case = synthetic.fp8_case(m, k, n, group_size=gs, seed=6900 + m, bf16=True)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device=dev, group_size=gs,
                               bf16=True, fp8=True)
    c = torch_ops.gemm(torch_ops.to_device(case["a"], dev), w)
    torch.cuda.synchronize()
    assert c.dtype == torch.bfloat16
    want = ref.w8a16_gemm(case["a"], case["qweight"], case["scales"], group_size=gs, bf16=True)
    res = ref.check(c.float().cpu().numpy(), want, **BF16_TOL)
    say(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} rel_frob={res['rel_frob']:.3e}")
    assert res["ok"], (label, res)


def fp8_proj(seed, k, cols, bf16=False):
    sc = synthetic.scales_bf16 if bf16 else synthetic.scales
    return dict(qweight=synthetic.fp8_words(seed, k, cols), scales=sc(seed + 1, k // 128, cols))


@pytest.mark.parametrize("m,k,i,bf16", [(1, 4096, 512, False), (4, 2048, 256, True),
                                        (300, 1024, 256, False), (130, 768, 256, True)])
def test_fp8_swiglu_activation(dev, m, k, i, bf16):
    """The SwiGLU epilogue over E4M3 gate/up weights (paired small-M kernel and tiled)."""
    label = f"fp8 swiglu m={m} k={k} i={i} bf16={bf16}"
    say(label)
    gate, up = fp8_proj(7000 + m, k, i, bf16), fp8_proj(7010 + m, k, i, bf16)
    a = (synthetic.activations_bf16 if bf16 else synthetic.activations)(7020 + m, m, k)
    w = torch_ops.PackedWeight.gate_up(gate, up, device=dev, bf16=bf16, fp8=True)
    act = torch_ops.gemm(torch_ops.to_device(a, dev), w)
    torch.cuda.synchronize()
    assert act.shape == (m, i)
    want = ref.swiglu_activation(a, gate, up, bf16=bf16, fp8=True)
    tol = BF16_TOL if bf16 else dict(rel_elem=2.0 ** -10)  # the activation's heavy tails
    res = ref.check(act.float().cpu().numpy(), want, **tol)
    say(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} rel_frob={res['rel_frob']:.3e}")
    assert res["ok"], (label, res)


def test_fp8_grouped_swiglu(dev):
    """MoE gate/up with E4M3 weights: grouped SwiGLU over pair rows."""
    tokens, experts, k, i = 200, 3, 512, 256
    say(f"fp8 grouped swiglu tokens={tokens} experts={experts} k={k} i={i}")
    moe = synthetic.moe_case(tokens, experts, k, 2 * i, seed=7100)
    ex = [dict(gate=fp8_proj(7200 + e, k, i), up=fp8_proj(7300 + e, k, i))
          for e in range(experts)]
    bank = torch_ops.ExpertBank(ex, device=dev, fp8=True)
    csr = wq.wq_csr_from_routes(moe["routes"], tokens, 2, experts)
    y = host(torch_ops.grouped_gemm(torch_ops.to_device(moe["a"], dev), bank, csr))
    torch.cuda.synchronize()
    ocsr = ref.csr_from_token_routes(experts, tokens, 2, moe["routes"])
    want = np.full((len(ocsr["ex_pairs"]), i), np.nan)
    for s_i, e in enumerate(ocsr["ex_ids"]):
        rows = [ocsr["ex_pairs"][j] for j in range(ocsr["ex_off"][s_i], ocsr["ex_off"][s_i + 1])]
        toks = [ocsr["pair_tok"][p] for p in rows]
        want[rows, :] = ref.swiglu_activation(moe["a"][toks, :], ex[e]["gate"], ex[e]["up"],
                                              fp8=True)
    res = ref.check(y, want, rel_elem=2.0 ** -10)
    say(f"fp8 grouped swiglu: max_err={res['max_err']:.3e} tol={res['tol']:.3e}")
    assert res["ok"], res
