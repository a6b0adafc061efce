"""Parity of the bf16-activation path (WQ_FLAG_BF16) with the CPU oracle, on an MI355X.

Activations, scales and outputs are bf16; codes and zero points are as on the fp16 path.
The dequant export and integer-valued products must match bit for bit.  GEMM outputs must
satisfy |C - ref| <= 2^-8 * |ref| + 2e-3 * rms(ref) + 1e-3 per element and
||C - ref||_F / ||ref||_F <= 4e-3 with no non-finite value: the rounding of one bf16
output is at most 2^-9 of its magnitude (2^-8 leaves room for the fp32 accumulation), and
uniform rounding noise of that size alone gives a Frobenius ratio near 2^-9 / sqrt(3).
Where the reference itself is a rounded bf16 value (the chain's activation), the two
roundings may land one bf16 ulp apart near a rounding boundary: up to 2^-7 of the value.
The chain's down projection is checked on the activation the GPU produced; end to end,
each output may also move by the activation's allowance carried through the weights,
2^-7 * sum_i |act_i| |W_ij|.
"""

import numpy as np
import pytest

import synthetic
from conftest import by_column_chunks
from oracle import reference as ref

torch = pytest.importorskip("torch")
wq = pytest.importorskip("weight_only_quantized_gemm_amd")
from weight_only_quantized_gemm_amd import torch_ops  # noqa: E402

pytestmark = pytest.mark.gpu

BF16_TOL = dict(rel_elem=2.0 ** -8, rel_frob=4e-3)
BF16_ROUNDED_REF_TOL = dict(rel_elem=2.0 ** -7, rel_frob=4e-3)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def say(*args):
    print(*args, flush=True)


def host(t):
    """Values of a result tensor as numpy (bf16 widened to fp32, which is exact)."""
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def assert_parity(c, want, label, tol=BF16_TOL):
    res = ref.check(c, want, **tol)
    say(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} "
        f"rel_frob={res['rel_frob']:.3e} nonfinite={res['nonfinite']}")
    assert res["ok"], (label, res)


def packed(case, dev):
    return torch_ops.PackedWeight(case["qweight"], case["scales"], case.get("zeros"),
                                  case.get("g_idx"), device=dev,
                                  group_size=case.get("group_size", 128), bf16=True)


def oracle_gemm(case, columns=None):
    return ref.w4a16_gemm(case["a"], case["qweight"], case["scales"], zeros=case.get("zeros"),
                          g_idx=case.get("g_idx"), group_size=case.get("group_size", 128),
                          columns=columns, bf16=True)


BF16_SHAPES = [
    # m, k, n, group_size, zp, act_order, fp32_reduce, split_k
    (1, 4096, 512, 128, False, False, False, 0),
    (1, 1024, 512, 128, True, False, True, 3),
    (5, 2048, 256, 64, True, False, True, 0),
    (16, 1024, 512, 32, False, True, False, 0),
    (3, 768, 256, 16, True, False, False, 0),
    (7, 1536, 256, 48, False, False, True, 0),
    (17, 1024, 256, 128, False, False, False, 0),
    (300, 1024, 512, 128, True, True, False, 0),
    (257, 768, 256, 48, True, False, False, 0),
    (513, 2048, 768, 256, False, True, False, 0),
    (64, 1024, 256, 32, True, False, False, 0),
    (130, 1536, 512, 16, False, False, False, 0),
    (40, 1024, 256, -1, True, False, False, 0),
    # direct activation tiles: 8 waves x 4 groups (one block), 4 waves x 8 (two blocks)
    (12, 4096, 4096, 64, True, False, False, 0),
    (16, 4096, 8192, 128, True, False, True, 0),
    # one row: biased operands on 4x4x4 products, every unit size
    (1, 2048, 512, 16, True, False, True, 0),
    (1, 1024, 768, 32, False, False, False, 0),
    (1, 2048, 256, 64, True, False, False, 0),
    (1, 1024, 256, -1, True, False, True, 0),
    # 9..16 rows with activation operands in registers
    (9, 2048, 256, 128, True, False, False, 0),
    (13, 1024, 512, 16, False, False, True, 2),
    # two column blocks per wave
    (16, 1024, 8192, 128, True, False, False, 0),
    (10, 2048, 8192, 16, False, False, True, 0),
    # tiled kernel split along K with the fp32 reduce (128-row tiles)
    (64, 2048, 512, 128, True, False, True, 0),
    (300, 1024, 768, 64, False, True, True, 0),
    # eight staged waves with two to four rows, each staging its own share
    (3, 8192, 256, 128, True, False, False, 0),
    (4, 6144, 512, -1, False, False, False, 0),
    # long K on sixteen waves, each staging its own groups' activations and scales
    (1, 14336, 512, 128, True, False, False, 0),
    (4, 12288, 256, 64, False, False, False, 0),
    (3, 20480, 256, 128, True, False, False, 0),
    # K split into ranges of at most 16 groups (four or more rows, grid beyond the CUs)
    (6, 14336, 4096, 128, True, False, True, 0),
    (4, 11008, 8192, 64, False, True, True, 0),
]


@pytest.mark.parametrize("m,k,n,gs,zp,act_order,fp32,split", BF16_SHAPES)
def test_bf16_gemm_matches_oracle(dev, m, k, n, gs, zp, act_order, fp32, split):
    label = (f"bf16 gemm m={m} k={k} n={n} group_size={gs} zp={zp} act_order={act_order} "
             f"fp32={fp32} split={split}")
    say(label)
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=5000 + m + k + gs, bf16=True)
    w = packed(case, dev)
    c = torch_ops.gemm(torch_ops.to_device(case["a"], dev), w, fp32_reduce=fp32, split_k=split)
    torch.cuda.synchronize()
    assert c.dtype == torch.bfloat16
    assert_parity(host(c), oracle_gemm(case), label)


@pytest.mark.parametrize("gs,k,zp", [(128, 1024, True), (32, 1024, False), (48, 768, True),
                                     (-1, 512, True)])
def test_bf16_dequant_export_bitwise(dev, gs, k, zp):
    n = 256
    say(f"bf16 dequant export group_size={gs} k={k} zp={zp}")
    case = synthetic.dense_case(1, k, n, zp=zp, group_size=gs, seed=5100 + k, bf16=True)
    w = packed(case, dev)
    out = torch.empty((k, n), dtype=torch.bfloat16, device=dev)
    flags = wq.WQ_FLAG_BF16 | (wq.WQ_FLAG_HAS_ZP if zp else 0)
    wq.wq_dequant(w.b, w.s, w.z, out, k=k, n=n, flags=flags, group_size=gs)
    torch.cuda.synchronize()
    exact = ref.w4a16_weights(case["qweight"], case["scales"], zeros=case.get("zeros"),
                              group_size=gs, bf16=True)
    assert np.array_equal(host(out).astype(np.float64), ref.round_bf16(exact))


@pytest.mark.parametrize("m,k,zp", [(1, 1024, False), (9, 512, True), (200, 512, True)])
def test_bf16_integer_products_are_bit_exact(dev, m, k, zp):
    """Unit scales and small-integer activations: every fp32 partial sum is an exact
    integer, so the output must be the bf16 rounding of the exact product, bit for bit."""
    n = 256
    say(f"bf16 integer products m={m} k={k} zp={zp}")
    rng = np.random.default_rng(5200 + m)
    a = rng.integers(-3, 4, size=(m, k)).astype(np.float32)
    a_bits = (a.view(np.uint32) >> 16).astype(np.uint16)  # small integers are exact in bf16
    groups = k // 128
    s_bits = np.full((groups, n), 0x3F80, dtype=np.uint16)  # 1.0
    qw = synthetic.qweight_words(5201 + m, k, n)
    zw = synthetic.zero_point_words(5202 + m, groups, n) if zp else None
    w = torch_ops.PackedWeight(qw, s_bits, zw, device=dev, bf16=True)
    c = host(torch_ops.gemm(torch_ops.to_device(a_bits, dev), w))
    torch.cuda.synchronize()
    exact = ref.w4a16_gemm(a_bits, qw, s_bits, zeros=zw, bf16=True)
    assert np.array_equal(c.astype(np.float64), ref.round_bf16(exact))


def test_bf16_decode_config_in_full(dev):
    m, k, n = 1, 4096, 14336
    say("bf16 decode config M=1 K=4096 N=14336 g128 (full)")
    case = synthetic.dense_case(m, k, n, seed=5300, bf16=True)
    w = packed(case, dev)
    c = torch_ops.gemm(torch_ops.to_device(case["a"], dev), w, fp32_reduce=True)
    torch.cuda.synchronize()
    assert_parity(host(c), oracle_gemm(case), "bf16 decode config")


def test_bf16_prefill_config_in_full(dev):
    m, k, n = 2048, 4096, 14336
    say("bf16 prefill config M=2048 K=4096 N=14336 g128 act_order (every output)")
    case = synthetic.dense_case(m, k, n, act_order=True, seed=5400, bf16=True)
    w = packed(case, dev)
    c = host(torch_ops.gemm(torch_ops.to_device(case["a"], dev), w))
    torch.cuda.synchronize()
    want = by_column_chunks(lambda cols: oracle_gemm(case, columns=cols), n)
    assert_parity(c, want, "bf16 prefill")


@pytest.mark.parametrize("tokens,experts,k,n,zp,weighted", [(40, 4, 256, 256, False, False),
                                                            (300, 3, 512, 512, True, True),
                                                            (700, 2, 256, 256, False, True)])
def test_bf16_grouped_matches_oracle(dev, tokens, experts, k, n, zp, weighted):
    label = f"bf16 grouped tokens={tokens} experts={experts} k={k} n={n} zp={zp} w={weighted}"
    say(label)
    moe = synthetic.moe_case(tokens, experts, k, n, seed=5500 + tokens, bf16=True)
    ex = [dict(e) for e in moe["experts"]]
    if zp:
        for i, e in enumerate(ex):
            e["zeros"] = synthetic.zero_point_words(5600 + i, k // 128, n)
    bank = torch_ops.ExpertBank(ex, device=dev, bf16=True)
    csr = wq.wq_csr_from_routes(moe["routes"], moe["n_tokens"], moe["top_k"], moe["n_expert"])
    wts = synthetic.routing_weights(5700 + tokens, tokens, 2) if weighted else None
    y = torch_ops.grouped_gemm(torch_ops.to_device(moe["a"], dev), bank, csr,
                               topk_weights=None if wts is None else torch_ops.to_device(wts, dev))
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    ocsr = ref.csr_from_token_routes(moe["n_expert"], moe["n_tokens"], moe["top_k"],
                                     moe["routes"])
    want = ref.grouped_w4a16_gemm(moe["a"], ex, ocsr, topk_weights=wts, bf16=True)
    assert_parity(host(y), want, label)


def bf16_weights(seed, k, cols, zp, group_size=128):
    groups = 1 if group_size == -1 else k // group_size
    w = dict(qweight=synthetic.qweight_words(seed, k, cols),
             scales=synthetic.scales_bf16(seed + 1, groups, cols))
    if zp:
        w["zeros"] = synthetic.zero_point_words(seed + 2, groups, cols)
    return w


@pytest.mark.parametrize("m,k,i,zp,gs", [(1, 4096, 1024, False, 128), (4, 1024, 256, True, 32),
                                         (300, 1024, 256, True, 128), (100, 768, 256, False, 48)])
def test_bf16_swiglu_activation_matches_oracle(dev, m, k, i, zp, gs):
    label = f"bf16 swiglu m={m} k={k} i={i} zp={zp} group_size={gs}"
    say(label)
    gate, up = bf16_weights(5800 + m, k, i, zp, gs), bf16_weights(5810 + m, k, i, zp, gs)
    a = synthetic.activations_bf16(5820 + m, m, k)
    w = torch_ops.PackedWeight.gate_up(gate, up, device=dev, group_size=gs, bf16=True)
    act = torch_ops.gemm(torch_ops.to_device(a, dev), w)
    torch.cuda.synchronize()
    assert act.shape == (m, i) and act.dtype == torch.bfloat16
    want = ref.swiglu_activation(a, gate, up, group_size=gs, bf16=True)
    assert_parity(host(act), want, label)


def test_bf16_swiglu_mlp_chain_matches_oracle(dev):
    m, h, i = 200, 512, 768
    say(f"bf16 swiglu mlp chain m={m} hidden={h} intermediate={i}")
    gate, up, down = bf16_weights(5900, h, i, True), bf16_weights(5910, h, i, True), \
        bf16_weights(5920, i, h, True)
    a = synthetic.activations_bf16(5930, m, h)
    wgu = torch_ops.PackedWeight.gate_up(gate, up, device=dev, bf16=True)
    wd = torch_ops.PackedWeight(down["qweight"], down["scales"], down["zeros"], device=dev,
                                bf16=True)
    act = torch_ops.gemm(torch_ops.to_device(a, dev), wgu)
    out = host(torch_ops.gemm(act, wd))
    torch.cuda.synchronize()
    act_want, want = ref.swiglu_mlp_bf16(a, gate, up, down)
    act_got = host(act).astype(np.float64)
    assert_parity(act_got, act_want, "bf16 chain activation", tol=BF16_ROUNDED_REF_TOL)
    w_down = ref.w4a16_weights(down["qweight"], down["scales"], zeros=down["zeros"], bf16=True)
    assert_parity(out, act_got @ w_down, "bf16 chain down projection on the GPU activation")
    carried = 2.0 ** -7 * (np.abs(act_want) @ np.abs(w_down))
    err = np.abs(out - want) - carried - 2.0 ** -8 * np.abs(want) - 1e-3
    say(f"bf16 chain end to end: worst excess {err.max():.3e}")
    assert err.max() <= 0.0
