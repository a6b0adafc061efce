"""Edge cases of the HIP path through the C ABI, against the CPU oracle on an MI355X:
zero scales (all-zero columns must come out exactly zero), the act_order group_index
check, strided bf16 activations, and the register-only MFMA rate helper."""

import numpy as np
import pytest

import synthetic
from oracle import reference as ref

torch = pytest.importorskip("torch")
wq = pytest.importorskip("weight_only_quantized_gemm_amd")
from weight_only_quantized_gemm_amd import torch_ops  # noqa: E402

pytestmark = pytest.mark.gpu

# bf16 outputs: the output's own rounding (<= 2^-8 of |ref| per element) on top of the GEMM
# bound, relative Frobenius 4e-3 (the bf16 rows' criterion)
BF16_TOL = dict(rel_elem=2.0 ** -8, rel_frob=4e-3)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def say(*args):
    print(*args, flush=True)


def host(t):
    return t.cpu().numpy()


def check(c, want, label, bf16):
    res = ref.check(c.astype(np.float64), want, **(BF16_TOL if bf16 else {}))
    say(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} "
        f"rel_frob={res['rel_frob']:.3e} nonfinite={res['nonfinite']}")
    assert res["ok"], (label, res)


def zero_scale_case(m, k, n, *, zp, bf16, seed):
    """Columns 0..15 have every scale zero, columns 16..31 have zero scales in every other
    group; the rest are ordinary."""
    case = synthetic.dense_case(m, k, n, zp=zp, seed=seed, bf16=bf16)
    s = case["scales"].copy()
    s[:, :16] = 0
    s[::2, 16:32] = 0
    case["scales"] = s
    return case


def run(case, dev, fp32):
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], case["zeros"], device=dev,
                               bf16=case["bf16"])
    c = torch_ops.gemm(torch_ops.to_device(case["a"], dev), w, fp32_reduce=fp32)
    torch.cuda.synchronize()
    out = host(c.view(torch.int16)).view(np.uint16) if case["bf16"] else host(c)
    return ref.bf16_value(out) if case["bf16"] else out.astype(np.float64)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("m,k,n,zp,fp32", [(1, 1024, 512, False, True),     # one-row path
                                           (7, 1024, 512, True, True),      # small-M, split
                                           (16, 2048, 512, True, False),    # small-M direct
                                           (300, 1024, 512, True, False),   # tiled
                                           (64, 2048, 1024, False, True)])  # tiled, split K
def test_zero_scales(dev, m, k, n, zp, fp32, bf16):
    label = f"zero scales m={m} k={k} n={n} zp={zp} fp32={fp32} bf16={bf16}"
    say(label)
    case = zero_scale_case(m, k, n, zp=zp, bf16=bf16, seed=900 + m)
    c = run(case, dev, fp32)
    assert np.all(c[:, :16] == 0), "an all-zero-scale column must be exactly zero"
    want = ref.w4a16_gemm(case["a"], case["qweight"], case["scales"], zeros=case["zeros"],
                          bf16=bf16)
    check(c, want, label, bf16)


@pytest.mark.parametrize("bf16", [False, True])
def test_zero_scales_grouped(dev, bf16):
    tokens, experts, k, n = 150, 3, 512, 512
    label = f"zero scales grouped bf16={bf16}"
    say(label)
    moe = synthetic.moe_case(tokens, experts, k, n, seed=950, bf16=bf16)
    ex = [dict(e) for e in moe["experts"]]
    for e in ex:
        s = e["scales"].copy()
        s[:, :16] = 0
        s[1::2, 16:32] = 0
        e["scales"] = s
    bank = torch_ops.ExpertBank(ex, device=dev, bf16=bf16)
    csr = wq.wq_csr_from_routes(moe["routes"], tokens, 2, experts)
    y = torch_ops.grouped_gemm(torch_ops.to_device(moe["a"], dev), bank, csr)
    torch.cuda.synchronize()
    yh = ref.bf16_value(host(y.view(torch.int16)).view(np.uint16)) if bf16 else host(y).astype(
        np.float64)
    assert np.all(yh[:, :16] == 0)
    ocsr = ref.csr_from_token_routes(experts, tokens, 2, moe["routes"])
    check(yh, ref.grouped_w4a16_gemm(moe["a"], ex, ocsr, bf16=bf16), label, bf16)


@pytest.mark.parametrize("m,k", [(5, 1024), (300, 1024), (3, 16512)])
def test_group_index_is_checked(dev, m, k):
    """The sorted per-position groups change no bit; a group_index that disagrees with the
    layout's groups turns every output into NaN.  K = 16512 takes the per-column gather
    (rows longer than the row-staged gather holds)."""
    n = 512
    case = synthetic.dense_case(m, k, n, act_order=True, seed=960 + m)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], None, case["g_idx"], device=dev)
    a = torch_ops.to_device(case["a"], dev)
    bufs = torch_ops.GemmBuffers(w, m, False)
    with_gi = host(torch_ops.gemm(a, w, buffers=bufs))
    saved = w.group_index
    w.group_index = None
    without = host(torch_ops.gemm(a, w, buffers=bufs))
    assert np.array_equal(with_gi.view(np.uint16), without.view(np.uint16))
    want = ref.w4a16_gemm(case["a"], case["qweight"], case["scales"], g_idx=case["g_idx"])
    check(with_gi, want, f"group_index m={m} k={k}", False)
    bad = saved.clone()
    bad[200] += 1                      # one position claims the next group
    w.group_index = bad
    broken = host(torch_ops.gemm(a, w, buffers=bufs))
    torch.cuda.synchronize()
    assert np.isnan(broken).all()
    w.group_index = saved


@pytest.mark.parametrize("m,fp32", [(20, False), (64, True), (5, True), (12, True)])
def test_strided_bf16_activations(dev, m, fp32):
    """lda > k with bf16 activations on the tiled kernel (unsplit and split) and the small-M
    kernel."""
    k, n = 512, 256
    case = synthetic.dense_case(m, k, n, seed=13, bf16=True)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device=dev, bf16=True)
    wide = torch.zeros((m, k + 64), dtype=torch.bfloat16, device=dev)
    wide[:, :k] = torch_ops.to_device(case["a"], dev)
    c = torch_ops.gemm(wide[:, :k], w, fp32_reduce=fp32)
    torch.cuda.synchronize()
    out = ref.bf16_value(host(c.view(torch.int16)).view(np.uint16))
    want = ref.w4a16_gemm(case["a"], case["qweight"], case["scales"], bf16=True)
    check(out, want, f"bf16 lda > k m={m} fp32={fp32}", True)


def test_mfma_rate_helper_runs(dev):
    """The register-only MFMA loop: the stored sums equal the closed form of its operands
    (every thread of a wave keeps the same 128 x 64 product), and the operation count is
    waves x iterations x 8 x 32768."""
    ops = torch.zeros((6, 64, 8), dtype=torch.float16, device=dev)
    ops[:4] = 1.0                       # A operands all ones
    ops[4:] = 2.0                       # B operands all twos
    sink = torch.zeros(256 * 512, dtype=torch.float32, device=dev)
    iters = 8
    flops = wq.wq_mfma_rate(ops, iters, sink, sink.numel())
    torch.cuda.synchronize()
    assert flops == 256 * 8 * iters * 8 * 32768
    # each accumulator element is iters * 16 * (1 * 2); a lane holds 4 x 2 blocks x 16
    assert torch.all(sink == iters * 16 * 2.0 * 8 * 16).item()
