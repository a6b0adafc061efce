"""wq_gemm_noalloc (the entry point for callers that cannot allocate) against wq_gemm with
caller-owned scratch, through the C ABI: the same kernels, so the same bits, and both within
the oracle's tolerance.  Each case runs two calls in a row, the second smaller, so that the
static scratch is reused with stale contents."""

import numpy as np
import pytest

import synthetic
from oracle import reference as ref

torch = pytest.importorskip("torch")
wq = pytest.importorskip("weight_only_quantized_gemm_amd")
from weight_only_quantized_gemm_amd import torch_ops  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def run_both(case, dev, fp32):
    """(wq_gemm output, wq_gemm_noalloc output, planned splits) as numpy fp16."""
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], case["zeros"], case["g_idx"],
                               device=dev)
    m, k, n = case["m"], case["k"], case["n"]
    a = torch_ops.to_device(case["a"], dev)
    flags = w.flags(fp32)
    _, splits = wq.wq_gemm_plan(m, n, k, flags=flags)
    with_bufs = torch_ops.gemm(a, w, fp32_reduce=fp32)
    out = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
    wq.wq_gemm_noalloc(a, w.b, out, w.s, m=m, n=n, k=k, zero_points=w.z, perm=w.perm,
                       group_index=w.group_index, flags=flags)
    torch.cuda.synchronize()
    return with_bufs.cpu().numpy(), out.cpu().numpy(), splits


# (first call, second smaller call): m, k, n, zp, act_order, fp32
PAIRS = [
    ((1, 2048, 512, False, False, True), (1, 1024, 256, False, False, True)),    # small-M split
    ((7, 2048, 512, True, False, True), (3, 1024, 256, True, False, True)),      # zp, split
    ((300, 1024, 512, False, True, False), (100, 512, 256, False, True, False)),  # act_order
    ((64, 4096, 8192, False, False, True), (24, 2048, 14336, False, False, True)),  # tiled split
    ((16, 1024, 512, False, True, True), (5, 512, 256, False, True, True)),      # both scratches
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_caller_scratch(dev, first, second):
    used = []
    for i, (m, k, n, zp, act, fp32) in enumerate((first, second)):
        label = f"noalloc call {i}: m={m} k={k} n={n} zp={zp} act_order={act} fp32={fp32}"
        print(label, flush=True)
        case = synthetic.dense_case(m, k, n, zp=zp, act_order=act, seed=1000 + 7 * m + k + i)
        base, got, splits = run_both(case, dev, fp32)
        used.append(splits > 1 or act)
        assert np.array_equal(base.view(np.uint16), got.view(np.uint16)), label
        want = ref.w4a16_gemm(case["a"], case["qweight"], case["scales"], zeros=case["zeros"],
                              g_idx=case["g_idx"])
        res = ref.check(got, want)
        print(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e}", flush=True)
        assert res["ok"], (label, res)
    assert all(used), "every case must use the static scratch"


def test_noalloc_shrinks_a_split_that_does_not_fit(dev):
    """A tiled split whose partials exceed the static array (1000 x 4096 outputs, K = 14336:
    the library's own choice is four splits, 64 MiB) runs with the largest split that fits
    (two, 31 MiB): the same bits as wq_gemm with split_k = 2, within the oracle's tolerance
    on sampled columns."""
    m, k, n = 1000, 14336, 4096
    fp32 = wq.WQ_FLAG_FP32_REDUCE
    _, auto = wq.wq_gemm_plan(m, n, k, flags=fp32)
    assert auto * m * n * 4 > wq.WQ_NOALLOC_SCRATCH_BYTES >= 2 * m * n * 4
    case = synthetic.dense_case(m, k, n, seed=1333)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device=dev)
    a = torch_ops.to_device(case["a"], dev)
    for i in range(2):   # twice: the second call reuses the array's stale partials
        base = torch_ops.gemm(a, w, fp32_reduce=True, split_k=2)
        out = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
        wq.wq_gemm_noalloc(a, w.b, out, w.s, m=m, n=n, k=k, flags=w.flags(True))
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(base.cpu().numpy().view(np.uint16), got.view(np.uint16)), i
    cols = np.r_[0:64, n - 64:n]
    want = ref.w4a16_gemm(case["a"], case["qweight"], case["scales"], columns=cols)
    res = ref.check(got[:, cols], want)
    print(f"noalloc shrunk split: max_err={res['max_err']:.3e} tol={res['tol']:.3e}", flush=True)
    assert res["ok"], res


def test_noalloc_rejects_oversized_scratch_before_launch(dev):
    """An act_order gather larger than the static array is refused with WQ_ERR_WORKSPACE."""
    m, k, n = 8192, 4096, 256          # 64 MiB of gathered activations
    assert m * k * 2 > wq.WQ_NOALLOC_SCRATCH_BYTES
    with pytest.raises(wq.WQError) as err:
        wq.wq_gemm_noalloc(0x1000, 0x2000, 0x3000, 0x4000, m=m, n=n, k=k, perm=0x5000,
                           flags=wq.WQ_FLAG_ACT_ORDER)
    assert err.value.code == wq.WQ_ERR_WORKSPACE
