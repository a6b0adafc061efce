"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Integer and byte work (repack, dequant export, integer-valued pins) must match bit for
bit; GEMM outputs must satisfy max |C - ref| <= 2e-3 * rms(ref) + 1e-3 and
||C - ref||_F / ||ref||_F <= 1e-3 with no non-finite value.
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


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def say(*args):
    print(*args, flush=True)


def host(t):
    return t.cpu().numpy()


def gpu_gemm(case, dev, *, fp32_reduce=False, split_k=0, a=None):
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], case.get("zeros"),
                               case.get("g_idx"), device=dev,
                               group_size=case.get("group_size", 128))
    a_d = torch_ops.to_device(case["a"] if a is None else a, dev)
    c = torch_ops.gemm(a_d, w, fp32_reduce=fp32_reduce, split_k=split_k)
    torch.cuda.synchronize()
    return host(c)


def oracle_gemm(case, columns=None):
    return ref.w4a16_gemm(case["a"], case["qweight"], case["scales"], zeros=case.get("zeros"),
                          g_idx=case.get("g_idx"), group_size=case.get("group_size", 128),
                          columns=columns)


def assert_parity(c, want, label, rel_elem=0.0):
    res = ref.check(c, want, rel_elem=rel_elem)
    say(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} "
        f"rel_frob={res['rel_frob']:.3e} nonfinite={res['nonfinite']}")
    assert res["ok"], (label, res)


# --------------------------------------------------------------------------- layout

@pytest.mark.parametrize("k,n,use_perm", [(128, 256, False), (1024, 512, False),
                                          (1024, 512, True), (4096, 4096, True)])
def test_repack_matches_reference_layout_bitwise(dev, k, n, use_perm):
    say(f"repack k={k} n={n} perm={use_perm}")
    qw = synthetic.qweight_words(100 + k + n, k, n)
    perm = synthetic.permutation(7, k).astype(np.int32) if use_perm else None
    out = torch.empty(k * n // 8, dtype=torch.int32, device=dev)
    wq.wq_repack_b(torch_ops.to_device(qw, dev), out, k, n,
                   perm=None if perm is None else torch_ops.to_device(perm, dev))
    torch.cuda.synchronize()
    want = layout.repack_b(qw, perm)
    assert np.array_equal(host(out).view(np.uint32), want)


def test_scale_and_zero_repack_bitwise(dev):
    k, n = 1024, 512
    s = synthetic.scales(1, k // 128, n)
    z = synthetic.zero_point_words(2, k // 128, n)
    s_out = torch.empty(s.size, dtype=torch.float16, device=dev)
    z_out = torch.empty(z.size, dtype=torch.int32, device=dev)
    wq.wq_repack_scales(torch_ops.to_device(s, dev), s_out, k, n)
    wq.wq_repack_zeros(torch_ops.to_device(z, dev), z_out, k, n)
    torch.cuda.synchronize()
    assert np.array_equal(host(s_out).view(np.uint16), layout.repack_scales(s).view(np.uint16))
    assert np.array_equal(host(z_out).view(np.uint32), layout.repack_zero_points(z))


@pytest.mark.parametrize("zp,act_order", [(False, False), (True, False), (False, True)])
def test_dequant_export_bitwise(dev, zp, act_order):
    k, n = 1024, 512
    say(f"dequant zp={zp} act_order={act_order}")
    case = synthetic.dense_case(1, k, n, zp=zp, act_order=act_order, seed=11)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], case["zeros"], case["g_idx"],
                               device=dev)
    out = torch.empty((k, n), dtype=torch.float16, device=dev)
    wq.wq_dequant(w.b, w.s, w.z, out, k=k, n=n, flags=wq.WQ_FLAG_HAS_ZP if zp else 0)
    torch.cuda.synchronize()
    exact = ref.w4a16_weights(case["qweight"], case["scales"], zeros=case["zeros"],
                              g_idx=case["g_idx"])
    if act_order:
        perm, _ = ref.act_order_perm(case["g_idx"], 128)
        exact = exact[perm, :]
    want = ref.dequantize_fp16(exact)
    assert np.array_equal(host(out).view(np.uint16), want.view(np.uint16))


# --------------------------------------------------------------------------- GEMM parity

SMALL_SHAPES = [
    # m, k, n, zp, act_order, fp32_reduce, split_k
    (1, 128, 256, False, False, False, 0),
    (1, 1024, 512, False, False, True, 0),
    (1, 1024, 512, True, False, True, 3),
    (3, 384, 256, True, False, False, 0),
    (7, 1024, 768, False, True, True, 0),
    (16, 1024, 256, False, False, False, 0),
    (16, 2048, 512, True, False, True, 0),
    (16, 2048, 512, False, False, True, 16),
    (17, 1024, 256, False, False, False, 0),
    (64, 512, 512, True, False, False, 0),
    (100, 1024, 512, False, True, False, 0),
    (255, 256, 256, False, False, False, 0),
    (257, 1024, 512, True, False, False, 0),
    (300, 640, 768, False, True, False, 0),
    (513, 256, 256, False, False, False, 0),
]


@pytest.mark.parametrize("m,k,n,zp,act_order,fp32,split", SMALL_SHAPES)
def test_gemm_matches_oracle_small(dev, m, k, n, zp, act_order, fp32, split):
    label = f"gemm m={m} k={k} n={n} zp={zp} act_order={act_order} fp32={fp32} split={split}"
    say(label)
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, seed=1000 + m + k + n)
    c = gpu_gemm(case, dev, fp32_reduce=fp32, split_k=split)
    assert_parity(c, oracle_gemm(case), label)


# Split-K on the tiled kernel (m > 16 with the fp32 reduce, when the output tiles are fewer
# than the CUs): both tile geometries, 128- and 64-row scale units (and 32-row units, which
# are not split), splits that do not divide the groups, act_order and zero points.
MID_SHAPES = [
    # m, k, n, zp, act_order, group_size
    (17, 4096, 2048, False, False, 128),    # 128-row tiles: 8 tiles, 16 splits
    (64, 2048, 512, True, False, 128),      # 2 tiles, 8 splits
    (128, 4096, 14336, False, False, 128),  # 56 tiles, 3 splits
    (300, 1024, 768, False, True, 128),     # 9 tiles, 4 splits
    (256, 1152, 512, True, False, 64),      # 64-row units, 9 groups over 4 splits
    (40, 1024, 256, False, False, 32),      # 32-row units (256-row tiles): K not split
    (1100, 4096, 2048, False, False, 128),  # 72 tiles, 2 splits
]


@pytest.mark.parametrize("m,k,n,zp,act_order,gs", MID_SHAPES)
def test_tiled_split_k_matches_oracle(dev, m, k, n, zp, act_order, gs):
    label = f"tiled split-K m={m} k={k} n={n} zp={zp} act_order={act_order} gs={gs}"
    say(label)
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=2000 + m + k + n)
    c = gpu_gemm(case, dev, fp32_reduce=True)
    assert_parity(c, oracle_gemm(case), label)
    again = gpu_gemm(case, dev, fp32_reduce=True)
    assert np.array_equal(c.view(np.uint16), again.view(np.uint16)), label


# act_order gathers: every LDS staging width of the row gather (K/8 granules over 256
# threads: 1, 2, 4, 8 per thread), its global-memory fallback beyond K = 16384, and more
# rows than the gather's 1024 work-groups, so that work-groups loop over rows.
ACT_ORDER_SHAPES = [(5, 256), (20, 2048), (1100, 4096), (40, 8192), (33, 16384), (17, 17408)]


@pytest.mark.parametrize("m,k", ACT_ORDER_SHAPES)
def test_act_order_gather_widths(dev, m, k):
    n = 256
    label = f"act_order m={m} k={k} n={n}"
    say(label)
    case = synthetic.dense_case(m, k, n, act_order=True, seed=2000 + m + k)
    c = gpu_gemm(case, dev)
    assert_parity(c, oracle_gemm(case), label)


# group sizes other than 128: channelwise (-1) and multiples of 128, whose scales and zero
# points the repack repeats per 128-row chunk, on both kernels, with zp and act_order.
GROUP_SHAPES = [
    # m, k, n, group_size, zp, act_order
    (1, 1024, 512, 32, True, False),
    (16, 512, 256, 64, False, False),
    (300, 1024, 512, 32, False, True),
    (513, 512, 256, 64, True, False),
    (64, 768, 512, 64, False, True),
    (130, 1024, 256, 32, True, False),
    (1, 1024, 512, -1, False, False),
    (16, 2048, 256, 256, True, False),
    (7, 1024, 512, 512, False, True),
    (300, 1024, 512, -1, True, False),
    (257, 2048, 256, 1024, False, True),
    (40, 4096, 256, 2048, True, False),
    # multiples of 16 that are not divisors or multiples of 128: units of 16, 32 or 64 rows
    (257, 1536, 512, 16, True, False),
    (300, 384, 256, 48, False, True),
    (64, 640, 256, 80, True, False),
    (130, 1152, 512, 96, True, True),
    (40, 768, 256, 192, False, False),
    (513, 1280, 256, 320, True, False),
]


@pytest.mark.parametrize("m,k,n,gs,zp,act_order", GROUP_SHAPES)
def test_group_sizes_match_oracle(dev, m, k, n, gs, zp, act_order):
    label = f"group_size={gs} m={m} k={k} n={n} zp={zp} act_order={act_order}"
    say(label)
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=3000 + m + k + gs)
    c = gpu_gemm(case, dev, fp32_reduce=True)
    assert_parity(c, oracle_gemm(case), label)


# The small-M kernel (m <= 16) with 2 or 4 scale groups per 128-row chunk: one split over a
# 32- or 64-chunk span, automatic and requested (ragged) splits, act_order, zero points, and
# a K that is not a multiple of the waves' share.
SMALL_GROUP_SHAPES = [
    # m, k, n, group_size, zp, act_order, fp32_reduce, split_k
    (1, 4096, 512, 32, False, False, False, 0),
    (1, 4096, 512, 32, True, False, True, 0),
    (5, 2048, 256, 64, True, False, True, 3),
    (16, 1024, 512, 32, True, True, False, 0),
    (3, 8192, 256, 64, False, False, False, 0),
    (8, 8192, 256, 32, True, False, False, 0),
    (2, 3968, 256, 32, False, False, True, 5),
    (12, 1536, 768, 64, False, True, True, 0),
    (1, 2048, 256, -1, True, False, True, 0),
    # 16-row units (two MFMA passes per step) and units repeated for 48/80/96-row groups
    (1, 4096, 512, 16, False, False, False, 0),
    (3, 1536, 256, 48, True, False, True, 0),
    (16, 768, 512, 16, True, True, False, 0),
    (7, 3840, 256, 80, False, False, True, 3),
    (2, 8192, 256, 16, True, False, False, 0),
    (5, 1152, 512, 96, True, False, False, 0),
]


@pytest.mark.parametrize("m,k,n,gs,zp,act_order,fp32,split", SMALL_GROUP_SHAPES)
def test_small_m_group_sizes_match_oracle(dev, m, k, n, gs, zp, act_order, fp32, split):
    label = (f"small-M group_size={gs} m={m} k={k} n={n} zp={zp} act_order={act_order} "
             f"fp32={fp32} split={split}")
    say(label)
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=3500 + m + k + gs)
    c = gpu_gemm(case, dev, fp32_reduce=fp32, split_k=split)
    assert_parity(c, oracle_gemm(case), label)


# 9..16 rows: each wave of the small-M kernel fetches its own groups' activation tiles,
# scales and zero points into its own LDS region (no shared slice, no barrier before the
# arithmetic); with enough column blocks each wave applies them to two blocks.
DIRECT_SHAPES = [
    # m, k, n, group_size, zp, act_order, fp32_reduce, split_k
    (9, 4096, 256, 16, True, False, False, 0),
    (11, 1024, 512, 128, False, True, True, 0),
    (13, 2048, 256, 64, True, False, True, 2),
    (16, 512, 256, -1, False, False, False, 0),
    (10, 4096, 512, 32, False, False, True, 4),
    # two column blocks per wave (at least 256 work-groups of two blocks)
    (16, 1024, 8192, 128, True, False, True, 0),
    (9, 2048, 8192, 16, True, False, False, 0),
    (12, 4096, 1024, 64, False, True, True, 8),
    (11, 1024, 8192, 32, False, False, False, 0),
    (14, 768, 8192, -1, True, False, False, 0),
    # 4 waves of 8 groups over two blocks; with 16-row units ten scale loads per block
    (16, 4096, 8192, 128, True, False, False, 0),
    (9, 4096, 8192, 16, True, False, False, 0),
    # 8 waves of 4 groups over one block, 16-row units (five scale loads)
    (16, 4096, 4096, 16, True, False, False, 0),
    (15, 3072, 4096, 48, False, True, True, 0),
]


@pytest.mark.parametrize("m,k,n,gs,zp,act_order,fp32,split", DIRECT_SHAPES)
def test_direct_activation_rows_match_oracle(dev, m, k, n, gs, zp, act_order, fp32, split):
    label = (f"direct rows m={m} k={k} n={n} group_size={gs} zp={zp} act_order={act_order} "
             f"fp32={fp32} split={split}")
    say(label)
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=3700 + m + k)
    c = gpu_gemm(case, dev, fp32_reduce=fp32, split_k=split)
    assert_parity(c, oracle_gemm(case), label)


# 2..4 rows on the small-M kernel's staged general path: slices of one to eight slots per
# thread (four or eight waves), every scale unit size and channelwise scales, zero points,
# act_order and requested splits.
FEW_ROW_SHAPES = [
    # m, k, n, group_size, zp, act_order, fp32_reduce, split_k
    (2, 128, 256, 128, False, False, False, 0),
    (3, 1024, 512, 128, True, False, True, 0),
    (4, 4096, 512, 128, False, False, False, 0),
    (4, 4096, 768, 128, True, False, True, 3),
    (2, 8192, 256, 128, False, True, False, 0),
    (3, 2048, 768, 64, True, False, False, 0),
    (4, 2048, 512, 32, False, False, True, 0),
    (2, 1024, 512, 16, True, False, False, 0),
    (4, 1024, 256, -1, True, False, False, 0),
    (3, 1536, 256, 48, False, True, False, 0),
    (4, 6144, 256, 16, True, False, True, 2),
]


# K beyond 64 groups on one work-group per column block: sixteen waves of eight (or, beyond
# 128 groups, sixteen) groups over a staged slice (up to four rows at K = 14336), with and
# without the fp32 reduce flag.
LONG_K_SHAPES = [
    # m, k, n, group_size, zp, act_order, fp32
    (1, 14336, 512, 128, False, False, False),
    (1, 11008, 2048, 128, True, False, True),
    (4, 14336, 256, 128, False, False, False),
    (3, 16384, 512, 64, True, False, False),
    (2, 12288, 256, 32, False, True, False),
    (1, 8320, 256, 16, True, False, False),
    (4, 9216, 2048, -1, False, False, True),
    # beyond 128 groups: sixteen groups per wave
    (1, 28672, 256, 128, False, False, False),
    (2, 20480, 512, 128, True, False, False),
    (1, 24576, 2048, 32, True, False, True),
]


@pytest.mark.parametrize("m,k,n,gs,zp,act_order,fp32", LONG_K_SHAPES)
def test_long_k_sixteen_waves_match_oracle(dev, m, k, n, gs, zp, act_order, fp32):
    label = (f"long K m={m} k={k} n={n} group_size={gs} zp={zp} act_order={act_order} "
             f"fp32={fp32}")
    say(label)
    flags = wq.WQ_FLAG_FP32_REDUCE if fp32 else 0
    kernel, splits = wq.wq_gemm_plan(m, n, k, group_size=gs, flags=flags)
    # (with the flag, beyond 128 groups the planner splits K into at most 64 groups)
    assert kernel == wq.WQ_KERNEL_SMALL_M and (splits == 1 or (fp32 and k // 128 > 128))
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=4300 + m + k + gs)
    c = gpu_gemm(case, dev, fp32_reduce=fp32)
    assert_parity(c, oracle_gemm(case), label)


# Eight staged waves (33 to 64 groups of K) with two to four rows per work-group: each wave
# stages its own share of the activation slice (the separate per-wave instances); row
# chunks of up to four rows take them too.
EIGHT_WAVE_SHAPES = [
    # m, k, n, group_size, zp, act_order, fp32
    (2, 8192, 512, 128, False, False, False),
    (3, 6144, 256, 64, True, False, False),
    (4, 5120, 768, 32, False, True, False),
    (4, 8192, 256, 16, True, False, False),
    (2, 4352, 4096, 128, False, False, True),
]


@pytest.mark.parametrize("m,k,n,gs,zp,act_order,fp32", EIGHT_WAVE_SHAPES)
def test_eight_wave_per_wave_staging_matches_oracle(dev, m, k, n, gs, zp, act_order, fp32):
    label = (f"eight waves m={m} k={k} n={n} group_size={gs} zp={zp} act_order={act_order} "
             f"fp32={fp32}")
    say(label)
    flags = wq.WQ_FLAG_FP32_REDUCE if fp32 else 0
    kernel, splits = wq.wq_gemm_plan(m, n, k, group_size=gs, flags=flags)
    assert kernel == wq.WQ_KERNEL_SMALL_M and splits == 1
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=4400 + m + k + gs)
    c = gpu_gemm(case, dev, fp32_reduce=fp32)
    assert_parity(c, oracle_gemm(case), label)


# Long K with the fp32 reduce flag where the grid exceeds the CUs: from four rows the planner
# splits K into ceil(groups / 16) ranges of at most 16 groups, on the staged and the direct
# forms; with one to three rows into ranges of at most 32; with act_order, zero points and
# 64-row units.
DEEP_SPLIT_SHAPES = [
    # m, k, n, group_size, zp, act_order, splits the planner takes
    (5, 14336, 4096, 128, False, False, 7),
    (4, 11008, 8192, 128, True, False, 6),
    (7, 12288, 4608, 64, False, True, 6),
    (6, 28672, 2048, 128, False, False, 14),
    (8, 16384, 4352, 64, True, False, 8),
    (12, 28672, 4096, 128, False, False, 14),
    (10, 11008, 4096, 128, True, False, 6),
    (16, 14336, 4352, 64, False, True, 7),
    # one to three rows: ranges of at most 32 groups beyond two work-groups per CU
    (3, 28672, 4096, 128, True, False, 7),
    (1, 14336, 8704, 128, False, False, 4),
    (2, 14336, 8704, 64, False, True, 4),
]


@pytest.mark.parametrize("m,k,n,gs,zp,act_order,want", DEEP_SPLIT_SHAPES)
def test_deep_split_matches_oracle(dev, m, k, n, gs, zp, act_order, want):
    label = f"deep split m={m} k={k} n={n} group_size={gs} zp={zp} act_order={act_order}"
    say(label)
    kernel, splits = wq.wq_gemm_plan(m, n, k, group_size=gs, flags=wq.WQ_FLAG_FP32_REDUCE)
    assert kernel == wq.WQ_KERNEL_SMALL_M and splits == want
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=4600 + m + k + gs)
    c = gpu_gemm(case, dev, fp32_reduce=True)
    assert_parity(c, oracle_gemm(case), label)
    again = gpu_gemm(case, dev, fp32_reduce=True)
    assert np.array_equal(c.view(np.uint16), again.view(np.uint16)), label


# More rows than one staged work-group holds at long K, without the fp32 reduce flag: row
# chunks of 8, 4 (or fewer) rows along grid z on sixteen waves.
LONG_K_CHUNK_SHAPES = [
    # m, k, n, group_size, zp
    (8, 14336, 256, 128, False),
    (16, 11008, 512, 128, True),
    (11, 12288, 256, 64, False),
    (24, 8192, 512, 128, True),
    (6, 16384, 256, 32, False),
    (4, 32768, 256, 64, True),
    (8, 28672, 256, 128, False),
]


@pytest.mark.parametrize("m,k,n,gs,zp", LONG_K_CHUNK_SHAPES)
def test_long_k_row_chunks_match_oracle(dev, m, k, n, gs, zp):
    label = f"long K row chunks m={m} k={k} n={n} group_size={gs} zp={zp}"
    say(label)
    assert wq.wq_gemm_plan(m, n, k, group_size=gs) == (wq.WQ_KERNEL_SMALL_M, 1)
    case = synthetic.dense_case(m, k, n, zp=zp, group_size=gs, seed=4400 + m + k + gs)
    c = gpu_gemm(case, dev)
    assert_parity(c, oracle_gemm(case), label)


# More than 16 rows without the fp32 reduce flag: the small-M kernel's direct form in 16-row
# chunks along grid z (single and paired column blocks, ragged last chunks, group sizes,
# zero points, act_order).
CHUNK_SHAPES = [
    # m, k, n, group_size, zp, act_order
    (17, 1024, 512, 128, False, False),
    (24, 4096, 256, 128, True, False),
    (32, 2048, 8192, 128, False, False),
    (33, 1024, 256, 64, True, False),
    (48, 768, 512, 16, False, False),
    (64, 4096, 1024, 128, False, True),
    (50, 1536, 256, 48, True, False),
    (61, 2048, 8192, 32, True, True),
    # up to sixteen chunks while their weight reads stay within the budget
    (80, 1024, 2048, 128, False, False),
    (200, 2048, 1024, 128, True, False),
    (256, 512, 512, 64, False, False),
    (130, 4096, 512, 128, False, True),
]


@pytest.mark.parametrize("m,k,n,gs,zp,act_order", CHUNK_SHAPES)
def test_row_chunks_match_oracle(dev, m, k, n, gs, zp, act_order):
    label = f"row chunks m={m} k={k} n={n} group_size={gs} zp={zp} act_order={act_order}"
    say(label)
    assert wq.wq_gemm_plan(m, n, k, group_size=gs)[0] == wq.WQ_KERNEL_SMALL_M
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=4100 + m + k + gs)
    c = gpu_gemm(case, dev)
    assert_parity(c, oracle_gemm(case), label)


@pytest.mark.parametrize("m,k,n,gs,zp,act_order,fp32,split", FEW_ROW_SHAPES)
def test_few_rows_match_oracle(dev, m, k, n, gs, zp, act_order, fp32, split):
    label = (f"few rows m={m} k={k} n={n} group_size={gs} zp={zp} act_order={act_order} "
             f"fp32={fp32} split={split}")
    say(label)
    case = synthetic.dense_case(m, k, n, zp=zp, act_order=act_order, group_size=gs,
                                seed=3800 + m + k + gs)
    c = gpu_gemm(case, dev, fp32_reduce=fp32, split_k=split)
    assert_parity(c, oracle_gemm(case), label)


@pytest.mark.parametrize("gs,k", [(-1, 1024), (32, 1024), (64, 1024), (256, 1024), (1024, 1024),
                                  (16, 1024), (48, 768), (80, 1280), (96, 1152)])
def test_group_size_repack_and_dequant_bitwise(dev, gs, k):
    n = 512
    say(f"repack/dequant group_size={gs}")
    groups = 1 if gs == -1 else k // gs
    s = synthetic.scales(90, groups, n)
    z = synthetic.zero_point_words(91, groups, n)
    qw = synthetic.qweight_words(92, k, n)
    w = torch_ops.PackedWeight(qw, s, z, device=dev, group_size=gs)
    assert np.array_equal(host(w.s).view(np.uint16), layout.repack_scales(s, k, gs).view(np.uint16))
    assert np.array_equal(host(w.z).view(np.uint32), layout.repack_zero_points(z, k, gs))
    out = torch.empty((k, n), dtype=torch.float16, device=dev)
    wq.wq_dequant(w.b, w.s, w.z, out, k=k, n=n, flags=wq.WQ_FLAG_HAS_ZP, group_size=gs)
    torch.cuda.synchronize()
    want = ref.dequantize_fp16(ref.w4a16_weights(qw, s, zeros=z, group_size=gs))
    assert np.array_equal(host(out).view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("name", ["tiny", "decode", "batched"])
def test_config_matches_oracle_in_full(dev, name):
    case = synthetic.config_case(name)
    say(f"config {name}: m={case['m']} k={case['k']} n={case['n']}")
    c = gpu_gemm(case, dev, fp32_reduce=case["fp32_reduce"])
    assert_parity(c, oracle_gemm(case), name)


def sample_columns(n, seed, count=256):
    cols = set(range(0, 128)) | set(range(n - 128, n))
    cols |= set(int(x) for x in synthetic.below(seed, count, n))
    return np.array(sorted(cols))


def test_prefill_config_matches_oracle_in_full(dev):
    case = synthetic.config_case("prefill")
    say("config prefill: m=2048 k=4096 n=14336 act_order, every output")
    c = gpu_gemm(case, dev)
    want = by_column_chunks(lambda cols: oracle_gemm(case, columns=cols), case["n"])
    assert_parity(c, want, "prefill")


# --------------------------------------------------------------------------- pins

# One-row products run on 4x4x4 MFMAs, each lane summing its column over one row class of
# every step, with the classes added by lane shuffles at the end.  The fp16 operands are
# the codes q themselves (fp16 subnormals, exact) and the zero point enters once per scale
# unit as z times the activations' sum over the lane's rows of the unit, so every partial
# is an fp32 sum of exact terms whose magnitudes add up to at most sum |a| (q + z) s,
# added along a tree of depth below 64 (the 32-term chains of a unit, the zero-point term,
# the scaled fold over units, the shuffles and the four-wave reduction): the unrounded
# result is within 64 * 2^-24 * sum |a| (q + z) s of the exact one.
ACCUMULATION_ROUNDINGS = 64


def accumulation_bound(case):
    k = case["qweight"].shape[0] * 8
    gs = case.get("group_size", 128)
    group = ref.group_of_rows(k, gs)
    q = ref.unpack_qweight(case["qweight"]).astype(np.float64)
    z = (8.0 if case.get("zeros") is None
         else ref.unpack_zero_points(case["zeros"]).astype(np.float64)[group, :])
    mag = (q + z) * ref.values16(case["scales"])[group, :]
    return ACCUMULATION_ROUNDINGS * 2.0 ** -24 * (np.abs(case["a"].astype(np.float64)) @ mag)


def test_all_eight_codes_give_zero(dev):
    """Codes equal to the zero point give zero: exactly on the tiled kernel and the
    small-M kernel's general path (the weights enter the products as exact zeros); within
    the accumulation bound on the one-row path, where q * a and z * a are summed apart."""
    for m in (1, 3, 16, 300):
        case = synthetic.dense_case(m, 512, 256, seed=3)
        case["qweight"][:] = 0x88888888
        c = gpu_gemm(case, dev, fp32_reduce=True).astype(np.float64)
        if m == 1:
            assert np.all(np.abs(c[0]) <= accumulation_bound(case)[0]), m
        else:
            assert np.all(c == 0.0), m


ONE_ROW_SHAPES = [
    # m, k, n, group_size, zp, all-positive activations, split_k
    (1, 4096, 512, 128, False, True, 0),
    (1, 4096, 512, 128, True, True, 0),
    (1, 4096, 512, 16, True, True, 0),
    (1, 2048, 512, 32, False, True, 0),
    (1, 1024, 512, 64, True, False, 0),
    (1, 1024, 768, -1, True, True, 0),
    (1, 4096, 256, 128, True, True, 3),
]


@pytest.mark.parametrize("m,k,n,gs,zp,positive,split", ONE_ROW_SHAPES)
def test_one_row_within_rounding_of_the_exact_product(dev, m, k, n, gs, zp, positive, split):
    label = (f"one row m={m} k={k} n={n} group_size={gs} zp={zp} positive={positive} "
             f"split={split}")
    say(label)
    case = synthetic.dense_case(m, k, n, zp=zp, group_size=gs, seed=3900 + k + n + gs + m)
    if positive:  # every activation of one sign: the largest partial sums for the result
        case["a"] = np.abs(case["a"])
    c = gpu_gemm(case, dev, fp32_reduce=True, split_k=split)
    want = oracle_gemm(case)
    assert_parity(c, want, label)
    err = np.abs(c.astype(np.float64) - want)
    allowed = (2.0 ** -11 * np.abs(want) + accumulation_bound(case) * (1 + 2.0 ** -11)
               + 2.0 ** -25)
    assert np.all(err <= allowed), (label, float(np.max(err - allowed)))


def test_unit_scales_integer_products_are_bit_exact(dev):
    for m in (1, 3, 16, 40):
        k, n = 1024, 256
        case = synthetic.dense_case(m, k, n, seed=4)
        case["a"] = (synthetic.below(5, m * k, 3) - 1).reshape(m, k).astype(np.float16)
        case["scales"] = np.ones_like(case["scales"])
        want = oracle_gemm(case)
        assert np.abs(want).max() <= 2048   # every integer below this is exact in fp16
        c = gpu_gemm(case, dev, fp32_reduce=True)
        assert np.array_equal(c.astype(np.float64), want), m


@pytest.mark.parametrize("rows", [[0, 1, 127, 128, 500, 1023], [0, 500, 1023], [129]])
def test_one_hot_rows_give_dequantized_rows_bitwise(dev, rows):
    k, n = 1024, 512
    for zp in (False, True):
        case = synthetic.dense_case(len(rows), k, n, zp=zp, seed=6)
        a = np.zeros((len(rows), k), dtype=np.float16)
        for i, r in enumerate(rows):
            a[i, r] = 1.0
        case["a"] = a
        c = gpu_gemm(case, dev)
        exact = ref.w4a16_weights(case["qweight"], case["scales"], zeros=case["zeros"])
        want = ref.dequantize_fp16(exact[rows, :])
        assert np.array_equal(c.view(np.uint16), want.view(np.uint16)), zp


@pytest.mark.parametrize("gs,zp", [(128, True), (64, False)])
def test_tile_geometries_agree_bitwise(dev, gs, zp):
    """1024 rows by 16384 columns run on 256 x 256 tiles (256 of them) and 896 rows on
    128 x 256 tiles; every output is the same sum in the same order either way, so the
    shared rows agree bit for bit."""
    k, n = 256, 16384
    case = synthetic.dense_case(1024, k, n, zp=zp, group_size=gs, seed=41)
    c_full = gpu_gemm(case, dev)
    c_part = gpu_gemm(case, dev, a=np.ascontiguousarray(case["a"][:896]))
    assert np.array_equal(c_full[:896].view(np.uint16), c_part.view(np.uint16))
    cols = sample_columns(n, 4, 64)
    assert_parity(c_part[:, cols], oracle_gemm(dict(case, a=case["a"][:896]), columns=cols),
                  f"896 rows gs={gs}")


def test_results_are_deterministic_and_split_independent(dev):
    for m, zp in ((1, False), (16, True)):
        case = synthetic.dense_case(m, 4096, 1024, zp=zp, seed=8)
        c1 = gpu_gemm(case, dev, fp32_reduce=True)
        c2 = gpu_gemm(case, dev, fp32_reduce=True)
        assert np.array_equal(c1.view(np.uint16), c2.view(np.uint16))
        want = oracle_gemm(case)
        for split in (1, 2, 5, 16):
            assert_parity(gpu_gemm(case, dev, fp32_reduce=True, split_k=split), want,
                          f"m={m} split={split}")


def test_act_order_equals_plain_product_on_permuted_operands(dev):
    k, n = 1024, 512
    for m in (4, 300):
        case = synthetic.dense_case(m, k, n, act_order=True, seed=9)
        perm, _ = ref.act_order_perm(case["g_idx"], 128)
        c_act = gpu_gemm(case, dev)
        codes = ref.unpack_qweight(case["qweight"])[perm, :]
        packed = np.zeros((k // 8, n), dtype=np.uint32)
        for i in range(8):
            packed |= codes[i::8].astype(np.uint32) << np.uint32(4 * i)
        plain = dict(case, qweight=packed, g_idx=None)
        c_plain = gpu_gemm(plain, dev, a=np.ascontiguousarray(case["a"][:, perm]))
        assert_parity(c_act, c_plain.astype(np.float64), f"act_order vs plain m={m}")


@pytest.mark.parametrize("m,fp32", [(20, False), (20, True), (5, True), (12, True)])
def test_strided_activations(dev, m, fp32):
    """lda > k on the tiled kernel (unsplit and split along K) and the small-M kernel."""
    k, n = 512, 256
    case = synthetic.dense_case(m, k, n, seed=12)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], device=dev)
    wide = torch.zeros((m, k + 64), dtype=torch.float16, device=dev)
    wide[:, :k] = torch_ops.to_device(case["a"], dev)
    c = torch_ops.gemm(wide[:, :k], w, fp32_reduce=fp32)
    torch.cuda.synchronize()
    assert_parity(host(c), oracle_gemm(case), f"lda > k m={m} fp32={fp32}")


# --------------------------------------------------------------------------- grouped (MoE)

def run_grouped(moe, dev, zeros=None, weights=None):
    experts = [dict(e) for e in moe["experts"]]
    if zeros is not None:
        for e, z in zip(experts, zeros):
            e["zeros"] = z
    bank = torch_ops.ExpertBank(experts, device=dev)
    csr = wq.wq_csr_from_routes(moe["routes"], moe["n_tokens"], moe["top_k"], moe["n_expert"])
    a = torch_ops.to_device(moe["a"], dev)
    w = None if weights is None else torch_ops.to_device(weights, dev)
    y = torch_ops.grouped_gemm(a, bank, csr, topk_weights=w)
    torch.cuda.synchronize()
    ocsr = ref.csr_from_token_routes(moe["n_expert"], moe["n_tokens"], moe["top_k"],
                                     moe["routes"])
    return host(y), experts, ocsr


@pytest.mark.parametrize("tokens,experts,k,n,zp,weighted", [(40, 4, 256, 256, False, False),
                                                            (300, 3, 512, 512, True, False),
                                                            (700, 2, 256, 256, False, False),
                                                            (40, 4, 256, 256, False, True),
                                                            (300, 3, 512, 512, True, True)])
def test_grouped_matches_oracle(dev, tokens, experts, k, n, zp, weighted):
    label = f"grouped tokens={tokens} experts={experts} k={k} n={n} zp={zp} weighted={weighted}"
    say(label)
    moe = synthetic.moe_case(tokens, experts, k, n, seed=200 + tokens)
    zeros = ([synthetic.zero_point_words(300 + e, k // 128, n) for e in range(experts)]
             if zp else None)
    w = synthetic.routing_weights(400 + tokens, tokens, 2) if weighted else None
    y, ex, ocsr = run_grouped(moe, dev, zeros, w)
    assert_parity(y, ref.grouped_w4a16_gemm(moe["a"], ex, ocsr, topk_weights=w), label)


@pytest.mark.parametrize("gs,k", [(256, 1024), (64, 1024), (32, 1024), (16, 1024), (48, 768)])
def test_grouped_with_other_group_sizes(dev, gs, k):
    tokens, experts, n = 120, 3, 256
    moe = synthetic.moe_case(tokens, experts, k, n, group_size=gs, seed=24)
    for e in moe["experts"]:
        e["group_size"] = gs
    y, ex, ocsr = run_grouped(moe, dev)
    assert_parity(y, ref.grouped_w4a16_gemm(moe["a"], ex, ocsr, group_size=gs),
                  f"grouped gs={gs}")


def test_grouped_unit_weights_change_nothing(dev):
    moe = synthetic.moe_case(90, 3, 256, 256, seed=23)
    y0, _, _ = run_grouped(moe, dev)
    y1, _, _ = run_grouped(moe, dev, weights=np.ones(180, np.float32))
    assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16))


def test_grouped_skips_inactive_experts(dev):
    moe = synthetic.moe_case(50, 6, 256, 256, seed=21)
    moe["routes"] = np.where(moe["routes"] % 2 == 0, 4, 1).astype(np.int32)
    moe["routes"][:, 1] = np.where(moe["routes"][:, 0] == 4, 1, 4)
    y, ex, ocsr = run_grouped(moe, dev)
    assert list(ocsr["ex_ids"]) == [1, 4]
    assert_parity(y, ref.grouped_w4a16_gemm(moe["a"], ex, ocsr), "inactive experts")


def test_grouped_single_expert_equals_dense(dev):
    k, n, tokens = 512, 512, 270
    moe = synthetic.moe_case(tokens, 1, k, n, seed=22)
    bank = torch_ops.ExpertBank(moe["experts"], device=dev)
    csr = wq.wq_csr_from_routes(np.zeros(tokens, np.int32), tokens, 1, 1)
    a = torch_ops.to_device(moe["a"], dev)
    y = host(torch_ops.grouped_gemm(a, bank, csr))
    dense = gpu_gemm(dict(a=moe["a"], qweight=moe["experts"][0]["qweight"],
                          scales=moe["experts"][0]["scales"]), dev)
    assert np.array_equal(y.view(np.uint16), dense.view(np.uint16))


# Segments of at most four rows (n_pairs - n_active + 1 <= 4) run on the small-M kernel, one
# work-group per 16-column block and segment: one-row segments on its one-row path, up to
# four rows on its general path; four waves of 1..8 groups, eight waves of 8 (K = 8192)
# or sixteen of 8 (K beyond 64 groups).
FEW_ROW_GROUPED = [
    # tokens, experts, k, n, group_size, zp, weighted, bf16
    (1, 8, 4096, 512, 128, False, False, False),
    (1, 8, 1024, 768, 128, True, True, False),
    (1, 1, 2048, 256, 128, False, False, False),      # both slots on one expert: two rows
    (2, 8, 2048, 512, 64, True, False, False),
    (3, 8, 8192, 256, 128, False, True, False),
    (2, 3, 1024, 512, 32, False, True, False),
    (1, 4, 4096, 256, 16, True, False, False),
    (3, 6, 768, 256, 256, False, False, False),
    (1, 8, 2048, 512, 128, False, True, True),
    (2, 8, 1024, 256, 64, True, False, True),
    (3, 5, 512, 512, 16, False, True, True),
    (4, 8, 1024, 256, 128, True, True, False),
    (5, 8, 1024, 512, 128, False, False, True),
    # a down projection's K (sixteen waves of eight groups, each staging its own share)
    (1, 8, 14336, 256, 128, False, True, False),
    (2, 8, 11008, 256, 64, True, False, False),
    (3, 4, 14336, 256, 128, False, True, True),
    (2, 2, 12288, 512, 32, True, True, False),
]


@pytest.mark.parametrize("tokens,experts,k,n,gs,zp,weighted,bf16", FEW_ROW_GROUPED)
def test_grouped_few_rows_match_oracle(dev, tokens, experts, k, n, gs, zp, weighted, bf16):
    label = (f"grouped few rows tokens={tokens} experts={experts} k={k} n={n} group_size={gs} "
             f"zp={zp} weighted={weighted} bf16={bf16}")
    say(label)
    seed = 5100 + tokens * 7 + experts + k + gs
    moe = synthetic.moe_case(tokens, experts, k, n, group_size=gs, seed=seed, bf16=bf16)
    groups = k // gs
    ex = []
    for i, e in enumerate(moe["experts"]):
        d = dict(e, group_size=gs)
        if zp:
            d["zeros"] = synthetic.zero_point_words(seed + 100 + i, groups, n)
        ex.append(d)
    bank = torch_ops.ExpertBank(ex, device=dev, bf16=bf16)
    csr = wq.wq_csr_from_routes(moe["routes"], tokens, 2, experts)
    assert csr["n_pairs"] - csr["n_active"] + 1 <= 4, "not a few-row product"
    wts = synthetic.routing_weights(seed + 200, tokens, 2) if weighted else None
    y = torch_ops.grouped_gemm(torch_ops.to_device(moe["a"], dev), bank, csr,
                               topk_weights=None if wts is None else torch_ops.to_device(wts, dev))
    torch.cuda.synchronize()
    ocsr = ref.csr_from_token_routes(experts, tokens, 2, moe["routes"])
    want = ref.grouped_w4a16_gemm(moe["a"], ex, ocsr, group_size=gs, topk_weights=wts,
                                  bf16=bf16)
    got = y.float().cpu().numpy() if bf16 else host(y)
    # bf16 outputs, and fp16 outputs scaled by routing weights, add their own rounding per
    # element (as the dense bf16 and the weighted MoE checks do)
    res = ref.check(got, want, rel_elem=(2.0 ** -8 if bf16 else 2.0 ** -11 if weighted else 0.0),
                    rel_frob=4e-3 if bf16 else 1e-3)
    say(f"{label}: max_err={res['max_err']:.3e} tol={res['tol']:.3e} "
        f"rel_frob={res['rel_frob']:.3e} nonfinite={res['nonfinite']}")
    assert res["ok"], (label, res)


@pytest.mark.parametrize("tokens,experts", [(1, 8), (1, 1), (2, 8)])
def test_grouped_few_rows_equal_dense_rows_bitwise(dev, tokens, experts):
    """A segment's rows give the same bits as the dense small-M product of its expert on
    those activation rows (the same plan: four waves, no split)."""
    k, n = 2048, 512
    moe = synthetic.moe_case(tokens, experts, k, n, seed=5200 + tokens + experts)
    bank = torch_ops.ExpertBank(moe["experts"], device=dev)
    csr = wq.wq_csr_from_routes(moe["routes"], tokens, 2, experts)
    y = host(torch_ops.grouped_gemm(torch_ops.to_device(moe["a"], dev), bank, csr))
    bound = csr["n_pairs"] - csr["n_active"] + 1
    for i, e in enumerate(csr["ex_ids"]):
        pairs = [int(p) for p in csr["ex_pairs"][csr["ex_off"][i]:csr["ex_off"][i + 1]]]
        rows = [int(csr["pair_tok"][p]) for p in pairs]
        # the instance is chosen by the bound: a shorter segment repeats its last row
        rows_b = rows + [rows[-1]] * (bound - len(rows))
        dense = gpu_gemm(dict(a=moe["a"][rows_b], qweight=moe["experts"][e]["qweight"],
                              scales=moe["experts"][e]["scales"]), dev)
        assert np.array_equal(y[pairs].view(np.uint16), dense[:len(rows)].view(np.uint16)), \
            (tokens, experts, e)


@pytest.mark.parametrize("weighted", [False, True])
def test_moe_config_matches_oracle_in_full(dev, weighted):
    say(f"config moe: 1024 tokens top-2 of 8 experts, k=4096 n=14336, every output, "
        f"weighted={weighted}")
    moe = synthetic.moe_case()
    w = synthetic.routing_weights(77, moe["n_tokens"], 2) if weighted else None
    y, ex, ocsr = run_grouped(moe, dev, weights=w)
    want = by_column_chunks(lambda cols: ref.grouped_w4a16_gemm(
        moe["a"], ex, ocsr, columns=cols, topk_weights=w), moe["n"])
    # Routing weights shrink rms(ref) while the largest outputs keep |y| near 20, where the
    # fp16 output's own rounding (half an ulp, at most 2^-11 |y|) exceeds 2e-3 rms + 1e-3:
    # the weighted check adds that rounding bound per element.
    assert_parity(y, want, "moe", rel_elem=2.0 ** -11 if weighted else 0.0)


# --------------------------------------------------------------------------- graph replay

@pytest.mark.parametrize("m,fp32", [(1, True), (16, True), (300, False), (64, True)])
def test_graph_replays_match_eager(dev, m, fp32):
    """Captured calls replay bit-identically, with eager work between replays."""
    case = synthetic.dense_case(m, 2048, 512, zp=(m == 16), act_order=(m == 300), seed=31)
    w = torch_ops.PackedWeight(case["qweight"], case["scales"], case["zeros"], case["g_idx"],
                               device=dev)
    a = torch_ops.to_device(case["a"], dev)
    bufs = torch_ops.GemmBuffers(w, m, fp32)
    eager = host(torch_ops.gemm(a, w, fp32_reduce=fp32, buffers=bufs))
    out = torch.empty((m, w.n), dtype=torch.float16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch_ops.gemm(a, w, out, fp32_reduce=fp32, buffers=bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        torch_ops.gemm(a, w, out, fp32_reduce=fp32, buffers=bufs)
    for rep in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint16), eager.view(np.uint16)), rep
        torch_ops.gemm(a, w, fp32_reduce=fp32, buffers=bufs)   # eager work in between
        torch.cuda.synchronize()


# --------------------------------------------------------------------------- measurement helper

def test_stream_read_reads_every_granule_once(dev):
    """The streaming-read helper's data-dependent store fires exactly for the wave whose
    lane read a planted word equal to its trigger value, so each planted position shows
    that its granule was read, by the wave that owns it."""
    magic = 0x9E3779B9
    nbytes = (1 << 20) + 16 * 37  # a ragged last wave
    granules = nbytes // 16
    for pos in (0, 511, 512, 12345, granules - 37, granules - 1):
        buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
        buf[4 * pos + (pos % 4)] = magic - (1 << 32)  # the same 32 bits as int32
        words = wq.wq_stream_read_sink_words(nbytes)
        sink = torch.zeros(words, dtype=torch.int32, device=dev)
        wq.wq_stream_read(buf, nbytes, sink, words)
        torch.cuda.synchronize()
        got = host(sink).view(np.uint32)
        owner = pos // 512
        if pos == granules - 1:
            # lanes past the end re-read the last granule: an even number of extra reads
            # cancels in the XOR unless exactly one lane reads it
            continue
        assert got[owner] == magic, (pos, owner, got[max(owner - 1, 0):owner + 2])
        assert np.count_nonzero(got) == 1, pos


# --------------------------------------------------------------------------- SwiGLU chain

# The SwiGLU activation is a product of two sums, so its values (and the down projection's
# outputs of them) are heavy-tailed: fp16 rounding alone (up to 2^-11 |x|) can exceed the
# GEMM bound at the largest elements, so these checks add twice that per-element rounding
# allowance.
ACT_REL = 2.0 ** -10

def mlp_weights(seed, k, i, h=None, zp=False, group_size=128):
    groups = 1 if group_size == -1 else k // group_size

    def one(s, kk, nn):
        g = 1 if group_size == -1 else kk // group_size
        w = dict(qweight=synthetic.qweight_words(s, kk, nn), scales=synthetic.scales(s + 1, g, nn))
        if zp:
            w["zeros"] = synthetic.zero_point_words(s + 2, g, nn)
        return w
    gate, up = one(seed, k, i), one(seed + 10, k, i)
    down = one(seed + 20, i, h) if h else None
    return gate, up, down


@pytest.mark.parametrize("bits,rows,cols", [(32, 128, 256), (16, 8, 512), (4, 8, 256)])
def test_interleave_gate_up_bitwise(dev, bits, rows, cols):
    per_word = 32 // bits
    words = cols // per_word
    g = synthetic.words_u32(95, rows * words).reshape(rows, words)
    u = synthetic.words_u32(96, rows * words).reshape(rows, words)
    out = torch.empty((rows, 2 * words), dtype=torch.int32, device=dev)
    wq.wq_interleave_gate_up(torch_ops.to_device(g, dev), torch_ops.to_device(u, dev), out,
                             rows, cols, bits)
    torch.cuda.synchronize()
    # a 16-column block is 16 words, 8 words (two fp16 per word) or 2 words
    want = layout.interleave_gate_up(g, u, cols_per_elem=per_word) if bits != 16 else \
        layout.interleave_gate_up(g.view(np.uint16).reshape(rows, cols),
                                  u.view(np.uint16).reshape(rows, cols)).view(np.uint32)
    assert np.array_equal(host(out).view(np.uint32), want.reshape(rows, 2 * words))


@pytest.mark.parametrize("m,k,i,zp,act_order,gs", [(1, 1024, 256, False, False, 128),
                                                    (16, 512, 512, True, False, 128),
                                                    (300, 1024, 256, False, True, 128),
                                                    (513, 256, 384, True, False, 128),
                                                    (100, 512, 256, True, False, 32),
                                                    # small-M paired form: 8 and 16 waves,
                                                    # and beyond it the tiled kernel
                                                    (1, 4096, 1024, False, False, 128),
                                                    (4, 8192, 256, True, False, 128),
                                                    (2, 12288, 256, False, False, 128),
                                                    # the paired form with 32/64-row groups
                                                    (1, 4096, 512, False, False, 32),
                                                    (4, 2048, 256, True, False, 64),
                                                    (2, 8192, 256, True, False, 32),
                                                    (1, 768, 256, False, False, 48),
                                                    (100, 768, 256, True, False, 16)])
def test_swiglu_activation_matches_oracle(dev, m, k, i, zp, act_order, gs):
    label = f"swiglu m={m} k={k} i={i} zp={zp} act_order={act_order} group_size={gs}"
    say(label)
    gate, up, _ = mlp_weights(500 + m, k, i, zp=zp, group_size=gs)
    a = synthetic.activations(501 + m, m, k)
    g_idx = synthetic.act_order_g_idx(502, k, 128) if act_order else None
    if act_order:
        gate["g_idx"] = up["g_idx"] = g_idx
    w = torch_ops.PackedWeight.gate_up(gate, up, device=dev, g_idx=g_idx, group_size=gs)
    act = host(torch_ops.gemm(torch_ops.to_device(a, dev), w))
    torch.cuda.synchronize()
    if act_order:  # the oracle reads g_idx through its own argument
        g = ref.w4a16_gemm(a, gate["qweight"], gate["scales"], zeros=gate.get("zeros"), g_idx=g_idx)
        u = ref.w4a16_gemm(a, up["qweight"], up["scales"], zeros=up.get("zeros"), g_idx=g_idx)
        want = ref.silu(g) * u
    else:
        want = ref.swiglu_activation(a, gate, up, group_size=gs)
    assert act.shape == (m, i)
    assert_parity(act, want, label, rel_elem=ACT_REL)


def test_swiglu_mlp_chain_matches_oracle(dev):
    m, h, i = 200, 512, 768
    say(f"swiglu mlp chain m={m} hidden={h} intermediate={i}")
    gate, up, down = mlp_weights(600, h, i, h, zp=True)
    a = synthetic.activations(601, m, h)
    wgu = torch_ops.PackedWeight.gate_up(gate, up, device=dev)
    wd = torch_ops.PackedWeight(down["qweight"], down["scales"], down["zeros"], device=dev)
    act = torch_ops.gemm(torch_ops.to_device(a, dev), wgu)
    out = host(torch_ops.gemm(act, wd))
    act16, want = ref.swiglu_mlp(a, gate, up, down)
    assert_parity(host(act), act16.astype(np.float64), "chain activation", rel_elem=ACT_REL)
    assert_parity(out, want, "chain output", rel_elem=ACT_REL)


# 300 tokens: row tiles; 1..3 tokens (every segment at most four rows): the small-M kernel,
# its SwiGLU pair for the gate/up projection and single blocks for the down projection.
@pytest.mark.parametrize("tokens,experts,h,i", [(300, 4, 512, 256), (1, 8, 1024, 512),
                                                (2, 8, 512, 256), (3, 4, 512, 256)])
def test_moe_swiglu_chain_matches_oracle(dev, tokens, experts, h, i):
    say(f"moe swiglu chain tokens={tokens} experts={experts} hidden={h} intermediate={i}")
    moe = synthetic.moe_case(tokens, experts, h, i, seed=610 + tokens)
    mats = [mlp_weights(620 + 30 * e, h, i, h) for e in range(experts)]
    gu_bank = torch_ops.ExpertBank([dict(gate=g, up=u) for g, u, _ in mats], device=dev)
    dn_bank = torch_ops.ExpertBank([d for _, _, d in mats], device=dev)
    csr = wq.wq_csr_from_routes(moe["routes"], tokens, 2, experts)
    a = torch_ops.to_device(moe["a"], dev)
    act = torch_ops.grouped_gemm(a, gu_bank, csr)            # [pairs][i], pair-major
    # the down projection reads pair rows: the same CSR with pair_tok = identity
    n_pairs = 2 * tokens
    ident = dict(csr)
    ident["pair_tok"] = np.arange(n_pairs, dtype=np.int32)
    wts = synthetic.routing_weights(611, tokens, 2)
    out = host(torch_ops.grouped_gemm(act, dn_bank, ident,
                                      topk_weights=torch_ops.to_device(wts, dev)))
    ocsr = ref.csr_from_token_routes(experts, tokens, 2, moe["routes"])
    act_want = np.full((n_pairs, i), np.nan)
    for seg, e in enumerate(ocsr["ex_ids"]):
        rows = [ocsr["ex_pairs"][j] for j in range(ocsr["ex_off"][seg], ocsr["ex_off"][seg + 1])]
        toks = [ocsr["pair_tok"][p] for p in rows]
        act_want[rows] = ref.swiglu_activation(moe["a"][toks], mats[e][0], mats[e][1])
    assert_parity(host(act), act_want, "moe swiglu activation", rel_elem=ACT_REL)
    act16 = ref.dequantize_fp16(act_want)
    oid = dict(ocsr)
    oid["pair_tok"] = list(range(n_pairs))
    want = ref.grouped_w4a16_gemm(act16, [d for _, _, d in mats], oid, topk_weights=wts)
    assert_parity(out, want, "moe swiglu chain output", rel_elem=ACT_REL)


@pytest.mark.parametrize("tokens,experts,k,n,gs,skew", [(600, 64, 512, 256, 128, False),
                                                       (700, 300, 256, 256, 128, False),
                                                       (900, 64, 512, 256, 128, True),
                                                       (700, 300, 256, 256, 32, False)])
def test_grouped_many_experts(dev, tokens, experts, k, n, gs, skew):
    """Many experts: the tile lookup scans the segments in parallel (several rounds of the
    work-group's threads beyond 256 or 512 segments); skewed routes mix full, partial and
    tail tiles; 32-row scale units take the 256 x 256 geometry (512 threads)."""
    label = f"grouped experts={experts} tokens={tokens} k={k} n={n} gs={gs} skew={skew}"
    say(label)
    moe = synthetic.moe_case(tokens, experts, k, n, group_size=gs, seed=500 + experts + tokens)
    if skew:  # most first choices on three experts: segments of hundreds of rows and of few
        r = moe["routes"]
        r[: 2 * tokens // 3, 0] = np.arange(2 * tokens // 3) % 3
        r[:, 1] = np.where(r[:, 1] == r[:, 0], (r[:, 0] + 7) % experts, r[:, 1])
    for e in moe["experts"]:
        e["group_size"] = gs
    y, ex, ocsr = run_grouped(moe, dev)
    assert len(ocsr["ex_ids"]) > 50
    assert_parity(y, ref.grouped_w4a16_gemm(moe["a"], ex, ocsr, group_size=gs), label)
