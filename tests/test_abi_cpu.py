"""Host-side checks of the C ABI: exports, status codes, validation, host helpers.

No GPU is needed: every call here either runs on the host (act_order perm, CSR builder,
workspace sizing) or fails validation before anything is launched.  Fake device pointers
(0x1000, 0x2000, ...) stand in for buffers, as in the pages' validation tests
(ferrum-kernels marlin.rs test module).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import synthetic
import weight_only_quantized_gemm_amd as wq
from conftest import ROOT, golden_csr_cases
from oracle import reference as ref

STAGE_ARGS, STAGE_SHAPE = wq.WQ_STAGE_ARGS, wq.WQ_STAGE_SHAPE


def status(stage, code):
    return (stage << 16) | code


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wq.LIB_PATH):
        pytest.fail("libwq.so is not built (run __graft_entry__.build())")
    return wq.lib()


def declared_functions():
    with open(os.path.join(ROOT, "include", "wq.h")) as f:
        text = f.read()
    # declarations start a line: "<type> [*]wq_name(" with an optional const
    return sorted(set(re.findall(r"^(?:const )?[a-z_0-9]+ ?\*? ?(wq_[a-z_0-9]+)\(", text,
                                 flags=re.M)))


def test_library_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(wq.EXPORTED)


def test_abi_version(L):
    assert wq.wq_abi_version() == wq.WQ_ABI_VERSION == 3


def test_status_strings_decode_stage_and_code(L):
    assert wq.wq_status_str(0) == "ok"
    assert wq.wq_status_str(status(STAGE_ARGS, wq.WQ_ERR_NULL)).startswith("args: null pointer")
    assert "shape" in wq.wq_status_str(status(STAGE_SHAPE, wq.WQ_ERR_SHAPE))
    assert wq.wq_status_str(status(6, 1)).startswith("kernel-launch:")
    assert wq.wq_status_str(17).startswith("unknown")


def gemm_args(**over):
    base = dict(abi_version=wq.WQ_ABI_VERSION, struct_size=ctypes.sizeof(wq.wq_gemm_args),
                a=0x1000, b=0x2000,
                c=0x3000, b_scales=0x4000, zero_points=None, perm=None, group_index=None,
                a_tmp=None,
                workspace=None, workspace_bytes=0, stream=None, m=16, n=256, k=1024, lda=1024,
                group_size=128, flags=0, split_k=0, reserved=0)
    base.update(over)
    return wq.wq_gemm_args(**base)


def call_gemm(L, **over):
    return L.wq_gemm(ctypes.byref(gemm_args(**over)))


@pytest.mark.parametrize("over,expect", [
    (dict(a=None), status(STAGE_ARGS, wq.WQ_ERR_NULL)),
    (dict(b=None), status(STAGE_ARGS, wq.WQ_ERR_NULL)),
    (dict(c=None), status(STAGE_ARGS, wq.WQ_ERR_NULL)),
    (dict(b_scales=None), status(STAGE_ARGS, wq.WQ_ERR_NULL)),
    (dict(a=0x1002), status(STAGE_ARGS, wq.WQ_ERR_ALIGN)),
    (dict(c=0x3008), status(STAGE_ARGS, wq.WQ_ERR_ALIGN)),
    (dict(k=1000, lda=1000), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    (dict(n=320), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    (dict(m=0), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    (dict(lda=512), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    (dict(lda=1028), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    # group sizes: -1 and multiples of 16 dividing k (k = 1024 here) are supported
    (dict(group_size=8), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),      # not a multiple of 16
    (dict(group_size=24), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),     # not a multiple of 16
    (dict(group_size=48), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),     # does not divide k
    (dict(group_size=96), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),     # does not divide k
    (dict(group_size=192), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),    # does not divide k
    (dict(group_size=2048), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),   # does not divide k
    (dict(group_size=-2), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    (dict(group_size=0), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    (dict(flags=wq.WQ_FLAG_HAS_ZP), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(zero_points=0x5000), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(flags=wq.WQ_FLAG_HAS_ZP, zero_points=0x5008), status(STAGE_ARGS, wq.WQ_ERR_ALIGN)),
    (dict(flags=wq.WQ_FLAG_ATOMIC_ADD), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(flags=1 << 10), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(flags=wq.WQ_FLAG_ACT_ORDER), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(perm=0x6000), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(flags=wq.WQ_FLAG_ACT_ORDER, perm=0x6000), status(STAGE_ARGS, wq.WQ_ERR_NULL)),
    # group_index: only with act_order (it checks the act_order layout's groups), 4-byte aligned
    (dict(group_index=0x6800), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(flags=wq.WQ_FLAG_ACT_ORDER, perm=0x6000, a_tmp=0x7000, group_index=0x6802),
     status(STAGE_ARGS, wq.WQ_ERR_ALIGN)),
    (dict(flags=wq.WQ_FLAG_ACT_ORDER, perm=0x6000, a_tmp=0x7000, group_index=0x6800, a=None),
     status(STAGE_ARGS, wq.WQ_ERR_NULL)),
    (dict(split_k=2), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(split_k=-1), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(flags=wq.WQ_FLAG_FP32_REDUCE, split_k=2), status(STAGE_ARGS, wq.WQ_ERR_WORKSPACE)),
    (dict(flags=wq.WQ_FLAG_FP32_REDUCE, split_k=2, workspace=0x7000, workspace_bytes=16),
     status(STAGE_ARGS, wq.WQ_ERR_WORKSPACE)),
    (dict(abi_version=wq.WQ_ABI_VERSION + 1), status(STAGE_ARGS, wq.WQ_ERR_ABI)),
    (dict(struct_size=8), status(STAGE_ARGS, wq.WQ_ERR_ABI)),
    (dict(reserved=1), status(STAGE_ARGS, wq.WQ_ERR_ABI)),
])
def test_gemm_rejects_bad_arguments_before_launch(L, over, expect):
    assert call_gemm(L, **over) == expect


def test_gemm_null_struct(L):
    assert L.wq_gemm(None) == status(STAGE_ARGS, wq.WQ_ERR_NULL)


def test_workspace_sizes():
    fp32 = wq.WQ_FLAG_FP32_REDUCE
    assert wq.wq_gemm_workspace_bytes(16, 4096, 4096, 0) == 0
    assert wq.wq_gemm_workspace_bytes(2048, 14336, 4096, fp32) == 0
    assert wq.wq_gemm_workspace_bytes(1, 256, 128, fp32) == 0   # one group: never split
    ws = wq.wq_gemm_workspace_bytes(1, 14336, 4096, fp32)
    assert ws == 16 * 1 * 14336 * 4          # fp32 partials of up to 16 splits
    assert wq.wq_gemm_workspace_bytes(16, 4096, 4096, fp32) >= 16 * 16 * 4096 * 4
    # m > 16: the tiled kernel's split, about one work-group per CU: 256 // 56 tiles = 4 at
    # n = 14336; none once the tiles fill most CUs (224 tiles at m = 512)
    assert wq.wq_gemm_workspace_bytes(128, 14336, 4096, fp32) == 4 * 128 * 14336 * 4
    assert wq.wq_gemm_workspace_bytes(512, 14336, 4096, fp32) == 0
    # from k = 8192, two work-groups per CU once the tiles fill half of them: 512 // 128 at
    # m = 1024, 512 // 256 at m = 2048; 256 // 64 below that
    assert wq.wq_gemm_workspace_bytes(1024, 4096, 14336, fp32) == 4 * 1024 * 4096 * 4
    assert wq.wq_gemm_workspace_bytes(2048, 4096, 14336, fp32) == 2 * 2048 * 4096 * 4
    assert wq.wq_gemm_workspace_bytes(512, 4096, 14336, fp32) == 4 * 512 * 4096 * 4
    assert wq.wq_gemm_workspace_bytes(128, 14336, 4096, 0) == 0
    # at most two groups of K per split: k = 512 allows 2
    assert wq.wq_gemm_workspace_bytes(100, 256, 512, fp32) == 2 * 100 * 256 * 4
    with pytest.raises(wq.WQError):
        wq.wq_gemm_workspace_bytes(1, 100, 4096, fp32)


def test_repack_and_dequant_validation(L):
    assert L.wq_repack_b(None, None, 0x2000, 1024, 256, None) == status(STAGE_ARGS, wq.WQ_ERR_NULL)
    assert L.wq_repack_b(0x1000, None, 0x2008, 1024, 256, None) == status(STAGE_ARGS,
                                                                         wq.WQ_ERR_ALIGN)
    assert L.wq_repack_b(0x1000, None, 0x2000, 1000, 256, None) == status(STAGE_SHAPE,
                                                                         wq.WQ_ERR_SHAPE)
    assert L.wq_repack_b(0x1000, 0x3002, 0x2000, 1024, 256, None) == status(STAGE_ARGS,
                                                                           wq.WQ_ERR_ALIGN)
    assert L.wq_repack_scales(0x1000, 0x2000, 1024, 256, 48, None) == status(STAGE_SHAPE,
                                                                            wq.WQ_ERR_SHAPE)
    assert L.wq_repack_zeros(0x1000, None, 1024, 256, 128, None) == status(STAGE_ARGS,
                                                                          wq.WQ_ERR_NULL)
    assert L.wq_dequant(0x1000, 0x2000, None, 1024, 256, 128, wq.WQ_FLAG_HAS_ZP, 0x3000,
                        None) == status(STAGE_ARGS, wq.WQ_ERR_FLAGS)
    # unknown flag bits (beyond HAS_ZP, ACT_ORDER, IS_K_FULL, BF16 and FP8) are rejected
    assert L.wq_dequant(0x1000, 0x2000, None, 1024, 256, 128, 1 << 10, 0x3000,
                        None) == status(STAGE_ARGS, wq.WQ_ERR_FLAGS)
    assert L.wq_dequant(0x1000, 0x2000, None, 1024, 256, 128, wq.WQ_FLAG_SWIGLU, 0x3000,
                        None) == status(STAGE_ARGS, wq.WQ_ERR_FLAGS)


def test_fp8_validation_before_launch(L):
    FP8 = wq.WQ_FLAG_FP8
    # the pages' E4M3 rules: group_size -1 or 128, no zero points; and no act_order here
    # (bf16 activations and the SwiGLU epilogue are valid, so no fake-pointer call uses them)
    assert call_gemm(L, flags=FP8, group_size=64) == status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)
    assert call_gemm(L, flags=FP8, group_size=256) == status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)
    assert call_gemm(L, flags=FP8 | wq.WQ_FLAG_HAS_ZP, zero_points=0x5000) == status(
        STAGE_ARGS, wq.WQ_ERR_FLAGS)
    assert call_gemm(L, flags=FP8 | wq.WQ_FLAG_BF16, group_size=32) == status(
        STAGE_SHAPE, wq.WQ_ERR_SHAPE)
    assert call_gemm(L, flags=FP8 | wq.WQ_FLAG_SWIGLU | wq.WQ_FLAG_HAS_ZP,
                     zero_points=0x5000) == status(STAGE_ARGS, wq.WQ_ERR_FLAGS)
    assert call_gemm(L, flags=FP8 | wq.WQ_FLAG_ACT_ORDER, perm=0x6000,
                     a_tmp=0x6100) == status(STAGE_ARGS, wq.WQ_ERR_FLAGS)
    assert L.wq_dequant(0x1000, 0x2000, None, 1024, 256, 64, FP8, 0x3000,
                        None) == status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)
    assert L.wq_dequant(0x1000, 0x2000, 0x4000, 1024, 256, 128, FP8 | wq.WQ_FLAG_HAS_ZP,
                        0x3000, None) == status(STAGE_ARGS, wq.WQ_ERR_FLAGS)
    assert L.wq_repack_fp8(None, 0x2000, 1024, 256, None) == status(STAGE_ARGS,
                                                                   wq.WQ_ERR_NULL)
    assert L.wq_repack_fp8(0x1000, 0x2008, 1024, 256, None) == status(STAGE_ARGS,
                                                                     wq.WQ_ERR_ALIGN)
    assert L.wq_repack_fp8(0x1000, 0x2000, 1000, 256, None) == status(STAGE_SHAPE,
                                                                     wq.WQ_ERR_SHAPE)
    for fn in (L.wq_repack_fp8_rows, L.wq_fp8_block_scales):
        assert fn(None, 0x2000, 1024, 256, None) == status(STAGE_ARGS, wq.WQ_ERR_NULL)
        assert fn(0x1000, 0x2008, 1024, 256, None) == status(STAGE_ARGS, wq.WQ_ERR_ALIGN)
        assert fn(0x1000, 0x2000, 1024, 320, None) == status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)
    assert L.wq_repack_fp8_rows(0x1002, 0x2000, 1024, 256, None) == status(STAGE_ARGS,
                                                                          wq.WQ_ERR_ALIGN)


def test_flag_values_match_the_header():
    with open(os.path.join(ROOT, "include", "wq.h")) as f:
        text = f.read()
    found = dict((name, int(bit)) for name, bit in
                 re.findall(r"#define (WQ_FLAG_[A-Z_0-9]+)\s+\(1u << (\d+)\)", text))
    assert found["WQ_FLAG_BF16"] == 8
    for name, bit in found.items():
        assert getattr(wq, name) == 1 << bit, name


def test_stream_read_sizing_and_validation(L):
    # one wave reads 64 lanes x 8 granules of 16 B; four waves per work-group
    assert wq.wq_stream_read_sink_words(29360128) == 3584
    assert wq.wq_stream_read_sink_words(16) == 4
    assert wq.wq_stream_read_sink_words(8192 * 5) == 8
    with pytest.raises(wq.WQError):
        wq.wq_stream_read_sink_words(100)
    with pytest.raises(wq.WQError):
        wq.wq_stream_read_sink_words(0)
    assert L.wq_stream_read(None, 1024, 0x2000, 4, None) == status(STAGE_ARGS, wq.WQ_ERR_NULL)
    assert L.wq_stream_read(0x1008, 1024, 0x2000, 4, None) == status(STAGE_ARGS,
                                                                      wq.WQ_ERR_ALIGN)
    assert L.wq_stream_read(0x1000, 1024, 0x2000, 3, None) == status(STAGE_ARGS,
                                                                      wq.WQ_ERR_WORKSPACE)
    assert L.wq_stream_read(0x1000, 1000, 0x2000, 4, None) == status(STAGE_SHAPE,
                                                                      wq.WQ_ERR_SHAPE)


def test_interleave_gate_up_validation(L):
    assert L.wq_interleave_gate_up(0x1000, 0x2000, 0x3000, 4, 32, 8, None) == status(
        STAGE_SHAPE, wq.WQ_ERR_SHAPE)                      # bits per column
    assert L.wq_interleave_gate_up(0x1000, 0x2000, 0x3000, 4, 24, 16, None) == status(
        STAGE_SHAPE, wq.WQ_ERR_SHAPE)                      # columns not a multiple of 16
    assert L.wq_interleave_gate_up(None, 0x2000, 0x3000, 4, 32, 16, None) == status(
        STAGE_ARGS, wq.WQ_ERR_NULL)
    assert L.wq_interleave_gate_up(0x1000, 0x2002, 0x3000, 4, 32, 16, None) == status(
        STAGE_ARGS, wq.WQ_ERR_ALIGN)


def test_repack_validation_of_group_sizes(L):
    # group sizes are -1 or multiples of 16 dividing k: at k = 1024, 48, 96 and 768 do not
    # divide it, 8, 24 and 40 are not multiples of 16; at k = 384, 80 does not divide it
    for k, gs in ((1024, 48), (1024, 96), (1024, 768), (1024, 8), (1024, 24), (1024, 40),
                  (1024, -2), (1024, 0), (384, 80), (384, 40)):
        assert L.wq_repack_scales(0x1000, 0x2000, k, 256, gs, None) == status(
            STAGE_SHAPE, wq.WQ_ERR_SHAPE), (k, gs)
        assert L.wq_repack_zeros(0x1000, 0x2000, k, 256, gs, None) == status(
            STAGE_SHAPE, wq.WQ_ERR_SHAPE), (k, gs)


def test_act_order_perm_with_other_group_sizes():
    g_idx = synthetic.act_order_g_idx(4, 1024, 256)
    perm, sorted_g = wq.wq_act_order_perm(g_idx, 256)
    operm, osorted = ref.act_order_perm(g_idx, 256)
    assert np.array_equal(perm, operm) and np.array_equal(sorted_g, osorted)
    # channelwise: one group of all rows, so the stable argsort is the identity
    perm, sorted_g = wq.wq_act_order_perm(np.zeros(512, np.int32), -1)
    assert perm.tolist() == list(range(512)) and not sorted_g.any()


def test_act_order_perm_matches_oracle_and_rejects_uneven_groups():
    for seed in (1, 2, 3):
        g_idx = synthetic.act_order_g_idx(seed, 4096, 128)
        perm, sorted_g = wq.wq_act_order_perm(g_idx, 128)
        operm, osorted = ref.act_order_perm(g_idx, 128)
        assert np.array_equal(perm, operm) and np.array_equal(sorted_g, osorted)
    with pytest.raises(wq.WQError) as e:
        wq.wq_act_order_perm(np.array([0, 0, 0, 1], np.int32), 2)
    assert e.value.code == wq.WQ_ERR_ACT_ORDER
    with pytest.raises(wq.WQError):
        wq.wq_act_order_perm(np.array([0, 5, 0, 1], np.int32), 2)


def test_csr_builder_reproduces_the_pages_examples():
    for case in golden_csr_cases():
        if case["kind"] != "token_routes":
            continue
        csr = wq.wq_csr_from_routes(case["selected"], case["n_tokens"][0], case["top_k"][0],
                                    case["n_expert"][0])
        for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok"):
            assert csr[key].tolist() == case[key], key


def test_csr_builder_matches_oracle_on_random_routes():
    routes = synthetic.top2_routes(5, 1024, 8)
    csr = wq.wq_csr_from_routes(routes, 1024, 2, 8)
    ocsr = ref.csr_from_token_routes(8, 1024, 2, routes)
    for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok"):
        assert csr[key].tolist() == list(ocsr[key]), key
    # inactive experts are left out
    few = np.array([[1, 5]] * 7, dtype=np.int32)
    csr = wq.wq_csr_from_routes(few, 7, 2, 8)
    assert csr["ex_ids"].tolist() == [1, 5] and csr["ex_off"].tolist() == [0, 7, 14]


def test_csr_builder_rejects_out_of_range_expert():
    with pytest.raises(wq.WQError) as e:
        wq.wq_csr_from_routes(np.array([0, 8], np.int32), 1, 2, 8)
    assert e.value.code == wq.WQ_ERR_CSR


def grouped_args(**over):
    base = dict(abi_version=wq.WQ_ABI_VERSION, struct_size=ctypes.sizeof(wq.wq_grouped_args),
                a=0x1000,
                b_bank=0x2000, b_stride_bytes=1024 * 256 // 2, s_bank=0x3000,
                s_stride_bytes=8 * 256 * 2, zp_bank=None, zp_stride_bytes=0, ex_ids=None,
                ex_off=0x4000, ex_pairs=0x5000, pair_tok=0x6000, y=0x7000, workspace=None,
                workspace_bytes=0, stream=None, n_expert=2, n_active=2, n_pairs=4, n_tokens=2,
                k=1024, n=256, group_size=128, flags=0, reserved=0)
    base.update(over)
    return wq.wq_grouped_args(**base)


@pytest.mark.parametrize("over,expect", [
    (dict(a=None), status(STAGE_ARGS, wq.WQ_ERR_NULL)),
    (dict(y=0x7004), status(STAGE_ARGS, wq.WQ_ERR_ALIGN)),
    (dict(ex_off=None), status(STAGE_ARGS, wq.WQ_ERR_NULL)),
    (dict(ex_pairs=0x5002), status(STAGE_ARGS, wq.WQ_ERR_ALIGN)),
    (dict(n_active=3), status(STAGE_ARGS, wq.WQ_ERR_CSR)),
    (dict(n_pairs=0), status(STAGE_ARGS, wq.WQ_ERR_CSR)),
    (dict(n_tokens=0), status(STAGE_ARGS, wq.WQ_ERR_CSR)),
    (dict(b_stride_bytes=1000), status(STAGE_ARGS, wq.WQ_ERR_SHAPE)),
    (dict(s_stride_bytes=16), status(STAGE_ARGS, wq.WQ_ERR_SHAPE)),
    (dict(flags=wq.WQ_FLAG_HAS_ZP), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(flags=wq.WQ_FLAG_ACT_ORDER), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    # routing weights: the flag and the pointer go together (marlin.rs MoE validation)
    (dict(flags=wq.WQ_FLAG_MUL_TOPK_WEIGHTS), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(topk_weights=0x8000), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(topk_weights=0x8002, flags=wq.WQ_FLAG_MUL_TOPK_WEIGHTS),
     status(STAGE_ARGS, wq.WQ_ERR_ALIGN)),
    (dict(k=1000), status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    (dict(struct_size=4), status(STAGE_ARGS, wq.WQ_ERR_ABI)),
    (dict(abi_version=1), status(STAGE_ARGS, wq.WQ_ERR_ABI)),
    # the SwiGLU activation takes no routing weight
    (dict(topk_weights=0x8000, flags=wq.WQ_FLAG_MUL_TOPK_WEIGHTS | wq.WQ_FLAG_SWIGLU),
     status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    (dict(flags=1 << 10), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
    # E4M3 banks: one byte per weight, so a 4-bit bank stride is too short; the pages'
    # group sizes (-1, 128) and no zero points
    (dict(flags=wq.WQ_FLAG_FP8), status(STAGE_ARGS, wq.WQ_ERR_SHAPE)),
    (dict(flags=wq.WQ_FLAG_FP8, group_size=64, b_stride_bytes=1024 * 256),
     status(STAGE_SHAPE, wq.WQ_ERR_SHAPE)),
    (dict(flags=wq.WQ_FLAG_FP8 | wq.WQ_FLAG_HAS_ZP, zp_bank=0x9000, zp_stride_bytes=4096,
          b_stride_bytes=1024 * 256), status(STAGE_ARGS, wq.WQ_ERR_FLAGS)),
])
def test_grouped_rejects_bad_arguments_before_launch(L, over, expect):
    assert L.wq_grouped_gemm(ctypes.byref(grouped_args(**over))) == expect


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(wq, "_LIB", None)
    monkeypatch.setattr(wq, "LIB_PATH", "/nonexistent/libwq.so")
    with pytest.raises(RuntimeError):
        wq.wq_abi_version()


def test_gemm_plan_names_the_kernel_and_split():
    """The planner's choice for the benchmarked shapes (host only, no device access)."""
    fp32, zp, act = wq.WQ_FLAG_FP32_REDUCE, wq.WQ_FLAG_HAS_ZP, wq.WQ_FLAG_ACT_ORDER
    small, t256, t128 = wq.WQ_KERNEL_SMALL_M, wq.WQ_KERNEL_TILE_256, wq.WQ_KERNEL_TILE_128
    # decode: 896 column blocks fill the CUs, so the fp32 reduce flag leads to no split
    assert wq.wq_gemm_plan(1, 14336, 4096, flags=fp32) == (small, 1)
    assert wq.wq_gemm_plan(16, 4096, 4096, flags=fp32 | zp) == (small, 1)
    assert wq.wq_gemm_plan(2048, 14336, 4096, flags=act) == (t256, 1)
    # few column blocks: split along K (at most a quarter of the groups, one per wave)
    assert wq.wq_gemm_plan(1, 256, 1024, flags=fp32) == (small, 2)
    assert wq.wq_gemm_plan(1, 256, 4096, flags=fp32, split_k=3) == (small, 3)
    assert wq.wq_gemm_plan(1, 256, 1024) == (small, 1)
    # mid-size m: 128-row tiles, split for about one work-group per CU (256 // 56 tiles)
    assert wq.wq_gemm_plan(64, 14336, 4096, flags=fp32) == (t128, 4)
    assert wq.wq_gemm_plan(256, 14336, 4096, flags=fp32) == (t128, 2)
    assert wq.wq_gemm_plan(256, 14336, 4096) == (t128, 1)
    # 17..64 rows without the fp32 reduce flag: the small-M kernel in 16-row chunks, unsplit
    for m in (17, 32, 48, 64):
        assert wq.wq_gemm_plan(m, 14336, 4096) == (small, 1), m
        assert wq.wq_gemm_plan(m, 14336, 4096, flags=fp32)[0] == t128, m
    assert wq.wq_gemm_plan(80, 14336, 4096) == (small, 1)    # five chunks, 147 MB of reads
    assert wq.wq_gemm_plan(81, 14336, 4096) == (t128, 1)     # six would pass the budget
    assert wq.wq_gemm_plan(256, 4096, 4096) == (small, 1)    # sixteen chunks of 8.4 MB
    assert wq.wq_gemm_plan(24, 28672, 8192) == (t128, 1)     # staged chunks past the budget
    # with the flag, direct chunks within K x 12 kB of weight reads (else split tiles)
    assert wq.wq_gemm_plan(64, 4096, 4096, flags=fp32) == (small, 1)
    assert wq.wq_gemm_plan(96, 4096, 4096, flags=fp32)[0] == t128
    assert wq.wq_gemm_plan(32, 14336, 4096, flags=wq.WQ_FLAG_SWIGLU)[0] != small
    # long K: sixteen waves on one work-group per column block (no flag: never split);
    # with the flag, beyond 128 groups, splits of at most 64 groups, and of at most 32 where
    # the grid exceeds two work-groups per CU (16 from four rows, beyond one per CU)
    assert wq.wq_gemm_plan(1, 4096, 14336) == (small, 1)
    assert wq.wq_gemm_plan(1, 8192, 28672) == (small, 1)
    assert wq.wq_gemm_plan(1, 8192, 28672, flags=fp32) == (small, 7)
    assert wq.wq_gemm_plan(1, 2048, 28672, flags=fp32) == (small, 4)
    assert wq.wq_gemm_plan(1, 14336, 14336, flags=fp32) == (small, 4)
    assert wq.wq_gemm_plan(1, 8192, 14336, flags=fp32) == (small, 1)
    assert wq.wq_gemm_plan(4, 4096, 14336, flags=fp32) == (small, 1)
    assert wq.wq_gemm_plan(8, 4096, 14336, flags=fp32) == (small, 7)
    assert wq.wq_gemm_plan(4, 8192, 8192, flags=fp32) == (small, 1)
    assert wq.wq_gemm_plan(12, 8192, 28672, flags=fp32) == (small, 14)
    assert wq.wq_gemm_plan(8, 4096, 14336) == (small, 1)   # two staged 4-row chunks
    # the planner's split always fits the workspace the library asks for
    for m, n in ((1, 256), (64, 14336), (256, 14336), (16, 512)):
        _, s = wq.wq_gemm_plan(m, n, 1024 if n == 256 else 4096, flags=fp32)
        need = wq.wq_gemm_workspace_bytes(m, n, 1024 if n == 256 else 4096, fp32)
        assert s == 1 or need >= s * m * n * 4
    with pytest.raises(wq.WQError):
        wq.wq_gemm_plan(1, 100, 4096)


def test_noalloc_rejects_caller_scratch_and_oversize(L):
    """wq_gemm_noalloc takes no caller scratch, and refuses problems whose scratch would
    exceed its static array, before touching any device."""
    ws = status(STAGE_ARGS, wq.WQ_ERR_WORKSPACE)
    assert L.wq_gemm_noalloc(ctypes.byref(gemm_args(workspace=0x7000, workspace_bytes=64))) == ws
    assert L.wq_gemm_noalloc(ctypes.byref(gemm_args(a_tmp=0x7000))) == ws
    big = gemm_args(m=8192, k=4096, lda=4096, flags=wq.WQ_FLAG_ACT_ORDER, perm=0x6000)
    assert L.wq_gemm_noalloc(ctypes.byref(big)) == ws
    assert L.wq_gemm_noalloc(None) == status(STAGE_ARGS, wq.WQ_ERR_NULL)
    assert L.wq_gemm_noalloc(ctypes.byref(gemm_args(abi_version=2))) == status(STAGE_ARGS,
                                                                               wq.WQ_ERR_ABI)
