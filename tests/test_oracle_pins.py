"""Pins of the CPU oracle to facts fixed by the pages and by plain arithmetic.

Each test checks the oracle against something other than itself: a value printed on a
page (golden fixtures), a closed form, or a brute-force computation in plain Python that
decodes words through their hexadecimal digits rather than through shifts.
"""

import struct

import math

import numpy as np
import pytest

from conftest import golden_csr_cases, read_golden
from oracle import layout, reference as ref
import synthetic


def hex_nibbles(word):
    """The eight 4-bit fields of a word, lowest first, read from its hex digits."""
    h = f"{int(word) & 0xFFFFFFFF:08x}"
    return [int(h[7 - i], 16) for i in range(8)]


def hex_word(nibbles):
    """Inverse of hex_nibbles: eight fields (lowest first) to a word via hex digits."""
    return int("".join(f"{v:x}" for v in reversed(nibbles)), 16)


def codes_bruteforce(qweight):
    """Codes [K][N] as nested Python lists, decoded digit by digit."""
    k8, n = qweight.shape
    out = [[0] * n for _ in range(8 * k8)]
    for r in range(k8):
        for c in range(n):
            for i, v in enumerate(hex_nibbles(qweight[r, c])):
                out[8 * r + i][c] = v
    return out


def zero_codes_bruteforce(zeros):
    g, n8 = zeros.shape
    return [[hex_nibbles(zeros[gi, c // 8])[c % 8] for c in range(8 * n8)] for gi in range(g)]


def gemm_bruteforce(a, codes, scales, group, zcodes=None):
    """Plain-Python triple loop with exact float products (fp64)."""
    m, k = a.shape
    n = len(codes[0])
    out = [[0.0] * n for _ in range(m)]
    for mi in range(m):
        for c in range(n):
            acc = 0.0
            for ki in range(k):
                z = 8 if zcodes is None else zcodes[group[ki]][c]
                w = (codes[ki][c] - z) * float(scales[group[ki], c])
                acc += float(a[mi, ki]) * w
            out[mi][c] = acc
    return np.array(out)


# --------------------------------------------------------------------------- formats

def test_zero_point_words_match_page_example():
    for parts in read_golden("zero_point_words.txt"):
        word = int(parts[0], 16)
        codes = [int(x) for x in parts[1:]]
        got = ref.unpack_zero_points(np.array([[word]], dtype=np.uint32))[0].tolist()
        assert got == codes
        assert hex_word(codes) == word


def test_qweight_rows_are_low_nibble_first():
    # column 0 holds rows 0..7 = 0..7 and column 1 rows = 15..8
    w0 = hex_word(list(range(8)))
    w1 = hex_word(list(range(15, 7, -1)))
    assert w0 == 0x76543210
    q = ref.unpack_qweight(np.array([[w0, w1]], dtype=np.uint32))
    assert q[:, 0].tolist() == list(range(8))
    assert q[:, 1].tolist() == list(range(15, 7, -1))


def test_unpack_matches_hex_digits_on_random_words():
    qw = synthetic.qweight_words(11, 64, 24)
    assert ref.unpack_qweight(qw).tolist() == codes_bruteforce(qw)
    zw = synthetic.zero_point_words(12, 3, 32)
    assert ref.unpack_zero_points(zw).tolist() == zero_codes_bruteforce(zw)


def test_group_counts_match_page():
    for k, gs, expect in read_golden("group_counts.txt"):
        if expect == "error":
            with pytest.raises(ValueError):
                ref.num_groups(int(k), int(gs))
        else:
            assert ref.num_groups(int(k), int(gs)) == int(expect)


# --------------------------------------------------------------------------- closed forms

def test_all_eight_codes_give_exact_zero():
    """u4b8 code 8 means 0, so C == 0 for any A and scales."""
    k, n = 256, 32
    a = synthetic.activations(1, 5, k)
    qw = np.full((k // 8, n), 0x88888888, dtype=np.uint32)
    s = synthetic.scales(2, k // 128, n)
    c = ref.w4a16_gemm(a, qw, s)
    assert np.all(c == 0.0)


def test_codes_equal_to_zero_points_give_exact_zero():
    """u4 with q == z in every group and column gives C == 0."""
    k, n = 256, 16
    zcodes = [[(3 * g + c) % 16 for c in range(n)] for g in range(2)]
    zeros = np.array([[hex_word(zcodes[g][8 * j:8 * j + 8]) for j in range(n // 8)]
                      for g in range(2)], dtype=np.uint32)
    qw = np.array([[hex_word([zcodes[(8 * r) // 128][c]] * 8) for c in range(n)]
                   for r in range(k // 8)], dtype=np.uint32)
    a = synthetic.activations(3, 4, k)
    s = synthetic.scales(4, 2, n)
    assert np.all(ref.w4a16_gemm(a, qw, s, zeros=zeros) == 0.0)


def test_unit_scales_match_integer_bruteforce():
    """s = 1 and A in {-1, 0, 1}: every output is the exact integer sum of (q - 8)."""
    m, k, n = 3, 256, 16
    rng_codes = synthetic.qweight_words(5, k, n)
    trits = (synthetic.below(6, m * k, 3) - 1).reshape(m, k).astype(np.float16)
    ones = np.ones((k // 128, n), dtype=np.float16)
    codes = codes_bruteforce(rng_codes)
    want = [[sum(int(trits[i, kk]) * (codes[kk][c] - 8) for kk in range(k)) for c in range(n)]
            for i in range(m)]
    got = ref.w4a16_gemm(trits, rng_codes, ones)
    assert got.tolist() == [[float(v) for v in row] for row in want]


def test_one_hot_rows_select_one_dequantized_weight_row():
    """A = e_k picks row k: C = (q[k, :] - 8) * s[k // 128, :], exactly."""
    k, n = 512, 32
    qw = synthetic.qweight_words(7, k, n)
    s = synthetic.scales(8, k // 128, n)
    rows = [0, 1, 127, 128, 200, 383, 384, 511]
    a = np.zeros((len(rows), k), dtype=np.float16)
    for i, r in enumerate(rows):
        a[i, r] = 1.0
    codes = codes_bruteforce(qw)
    got = ref.w4a16_gemm(a, qw, s)
    for i, r in enumerate(rows):
        want = [(codes[r][c] - 8) * float(s[r // 128, c]) for c in range(n)]
        assert got[i].tolist() == want


def test_zero_point_product_matches_bruteforce():
    m, k, n = 2, 256, 16
    a = synthetic.activations(9, m, k)
    qw = synthetic.qweight_words(10, k, n)
    s = synthetic.scales(11, 2, n)
    zw = synthetic.zero_point_words(12, 2, n)
    group = [kk // 128 for kk in range(k)]
    want = gemm_bruteforce(a, codes_bruteforce(qw), s, group, zero_codes_bruteforce(zw))
    got = ref.w4a16_gemm(a, qw, s, zeros=zw)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_act_order_product_matches_bruteforce():
    m, k, n = 2, 256, 16
    a = synthetic.activations(13, m, k)
    qw = synthetic.qweight_words(14, k, n)
    s = synthetic.scales(15, 2, n)
    g_idx = synthetic.act_order_g_idx(16, k, 128)
    want = gemm_bruteforce(a, codes_bruteforce(qw), s, [int(x) for x in g_idx])
    got = ref.w4a16_gemm(a, qw, s, g_idx=g_idx)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_act_order_equals_plain_product_on_permuted_operands():
    """Gathering A's columns and B's rows by perm = argsort(g_idx) leaves C unchanged."""
    m, k, n = 4, 512, 32
    a = synthetic.activations(17, m, k)
    qw = synthetic.qweight_words(18, k, n)
    s = synthetic.scales(19, k // 128, n)
    g_idx = synthetic.act_order_g_idx(20, k, 128)
    perm = sorted(range(k), key=lambda r: (int(g_idx[r]), r))
    codes = codes_bruteforce(qw)
    qw_perm = np.array([[hex_word([codes[perm[8 * r + i]][c] for i in range(8)])
                         for c in range(n)] for r in range(k // 8)], dtype=np.uint32)
    plain = ref.w4a16_gemm(a[:, perm], qw_perm, s)
    ordered = ref.w4a16_gemm(a, qw, s, g_idx=g_idx)
    np.testing.assert_allclose(ordered, plain, rtol=1e-12, atol=1e-12)
    p, sorted_g = ref.act_order_perm(g_idx, 128)
    assert p.tolist() == perm
    assert sorted_g.tolist() == [i // 128 for i in range(k)]


def test_act_order_perm_keeps_ties_in_row_order_and_rejects_uneven_groups():
    g_idx = np.array([1, 0, 1, 0], dtype=np.int32)
    p, sg = ref.act_order_perm(g_idx, 2)
    assert p.tolist() == [1, 3, 0, 2] and sg.tolist() == [0, 0, 1, 1]
    with pytest.raises(ValueError):
        ref.act_order_perm(np.array([0, 0, 0, 1], dtype=np.int32), 2)


def test_fp16_dequant_is_one_round_to_nearest_even():
    s = synthetic.scales(21, 1, 64)[0]
    for d in range(-15, 16):
        q = np.full((1, 64), max(d, 0), dtype=np.uint8)
        z = np.full((1, 64), max(-d, 0), dtype=np.uint8)
        w = ref.dequantize(q, s[None, :], np.zeros(1, dtype=np.int64), z)
        got = ref.dequantize_fp16(w)[0]
        for c in range(64):
            exact = d * float(s[c])
            want = struct.unpack("<e", struct.pack("<e", exact))[0]
            assert float(got[c]) == want


# --------------------------------------------------------------------------- CSR

def test_csr_worked_examples_from_page():
    for case in golden_csr_cases():
        if case["kind"] == "token_routes":
            csr = ref.csr_from_token_routes(case["n_expert"][0], case["n_tokens"][0],
                                            case["top_k"][0], case["selected"])
        else:
            csr = ref.csr_from_pair_rows(case["n_expert"][0], case["n_tokens"][0],
                                         case["selected"], case["pair_tok_in"])
        for key in ("ex_ids", "ex_off", "ex_pairs", "pair_tok"):
            assert list(csr[key]) == case[key], key


def test_csr_rejects_the_pages_bad_routes_and_parts():
    with pytest.raises(ref.CsrError):
        ref.csr_from_token_routes(4, 2, 3, [0, 1])
    with pytest.raises(ref.CsrError):
        ref.csr_from_pair_rows(2, 1, [2], [0])
    with pytest.raises(ref.CsrError):
        ref.csr_from_pair_rows(2, 1, [0], [1])
    with pytest.raises(ref.CsrError):
        ref.validate_csr(dict(ex_ids=[0, 1], ex_off=[0, 1, 2], ex_pairs=[0, 0],
                              pair_tok=[0, 1], n_expert=2, n_tokens=2))
    with pytest.raises(ref.CsrError):
        ref.validate_csr(dict(ex_ids=[1, 0], ex_off=[0, 1, 2], ex_pairs=[0, 1],
                              pair_tok=[0, 1], n_expert=2, n_tokens=2))


def test_grouped_product_equals_dense_rows():
    """Every pair's row equals the dense product of its token row with its expert."""
    k, n, tokens, experts = 256, 32, 6, 3
    a = synthetic.activations(22, tokens, k)
    ex = [dict(qweight=synthetic.qweight_words(23 + e, k, n),
               scales=synthetic.scales(30 + e, 2, n)) for e in range(experts)]
    routes = np.array([[0, 2], [1, 0], [2, 1], [2, 0], [1, 2], [0, 1]])
    csr = ref.csr_from_token_routes(experts, tokens, 2, routes)
    y = ref.grouped_w4a16_gemm(a, ex, csr)
    for p in range(2 * tokens):
        t, e = p // 2, int(routes.reshape(-1)[p])
        dense = ref.w4a16_gemm(a[t:t + 1], ex[e]["qweight"], ex[e]["scales"])
        assert y[p].tolist() == dense[0].tolist()


def test_larger_and_channelwise_groups_equal_repeated_128_row_groups():
    """A group of 256 or 512 rows (or one channelwise group) is the same as 128-row groups
    repeating its scales and zero points: the row -> group map must use the group size."""
    k, n, m = 1024, 32, 3
    a = synthetic.activations(60, m, k)
    qw = synthetic.qweight_words(61, k, n)
    for gs in (256, 512, -1):
        groups = ref.num_groups(k, gs)
        rep = (k // 128) // groups
        s = synthetic.scales(62 + gs % 7, groups, n)
        z = synthetic.zero_point_words(63, groups, n)
        got = ref.w4a16_gemm(a, qw, s, zeros=z, group_size=gs)
        want = ref.w4a16_gemm(a, qw, np.repeat(s, rep, axis=0), zeros=np.repeat(z, rep, axis=0),
                              group_size=128)
        assert got.tolist() == want.tolist(), gs
        assert np.array_equal(layout.repack_scales(s, k, gs),
                              layout.repack_scales(np.repeat(s, rep, axis=0)))
        assert np.array_equal(layout.repack_zero_points(z, k, gs),
                              layout.repack_zero_points(np.repeat(z, rep, axis=0)))
    # groups of 64 rows equal groups of 32 rows repeating each scale and zero point twice
    s = synthetic.scales(64, k // 64, n)
    z = synthetic.zero_point_words(65, k // 64, n)
    got = ref.w4a16_gemm(a, qw, s, zeros=z, group_size=64)
    want = ref.w4a16_gemm(a, qw, np.repeat(s, 2, axis=0), zeros=np.repeat(z, 2, axis=0),
                          group_size=32)
    assert got.tolist() == want.tolist()
    assert ref.group_of_rows(256, 32)[[31, 32, 63, 64]].tolist() == [0, 1, 1, 2]
    # with 256-row groups, row 128 is in group 0 and row 256 in group 1
    assert ref.group_of_rows(1024, 256)[[127, 128, 255, 256]].tolist() == [0, 0, 0, 1]
    assert ref.group_of_rows(1024, -1).max() == 0


def test_multiple_of_16_group_sizes_match_bruteforce():
    """Any multiple of 16 dividing K is a valid group size (16, 48, 80 here, none of which
    divides 128 or is divided by it): row r belongs to group r // group_size."""
    m, n = 2, 16
    for gs, k in ((16, 64), (48, 96), (80, 160)):
        a = synthetic.activations(70 + gs, m, k)
        qw = synthetic.qweight_words(71 + gs, k, n)
        s = synthetic.scales(72 + gs, k // gs, n)
        zw = synthetic.zero_point_words(73 + gs, k // gs, n)
        group = [kk // gs for kk in range(k)]
        want = gemm_bruteforce(a, codes_bruteforce(qw), s, group, zero_codes_bruteforce(zw))
        got = ref.w4a16_gemm(a, qw, s, zeros=zw, group_size=gs)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12, err_msg=str(gs))


def test_scale_units_are_the_gcd_with_the_chunk():
    for gs in range(16, 2049, 16):
        assert layout.unit_rows(gs) == math.gcd(gs, 128), gs
    assert layout.unit_rows(-1) == 128


def test_groups_straddling_chunks_equal_repeated_smaller_units():
    """A 48-, 96- or 192-row group is stored as 3 units of 16, 32 or 64 rows: its layout and
    its product equal those of the unit-sized groups with each row repeated 3 times."""
    k, n, m = 384, 32, 2
    a = synthetic.activations(80, m, k)
    qw = synthetic.qweight_words(81, k, n)
    for gs, unit in ((48, 16), (96, 32), (192, 64)):
        s = synthetic.scales(82 + gs, k // gs, n)
        z = synthetic.zero_point_words(83 + gs, k // gs, n)
        sr, zr = np.repeat(s, 3, axis=0), np.repeat(z, 3, axis=0)
        assert np.array_equal(layout.repack_scales(s, k, gs), layout.repack_scales(sr, k, unit))
        assert np.array_equal(layout.repack_zero_points(z, k, gs),
                              layout.repack_zero_points(zr, k, unit))
        got = ref.w4a16_gemm(a, qw, s, zeros=z, group_size=gs)
        want = ref.w4a16_gemm(a, qw, sr, zeros=zr, group_size=unit)
        assert got.tolist() == want.tolist(), gs
    # 16-row units by hand: block nb, unit u, column c
    s = synthetic.scales(90, 4, 32)
    rs = layout.repack_scales(s, 64, 16)
    for nb in range(2):
        for u in range(4):
            for c in range(16):
                assert rs[(nb * 4 + u) * 16 + c] == s[u, 16 * nb + c]


def test_bf16_values_of_known_bit_patterns():
    """bfloat16 = sign, 8 exponent bits (bias 127), 7 mantissa bits."""
    cases = {0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC040: -3.0,
             0x3F00: 0.5, 0x4049: 3.140625, 0x3F81: 1.0 + 2.0 ** -7, 0x7F7F: 255 * 2.0 ** 120,
             0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x4300: 128.0, 0x4380: 256.0}
    bits = np.array(list(cases), dtype=np.uint16)
    assert ref.bf16_value(bits).tolist() == list(cases.values())


def test_bf16_rounding_is_nearest_even_by_brute_force():
    """round_bf16 against a search over every finite positive bf16 value: the nearest one,
    and on a tie the one with an even last mantissa bit."""
    table_bits = np.arange(0x0000, 0x7F80, dtype=np.uint16)   # zero, subnormals, normals
    table = ref.bf16_value(table_bits)
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.uniform(2.0 ** -20, 2.0 ** 20, 300),
                         rng.uniform(2.0 ** -134, 2.0 ** -124, 100),  # around the subnormals
                         # exact midpoints between neighbours: ties (normal, then subnormal)
                         (table[1000:1100] + table[1001:1101]) / 2,
                         (table[5:60] + table[6:61]) / 2,
                         table[2000:2050]])
    got = ref.round_bf16(xs)
    for x, g in zip(xs, got):
        d = np.abs(table - x)
        best = np.flatnonzero(d == d.min())
        pick = best[0] if len(best) == 1 else [i for i in best if table_bits[i] % 2 == 0][0]
        assert g == table[pick], x
    assert ref.round_bf16(-xs).tolist() == (-got).tolist()


def test_bf16_product_matches_bruteforce():
    """bf16 activations and scales (bit patterns) decoded and multiplied exactly."""
    m, k, n = 2, 256, 16
    a = synthetic.activations_bf16(20, m, k)
    qw = synthetic.qweight_words(21, k, n)
    s = synthetic.scales_bf16(22, 2, n)
    zw = synthetic.zero_point_words(23, 2, n)
    group = [kk // 128 for kk in range(k)]
    want = gemm_bruteforce(ref.bf16_value(a), codes_bruteforce(qw), ref.bf16_value(s), group,
                           zero_codes_bruteforce(zw))
    got = ref.w4a16_gemm(a, qw, s, zeros=zw, bf16=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_e4m3_values_of_known_codes():
    """E4M3 (fn): bias 7, subnormals below exponent 1, 0x7F / 0xFF NaN, no infinities."""
    cases = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0,
             0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x30: 0.5, 0x77: 240.0, 0x57: 15.0, 0x5F: 30.0}
    got = ref.e4m3_value(np.array(list(cases), dtype=np.uint8))
    assert got.tolist() == list(cases.values())
    assert np.isnan(ref.e4m3_value(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    assert np.signbit(ref.e4m3_value(np.array([0x80], dtype=np.uint8)))[0]


def test_e4m3_values_match_torch_for_every_code():
    """Every byte against torch's float8_e4m3fn decode (a library routine the oracle does
    not use)."""
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = ref.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_fp8_words_are_k_major_little_endian():
    w = np.array([[0x04030201, 0xA0B0C0D0]], dtype=np.uint32)
    assert ref.unpack_fp8_words(w).tolist() == [[1, 0xD0], [2, 0xC0], [3, 0xB0], [4, 0xA0]]


def test_w8a16_product_matches_bruteforce():
    m, k, n = 2, 256, 16
    for gs, bf16 in ((128, False), (-1, False), (128, True)):
        a = (synthetic.activations_bf16 if bf16 else synthetic.activations)(30, m, k)
        words = synthetic.fp8_words(31, k, n)
        groups = 1 if gs == -1 else k // gs
        s = (synthetic.scales_bf16 if bf16 else synthetic.scales)(32, groups, n)
        codes = ref.unpack_fp8_words(words)
        av = ref.bf16_value(a) if bf16 else a.astype(np.float64)
        sv = ref.bf16_value(s) if bf16 else s.astype(np.float64)
        want = np.zeros((m, n))
        for mi in range(m):
            for c in range(n):
                acc = 0.0
                for kk in range(k):
                    g = 0 if gs == -1 else kk // gs
                    acc += float(av[mi, kk]) * float(ref.e4m3_value(codes[kk, c])) * sv[g, c]
                want[mi, c] = acc
        got = ref.w8a16_gemm(a, words, s, group_size=gs, bf16=bf16)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12, err_msg=str((gs, bf16)))
    with pytest.raises(ValueError):
        ref.w8a16_weights(words, s, group_size=64)


def test_block_fp8_checkpoint_product_matches_bruteforce():
    """The pages' block-FP8 reference: decoded weight = e4m3(w[n][k]) * inv[n/128][k/128],
    with the pages' inverse-scale values (bf16 0x3b80 + 0x20 r, r < 5)."""
    n, k, m = 256, 256, 2
    rng = np.random.default_rng(40)
    w_nk = synthetic.FP8_CODES[rng.integers(0, 254, size=(n, k))].astype(np.uint8)
    inv = (0x3B80 + 0x20 * rng.integers(0, 5, size=(n // 128, k // 128))).astype(np.uint16)
    a = synthetic.activations(41, m, k)
    want = np.zeros((m, n))
    for mi in range(m):
        for o in range(n):
            acc = 0.0
            for kk in range(k):
                wv = float(ref.e4m3_value(w_nk[o, kk])) * float(ref.bf16_value(inv[o // 128, kk // 128]))
                acc += float(a[mi, kk]) * wv
            want[mi, o] = acc
    got = ref.w8a16_gemm(a, ref.fp8_rows_to_words(w_nk), ref.fp8_block_scales(inv))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # the words are the transposed rows, four K-consecutive bytes each
    assert np.array_equal(ref.unpack_fp8_words(ref.fp8_rows_to_words(w_nk)), w_nk.T)


def test_fp8_layout_loops_and_inverse_agree():
    codes = np.random.default_rng(33).integers(0, 256, size=(256, 32)).astype(np.uint8)
    words = layout.repack_fp8_loops(codes)
    assert words.size * 4 == codes.size          # a permutation of the bytes
    assert np.array_equal(layout.unrepack_fp8(words, 256, 32), codes)
    # word d of lane l = c + 16*qd in block 0, group 0, half 0: rows 32*(d//2) + 8qd + 4(d%2)
    for lane in (0, 17, 63):
        c, qd = lane % 16, lane // 16
        for d in range(4):
            rows = [32 * (d // 2) + 8 * qd + 4 * (d % 2) + i for i in range(4)]
            word = int(words[lane * 4 + d])
            assert [(word >> (8 * i)) & 0xFF for i in range(4)] == [codes[r, c] for r in rows]


def test_act_order_with_256_row_groups_equals_plain_product():
    k, n, m, gs = 1024, 32, 4, 256
    a = synthetic.activations(70, m, k)
    qw = synthetic.qweight_words(71, k, n)
    s = synthetic.scales(72, k // gs, n)
    g_idx = (synthetic.permutation(73, k) // gs).astype(np.int32)
    perm, sorted_g = ref.act_order_perm(g_idx, gs)
    assert sorted_g.tolist() == (np.arange(k) // gs).tolist()
    got = ref.w4a16_gemm(a, qw, s, g_idx=g_idx, group_size=gs)
    # permuted operands: rows of W in sorted order (codes moved with their rows), A columns
    q = ref.unpack_qweight(qw)[perm, :]
    w = (q.astype(np.float64) - 8) * s.astype(np.float64)[np.arange(k) // gs, :]
    want = a.astype(np.float64)[:, perm] @ w
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_silu_closed_forms():
    e = np.e
    got = ref.silu(np.array([0.0, 1.0, -1.0, 2.0]))
    assert got[0] == 0.0
    assert abs(got[1] - e / (1 + e)) < 1e-15 and abs(got[2] + 1 / (1 + e)) < 1e-15
    assert abs(got[3] - 2 * e * e / (1 + e * e)) < 1e-15
    x = np.linspace(-12, 12, 97)
    assert np.allclose(ref.silu(x) - ref.silu(-x), x, rtol=0, atol=1e-13)  # x*(s(x)+s(-x))
    assert np.all(ref.silu(np.array([40.0, 60.0])) == np.array([40.0, 60.0]))  # exp(-x) < ulp


def test_swiglu_activation_by_brute_force():
    """act[m][j] = silu(sum_k a*wg) * (sum_k a*wu), summed here by plain loops over codes
    read from the hex digits of the words (ternary A, unit scales: exact integers)."""
    k, n, m = 128, 16, 2
    rng_a = synthetic.below(80, m * k, 3).reshape(m, k).astype(np.float64) - 1.0
    a = rng_a.astype(np.float16)
    gq, uq = synthetic.qweight_words(81, k, n), synthetic.qweight_words(82, k, n)
    ones = np.ones((1, n), np.float16)
    act = ref.swiglu_activation(a, dict(qweight=gq, scales=ones), dict(qweight=uq, scales=ones))
    for i in range(m):
        for j in range(n):
            g = u = 0.0
            for kk in range(k):
                qg = int(f"{int(gq[kk // 8, j]):08x}"[7 - kk % 8], 16) - 8
                qu = int(f"{int(uq[kk // 8, j]):08x}"[7 - kk % 8], 16) - 8
                g += float(rng_a[i, kk]) * qg
                u += float(rng_a[i, kk]) * qu
            assert act[i, j] == g / (1.0 + np.exp(-g)) * u


def test_gate_up_interleave_and_mlp_chain_shapes():
    g = np.arange(4 * 32).reshape(4, 32)
    u = 1000 + np.arange(4 * 32).reshape(4, 32)
    out = layout.interleave_gate_up(g, u)
    assert out.shape == (4, 64)
    assert out[0, :16].tolist() == g[0, :16].tolist() and out[0, 16:32].tolist() == u[0, :16].tolist()
    assert out[3, 32:48].tolist() == g[3, 16:32].tolist() and out[3, 48:].tolist() == u[3, 16:32].tolist()
    z = layout.interleave_gate_up(g[:, :4], u[:, :4], cols_per_elem=8)  # 2 words per block
    assert z[1].tolist() == [g[1, 0], g[1, 1], u[1, 0], u[1, 1], g[1, 2], g[1, 3], u[1, 2], u[1, 3]]
    k, h, i, m = 256, 256, 128, 3
    a = synthetic.activations(84, m, k)
    mk = lambda s, kk, nn: dict(qweight=synthetic.qweight_words(s, kk, nn),
                                scales=synthetic.scales(s + 1, kk // 128, nn))
    act16, out = ref.swiglu_mlp(a, mk(85, k, i), mk(87, k, i), mk(89, i, h))
    assert act16.dtype == np.float16 and act16.shape == (m, i) and out.shape == (m, h)


def fp16_nearest(x):
    """Nearest fp16 value, ties to even, by Python's own half-precision packing."""
    return struct.unpack("<e", struct.pack("<e", float(x)))[0]


BF16_ALL = np.array([struct.unpack("<f", struct.pack("<I", b << 16))[0] for b in range(0x8000)
                     if (b & 0x7F80) != 0x7F80])  # every finite non-negative bf16 value


def bf16_nearest(x):
    """Nearest bf16 value, ties to the even bit pattern, by searching every finite bf16
    value (decoded through struct, not the oracle)."""
    mag = abs(float(x))
    d = np.abs(BF16_ALL - mag)
    best = np.flatnonzero(d == d.min())
    pick = best[0] if best.size == 1 else [b for b in best if b % 2 == 0][0]
    return float(np.copysign(BF16_ALL[pick], x))


def chain_bruteforce(a_vals, gq, uq, dq, d_scales, d_zeros, round16):
    """The SwiGLU chain by plain loops: gate and up sums of unit-scale codes read from hex
    digits, act = round16(silu(g) * u), then the down projection of act with per-group
    scales and zero-point codes (also from hex digits), all exact in fp64."""
    m, k = len(a_vals), len(a_vals[0])
    i = gq.shape[1]
    h = dq.shape[1]
    act = [[0.0] * i for _ in range(m)]
    for r in range(m):
        for j in range(i):
            g = u = 0.0
            for kk in range(k):
                g += a_vals[r][kk] * (hex_nibbles(gq[kk // 8, j])[kk % 8] - 8)
                u += a_vals[r][kk] * (hex_nibbles(uq[kk // 8, j])[kk % 8] - 8)
            act[r][j] = round16(g / (1.0 + math.exp(-g)) * u)
    out = [[0.0] * h for _ in range(m)]
    for r in range(m):
        for c in range(h):
            acc = 0.0
            for j in range(i):
                grp = j // 128
                w = (hex_nibbles(dq[j // 8, c])[j % 8] - hex_nibbles(d_zeros[grp, c // 8])[c % 8])
                acc += act[r][j] * (w * d_scales[grp][c])
            out[r][c] = acc
    return np.array(act), np.array(out)


def test_swiglu_mlp_chain_by_brute_force():
    """swiglu_mlp: the fp16-rounded activation and the down projection with zero points,
    against plain loops (ternary A and unit gate/up scales keep the sums exact integers,
    so the activation's fp16 rounding is the only rounding; the down scales are not 1)."""
    k, i, h, m = 128, 256, 16, 2
    tern = synthetic.below(90, m * k, 3).reshape(m, k).astype(np.float64) - 1.0
    a = tern.astype(np.float16)
    gq, uq = synthetic.qweight_words(91, k, i), synthetic.qweight_words(92, k, i)
    dq = synthetic.qweight_words(93, i, h)
    ds = synthetic.scales(94, i // 128, h)
    dz = synthetic.zero_point_words(95, i // 128, h)
    ones = np.ones((1, i), np.float16)
    act16, out = ref.swiglu_mlp(a, dict(qweight=gq, scales=ones), dict(qweight=uq, scales=ones),
                                dict(qweight=dq, scales=ds, zeros=dz))
    want_act, want_out = chain_bruteforce(tern.tolist(), gq, uq, dq, ds.astype(np.float64).tolist(),
                                          dz, fp16_nearest)
    assert act16.dtype == np.float16
    assert act16.astype(np.float64).tolist() == want_act.tolist()
    assert np.any(want_act != np.round(want_act))   # the rounding is visible in the sums
    assert np.allclose(out, want_out, rtol=1e-12, atol=1e-9)


def test_swiglu_mlp_bf16_chain_by_brute_force():
    """swiglu_mlp_bf16: activations and scales as bf16 bit patterns; the activation is
    rounded to bf16 (nearest even, by searching every bf16 value) before the down
    projection with zero points."""
    k, i, h, m = 128, 128, 16, 2
    tern = synthetic.below(96, m * k, 3).reshape(m, k).astype(np.float64) - 1.0
    a_bits = np.where(tern > 0, 0x3F80, np.where(tern < 0, 0xBF80, 0)).astype(np.uint16)
    gq, uq = synthetic.qweight_words(97, k, i), synthetic.qweight_words(98, k, i)
    dq = synthetic.qweight_words(99, i, h)
    ds = synthetic.scales_bf16(100, i // 128, h)
    dz = synthetic.zero_point_words(101, i // 128, h)
    ones = np.full((1, i), 0x3F80, np.uint16)
    act, out = ref.swiglu_mlp_bf16(a_bits, dict(qweight=gq, scales=ones),
                                   dict(qweight=uq, scales=ones),
                                   dict(qweight=dq, scales=ds, zeros=dz))
    ds_vals = [[struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in row] for row in ds]
    want_act, want_out = chain_bruteforce(tern.tolist(), gq, uq, dq, ds_vals, dz, bf16_nearest)
    assert np.asarray(act).tolist() == want_act.tolist()
    assert np.any(want_act != np.round(want_act))
    assert np.allclose(out, want_out, rtol=1e-12, atol=1e-9)


def test_routing_weights_scale_each_pair_row():
    """Row p is the dense product of its token row and expert times topk_weights[p]: the
    weights follow pair order, not CSR position or token; unit weights change nothing."""
    k, n, tokens, experts = 256, 32, 6, 3
    a = synthetic.activations(24, tokens, k)
    ex = [dict(qweight=synthetic.qweight_words(25 + e, k, n),
               scales=synthetic.scales(33 + e, 2, n)) for e in range(experts)]
    routes = np.array([[0, 2], [1, 0], [2, 1], [2, 0], [1, 2], [0, 1]])
    csr = ref.csr_from_token_routes(experts, tokens, 2, routes)
    assert list(csr["ex_pairs"]) != list(range(2 * tokens))  # CSR order differs from pairs
    w = np.array([0.5, 2.0, -1.25, 3.0, 0.0, 1.0, 0.75, -2.0, 1.5, 0.25, 4.0, -0.5],
                 dtype=np.float32)
    y = ref.grouped_w4a16_gemm(a, ex, csr, topk_weights=w)
    for p in range(2 * tokens):
        t, e = p // 2, int(routes.reshape(-1)[p])
        dense = ref.w4a16_gemm(a[t:t + 1], ex[e]["qweight"], ex[e]["scales"])
        assert y[p].tolist() == (float(w[p]) * dense[0]).tolist()
    ones = ref.grouped_w4a16_gemm(a, ex, csr, topk_weights=np.ones(2 * tokens, np.float32))
    assert ones.tolist() == ref.grouped_w4a16_gemm(a, ex, csr).tolist()
    r = synthetic.routing_weights(5, 100, 2)
    assert r.dtype == np.float32 and np.allclose(r.reshape(100, 2).sum(axis=1), 1.0, atol=1e-6)


# --------------------------------------------------------------------------- checker

def test_checker_element_allowance():
    r = np.ones((50, 50))
    r[0, 0] = 40.0           # rms 1.28: the bound is 3.6e-3; 2^-10 * 40 = 0.039
    c = r.copy()
    c[0, 0] += 0.03
    assert not ref.check(c, r)["ok"] and ref.check(c, r, rel_elem=2.0 ** -10)["ok"]
    c[0, 0] = 40.0 + 0.045   # beyond the allowance plus the bound
    assert not ref.check(c, r, rel_elem=2.0 ** -10)["ok"]


def test_checker_accepts_exact_and_rejects_large_error_and_nan():
    r = np.linspace(-3, 3, 64).reshape(8, 8)
    good = r.astype(np.float16)
    assert ref.check(good, r)["ok"]
    bad = good.copy()
    bad[3, 3] += np.float16(0.5)
    out = ref.check(bad, r)
    assert not out["ok"] and out["violations"] == 1
    nan = good.copy()
    nan[0, 0] = np.nan
    assert ref.check(nan, r)["nonfinite"] == 1 and not ref.check(nan, r)["ok"]


# --------------------------------------------------------------------------- layout

def test_layout_words_by_hand():
    """Rows 0..7 of column 0 carry codes 0..7: slots [0,4,1,5,2,6,3,7] give 0x75316420."""
    k, n = 128, 16
    codes = np.array([[kk % 16] * n for kk in range(k)], dtype=np.uint8)
    words = layout.repack_b_loops(codes)
    assert words[0] == 0x75316420          # lane 0, dword 0: rows 0..7
    assert words[1] == 0x75316420          # lane 0, dword 1: rows 32..39
    assert words[16 * 4] == 0xFDB9ECA8     # lane 16 (q = 1), dword 0: rows 8..15
    assert words[1 * 4] == 0x75316420      # lane 1 is column 1, rows 0..7


def test_layout_vectorized_matches_loops_and_round_trips():
    k, n = 256, 32
    qw = synthetic.qweight_words(40, k, n)
    codes = ref.unpack_qweight(qw)
    perm = synthetic.permutation(41, k)
    for p in (None, perm):
        loops = layout.repack_b_loops(codes, p)
        vec = layout.repack_b(qw, p)
        assert np.array_equal(loops, vec)
        assert vec.size * 8 == k * n   # same byte count as the plain format
        back = layout.unrepack_b(vec, k, n)
        assert np.array_equal(back, codes if p is None else codes[p])


def test_scale_and_zero_point_layouts():
    s = synthetic.scales(42, 2, 32)
    rs = layout.repack_scales(s)
    for nb in range(2):
        for g in range(2):
            for c in range(16):
                assert rs[(nb * 2 + g) * 16 + c] == s[g, 16 * nb + c]
    z = synthetic.zero_point_words(43, 2, 32)
    rz = layout.repack_zero_points(z)
    for nb in range(2):
        for g in range(2):
            for h in range(2):
                assert rz[(nb * 2 + g) * 2 + h] == z[g, 2 * nb + h]
