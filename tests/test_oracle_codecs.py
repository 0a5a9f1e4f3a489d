"""Pins for the oracle's number formats: bf16/fp32 storage rounding, E4M3FN,
E8M0 and the MXFP8 block quantiser, plus facts the pages state
(tests/golden/page_facts.json).
"""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _fp32_specials():
    bits = np.array([0x00000001, 0x007FFFFF, 0x00800000, 0x00808000, 0x00818000, 0x3F808000,
                     0x3F818000, 0x3F80FFFF, 0x3F817FFF, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF,
                     0x80000001, 0xBF808000, 0xFF7FFFFF, 0x00000000, 0x80000000,
                     0x00018000, 0x00008000], np.uint32)
    return bits.view(np.float32)


def test_bf16_rounding_matches_torch(oracle_lib):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    v = np.concatenate([v, _fp32_specials(), rng.standard_normal(10000).astype(np.float32)])
    ours = oracle_lib.round_(v.astype(np.float64), oracle_lib.BF16)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_fp32_rounding_matches_numpy(oracle_lib):
    v = np.random.default_rng(1).standard_normal(10000) * 1e3
    np.testing.assert_array_equal(oracle_lib.round_(v, oracle_lib.FP32),
                                  v.astype(np.float32).astype(np.float64))


def test_e4m3_decode_all_codes_match_torch(oracle_lib):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle_lib.e4m3_decode(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == GOLDEN["e4m3_max"]["value"]
    assert oracle_lib.e4m3_decode(0x7E) == 448.0


def test_e4m3_encode_rne_matches_torch(oracle_lib):
    finite = np.array([oracle_lib.e4m3_decode(c) for c in range(256)])
    finite = np.unique(finite[~np.isnan(finite)])
    mids = (finite[:-1] + finite[1:]) / 2                      # exact ties
    rng = np.random.default_rng(2)
    rand = rng.uniform(-448, 448, 20000)
    small = rng.uniform(-0.02, 0.02, 20000)                    # subnormal range
    v = np.concatenate([finite, mids, rand, small]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle_lib.e4m3_encode(float(a)) for a in v], np.uint8)
    # torch keeps the sign of zero; so do we
    np.testing.assert_array_equal(ours, ref)


def test_e8m0_decode_matches_torch(oracle_lib):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = np.array([oracle_lib.e8m0_decode(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert GOLDEN["e8m0_is_power_of_two"]["value"]
    assert all(np.log2(ours[ok]) == np.round(np.log2(ours[ok])))


@pytest.mark.parametrize("e", [-20, -8, -1, 0, 3, 10])
def test_scale_rule_at_and_above_boundary(oracle_lib, e):
    amax = 448.0 * 2.0 ** e
    assert oracle_lib.mx_scale_exp(amax) == e
    assert oracle_lib.mx_scale_exp(np.nextafter(amax, np.inf)) == e + 1
    assert oracle_lib.mx_scale_exp(np.nextafter(amax, 0)) == e
    assert oracle_lib.mx_scale_exp(amax / 2 * 1.0000001) == e
    # a block whose maximum is exactly 448 * 2^e encodes its max as 0x7E
    v = np.zeros((1, 32))
    v[0, 5] = -amax
    v[0, 9] = amax / 3
    codes, scales = oracle_lib.mx_quantize_rows(v)
    assert scales[0, 0] == e + 127
    assert codes[0, 5] == 0xFE and codes[0, 0] == 0


def test_zero_block_scale(oracle_lib):
    codes, scales = oracle_lib.mx_quantize_rows(np.zeros((2, 64)))
    assert np.all(scales == 0) and np.all(codes == 0)


def test_block_max_never_overflows_and_scale_is_smallest(oracle_lib):
    """The tutorial's MXFP8 scale rule: divide the block max by 448 and take a
    power of two so the block max just does not overflow."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    codes, scales = oracle_lib.mx_quantize_rows(v)
    B = GOLDEN["mx_block_elems"]["value"]
    for r in range(64):
        for b in range(96 // B):
            blk = v[r, b * B:(b + 1) * B]
            s = 2.0 ** (int(scales[r, b]) - 127)
            amax = np.abs(blk).max()
            assert amax / s <= 448.0
            assert amax / (s / 2) > 448.0                   # the next smaller power overflows


def test_mx_roundtrip_error_bound_and_idempotence(oracle_lib):
    rng = np.random.default_rng(4)
    v = rng.standard_normal((32, 128)) * 0.02
    codes, scales = oracle_lib.mx_quantize_rows(v)
    dq = oracle_lib.mx_dequant_rows(codes, scales)
    # 3 mantissa bits: relative error at most 2^-4 for values on the normal grid
    s = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    normal = np.abs(v) / s >= 2.0 ** -6
    assert np.all(np.abs(dq - v)[normal] <= 2 ** -4 * np.abs(v)[normal])
    assert np.all(np.abs(dq - v)[~normal] <= 2 ** -10 * s[~normal])
    np.testing.assert_array_equal(oracle_lib.mx_qdq_rows(v), dq)
    # quantise-dequantise is idempotent on values.  (Codes are not always
    # reproduced: a block max that rounds down to exactly 224 * 2^e is
    # re-quantised with the next smaller scale, representing the same values.)
    np.testing.assert_array_equal(oracle_lib.mx_qdq_rows(dq), dq)
    c2, s2 = oracle_lib.mx_quantize_rows(dq)
    blk_max = np.abs(dq).reshape(32, 4, 32).max(-1)
    same = blk_max != 224.0 * 2.0 ** (scales.astype(np.float64) - 127)
    np.testing.assert_array_equal(s2[same], scales[same])
    np.testing.assert_array_equal(s2[~same], scales[~same] - 1)
    np.testing.assert_array_equal(np.repeat(same, 32, axis=1) * c2,
                                  np.repeat(same, 32, axis=1) * codes)


def test_mx_storage_bits_per_element(oracle_lib):
    v = np.random.default_rng(5).standard_normal((8, 4096))
    codes, scales = oracle_lib.mx_quantize_rows(v)
    bits = 8.0 * (codes.nbytes + scales.nbytes) / v.size
    assert bits == GOLDEN["mx_bits_per_elem"]["value"]


def test_colwise_quantisation_is_rowwise_of_each_group_transposed(oracle_lib):
    rng = np.random.default_rng(6)
    v = rng.standard_normal((100, 40))
    go = np.array([0, 33, 33, 70, 100])
    codes, scales = oracle_lib.mx_quantize_cols(v, go)
    sb = 0
    for e in range(4):
        g0, g1 = go[e], go[e + 1]
        nb = (g1 - g0 + 31) // 32
        if g1 > g0:
            c_ref, s_ref = oracle_lib.mx_quantize_rows(v[g0:g1].T)
            np.testing.assert_array_equal(codes[g0:g1].T, c_ref)
            np.testing.assert_array_equal(scales[:, sb:sb + nb], s_ref)
        sb += nb
    dq = oracle_lib.mx_qdq_cols(v, go)
    for e in range(4):
        g0, g1 = go[e], go[e + 1]
        if g1 > g0:
            np.testing.assert_array_equal(dq[g0:g1], oracle_lib.mx_qdq_rows(v[g0:g1].T).T)
