"""Pins for the oracle's format decoders and bf16 rounding (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as fm

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "format_values.json")))


def _same(a, b):
    return (a == b and np.signbit(a) == np.signbit(b)) or (np.isnan(a) and np.isnan(b))


def test_e2m1_worked_values():
    for code, v in GOLDEN["e2m1"].items():
        assert _same(fm.E2M1_TABLE[int(code, 16)], v), code


def test_e2m1_value_set():
    mags = sorted(set(abs(v) for v in fm.E2M1_TABLE))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):  # sign bit mirrors
        assert fm.E2M1_TABLE[c | 8] == -fm.E2M1_TABLE[c]


def test_e4m3_worked_values():
    for code, v in GOLDEN["e4m3"].items():
        assert _same(fm.E4M3_TABLE[int(code, 16)], v), code
    for code in GOLDEN["e4m3_nan"]:
        assert np.isnan(fm.E4M3_TABLE[int(code, 16)])


def test_e4m3_matches_torch_all_codes():
    # independent implementation: torch's float8_e4m3fn
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(t), np.isnan(fm.E4M3_TABLE))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], fm.E4M3_TABLE[ok])


def test_e4m3_structure():
    pos = fm.E4M3_TABLE[:0x7F]
    assert len(pos) == 127 and np.all(np.diff(pos) > 0)
    assert pos[1] == 2.0 ** -9 and pos[-1] == 448.0


def test_e8m0_worked_values_and_torch():
    for code, v in GOLDEN["e8m0"].items():
        assert fm.E8M0_TABLE[int(code, 16)] == v, code
    assert np.isnan(fm.E8M0_TABLE[255])
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(t[:255], fm.E8M0_TABLE[:255])


def test_fp4_nibble_order():
    # low nibble = even element
    codes = np.array([[0x21, 0x7F]], dtype=np.uint8)
    assert fm.unpack_fp4(codes).tolist() == [[1, 2, 15, 7]]


def test_dequant_nvfp4_worked():
    # 16 elements: byte 0x21 -> [0.5, 1.0], rest zero; scale code 0x38 (1.0) * tau 2
    codes = np.zeros((1, 8), np.uint8); codes[0, 0] = 0x21; codes[0, 7] = 0xF0
    scales = np.array([[0x38]], np.uint8)
    w = fm.dequant_nvfp4(codes, scales, np.float32(2.0))
    exp = np.zeros(16); exp[0], exp[1], exp[15] = 1.0, 2.0, -12.0
    assert np.array_equal(w[0], exp)
    # second block uses its own scale
    codes2 = np.full((1, 16), 0x22, np.uint8)
    scales2 = np.array([[0x38, 0x40]], np.uint8)   # 1.0 and 2.0
    w2 = fm.dequant_nvfp4(codes2, scales2, np.float32(1.0))
    assert np.all(w2[0, :16] == 1.0) and np.all(w2[0, 16:] == 2.0)


def test_dequant_mxfp4_worked():
    codes = np.full((2, 32), 0x77, np.uint8)     # all 6.0
    scales = np.array([[127, 125], [130, 0]], np.uint8)
    w = fm.dequant_mxfp4(codes, scales)
    assert np.all(w[0, :32] == 6.0) and np.all(w[0, 32:] == 1.5)
    assert np.all(w[1, :32] == 48.0) and np.all(w[1, 32:] == 6.0 * 2.0 ** -127)


def test_dequant_fp8_worked():
    codes = np.zeros((1, 256), np.uint8); codes[0, 0] = 0x38; codes[0, 128] = 0xB8; codes[0, 255] = 0x7E
    scales = np.array([[0.5, 3.0]], np.float32)
    w = fm.dequant_fp8(codes, scales)
    assert w[0, 0] == 0.5 and w[0, 128] == -3.0 and w[0, 255] == 1344.0
    assert np.count_nonzero(w) == 3


def test_bf16_rne_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    ours = fm.to_bf16_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_single_rounding_from_f64():
    # 1 + 2^-8 + 2^-40 is above the bf16 midpoint: rounds up to 1 + 2^-7.
    # (Rounding through fp32 first would land exactly on the midpoint and go to 1.0.)
    v = fm.bf16_round_f64(np.array([1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8, 1 + 3 * 2 ** -8]))
    assert v.tolist() == [1 + 2 ** -7, 1.0, 1 + 2 ** -6]
    # subnormals: quantum 2^-133, ties to even
    s = fm.to_bf16_rne(np.array([2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, -2.0 ** -133]))
    assert s.tolist() == [0x0001, 0x0000, 0x0002, 0x8001]
    # overflow: bf16 max = (2 - 2^-7) * 2^127; max + half ulp rounds to inf
    mx = (2 - 2 ** -7) * 2.0 ** 127
    o = fm.to_bf16_rne(np.array([mx, mx + 2.0 ** 119, np.inf, np.nan]))
    assert o.tolist() == [0x7F7F, 0x7F80, 0x7F80, 0x7FC0]


def test_bf16_decode():
    assert fm.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0001], np.uint16)).tolist() == [1.0, -2.0, 2.0 ** -133]


def test_f32_rne_ties_to_even_and_specials():
    """to_f32_rne (the oracle's fp32 rounding of logits and routing weights)
    against IEEE binary32 round-to-nearest-even, worked by hand: halfway cases
    go to the even significand, just above halfway rounds up, and overflow,
    signed zeros and subnormals follow IEEE."""
    one = 1.0
    ulp = 2.0 ** -23
    cases = {
        one + ulp / 2: one,                        # tie, 1.0 has an even significand
        one + 3 * ulp / 2: one + 2 * ulp,          # tie, rounds up to the even one
        one + ulp / 2 + 2.0 ** -50: one + ulp,     # just above the tie
        -(one + ulp / 2): -one,
        2.0 ** 128: np.inf,                        # beyond the largest finite value
        (2.0 - 2.0 ** -24) * 2.0 ** 127: np.inf,   # tie at the top rounds to even = overflow
        2.0 ** -149: 2.0 ** -149,                  # smallest subnormal
        2.0 ** -150: 0.0,                          # tie between 0 and the smallest subnormal
        3 * 2.0 ** -151: 2.0 ** -149,              # above that tie
        -0.0: -0.0,
    }
    with np.errstate(over="ignore"):  # the two overflow cases
        got = fm.to_f32_rne(np.array(list(cases), dtype=np.float64))
    assert got.dtype == np.float32
    for (x, want), g in zip(cases.items(), got):
        assert g == np.float32(want), (x, g, want)
        assert np.signbit(g) == np.signbit(want), x
    # agrees with torch's float64 -> float32 cast on random values of every magnitude
    rng = np.random.default_rng(0)
    x = rng.normal(size=4096) * 10.0 ** rng.integers(-40, 39, size=4096)
    t = torch.from_numpy(x).to(torch.float32).numpy()
    assert np.array_equal(fm.to_f32_rne(x), t)
