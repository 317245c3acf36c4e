"""The seeded input generator and the test-data quantizers (CPU only).

The encoders are pinned against the format definitions: the round-to-nearest-
even midpoint list, saturation, decode(encode(v)) == v for every representable
value, and an independent encoder (torch's float8_e4m3fn cast) in range.
"""
import json
import os

import numpy as np
import torch

from oracle import formats as fm

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "format_values.json")))


def test_philox_known_answers(synth):
    # Known-answer vectors published with Random123 for philox4x32-10.
    assert synth.philox4x32_10([0, 0, 0, 0], [0, 0]).tolist() == \
        [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]
    assert synth.philox4x32_10([0xffffffff] * 4, [0xffffffff] * 2).tolist() == \
        [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]
    assert synth.philox4x32_10([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344],
                               [0xa4093822, 0x299f31d0]).tolist() == \
        [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]


def test_normal_moments_and_determinism(synth):
    st = synth.stream(0, 7, 1)
    x = synth.normal(st, 400000, 0.0, 2.0)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 2.0) < 0.02
    assert np.array_equal(x, synth.normal(st, 400000, 0.0, 2.0))
    # element i is addressable on its own (counter-based)
    assert np.array_equal(x[1001:1010], synth.normal(st, 9, 0.0, 2.0, first=1001))
    assert not np.array_equal(x[:100], synth.normal(synth.stream(0, 7, 1, attempt=1), 100, 0.0, 2.0))


def test_e2m1_encoder_ties_and_saturation(synth):
    for v, exp in GOLDEN["e2m1_rne_ties"].items():
        if v.startswith("_"):
            continue
        assert fm.E2M1_TABLE[synth.e2m1_encode(float(v))] == exp, v


def test_e2m1_encoder_round_trip(synth):
    for c in range(16):
        v = fm.E2M1_TABLE[c]
        assert fm.E2M1_TABLE[synth.e2m1_encode(v)] == v


def test_e4m3_encoder_round_trip_and_torch(synth):
    for c in range(256):
        v = fm.E4M3_TABLE[c]
        if np.isnan(v):
            continue
        assert fm.E4M3_TABLE[synth.e4m3_encode(v)] == v, hex(c)
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.uniform(-460, 460, 5000), rng.uniform(-0.02, 0.02, 5000)]).astype(np.float32)
    ours = np.array([synth.e4m3_encode(float(v)) for v in vals], np.uint8)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fm.E4M3_TABLE[ours], fm.E4M3_TABLE[ref])
    assert synth.e4m3_encode(1e6) == 0x7E and synth.e4m3_encode(-1e6) == 0xFE


def test_quantize_block_invariants(synth):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    w[3, 32:64] = 0.0                               # a zero MX block
    # NVFP4: block amax maps near 6 * s * tau, error bounded by half a step
    q = synth.quantize(fm.NVFP4, w)
    d = fm.dequant_nvfp4(q["codes"], q["scales"], q["tau"])
    assert q["tau"] == np.float32(np.abs(w).max() / (6 * 448))
    blk = np.abs(w).reshape(8, 16, 16).max(-1)
    s = fm.E4M3_TABLE[q["scales"]] * float(q["tau"])
    assert np.all(np.abs(d - w).reshape(8, 16, 16).max(-1) <= s * 1.0 + 1e-12)
    nzb = blk > 0
    assert np.all(s[~nzb] == 0) and np.all(fm.unpack_fp4(q["codes"])[3, 32:64] == 0)
    assert np.all(np.abs(blk[nzb] / s[nzb] - 6) <= 6 * 2 ** -3 + 1e-9)   # 3 mantissa bits
    # MXFP4: scale = 2^(floor(log2 amax) - 2), element magnitudes <= 6
    q = synth.quantize(fm.MXFP4, w)
    amax = np.abs(w).reshape(8, 8, 32).max(-1)
    nz = amax > 0
    exp_code = np.floor(np.log2(amax[nz])) - 2 + 127
    assert np.array_equal(q["scales"][nz].astype(np.float64), exp_code)
    assert q["scales"][3, 1] == 127 and np.all(fm.unpack_fp4(q["codes"])[3, 32:64] == 0)
    # FP8: sigma = amax/448 so the block max encodes to 448 exactly
    q = synth.quantize(fm.FP8, w)
    d = fm.dequant_fp8(q["codes"], q["scales"])
    sig = np.abs(w).reshape(8, 2, 128).max(-1) / 448.0
    assert np.allclose(q["scales"], sig.astype(np.float32), rtol=0, atol=0)
    assert np.all(np.abs(d - w) <= np.repeat(q["scales"].astype(np.float64), 128, 1) * 16 + 1e-12)


def test_experts_batch_matches_single_quantize(synth):
    b = synth.experts(fm.NVFP4, 0, 0, 0, 3, 2, 256, 512, 0.02)
    # re-derive expert 4's gate from its stream and the single-matrix quantizer
    st = synth.stream(0, 0, synth.KIND_W, 0, 4, 0, 0)
    w = synth.normal(st, 512 * 256, 0.0, 0.02).reshape(512, 256)
    q = synth.quantize(fm.NVFP4, w)
    assert np.array_equal(b["codes_g"][1], q["codes"]) and np.array_equal(b["scales_g"][1], q["scales"])
    assert b["tau"][1, 0] == q["tau"]


def test_ar1_recipe(synth):
    seq = synth.ar1_sequence(0, 1, 4, 2048)
    h0 = fm.bf16_to_f64(seq[0])
    assert abs(h0.std() - 1.0) < 0.05
    eps = synth.normal(synth.stream(0, 1, synth.KIND_EPS, 0, 1, 0, 0), 2048).astype(np.float64)
    exp = fm.to_bf16_rne(np.float32(0.9 * h0 + 0.44 * eps).astype(np.float64))
    assert np.array_equal(seq[1], exp)
