"""Pins for the oracle's layer arithmetic (CPU only).

Each check rests on something other than the oracle's own formula: exact
integer arithmetic, a brute-force sort, scipy's softmax, a dense all-experts
evaluation, hand-derived closed forms, and special cases that collapse to a
plain FFN or a dense softmax mixture.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import formats as fm, moe
from block_scaled_fp4_gemv_amd import synth as sy


def _bf16(a):
    return fm.to_bf16_rne(np.asarray(a, np.float64))


def test_router_logits_exact_on_integers():
    rng = np.random.default_rng(0)
    x = rng.integers(-8, 8, (5, 64))
    r = rng.integers(-8, 8, (7, 64))
    z = moe.router_logits(_bf16(x), r.astype(np.float32))
    assert np.array_equal(z, (x @ r.T).astype(np.float32))      # exact in int64
    assert z.dtype == np.float32


def test_softmax_against_scipy_and_invariants():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((9, 256)).astype(np.float32) * 3
    p = moe.softmax(z)
    assert np.allclose(p, scipy.special.softmax(z.astype(np.float64), axis=-1), rtol=1e-14, atol=0)
    assert np.all(np.abs(p.sum(-1) - 1) < 1e-15 * 256)
    assert np.allclose(moe.softmax(z.astype(np.float64) + 7.0), p, rtol=1e-12)


def test_topk_against_brute_force_sort():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((50, 40)).astype(np.float32)
    z[:, 5] = z[:, 9]            # ties: lower index must come first
    z[:, 30] = z[:, 2]
    z[0, :] = 0.0                # all equal
    z[1, 3] = -0.0
    for k in (1, 3, 8, 40):
        idx = moe.topk(z, k)
        for t in range(z.shape[0]):
            brute = sorted(range(z.shape[1]), key=lambda e: (-float(z[t, e]), e))[:k]
            assert idx[t].tolist() == brute


def test_ties_from_duplicated_router_rows():
    rng = np.random.default_rng(3)
    R = (rng.standard_normal((16, 64)) * 0.05).astype(np.float32)
    R[11] = R[4]                 # experts 4 and 11 always tie
    R[4] += 1.0                  # and win
    R[11] += 1.0
    x = _bf16(rng.standard_normal((6, 64)) + 1.0)
    idx, w, z = moe.route(x, R, 3)
    assert np.all(z[:, 4] == z[:, 11])
    assert np.all(np.where(idx == 4)[1] < np.where(idx == 11)[1])
    assert np.all(w[:, 0] == w[np.arange(6), np.where(idx == 11)[1]])


def test_route_weights_are_probabilities():
    rng = np.random.default_rng(4)
    R = (rng.standard_normal((32, 128)) * 0.05).astype(np.float32)
    x = _bf16(rng.standard_normal((4, 128)))
    idx, w, z = moe.route(x, R, 4)
    p = scipy.special.softmax(z.astype(np.float64), axis=-1)
    assert np.allclose(w, np.take_along_axis(p, idx.astype(np.int64), -1), rtol=1e-7)
    assert np.all(np.diff(w, axis=-1) <= 0)
    _, wr, _ = moe.route(x, R, 4, renorm=True)
    assert np.allclose(wr.sum(-1), 1.0, atol=1e-6)


def test_silu_closed_forms():
    assert moe.silu(np.array([0.0]))[0] == 0.0
    assert moe.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, abs=1e-16)
    assert moe.silu(np.array([-1.0]))[0] == pytest.approx(-0.2689414213699951, abs=1e-16)
    assert moe.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert moe.silu(np.array([-800.0]))[0] == 0.0


def _mx_onehot_expert(H, F, g_pos, g_code, u_pos, u_code, d_map, d_code):
    """MXFP4 expert with all scales 1.0 and a single nonzero code per row."""
    def mat(N, K, pos_of_row, code):
        codes = np.zeros((N, K), np.uint8)
        for n in range(N):
            p = pos_of_row(n)
            if p is not None:
                codes[n, p] = code
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        return packed, np.full((N, K // 32), 127, np.uint8)
    cg, sg = mat(F, H, g_pos, g_code)
    cu, su = mat(F, H, u_pos, u_code)
    cd, sd = mat(H, F, d_map, d_code)
    return dict(codes_g=cg, scales_g=sg, codes_u=cu, scales_u=su, codes_d=cd, scales_d=sd)


def test_worked_layer_closed_form():
    """Hand-derived: H=64, F=32, E=2, k=1.

    G[f, 2f] = 1, U[f, 2f+1] = 2, D[n, n//2] = 1 (expert 0); x[2f] = 1, x[2f+1] = 0.5.
    g_f = 1, u_f = 1, h_f = bf16(silu(1)) = 0.73046875 (187/256), y[n] = h[n//2].
    Router rows are zero -> logits tie at 0 -> expert 0 wins, p = 0.5.
    out[n] = bf16(0.5 * 0.73046875) = 0.365234375.
    Expert 1 = expert 0 with D[n, n//2] = -1 (never selected).
    """
    H, F = 64, 32
    e0 = _mx_onehot_expert(H, F, lambda f: 2 * f, 0x2, lambda f: 2 * f + 1, 0x4, lambda n: n // 2, 0x2)
    e1 = _mx_onehot_expert(H, F, lambda f: 2 * f, 0x2, lambda f: 2 * f + 1, 0x4, lambda n: n // 2, 0xA)
    x = np.zeros((1, H)); x[0, 0::2] = 1.0; x[0, 1::2] = 0.5
    res = moe.moe_layer(fm.MXFP4, _bf16(x), np.zeros((2, H), np.float32), [e0, e1], k=1, return_h=True)
    assert res["idx"].tolist() == [[0]]
    assert res["w"][0, 0] == np.float32(0.5)
    assert np.all(res["h"][(0, 0)] == 0.73046875)
    assert np.all(res["y"][0, 0] == 0.73046875)
    assert np.all(fm.bf16_to_f64(res["out"]) == 0.365234375)


def test_transposed_down_is_detected():
    """D maps h[f] to output n = 2f only: a transposed or mis-indexed D fails."""
    H, F = 64, 32
    e = _mx_onehot_expert(H, F, lambda f: f, 0x2, lambda f: f, 0x2,
                          lambda n: n // 2 if n % 2 == 0 else None, 0x2)
    x = np.zeros((1, H)); x[0, :F] = np.arange(F) / 8.0
    res = moe.moe_layer(fm.MXFP4, _bf16(x), np.zeros((1, H), np.float32), [e], k=1)
    xv = np.arange(F) / 8.0
    h = fm.bf16_round_f64(xv * xv / (1 + np.exp(-xv)))
    exp = np.zeros(H); exp[0::2] = h
    assert np.array_equal(res["y"][0, 0], exp)


def _random_layer(fmt, H, E, F, T, seed=0):
    b = sy.experts(fmt, seed, 99, 0, 0, E, H, F, 0.02)
    R = sy.router(seed, 99, 0, E, H)
    x = sy.token_rows(seed, 99, T, H)
    return sy.ExpertList(b), R, x


@pytest.mark.parametrize("fmt", [fm.NVFP4, fm.MXFP4, fm.FP8])
def test_sparse_equals_dense_masked(fmt):
    experts, R, x = _random_layer(fmt, 256, 8, 512, 16)
    for renorm in (False, True):
        res = moe.moe_layer(fmt, x, R, experts, k=2, renorm=renorm)
        dense = moe.dense_masked_layer(fmt, x, R, experts, 8, 2, renorm=renorm)
        sparse = moe.combine_f64(res["y"], res["w"])
        assert np.max(np.abs(dense - sparse)) <= 1e-12 * max(1.0, np.abs(dense).max())
        assert np.array_equal(res["out"], fm.to_bf16_rne(sparse))


def test_single_expert_reduces_to_ffn():
    """E=1, k=1: w = 1 and out = bf16(D bf16(silu(Gx) * Ux)) with scipy's expit."""
    experts, R, x = _random_layer(fm.MXFP4, 256, 1, 512, 4)
    res = moe.moe_layer(fm.MXFP4, x, R, experts, k=1)
    assert np.all(res["w"] == 1.0)
    G, U, D = moe.dequant_expert(fm.MXFP4, experts[0])
    xf = fm.bf16_to_f64(x)
    g = xf @ G.T
    h = fm.bf16_round_f64(g * scipy.special.expit(g) * (xf @ U.T))
    assert np.allclose(fm.bf16_to_f64(res["out"]), fm.bf16_round_f64(h @ D.T), rtol=0, atol=0)


def test_k_equals_E_with_renorm_is_dense_softmax_mixture():
    experts, R, x = _random_layer(fm.NVFP4, 256, 4, 512, 3)
    res = moe.moe_layer(fm.NVFP4, x, R, experts, k=4, renorm=True)
    p = scipy.special.softmax(moe.router_logits(x, R).astype(np.float64), axis=-1)
    xf = fm.bf16_to_f64(x)
    acc = np.zeros_like(xf)
    for e in range(4):
        G, U, D = moe.dequant_expert(fm.NVFP4, experts[e])
        g = xf @ G.T
        acc += p[:, e:e + 1] * (fm.bf16_round_f64(g * scipy.special.expit(g) * (xf @ U.T)) @ D.T)
    got = moe.combine_f64(res["y"], res["w"])
    assert np.allclose(got, acc, rtol=1e-6, atol=1e-9)    # w is fp32-rounded p


def test_combine_order_and_rounding():
    y = np.zeros((1, 3, 2)); y[0, :, 0] = [1.0, 2.0, 4.0]; y[0, :, 1] = [1.0, -1.0, 2.0 ** -9]
    w = np.array([[0.5, 0.25, 0.125]], np.float32)
    out = fm.bf16_to_f64(moe.combine(y, w))
    assert out.tolist() == [[1.5, 0.25]]   # 0.5 - 0.25 + 2^-12 rounds to 0.25 in bf16


def test_top_margins():
    z = np.array([[3.0, 1.0, 2.0, 2.0005]], np.float32)
    assert moe.top_margins(z, 2)[0] == pytest.approx(0.0005, abs=1e-6)
