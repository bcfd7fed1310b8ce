"""Pins of the oracle's per-slot parts (forward_detail, forward_fp8_detail),
which the GPU parity checks use to tell a rounding-boundary flip from an
error: the parts recombine into the layer the oracle's forward functions
give, and on one-hot expert weights they equal the closed form written with
scipy's sigmoid and torch's e4m3 cast."""

import numpy as np
from scipy.special import expit

import oracle
from oracle import codecs
from test_oracle_fp8 import SCALE, _bf16_nearest, _one_hot_fp8_layer, _torch_e4m3


def _bf16_layer(seed, T=40, d=128, E=10, F=32):
    rng = np.random.default_rng(seed)
    x = codecs.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    gu = codecs.f32_to_bf16_bits((rng.standard_normal((E, 2 * F, d)) * 0.1).astype(np.float32))
    dn = codecs.f32_to_bf16_bits((rng.standard_normal((E, d, F)) * 0.1).astype(np.float32))
    sgu = codecs.f32_to_bf16_bits((rng.standard_normal((2 * F, d)) * 0.1).astype(np.float32))
    sdn = codecs.f32_to_bf16_bits((rng.standard_normal((d, F)) * 0.1).astype(np.float32))
    return x, Wg, gu, dn, sgu, sdn


def _recombine(det):
    return np.einsum("ts,tsc->tc", det.w, codecs.round_to_bf16(det.y))


def test_detail_recombines_into_forward_and_block():
    x, Wg, gu, dn, sgu, sdn = _bf16_layer(95)
    k = 4
    out, r = oracle.forward(x, Wg, gu, dn, k, SCALE)
    toks = np.array([0, 3, 17, 39])
    det = oracle.forward_detail(toks, x, r, gu, dn)
    assert det.y.shape == (4, k, 128) and det.h.shape == (4, k, 32)
    assert np.array_equal(det.expert, r.idx[toks])
    np.testing.assert_allclose(_recombine(det), out[toks], rtol=0, atol=1e-13 * np.abs(out).max())
    blk, rb = oracle.forward_block(x, Wg, gu, dn, sgu, sdn, k, SCALE)
    detb = oracle.forward_detail(toks, x, rb, gu, dn, sgu, sdn)
    assert np.all(detb.expert[:, k] == -1) and np.all(detb.w[:, k] == 1.0)
    np.testing.assert_allclose(_recombine(detb), blk[toks], rtol=0, atol=1e-13 * np.abs(blk).max())


def test_detail_parts_closed_form_one_hot():
    """One-hot bf16 weights: gate/up row f picks x column ig/iu with weight
    wg/wu, down row c picks activation fd[c] with weight wd[c]; then
    h = g * sigmoid(g) * u and y[c] = bf16(h)[fd[c]] * wd[c], exactly."""
    rng = np.random.default_rng(96)
    T, d, E, F, k = 9, 64, 3, 16, 3
    x = codecs.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wg = (rng.standard_normal((E, d)) / 8).astype(np.float32)
    ig, iu, fd = rng.integers(0, d, (E, F)), rng.integers(0, d, (E, F)), rng.integers(0, F, (E, d))
    wv = lambda s: codecs.bf16_bits_to_f64(codecs.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32)))
    wg, wu, wd = wv((E, F)), wv((E, F)), wv((E, d))
    gu = np.zeros((E, 2 * F, d))
    dn = np.zeros((E, d, F))
    for e in range(E):
        gu[e, np.arange(F), ig[e]] = wg[e]
        gu[e, F + np.arange(F), iu[e]] = wu[e]
        dn[e, np.arange(d), fd[e]] = wd[e]
    gu_bits = codecs.f32_to_bf16_bits(gu.astype(np.float32))
    dn_bits = codecs.f32_to_bf16_bits(dn.astype(np.float32))
    _, r = oracle.forward(x, Wg, gu_bits, dn_bits, k, SCALE)
    det = oracle.forward_detail(np.arange(T), x, r, gu_bits, dn_bits)
    x64 = codecs.bf16_bits_to_f64(x)
    for t in range(T):
        for j in range(k):
            e = det.expert[t, j]
            g, u = x64[t, ig[e]] * wg[e], x64[t, iu[e]] * wu[e]
            h = g * expit(g) * u
            np.testing.assert_allclose(det.h[t, j], h, rtol=1e-15, atol=0)
            assert np.array_equal(det.y[t, j], _bf16_nearest(det.h[t, j])[fd[e]] * wd[e])


def test_fp8_detail_recombines_and_matches_the_closed_form():
    for x_exact in (True, False):
        L, expect = _one_hot_fp8_layer(97, x_exact)
        out, r = oracle.forward_fp8(L["x"], L["Wg"], L["Wq_gu"], L["s_gu"], L["Wq_dn"], L["s_dn"], L["k"], SCALE)
        T = L["x"].shape[0]
        det = oracle.forward_fp8_detail(np.arange(T), L["x"], r, L["Wq_gu"], L["s_gu"], L["Wq_dn"], L["s_dn"])
        np.testing.assert_allclose(_recombine(det), out, rtol=0, atol=1e-13 * np.abs(out).max())
        assert np.max(np.abs(_recombine(det) - expect)) <= 1e-12 * np.abs(expect).max()
        # h is the activation before its bf16 rounding: the closed form's, slot j being expert r.idx[t, j]
        a = L["a"][np.arange(T)[:, None], r.idx]
        np.testing.assert_allclose(det.h, a, rtol=1e-12, atol=0)
        # the dequantised activations are torch's e4m3 cast of the scaled values times the row scale
        _, vals = _torch_e4m3(det.scaled)
        assert np.array_equal(det.a_deq, vals * det.s_a.astype(np.float64)[..., None])
        # each row's largest scaled magnitude is 448 (to float32 rounding of amax * r)
        peak = np.max(np.abs(det.scaled.astype(np.float64)), axis=2)
        assert np.all(np.abs(peak - 448.0) <= 448.0 * 2.0 ** -22)


def test_detail_of_no_tokens():
    x, Wg, gu, dn, _, _ = _bf16_layer(98, T=8)
    _, r = oracle.forward(x, Wg, gu, dn, 2, SCALE)
    det = oracle.forward_detail(np.zeros(0, np.int64), x, r, gu, dn)
    assert det.y.shape[0] == 0 and det.w.shape == (0, 2)


def test_predecoded_float64_weights_give_the_same_layer():
    """The oracle takes expert weights as bf16 bit patterns or already decoded
    to float64 (the CPU baseline decodes them outside its timed region): the
    outputs are identical."""
    x, Wg, gu, dn, sgu, sdn = _bf16_layer(99)
    a, ra = oracle.forward(x, Wg, gu, dn, 3, SCALE)
    b, rb = oracle.forward(x, Wg, codecs.bf16_bits_to_f64(gu), codecs.bf16_bits_to_f64(dn), 3, SCALE)
    assert np.array_equal(a, b) and np.array_equal(ra.idx, rb.idx)
    c, _ = oracle.forward_block(x, Wg, gu, dn, sgu, sdn, 3, SCALE)
    d_, _ = oracle.forward_block(x, Wg, codecs.bf16_bits_to_f64(gu), codecs.bf16_bits_to_f64(dn),
                                 codecs.bf16_bits_to_f64(sgu), codecs.bf16_bits_to_f64(sdn), 3, SCALE)
    assert np.array_equal(c, d_)
