"""Pins of the oracle's FP8 path: the row quantiser against torch's e4m3 cast
and the format's error bound, exact cases, and the FP8 layer against the bf16
layer on the same (e4m3-representable) weights within the quantisation bound."""

import numpy as np
import torch

import oracle
from oracle import codecs

SCALE = float(np.float32(2.826))


def test_row_quantiser_matches_torch_cast_and_bound():
    rng = np.random.default_rng(20)
    for scale in (1.0, 1e-3, 37.0, 1e-6):
        v = (rng.standard_normal(4096) * scale).astype(np.float32)
        q, s = oracle.quant_row_e4m3(v)
        amax = np.max(np.abs(v))
        assert s == np.float32(amax) / np.float32(448)
        r = np.float32(448) / np.float32(amax)
        ref = torch.from_numpy((v * r).clip(-448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q, ref)
        # the largest magnitude maps onto the largest code
        assert codecs.e4m3_bits_to_f64(q[np.argmax(np.abs(v))]) in (448.0, -448.0)
        # error bound: half an e4m3 step (relative 2^-4 for normals, 2^-10 * s absolute
        # for subnormals), plus float32 rounding of the scale and of v * r
        deq = codecs.e4m3_bits_to_f64(q) * np.float64(s)
        bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * np.float64(s)) * (1 + 1e-6)
        assert np.all(np.abs(deq - v) <= bound)


def test_row_quantiser_zero_and_exact_rows():
    q, s = oracle.quant_row_e4m3(np.zeros(64, np.float32))
    assert s == 1.0 and not q.any()
    # a row of e4m3 values times a power of two whose magnitude peaks at 448 * 2^m
    # quantises exactly
    codes = np.random.default_rng(21).integers(0, 0x7E, 256).astype(np.uint8)
    codes[7] = 0x7E
    v = (codecs.e4m3_bits_to_f64(codes) * 2.0 ** -5).astype(np.float32)
    q, s = oracle.quant_row_e4m3(v)
    assert s == np.float32(2.0 ** -5)
    assert np.array_equal(q, codes)


def test_fp8_layer_close_to_bf16_layer_on_same_weights():
    """Per-row weight scales of 1 and e4m3 weight codes: the dequantised weights
    are exactly bf16-representable, so the bf16 layer on them differs from the
    FP8 layer only by the two activation quantisations."""
    rng = np.random.default_rng(22)
    T, d, E, F, k = 24, 128, 12, 32, 4
    x = codecs.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    qgu = codecs.f32_to_e4m3_bits((rng.standard_normal((E, 2 * F, d)) * 0.1).astype(np.float32))
    qdn = codecs.f32_to_e4m3_bits((rng.standard_normal((E, d, F)) * 0.1).astype(np.float32))
    sgu = np.ones((E, 2 * F), np.float32)
    sdn = np.ones((E, d), np.float32)
    out8, r8 = oracle.forward_fp8(x, Wg, qgu, sgu, qdn, sdn, k, SCALE)
    Wgu = codecs.f32_to_bf16_bits(codecs.e4m3_bits_to_f64(qgu).astype(np.float32))
    Wdn = codecs.f32_to_bf16_bits(codecs.e4m3_bits_to_f64(qdn).astype(np.float32))
    assert np.array_equal(codecs.bf16_bits_to_f64(Wgu), codecs.e4m3_bits_to_f64(qgu))
    out16, r16 = oracle.forward(x, Wg, Wgu, Wdn, k, SCALE)
    assert np.array_equal(r8.idx, r16.idx)
    rel = np.sqrt(np.mean((out8 - out16) ** 2)) / np.sqrt(np.mean(out16 ** 2))
    assert 1e-4 < rel < 6e-2            # quantisation noise is present but small
    # with a zero router-chosen token row, both are zero
    x0 = x.copy()
    x0[3] = 0
    o8, _ = oracle.forward_fp8(x0, Wg, qgu, sgu, qdn, sdn, k, SCALE)
    assert np.all(o8[3] == 0)


def test_fp8_routing_equals_bf16_routing():
    """The router never sees the expert weights' format."""
    rng = np.random.default_rng(23)
    T, d, E, F = 16, 64, 10, 16
    x = codecs.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    qgu = rng.integers(0, 0x7E, (E, 2 * F, d)).astype(np.uint8)
    qdn = rng.integers(0, 0x7E, (E, d, F)).astype(np.uint8)
    s1 = np.full((E, 2 * F), 1e-3, np.float32)
    s2 = np.full((E, d), 1e-3, np.float32)
    _, r8 = oracle.forward_fp8(x, Wg, qgu, s1, qdn, s2, 4, SCALE)
    r = oracle.route(x, Wg, 4, SCALE)
    assert np.array_equal(r8.idx, r.idx) and np.array_equal(r8.w, r.w)


def _fp8_layer(rng, T, d, E, F):
    x = codecs.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    qgu = codecs.f32_to_e4m3_bits((rng.standard_normal((E, 2 * F, d)) * 0.1).astype(np.float32))
    qdn = codecs.f32_to_e4m3_bits((rng.standard_normal((E, d, F)) * 0.1).astype(np.float32))
    return x, Wg, qgu, qdn


def test_block_scales_constant_along_k_equal_row_scales():
    """128 x 128 block scales that depend only on the row block give the same
    layer as per-row scales repeated over each block's 128 rows."""
    rng = np.random.default_rng(24)
    T, d, E, F, k = 20, 256, 6, 128, 3
    x, Wg, qgu, qdn = _fp8_layer(rng, T, d, E, F)
    cgu = (2.0 ** rng.integers(-9, -3, (E, 2 * F // 128)) * (1 + rng.random((E, 2 * F // 128)))).astype(np.float32)
    cdn = (2.0 ** rng.integers(-9, -3, (E, d // 128)) * (1 + rng.random((E, d // 128)))).astype(np.float32)
    bgu = np.repeat(cgu[:, :, None], d // 128, axis=2)
    bdn = np.repeat(cdn[:, :, None], F // 128, axis=2)
    rgu = np.repeat(cgu, 128, axis=1)
    rdn = np.repeat(cdn, 128, axis=1)
    out_b, rb = oracle.forward_fp8(x, Wg, qgu, bgu, qdn, bdn, k, SCALE)
    out_r, rr = oracle.forward_fp8(x, Wg, qgu, rgu, qdn, rdn, k, SCALE)
    assert np.array_equal(rb.idx, rr.idx)
    assert np.array_equal(out_b, out_r)


def test_block_scale_acts_on_its_own_k_range_only():
    """A zero scale on k-block j of every row block is the same layer as
    zero codes in columns 128 j .. 128 j + 127 with unit scales; a zero scale
    on row block m zeroes exactly that block's output channels of down."""
    rng = np.random.default_rng(25)
    T, d, E, F, k = 20, 384, 5, 256, 2
    x, Wg, qgu, qdn = _fp8_layer(rng, T, d, E, F)
    bgu = np.ones((E, 2 * F // 128, d // 128), np.float32)
    bdn = np.ones((E, d // 128, F // 128), np.float32)
    bgu[:, :, 1] = 0.0                                  # k columns 128..255 of gate_up
    bdn[:, :, 0] = 0.0                                  # k columns 0..127 of down
    zgu = qgu.copy()
    zgu[:, :, 128:256] = 0
    zdn = qdn.copy()
    zdn[:, :, 0:128] = 0
    out_b, _ = oracle.forward_fp8(x, Wg, qgu, bgu, qdn, bdn, k, SCALE)
    out_z, _ = oracle.forward_fp8(x, Wg, zgu, np.ones((E, 2 * F), np.float32), zdn,
                                  np.ones((E, d), np.float32), k, SCALE)
    assert np.array_equal(out_b, out_z)
    assert np.any(out_b != 0)
    bdn2 = np.ones((E, d // 128, F // 128), np.float32)
    bdn2[:, 2, :] = 0.0                                 # output channels 256..383
    out_m, _ = oracle.forward_fp8(x, Wg, qgu, np.ones_like(bgu), qdn, bdn2, k, SCALE)
    assert np.all(out_m[:, 256:384] == 0) and np.all(out_m[:, :256] != 0)


def test_block_dequantisation_element_by_element():
    """dequant_e4m3 with block scales against a per-element loop."""
    rng = np.random.default_rng(26)
    q = rng.integers(0, 256, (256, 384)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0                            # no NaN codes
    s = rng.random((2, 3)).astype(np.float32)
    w = oracle.dequant_e4m3(q, s)
    lut = codecs.e4m3_bits_to_f64(np.arange(256, dtype=np.uint8))
    for n in range(0, 256, 7):
        for i in range(0, 384, 5):
            assert w[n, i] == lut[q[n, i]] * float(s[n // 128, i // 128])
