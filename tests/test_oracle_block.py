"""Pins of the oracle's full-block pieces against what mathematics and library
routines fix:

* rms_norm_bf16 ("Tencent Hy3-Flash Q&A", Q4.9, route_norm): torch's own
  rms_norm within the two bf16 roundings, exact invariance under power-of-two
  scaling of a row (eps = 0), and the closed form for rows of equal magnitude;
* the selection-only score bias ("Tencent Hy3-Flash Q&A", Q4.3; "Tencent
  Hy3-295B architecture teardown", section 4.1 step 2): a zero bias changes
  nothing, a dominant bias forces the chosen set, and brute-force subset
  enumeration (choice values below zero included) finds the same set, with
  weights from the unbiased scores;
* forward_block ("Tencent Hy3-Flash Q&A", Q4.7): with zero routed experts it
  is the dense SwiGLU of the shared expert (torch matmul and silu); with the
  shared expert equal to every routed expert it is (scale + 1) times that
  expert; route_norm makes the routing blind to the row's scale."""

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
from oracle import codecs

SCALE = float(np.float32(2.826))


def _bits(a):
    return codecs.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _layer(rng, T, d, E, F, w_std=0.02):
    x = _bits(rng.standard_normal((T, d)))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    Wgu = _bits(rng.standard_normal((E, 2 * F, d)) * w_std)
    Wdn = _bits(rng.standard_normal((E, d, F)) * w_std)
    Wsgu = _bits(rng.standard_normal((2 * F, d)) * w_std)
    Wsdn = _bits(rng.standard_normal((d, F)) * w_std)
    return x, Wg, Wgu, Wdn, Wsgu, Wsdn


def _torch_swiglu_bf16(x_bits, Wgu_bits, Wdn_bits):
    """Dense SwiGLU with torch matmul and silu in float64, h and y rounded to
    bf16 through torch's own float -> bfloat16 cast."""
    x = torch.from_numpy(codecs.bf16_bits_to_f64(x_bits))
    Wgu = torch.from_numpy(codecs.bf16_bits_to_f64(Wgu_bits))
    Wdn = torch.from_numpy(codecs.bf16_bits_to_f64(Wdn_bits))
    F = Wdn.shape[1]
    h = Fn.silu(x @ Wgu[:F].T) * (x @ Wgu[F:].T)
    h = h.to(torch.bfloat16).to(torch.float64)
    return (h @ Wdn.T).to(torch.bfloat16).to(torch.float64).numpy()


# ----------------------------------------------------------------------------- rms_norm_bf16

def test_rms_norm_matches_torch_within_bf16_rounding():
    rng = np.random.default_rng(50)
    x = _bits(rng.standard_normal((64, 512)) * 3)
    w = _bits(1 + 0.1 * rng.standard_normal(512))
    got = codecs.bf16_bits_to_f64(oracle.rms_norm_bf16(x, w, 1e-6))
    ref = Fn.rms_norm(torch.from_numpy(codecs.bf16_bits_to_f64(x)), (512,),
                      weight=torch.from_numpy(codecs.bf16_bits_to_f64(w)), eps=1e-6).numpy()
    # two bf16 roundings (normalised row, then the weighted product): at most
    # 2^-8 + 2^-8 (1 + 2^-8) relative
    assert np.all(np.abs(got - ref) <= (2.0 ** -7 + 2.0 ** -15) * np.abs(ref) + 1e-30)
    # with a unit weight the second rounding is exact, so the result is torch's
    # float32 rms_norm rounded once to bf16, up to torch's float32 rsqrt
    # (not correctly rounded) tipping a product across a bf16 rounding boundary
    one = _bits(np.ones(512))
    got1 = codecs.bf16_bits_to_f64(oracle.rms_norm_bf16(x, one, 1e-6))
    ref1 = Fn.rms_norm(torch.from_numpy(codecs.bf16_bits_to_f64(x)).float(), (512,), eps=1e-6).numpy()
    once = codecs.bf16_bits_to_f64(codecs.f32_to_bf16_bits(ref1))
    assert np.mean(got1 == once) > 0.999
    assert np.all(np.abs(got1 - once) <= 2.0 ** -7 * np.abs(once))


def test_rms_norm_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(51)
    x = _bits(rng.standard_normal((16, 256)))
    w = _bits(1 + 0.1 * rng.standard_normal(256))
    base = oracle.rms_norm_bf16(x, w, 0.0)
    for shift in (-6, -1, 3, 9):
        xs = _bits(codecs.bf16_bits_to_f64(x) * 2.0 ** shift)        # exact in bf16
        assert np.array_equal(oracle.rms_norm_bf16(xs, w, 0.0), base)


def test_rms_norm_equal_magnitude_rows_closed_form():
    d = 128
    for c in (0.5, 3.0, 1e-3):
        for eps in (0.0, 1e-6, 0.25):
            cb = float(np.ravel(codecs.bf16_bits_to_f64(_bits(c)))[0])
            signs = np.where(np.arange(d) % 3 == 0, -1.0, 1.0)
            x = _bits(signs * cb)[None, :]
            w = _bits(np.full(d, 2.0))
            r = np.float32(1.0 / np.sqrt(cb * cb + eps))
            a = float(np.ravel(codecs.bf16_bits_to_f64(_bits(np.float32(cb) * r)))[0])
            expect = signs * float(np.ravel(codecs.bf16_bits_to_f64(_bits(a * 2.0)))[0])
            assert np.array_equal(codecs.bf16_bits_to_f64(oracle.rms_norm_bf16(x, w, eps))[0], expect)


def test_rms_norm_zero_row_and_empty():
    z = np.zeros((2, 64), np.uint16)
    w = _bits(np.ones(64))
    assert np.array_equal(oracle.rms_norm_bf16(z, w, 1e-6), z)       # 0 * r = 0
    assert oracle.rms_norm_bf16(np.zeros((0, 64), np.uint16), w, 1e-6).shape == (0, 64)


# ----------------------------------------------------------------------------- score bias

def test_zero_score_bias_changes_nothing():
    rng = np.random.default_rng(52)
    x, Wg, *_ = _layer(rng, 200, 256, 32, 64)
    a = oracle.route(x, Wg, 8, SCALE)
    b = oracle.route(x, Wg, 8, SCALE, score_bias=np.zeros(32, np.float32))
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.w, b.w)
    assert np.array_equal(a.near_tie, b.near_tie)


def test_dominant_score_bias_forces_the_set_weights_from_scores():
    rng = np.random.default_rng(53)
    x, Wg, *_ = _layer(rng, 50, 256, 32, 64)
    forced = [30, 3, 17, 9]
    bias = np.zeros(32, np.float32)
    bias[forced] = [10.0, 10.0, 12.0, 10.0]           # scores lie in (0, 1)
    r = oracle.route(x, Wg, 4, SCALE, score_bias=bias)
    s = r.scores.astype(np.float64)
    for t in range(50):
        assert sorted(r.idx[t]) == sorted(forced)
        assert r.idx[t][0] == 17                                   # the largest bias leads
        sel = s[t, r.idx[t]]
        assert np.allclose(r.w[t], SCALE * sel / sel.sum(), rtol=0, atol=1e-15)
        assert abs(r.w[t].sum() - SCALE) < 1e-12


def _brute_force_choice(c_row, s_row, k, scale):
    """Unique k-subset whose members all precede every non-member in
    (choice descending, index ascending) order == the subset maximising the
    exact sum of choice values, ties broken towards the lexicographically
    smallest index set.  Weights from the scores s."""
    E = len(c_row)
    best, best_key = None, None
    for sub in itertools.combinations(range(E), k):
        total = sum(Fraction(float(c_row[e])) for e in sub)
        key = (total, tuple(-e for e in sub))
        if best_key is None or key > best_key:
            best, best_key = sub, key
    order = sorted(best, key=lambda e: (-float(c_row[e]), e))
    sel = np.array([float(s_row[e]) for e in order])
    return order, scale * sel / sel.sum()


@pytest.mark.parametrize("E,k,seed", [(10, 3, 54), (12, 4, 55), (9, 1, 56)])
def test_score_bias_brute_force_with_negative_choice_values(E, k, seed):
    rng = np.random.default_rng(seed)
    d = 32
    x = _bits(rng.standard_normal((40, d)))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.6 - 0.5).astype(np.float32)  # many choice values < 0
    r = oracle.route(x, Wg, k, SCALE, score_bias=bias)
    assert np.mean(r.choice < 0) > 0.2
    for t in range(40):
        if r.order_tie[t]:
            continue
        order, w = _brute_force_choice(r.choice[t], r.scores[t], k, SCALE)
        assert list(r.idx[t]) == order
        assert np.allclose(r.w[t], w, rtol=0, atol=1e-15)


def test_choice_is_a_float32_addition():
    rng = np.random.default_rng(57)
    x, Wg, *_ = _layer(rng, 30, 128, 16, 64)
    bias = (rng.standard_normal(16) * 1e-3).astype(np.float32)
    r = oracle.route(x, Wg, 4, SCALE, score_bias=bias)
    # float32 + float32 rounded once: the float64 sum rounded to float32 (exact
    # here: operands within 2^29 of each other's scale)
    expect = (r.scores.astype(np.float64) + bias.astype(np.float64)).astype(np.float32)
    assert np.array_equal(r.choice, expect)


# ----------------------------------------------------------------------------- forward_block

def test_block_with_zero_routed_experts_is_the_shared_dense_swiglu():
    rng = np.random.default_rng(58)
    x, Wg, Wgu, Wdn, Wsgu, Wsdn = _layer(rng, 24, 128, 16, 64)
    zgu = np.zeros_like(Wgu)
    zdn = np.zeros_like(Wdn)
    out, _ = oracle.forward_block(x, Wg, zgu, zdn, Wsgu, Wsdn, 4, SCALE,
                                  norm_w_bits=_bits(np.ones(128)), eps=1e-6)
    assert np.array_equal(out, _torch_swiglu_bf16(x, Wsgu, Wsdn))


def test_block_with_shared_equal_to_every_routed_expert():
    rng = np.random.default_rng(59)
    x, Wg, Wgu, Wdn, Wsgu, Wsdn = _layer(rng, 24, 128, 8, 64)
    Wgu[:] = Wsgu
    Wdn[:] = Wsdn
    # route_norm and the score bias change which experts are picked, never
    # what the experts are fed: all of them see x itself
    out, r = oracle.forward_block(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 3, SCALE,
                                  norm_w_bits=_bits(1.5 + 0.1 * rng.standard_normal(128)), eps=1e-6,
                                  score_bias=(rng.standard_normal(8) * 0.1).astype(np.float32))
    y = _torch_swiglu_bf16(x, Wsgu, Wsdn)
    assert np.allclose(out, (SCALE + 1.0) * y, rtol=1e-13, atol=1e-15)


def test_block_without_extras_is_forward_plus_shared():
    rng = np.random.default_rng(60)
    x, Wg, Wgu, Wdn, Wsgu, Wsdn = _layer(rng, 40, 128, 16, 64)
    out, r = oracle.forward_block(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE)
    routed, r0 = oracle.forward(x, Wg, Wgu, Wdn, 4, SCALE)
    assert np.array_equal(r.idx, r0.idx)
    assert np.allclose(out, routed + _torch_swiglu_bf16(x, Wsgu, Wsdn), rtol=0, atol=1e-15)


def test_route_norm_makes_routing_scale_blind():
    rng = np.random.default_rng(61)
    x, Wg, Wgu, Wdn, Wsgu, Wsdn = _layer(rng, 64, 128, 16, 64)
    x4 = _bits(codecs.bf16_bits_to_f64(x) * 4.0)
    w = _bits(1 + 0.1 * rng.standard_normal(128))
    _, ra = oracle.forward_block(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE, norm_w_bits=w, eps=0.0)
    _, rb = oracle.forward_block(x4, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE, norm_w_bits=w, eps=0.0)
    assert np.array_equal(ra.idx, rb.idx) and np.array_equal(ra.w, rb.w)
    # without route_norm the router sees the scale (logits x4)
    _, rc = oracle.forward_block(x4, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE)
    _, rd = oracle.forward_block(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE)
    assert not np.array_equal(rc.w, rd.w)


def test_block_tokens_are_independent():
    rng = np.random.default_rng(62)
    x, Wg, Wgu, Wdn, Wsgu, Wsdn = _layer(rng, 30, 128, 16, 64)
    kw = dict(norm_w_bits=_bits(np.ones(128)), eps=1e-6, score_bias=np.linspace(-0.1, 0.1, 16).astype(np.float32))
    out, _ = oracle.forward_block(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE, **kw)
    sub = [0, 7, 29]
    part, _ = oracle.forward_block_tokens(sub, x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE, **kw)
    assert np.array_equal(part, out[sub])


# ----------------------------------------------------------------------------- residual branch

def test_residual_branch_with_zero_experts_is_the_residual():
    rng = np.random.default_rng(63)
    x, Wg, Wgu, Wdn, Wsgu, Wsdn = _layer(rng, 20, 128, 16, 64)
    res = _bits(rng.standard_normal((20, 128)))
    out, _ = oracle.forward_block_residual(x, Wg, Wgu, np.zeros_like(Wdn), Wsgu, np.zeros_like(Wsdn), 4,
                                           SCALE, residual_bits=res)
    assert np.array_equal(out, codecs.bf16_bits_to_f64(res))


def test_residual_branch_adds_the_residual_to_the_block():
    rng = np.random.default_rng(64)
    x, Wg, Wgu, Wdn, Wsgu, Wsdn = _layer(rng, 20, 128, 16, 64)
    res = _bits(rng.standard_normal((20, 128)))
    kw = dict(norm_w_bits=_bits(np.ones(128)), eps=1e-6)
    blk, r0 = oracle.forward_block(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE, **kw)
    none, r1 = oracle.forward_block_residual(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE, **kw)
    out, r2 = oracle.forward_block_residual(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE, residual_bits=res, **kw)
    assert np.array_equal(none, blk) and np.array_equal(r2.idx, r0.idx)
    # the residual is x itself here: out = x + block(x), element by element
    same, _ = oracle.forward_block_residual(x, Wg, Wgu, Wdn, Wsgu, Wsdn, 4, SCALE, residual_bits=x, **kw)
    assert np.array_equal(same, codecs.bf16_bits_to_f64(x) + blk)
    assert np.allclose(out - blk, codecs.bf16_bits_to_f64(res), rtol=0, atol=1e-14)
