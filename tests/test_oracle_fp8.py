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


# ----------------------------------------------------------------------------- where the layer quantises
#
# One-hot expert weights make the FP8 layer a closed form.  Gate row f of
# expert e picks one x column, ig[e, f], with one e4m3 code and a power-of-two
# row scale, so g = dequant(x)[ig] * w_g exactly (likewise u); down row c
# picks one activation column, fd[e, c], so y_c = dequant(a)[fd] * w_d
# exactly.  The expected output is then written with torch's e4m3 cast and
# scipy's sigmoid, independently of the oracle's codecs: x quantised per
# token row, the activation a rounded to bf16 (where the layer stores it) and
# its bf16 values quantised per (token, slot) row,
# r = float32(448 / amax), codes = e4m3(float32(a * r)), scale
# float32(amax / 448), dequantised as codes * scale ("DeepSeek V4-Flash
# architecture Q&A", Q7.2 and Q7.4).  Mutant copies of the oracle that move
# or drop either quantisation must fail the same check.

def _torch_e4m3(v32):
    """torch's float8_e4m3fn cast of float32 values clipped to +-448: (codes, values)."""
    t = torch.from_numpy(np.clip(np.asarray(v32, np.float32), -448.0, 448.0)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy(), t.to(torch.float64).numpy()


def _torch_e4m3_value(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_quant_rows(M32):
    """Dequantised per-row e4m3 quantisation of float32 rows (numpy float32
    arithmetic for r, v * r and the scale; torch for the rounding)."""
    M32 = np.asarray(M32, np.float32)
    out = np.zeros(M32.shape)
    for i, v in enumerate(M32):
        amax = np.max(np.abs(v))
        if amax == 0:
            continue
        r = np.float32(448.0) / amax
        _, vals = _torch_e4m3(v * r)
        out[i] = vals * np.float64(amax / np.float32(448.0))
    return out


def _bf16_nearest(v):
    """Nearest bf16 value (8 significant bits, ties to even) via frexp."""
    m, e = np.frexp(np.asarray(v, np.float64))
    return np.ldexp(np.round(m * 256.0), e - 8)          # np.round: half to even; m * 256 exact


def _one_hot_fp8_layer(seed, x_exact):
    rng = np.random.default_rng(seed)
    T, d, E, F = 12, 128, 3, 64
    if x_exact:
        # rows of e4m3 values times 2^m whose largest magnitude is 448 * 2^m:
        # quantising them is exact, so the layer sees x itself
        codes = rng.integers(0x20, 0x7E, (T, d)).astype(np.uint8) | (rng.integers(0, 2, (T, d)) << 7).astype(np.uint8)
        codes[:, 5] = 0x7E
        xv = _torch_e4m3_value(codes) * np.ldexp(1.0, rng.integers(-9, -5, T))[:, None]
    else:
        xv = rng.standard_normal((T, d))
    x = codecs.f32_to_bf16_bits(xv.astype(np.float32))
    assert not x_exact or np.array_equal(codecs.bf16_bits_to_f64(x), xv)
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    sel = lambda n, hi: rng.integers(0, hi, n)
    wcode = lambda n: (rng.integers(0x30, 0x48, n) | (rng.integers(0, 2, n) << 7)).astype(np.uint8)
    ig, iu, fd = sel((E, F), d), sel((E, F), d), sel((E, d), F)
    cg, cu, cd = wcode((E, F)), wcode((E, F)), wcode((E, d))
    pg, pu, pd = (rng.integers(-4, 0, s).astype(np.float64) for s in ((E, F), (E, F), (E, d)))
    Wq_gu = np.zeros((E, 2 * F, d), np.uint8)
    Wq_dn = np.zeros((E, d, F), np.uint8)
    ee, ff = np.meshgrid(np.arange(E), np.arange(F), indexing="ij")
    Wq_gu[ee, ff, ig] = cg
    Wq_gu[ee, F + ff, iu] = cu
    ec, cc = np.meshgrid(np.arange(E), np.arange(d), indexing="ij")
    Wq_dn[ec, cc, fd] = cd
    s_gu = np.concatenate([np.ldexp(1.0, pg.astype(int)), np.ldexp(1.0, pu.astype(int))], axis=1).astype(np.float32)
    s_dn = np.ldexp(1.0, pd.astype(int)).astype(np.float32)
    layer = dict(x=x, Wg=Wg, Wq_gu=Wq_gu, s_gu=s_gu, Wq_dn=Wq_dn, s_dn=s_dn, k=E)
    # the closed form's activation before its bf16 rounding, [T, E, F] by expert
    # ---- the closed form
    from scipy.special import expit
    x64 = codecs.bf16_bits_to_f64(x)
    xd = x64 if x_exact else _torch_quant_rows(x64.astype(np.float32))
    wg = _torch_e4m3_value(cg) * s_gu[:, :F]
    wu = _torch_e4m3_value(cu) * s_gu[:, F:]
    wd = _torch_e4m3_value(cd) * s_dn
    g = xd[:, ig] * wg[None]                                 # [T, E, F], exact
    u = xd[:, iu] * wu[None]
    layer["a"] = g * expit(g) * u
    a16 = _bf16_nearest(layer["a"]).astype(np.float32)                # exact in float32
    ad = _torch_quant_rows(a16.reshape(T * E, F)).reshape(T, E, F)
    y = np.take_along_axis(ad, np.broadcast_to(fd[None], (T, E, d)), axis=2) * wd[None]   # exact
    s = expit(x64 @ Wg.astype(np.float64).T).astype(np.float32).astype(np.float64)
    w = np.float64(np.float32(SCALE)) * s / s.sum(axis=1, keepdims=True)
    expect = np.einsum("te,tec->tc", w, _bf16_nearest(y))
    return layer, expect


def _fp8_closed_form_holds(forward_fp8, seed, x_exact):
    L, expect = _one_hot_fp8_layer(seed, x_exact)
    out, _ = forward_fp8(L["x"], L["Wg"], L["Wq_gu"], L["s_gu"], L["Wq_dn"], L["s_dn"], L["k"], SCALE)
    return bool(np.max(np.abs(out - expect)) <= 1e-12 * np.max(np.abs(expect)))


def _mutant_fp8(kind):
    """A scratch copy of the oracle's FP8 layer with one deliberate change:
    no_h_quant (the down product takes float64 a), h_fp32 (a quantised from
    its float32 value, without the bf16 rounding), h_per_token (one scale over
    a token's k
    activation rows), no_x_quant (the gate_up product takes x itself).  The
    scale's exact float32 value is pinned by the quantiser tests above: a
    one-ulp change of it does not survive the bf16 rounding of y."""
    def fwd(x_bits, W_gate, Wq_gu, s_gu, Wq_dn, s_dn, k, scale):
        r = oracle.route(x_bits, W_gate, k, scale)
        x = codecs.bf16_bits_to_f64(x_bits)
        T, F = x.shape[0], Wq_dn.shape[2]
        if kind == "no_x_quant":
            xd = x
        else:
            qx, sx = oracle.quant_rows_e4m3(x.astype(np.float32))
            xd = codecs.e4m3_bits_to_f64(qx) * sx.astype(np.float64)[:, None]
        a = np.zeros((T, k, F))
        for e in np.unique(r.idx):
            t, j = np.nonzero(r.idx == e)
            Wgu = oracle.dequant_e4m3(Wq_gu[e], s_gu[e])
            g, u = xd[t] @ Wgu[:F].T, xd[t] @ Wgu[F:].T
            a[t, j] = g / (1.0 + np.exp(-g)) * u
        if kind == "no_h_quant":
            ad = a
        elif kind == "h_per_token":
            ad = np.stack([_oracle_deq_rows(codecs.round_to_bf16(a[t]).reshape(1, -1)).reshape(k, F)
                           for t in range(T)])
        else:
            src = a if kind == "h_fp32" else codecs.round_to_bf16(a)
            ad = _oracle_deq_rows(src.reshape(T * k, F)).reshape(T, k, F)
        out = np.zeros(x.shape)
        for e in np.unique(r.idx):
            t, j = np.nonzero(r.idx == e)
            y = ad[t, j] @ oracle.dequant_e4m3(Wq_dn[e], s_dn[e]).T
            out[t] += r.w[t, j][:, None] * codecs.round_to_bf16(y)
        return out, r
    return fwd


def _oracle_deq_rows(M):
    q, s = oracle.quant_rows_e4m3(np.asarray(M, np.float32))
    return codecs.e4m3_bits_to_f64(q) * s.astype(np.float64)[:, None]


def test_fp8_quantisation_placement_closed_form():
    """The oracle's FP8 layer equals the one-hot closed form, with x exactly
    e4m3-representable (pins the activation quantisation alone) and with
    general bf16 x (pins both quantisations)."""
    for seed in (90, 91):
        assert _fp8_closed_form_holds(oracle.forward_fp8, seed, x_exact=True)
        assert _fp8_closed_form_holds(oracle.forward_fp8, seed, x_exact=False)


def test_fp8_closed_form_rejects_moved_quantisations():
    """Each mutant fails the closed-form check: the check is sharp enough to
    catch a dropped or moved quantisation of either operand."""
    for kind in ("no_h_quant", "h_fp32", "h_per_token"):
        assert not _fp8_closed_form_holds(_mutant_fp8(kind), 90, x_exact=True), kind
    # x itself is exact in the first form, so dropping its quantisation needs the second
    assert _fp8_closed_form_holds(_mutant_fp8("no_x_quant"), 90, x_exact=True)
    assert not _fp8_closed_form_holds(_mutant_fp8("no_x_quant"), 90, x_exact=False)
    # the scratch copy itself, unmutated in effect, agrees with the closed form
    assert _fp8_closed_form_holds(_mutant_fp8("none"), 90, x_exact=False)
