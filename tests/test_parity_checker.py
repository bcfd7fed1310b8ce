"""The output check of the GPU parity tests (parity.check_output_flips),
exercised on the CPU: a float32 implementation of the layer in torch, which
rounds h and y to bf16 where the layer stores them (as the GPU does, with
another summation order), exceeds the plain 1e-2 * rms bound on some
elements and passes the flip check; the same implementation with a planted
error fails it."""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs
from parity import bf16_flip_model, check_output_flips, fp8_flip_model

SCALE = float(np.float32(2.826))


def _bf16_case(seed, T=3000, d=256, E=8, k=2, F=128):
    rng = np.random.default_rng(seed)
    x = codecs.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    gu = codecs.f32_to_bf16_bits((rng.standard_normal((E, 2 * F, d)) * 0.06).astype(np.float32))
    dn = codecs.f32_to_bf16_bits((rng.standard_normal((E, d, F)) * 0.06).astype(np.float32))
    return x, Wg, gu, dn, k


def _t(bits):
    return torch.from_numpy(codecs.bf16_bits_to_f64(bits).astype(np.float32))


def _torch_fp32_layer(x, gu, dn, r, w_scale=1.0, silu_on_up=False):
    """out[t] = sum_j w * bf16(bf16(SiLU(g) u) Wd^T), float32 sums (torch CPU)."""
    xt = _t(x)
    F = dn.shape[2]
    out = torch.zeros(xt.shape, dtype=torch.float32)
    w = torch.from_numpy(r.w.astype(np.float32)) * w_scale
    for e in np.unique(r.idx):
        t, j = np.nonzero(r.idx == e)
        Wgu, Wdn = _t(gu[e]), _t(dn[e])
        g = xt[t] @ Wgu[:F].T
        u = xt[t] @ Wgu[F:].T
        h = (u * torch.sigmoid(u) * g) if silu_on_up else (g * torch.sigmoid(g) * u)
        y = (h.to(torch.bfloat16).float() @ Wdn.T).to(torch.bfloat16).float()
        out[t] += w[t, j][:, None] * y
    return out.numpy()


def test_flip_check_accepts_a_float32_layer_the_plain_bound_rejects():
    x, Wg, gu, dn, k = _bf16_case(110)
    ref, r = oracle.forward(x, Wg, gu, dn, k, SCALE)
    out = _torch_fp32_layer(x, gu, dn, r)
    stats = check_output_flips(out, ref, None, 1e-2, **bf16_flip_model(x, r, gu, dn))
    assert stats["elems_over_tol"] > 0          # the plain bound alone would fail here
    assert stats["max_ratio"] < 2e-2


@pytest.mark.parametrize("plant", ["weights_1pct", "silu_on_up"])
def test_flip_check_rejects_planted_errors(plant):
    x, Wg, gu, dn, k = _bf16_case(111)
    ref, r = oracle.forward(x, Wg, gu, dn, k, SCALE)
    out = _torch_fp32_layer(x, gu, dn, r, w_scale=1.01 if plant == "weights_1pct" else 1.0,
                            silu_on_up=plant == "silu_on_up")
    with pytest.raises(AssertionError, match="not explained by rounding flips"):
        check_output_flips(out, ref, None, 1e-2, **bf16_flip_model(x, r, gu, dn))


def _torch_fp32_fp8_layer(x, qgu, sgu, qdn, sdn, r, F, per_token_h=False):
    """The e4m3 layer with torch's float32 arithmetic and e4m3 cast."""
    def q_rows(M):
        amax = M.abs().amax(dim=1, keepdim=True)
        c448 = torch.full_like(amax, 448.0)         # tensor / tensor: a correctly rounded division
        rr = torch.where(amax > 0, c448 / amax, torch.ones_like(amax))
        s = torch.where(amax > 0, amax / c448, torch.ones_like(amax))
        return (M * rr).clamp(-448, 448).to(torch.float8_e4m3fn).float() * s
    xt = q_rows(_t(x))
    out = torch.zeros(xt.shape, dtype=torch.float32)
    w = torch.from_numpy(r.w.astype(np.float32))
    T, k = r.idx.shape
    hs = torch.zeros((T, k, F))
    for e in np.unique(r.idx):
        t, j = np.nonzero(r.idx == e)
        Wgu = torch.from_numpy(oracle.dequant_e4m3(qgu[e], sgu[e]).astype(np.float32))
        g, u = xt[t] @ Wgu[:F].T, xt[t] @ Wgu[F:].T
        hs[t, j] = (g * torch.sigmoid(g) * u).to(torch.bfloat16).float()     # h is stored in bf16
    hq = q_rows(hs.reshape(T, k * F)).reshape(T, k, F) if per_token_h else q_rows(hs.reshape(T * k, F)).reshape(T, k, F)
    for e in np.unique(r.idx):
        t, j = np.nonzero(r.idx == e)
        Wdn = torch.from_numpy(oracle.dequant_e4m3(qdn[e], sdn[e]).astype(np.float32))
        out[t] += w[t, j][:, None] * (hq[t, j] @ Wdn.T).to(torch.bfloat16).float()
    return out.numpy()


@pytest.mark.parametrize("plant", [None, "per_token_h"])
def test_fp8_flip_check(plant):
    """d_ff = 64 and k = 2: an e4m3 code flip of one activation moves a whole
    output row by several 1e-3 of rms.  The check runs at 1e-2 * rms here
    (sharper than the layer's 3e-2) so that such flips exceed the plain bound
    and the e4m3 branch of the allowance has to explain them."""
    rng = np.random.default_rng(114)
    T, d, E, k, F = 3000, 256, 8, 2, 64
    x = codecs.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    qgu = codecs.f32_to_e4m3_bits((rng.standard_normal((E, 2 * F, d)) * 60).astype(np.float32))
    qdn = codecs.f32_to_e4m3_bits((rng.standard_normal((E, d, F)) * 60).astype(np.float32))
    sgu = np.full((E, 2 * F), 1e-3, np.float32)
    sdn = np.full((E, d), 1e-3, np.float32)
    ref, r = oracle.forward_fp8(x, Wg, qgu, sgu, qdn, sdn, k, SCALE)
    out = _torch_fp32_fp8_layer(x, qgu, sgu, qdn, sdn, r, F, per_token_h=plant == "per_token_h")
    model = fp8_flip_model(x, r, qgu, sgu, qdn, sdn)
    if plant is None:
        stats = check_output_flips(out, ref, None, 1e-2, **model)
        assert stats["elems_over_tol"] > 0 and stats["max_ratio"] < 6e-2
    else:
        with pytest.raises(AssertionError, match="not explained by rounding flips"):
            check_output_flips(out, ref, None, 1e-2, **model)
