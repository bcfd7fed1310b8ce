"""GPU parity on a seeded sweep of small random shapes: the bf16 layer, the
e4m3 layer (per-channel and 128 x 128 block scales) and the full block, every
token compared with the oracle.

The shapes are drawn once from a fixed generator, so every run tests the same
cases.  About half of each kind is drawn to take the weight-streaming decode
kernels (T * k <= 11 E, or 20 E where T * k >= 8 E, d and d_ff whole 256-byte
batches) and the rest the grouped GEMMs, with expert counts, k, d and d_ff in
the ranges the library takes (d and d_ff multiples of 64, of 128 with e4m3
experts; k <= min(E, 16)).
Criteria as in the other parity tests: routing bit-exact except flagged
near-ties; outputs within 1e-2 * rms(ref) with bf16 experts and 3e-2 * rms(ref)
with e4m3 experts, element by element, an element exceeding it only by the
rounding-boundary flips check_output_flips predicts from the oracle."""

import numpy as np
import pytest
import torch

import oracle
from parity import bf16_flip_model, check_output_flips, check_routing, fp8_flip_model
from sparse_moe_layer_wave_amd import inputs

pytestmark = pytest.mark.gpu
TOL_BF16 = 1e-2
TOL_FP8 = 3e-2
EPS = float(np.float32(1e-6))


def _draw(n, seed, esz, max_e=96):
    """n shapes (T, d, E, k, F); even draws satisfy the decode-path switch."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(4, max_e + 1))
        k = int(rng.integers(1, min(E, 16) + 1))
        if i % 2 == 0:                                  # decode-path sized
            unit = 256 // esz                           # whole 256-byte batches
            d = unit * int(rng.integers(1, max(2, 512 // unit + 1)))
            F = unit * int(rng.integers(1, max(2, 384 // unit + 1)))
            T = int(rng.integers(1, max(2, 11 * E // k + 1)))
        else:                                           # grouped-GEMM sized
            step = 64 if esz == 2 else 128              # e4m3: whole 128-byte K slices
            d = step * int(rng.integers(1, 512 // step + 1))
            F = step * int(rng.integers(1, 384 // step + 1))
            T = int(rng.integers(1, 701))
        out.append((T, d, E, k, F))
    return out


BF16_CASES = _draw(12, 2024, 2)
FP8_CASES = _draw(6, 2025, 1)
BLOCK_CASES = _draw(6, 2026, 2)
# 128 x 128 block scales: d and d_ff in whole 256-element batches
BLK128_CASES = [(T, 256 * ((d + 255) // 256), E, k, 256 * ((F + 255) // 256))
                for T, d, E, k, F in _draw(6, 2027, 1)]


def _ids(cases):
    return [f"T{T}-d{d}-E{E}-k{k}-F{F}" for T, d, E, k, F in cases]


def _set_eq(idx, r):
    return np.array([set(a) == set(b) for a, b in zip(idx.tolist(), r.idx.tolist())], dtype=bool)


@pytest.mark.parametrize("T,d,E,k,F", BF16_CASES, ids=_ids(BF16_CASES))
def test_sweep_bf16(gpu_lib, T, d, E, k, F):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    skew = (T + E) % 3 == 0                           # a third of the cases with the skewed logit bias
    c = dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=T, d=d, E=E, k=k, F=F, seed=500 + T, skew=skew)
    inp = inputs.make_inputs(c, device="cpu")
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    out, idx, w = hy.forward(dev["x"], dev["W_gate"], dev["W_gu"], dev["W_dn"], k, inp["scale"],
                             bias=dev["bias"], return_routing=True)
    torch.cuda.synchronize()
    b = None if inp["bias"] is None else inp["bias"].numpy()
    ref, r = oracle.forward(inputs.bits(inp["x"]), inp["W_gate"].numpy(), inputs.bits(inp["W_gu"]),
                            inputs.bits(inp["W_dn"]), k, inp["scale"], b)
    idx = idx.cpu().numpy()
    stats = check_routing(idx, w.cpu().numpy(), r, inp["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, _set_eq(idx, r), TOL_BF16,
                                    **bf16_flip_model(inputs.bits(inp["x"]), r, inputs.bits(inp["W_gu"]),
                                                      inputs.bits(inp["W_dn"]))))
    print(T, d, E, k, F, "skew" if skew else "", stats)


@pytest.mark.parametrize("T,d,E,k,F", FP8_CASES, ids=_ids(FP8_CASES))
def test_sweep_fp8(gpu_lib, T, d, E, k, F):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = dict(inputs.CONFIGS["hy3_fp8_T8192"], T=T, d=d, E=E, k=k, F=F, seed=600 + T)
    inp = inputs.make_inputs(c, device="cpu")
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    out, idx, w = hy.forward_fp8(dev["x"], dev["W_gate"], dev["Wq_gu"], dev["s_gu"], dev["Wq_dn"],
                                 dev["s_dn"], k, inp["scale"], return_routing=True)
    torch.cuda.synchronize()
    ref, r = oracle.forward_fp8(inputs.bits(inp["x"]), inp["W_gate"].numpy(), inputs.bits(inp["Wq_gu"]),
                                inp["s_gu"].numpy(), inputs.bits(inp["Wq_dn"]), inp["s_dn"].numpy(),
                                k, inp["scale"])
    idx = idx.cpu().numpy()
    stats = check_routing(idx, w.cpu().numpy(), r, inp["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, _set_eq(idx, r), TOL_FP8,
                                    **fp8_flip_model(inputs.bits(inp["x"]), r, inputs.bits(inp["Wq_gu"]),
                                                     inp["s_gu"].numpy(), inputs.bits(inp["Wq_dn"]),
                                                     inp["s_dn"].numpy())))
    print(T, d, E, k, F, stats)


@pytest.mark.parametrize("T,d,E,k,F", BLOCK_CASES, ids=_ids(BLOCK_CASES))
def test_sweep_block(gpu_lib, T, d, E, k, F):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = dict(inputs.CONFIGS["hy3_block_decode_T64"], T=T, d=d, E=E, k=k, F=F, seed=700 + T)
    inp = inputs.make_inputs(c, device="cpu")
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    out, idx, w = hy.block_forward(dev["x"], dev["W_gate"], dev["W_gu"], dev["W_dn"], dev["Ws_gu"],
                                   dev["Ws_dn"], k, inp["scale"], norm_weight=dev["norm_w"], norm_eps=EPS,
                                   score_bias=dev["score_bias"], return_routing=True)
    torch.cuda.synchronize()
    ref, r = oracle.forward_block(inputs.bits(inp["x"]), inputs.bits(inp["W_gate"]), inputs.bits(inp["W_gu"]),
                                  inputs.bits(inp["W_dn"]), inputs.bits(inp["Ws_gu"]), inputs.bits(inp["Ws_dn"]),
                                  k, inp["scale"], norm_w_bits=inputs.bits(inp["norm_w"]), eps=EPS,
                                  score_bias=inputs.bits(inp["score_bias"]))
    idx = idx.cpu().numpy()
    stats = check_routing(idx, w.cpu().numpy(), r, inp["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, _set_eq(idx, r), TOL_BF16,
                                    **bf16_flip_model(inputs.bits(inp["x"]), r, inputs.bits(inp["W_gu"]),
                                                      inputs.bits(inp["W_dn"]), inputs.bits(inp["Ws_gu"]),
                                                      inputs.bits(inp["Ws_dn"]))))
    print(T, d, E, k, F, stats)


@pytest.mark.parametrize("T,d,E,k,F", BLK128_CASES, ids=_ids(BLK128_CASES))
def test_sweep_fp8_block128(gpu_lib, T, d, E, k, F):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = dict(inputs.CONFIGS["hy3_fp8_block128_decode_T64"], T=T, d=d, E=E, k=k, F=F, seed=800 + T)
    inp = inputs.make_inputs(c, device="cpu")
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    out, idx, w = hy.forward_fp8_block128(dev["x"], dev["W_gate"], dev["Wq_gu"], dev["s_gu"], dev["Wq_dn"],
                                          dev["s_dn"], k, inp["scale"], return_routing=True)
    torch.cuda.synchronize()
    ref, r = oracle.forward_fp8(inputs.bits(inp["x"]), inp["W_gate"].numpy(), inputs.bits(inp["Wq_gu"]),
                                inp["s_gu"].numpy(), inputs.bits(inp["Wq_dn"]), inp["s_dn"].numpy(),
                                k, inp["scale"])
    idx = idx.cpu().numpy()
    stats = check_routing(idx, w.cpu().numpy(), r, inp["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, _set_eq(idx, r), TOL_FP8,
                                    **fp8_flip_model(inputs.bits(inp["x"]), r, inputs.bits(inp["Wq_gu"]),
                                                     inp["s_gu"].numpy(), inputs.bits(inp["Wq_dn"]),
                                                     inp["s_dn"].numpy())))
    print(T, d, E, k, F, stats)
