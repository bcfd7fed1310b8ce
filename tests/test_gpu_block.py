"""GPU parity of the full Hy3 MoE block (hy3moe_block_forward, hy3moe_route_ex)
against the oracle's forward_block / route: shared expert ("Tencent Hy3-Flash
Q&A", Q4.7), route_norm (Q4.9) and the selection-only score bias (Q4.3).

Routing is compared on every token (bit-exact indices except flagged
near-ties of the choice values), outputs within 1e-2 * rms(ref) element by
element on every token, small cases and Hy3-sized workloads alike (an element
may exceed the bound only by the rounding-boundary flips check_output_flips
predicts from the oracle's own values)."""

import numpy as np
import pytest
import torch

import oracle
from parity import LazyExperts, bf16_flip_model, check_output_flips, check_routing, set_equal
from sparse_moe_layer_wave_amd import inputs

pytestmark = pytest.mark.gpu
TOL_BF16 = 1e-2
EPS = float(np.float32(1e-6))     # the library takes eps as a float32


def _case(T, d, E, k, F, seed, **over):
    c = dict(inputs.CONFIGS["hy3_block_decode_T64"], T=T, d=d, E=E, k=k, F=F, seed=seed)
    c.update(over)
    return inputs.make_inputs(c, device="cpu")


def _gpu(inp):
    return {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}


def _oracle_block(inp, norm=True, sbias=True, tokens=None):
    c = inp["cfg"]
    args = (inputs.bits(inp["W_gate"]), _lazy_or_bits(inp["W_gu"]), _lazy_or_bits(inp["W_dn"]),
            inputs.bits(inp["Ws_gu"]), inputs.bits(inp["Ws_dn"]), c["k"], inp["scale"])
    kw = dict(norm_w_bits=inputs.bits(inp["norm_w"]) if norm else None, eps=EPS,
              score_bias=inputs.bits(inp["score_bias"]) if sbias else None)
    x_bits = inputs.bits(inp["x"])
    if tokens is None:
        return oracle.forward_block(x_bits, *args, **kw)
    return oracle.forward_block_tokens(tokens, x_bits, *args, **kw)


def _lazy_or_bits(t):
    return LazyExperts(t) if t.is_cuda else inputs.bits(t)


def _oracle_route(inp, norm=True, sbias=True):
    c = inp["cfg"]
    x_bits = inputs.bits(inp["x"])
    if norm:
        x_bits = oracle.rms_norm_bf16(x_bits, inputs.bits(inp["norm_w"]), EPS)
    return oracle.route(x_bits, inputs.bits(inp["W_gate"]), c["k"], inp["scale"],
                        score_bias=inputs.bits(inp["score_bias"]) if sbias else None)


def _run_block(inp, norm=True, sbias=True):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = inp["cfg"]
    torch.cuda.synchronize()
    out, idx, w = hy.block_forward(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], inp["Ws_gu"],
                                   inp["Ws_dn"], c["k"], inp["scale"],
                                   norm_weight=inp["norm_w"] if norm else None, norm_eps=EPS,
                                   score_bias=inp["score_bias"] if sbias else None,
                                   return_routing=True)
    torch.cuda.synchronize()
    return out, idx, w


def _flips(inp, r):
    """The flip model of the block (the shared expert as slot k)."""
    return bf16_flip_model(inputs.bits(inp["x"]), r, _lazy_or_bits(inp["W_gu"]), _lazy_or_bits(inp["W_dn"]),
                           inputs.bits(inp["Ws_gu"]), inputs.bits(inp["Ws_dn"]))


def _compare_full(inp_cpu, norm=True, sbias=True):
    out, idx, w = _run_block(_gpu(inp_cpu), norm, sbias)
    ref, r = _oracle_block(inp_cpu, norm, sbias)
    idx_np = idx.cpu().numpy()
    stats = check_routing(idx_np, w.cpu().numpy(), r, inp_cpu["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, set_equal(idx_np, r), TOL_BF16,
                                    **_flips(inp_cpu, r)))
    return stats


# ----------------------------------------------------------------------------- router

@pytest.mark.parametrize("norm,sbias", [(False, True), (True, False), (True, True)])
def test_route_ex_parity(gpu_lib, norm, sbias):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp_cpu = _case(700, 512, 48, 8, 128, seed=70)
    inp = _gpu(inp_cpu)
    c = inp["cfg"]
    idx, w = hy.route_ex(inp["x"], inp["W_gate"], c["k"], inp["scale"],
                         norm_weight=inp["norm_w"] if norm else None, norm_eps=EPS,
                         score_bias=inp["score_bias"] if sbias else None)
    torch.cuda.synchronize()
    r = _oracle_route(inp_cpu, norm, sbias)
    stats = check_routing(idx.cpu().numpy(), w.cpu().numpy(), r, inp_cpu["scale"])
    print(norm, sbias, stats)
    if sbias:
        # the bias really moves choices: differs from the unbiased selection
        r0 = _oracle_route(inp_cpu, norm, False)
        assert np.mean(np.any(r0.idx != r.idx, axis=1)) > 0.2


def test_route_ex_large_batch(gpu_lib):
    """4096 tokens or more: the LDS-staged logits kernel, here with route_norm
    and the score bias, a ragged last token tile and a partial expert group."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp_cpu = _case(4500, 256, 200, 8, 64, seed=77)
    inp = _gpu(inp_cpu)
    c = inp["cfg"]
    idx, w = hy.route_ex(inp["x"], inp["W_gate"], c["k"], inp["scale"], norm_weight=inp["norm_w"],
                         norm_eps=EPS, score_bias=inp["score_bias"])
    torch.cuda.synchronize()
    r = _oracle_route(inp_cpu, True, True)
    print(check_routing(idx.cpu().numpy(), w.cpu().numpy(), r, inp_cpu["scale"]))


def test_route_ex_negative_choice_values(gpu_lib):
    """A bias that makes most choice values negative still orders by value."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp_cpu = _case(300, 256, 40, 6, 64, seed=71)
    inp_cpu["score_bias"] = (torch.randn(40, generator=torch.Generator().manual_seed(5)) * 0.5
                             - 0.8).to(torch.float32)
    inp = _gpu(inp_cpu)
    idx, w = hy.route_ex(inp["x"], inp["W_gate"], 6, inp["scale"], score_bias=inp["score_bias"])
    torch.cuda.synchronize()
    r = _oracle_route(inp_cpu, norm=False, sbias=True)
    assert np.mean(r.choice < 0) > 0.5
    print(check_routing(idx.cpu().numpy(), w.cpu().numpy(), r, inp_cpu["scale"]))


# ----------------------------------------------------------------------------- block

def test_block_tiny_full_parity(gpu_lib):
    print(_compare_full(_case(128, 512, 32, 8, 128, seed=72)))


@pytest.mark.parametrize("T,k,E,F,norm,sbias", [
    (1, 8, 32, 128, True, True), (37, 8, 32, 128, True, False), (333, 4, 48, 192, False, True),
    (1000, 8, 32, 64, True, True), (130, 16, 64, 128, False, False), (520, 2, 24, 256, True, True)])
def test_block_ragged_and_small_shapes(gpu_lib, T, k, E, F, norm, sbias):
    print(T, k, E, F, _compare_full(_case(T, 512, E, k, F, seed=73 + T), norm, sbias))


@pytest.mark.parametrize("T", [16, 64])
def test_block_decode_path_shapes(gpu_lib, T):
    """T * k + 2 T <= 11 E (20 E with two row groups) with d, d_ff multiples
    of 128: the weight-streaming kernels, the shared expert as their last
    expert with all T rows."""
    print(T, _compare_full(_case(T, 1024, 192, 8, 256, seed=80 + T)))


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (16, 1, 1), (300, 1, 1), (4, 4, 4), (500, 4, 4)])
def test_block_degenerate_expert_counts(gpu_lib, T, k, E):
    """One routed expert and k = E beside the shared expert, with route_norm
    and the score bias, on the weight-streaming (T = 1 and T = 4: the shared
    expert's rows count twice, so T = 16 already takes the grouped GEMMs) and
    the grouped GEMMs, every token."""
    print(T, k, E, _compare_full(_case(T, 512, E, k, 256, seed=210 + T + E)))


def test_block_maximum_experts(gpu_lib):
    """E = 1023 routed experts plus the shared one: 1024 experts in the
    dispatch order, the most it takes."""
    print(_compare_full(_case(200, 256, 1023, 16, 64, seed=76)))


def test_block_zero_routed_experts_is_the_shared_expert(gpu_lib):
    inp_cpu = _case(200, 512, 32, 8, 128, seed=74)
    inp_cpu["W_gu"] = torch.zeros_like(inp_cpu["W_gu"])
    inp_cpu["W_dn"] = torch.zeros_like(inp_cpu["W_dn"])
    print(_compare_full(inp_cpu))
    # and the oracle's reference here is the dense shared SwiGLU alone
    ref, _ = _oracle_block(inp_cpu)
    dense = oracle.expert_swiglu(oracle.bf16_bits_to_f64(inputs.bits(inp_cpu["x"])),
                                 oracle.bf16_bits_to_f64(inputs.bits(inp_cpu["Ws_gu"])),
                                 oracle.bf16_bits_to_f64(inputs.bits(inp_cpu["Ws_dn"])))
    assert np.array_equal(ref, dense)


def test_block_deterministic(gpu_lib):
    inp = _gpu(_case(600, 512, 32, 8, 128, seed=75))
    a = _run_block(inp)
    b = _run_block(inp)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def _hy3_block_case(cfg):
    """Routing and every output element of a Hy3-sized block workload."""
    inp = inputs.make_inputs(cfg, device="cuda")
    out, idx, w = _run_block(inp)
    idx_np = idx.cpu().numpy()
    ref, r = _oracle_block(inp)
    stats = check_routing(idx_np, w.cpu().numpy(), r, inp["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, set_equal(idx_np, r), TOL_BF16, **_flips(inp, r)))
    return stats


def test_hy3_block_decode_T64(gpu_lib):
    print("block decode", _hy3_block_case("hy3_block_decode_T64"))


def test_hy3_block_prefill_T8192(gpu_lib):
    print("block prefill", _hy3_block_case("hy3_block_prefill_T8192"))


# ----------------------------------------------------------------------------- bf16 output + residual

@pytest.mark.parametrize("T,d,E,k,F", [(64, 512, 32, 8, 256), (300, 512, 32, 8, 128)],
                         ids=["decode-path", "grouped-path"])
def test_block_bf16_output_with_residual(gpu_lib, T, d, E, k, F):
    """hy3moe_block_forward_bf16 against the oracle's residual branch, and bit
    for bit against the fp32 block output plus the residual rounded once to
    bf16 (the fused combine does the same fp32 additions), also in place
    (out = residual) and with no residual."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = _case(T, d, E, k, F, seed=900 + T)
    res_cpu = inputs.make_residual(T, d, 900 + T)
    g = _gpu(inp)
    res = res_cpu.cuda()
    kw = dict(norm_weight=g["norm_w"], norm_eps=EPS, score_bias=g["score_bias"])
    args = (g["x"], g["W_gate"], g["W_gu"], g["W_dn"], g["Ws_gu"], g["Ws_dn"], k, inp["scale"])
    out, idx, w = hy.block_forward_bf16(*args, residual=res, return_routing=True, **kw)
    out32 = hy.block_forward(*args, **kw)
    plain = hy.block_forward_bf16(*args, **kw)
    inplace = res.clone()
    hy.block_forward_bf16(*args, residual=inplace, out=inplace, **kw)
    torch.cuda.synchronize()
    expect = (out32.cpu() + res_cpu.float()).to(torch.bfloat16)
    assert torch.equal(out.cpu().view(torch.int16), expect.view(torch.int16))
    assert torch.equal(inplace.cpu().view(torch.int16), expect.view(torch.int16))
    assert torch.equal(plain.cpu().view(torch.int16), out32.cpu().to(torch.bfloat16).view(torch.int16))

    x_bits = inputs.bits(inp["x"])
    ref, r = oracle.forward_block_residual(
        x_bits, inputs.bits(inp["W_gate"]), inputs.bits(inp["W_gu"]), inputs.bits(inp["W_dn"]),
        inputs.bits(inp["Ws_gu"]), inputs.bits(inp["Ws_dn"]), k, inp["scale"],
        norm_w_bits=inputs.bits(inp["norm_w"]), eps=EPS, score_bias=inputs.bits(inp["score_bias"]),
        residual_bits=inputs.bits(res_cpu))
    idx_np = idx.cpu().numpy()
    stats = check_routing(idx_np, w.cpu().numpy(), r, inp["scale"])
    # the output is rounded once to bf16: half a bf16 step of it is allowed on
    # top of the layer's 1e-2 * rms(ref) and its flips
    gpu = out.cpu().float().numpy().astype(np.float64)
    stats.update(check_output_flips(gpu, ref, set_equal(idx_np, r), TOL_BF16, out_bf16=True, **_flips(inp, r)))
    print(T, d, E, k, F, stats)


def test_hy3_block_residual_T8192(gpu_lib):
    """The bf16-output block with the residual at the Hy3 prefill size (the
    grouped kernels): every element against the oracle's residual branch, and
    bit for bit against the fp32 block output plus the residual rounded once
    to bf16."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = inputs.make_inputs("hy3_block_residual_T8192", device="cuda")
    c = inp["cfg"]
    k = c["k"]
    kw = dict(norm_weight=inp["norm_w"], norm_eps=EPS, score_bias=inp["score_bias"])
    args = (inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], inp["Ws_gu"], inp["Ws_dn"], k, inp["scale"])
    out, idx, w = hy.block_forward_bf16(*args, residual=inp["residual"], return_routing=True, **kw)
    out32 = hy.block_forward(*args, **kw)
    expect = (out32 + inp["residual"].float()).to(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), expect.view(torch.int16))
    del out32, expect
    blk, r = _oracle_block(inp)
    ref = blk + oracle.bf16_bits_to_f64(inputs.bits(inp["residual"]))
    del blk
    idx_np = idx.cpu().numpy()
    stats = check_routing(idx_np, w.cpu().numpy(), r, inp["scale"])
    gpu = out.float().cpu().numpy().astype(np.float64)
    stats.update(check_output_flips(gpu, ref, set_equal(idx_np, r), TOL_BF16, out_bf16=True, **_flips(inp, r)))
    print("block residual prefill", stats)
