"""GPU parity of the e4m3 expert path (through the C ABI) against the oracle's
FP8 definition: the x row quantiser bit-exactly, the whole layer within
3e-2 * rms(ref) element by element on every token (check_output_flips: an
element may exceed the bound only by the e4m3 and bf16 rounding-boundary
flips the oracle's own values allow), on small cases and on the Hy3 FP8
workloads (prefill-sized grouped kernels and the decode-sized
weight-streaming ones)."""

import numpy as np
import pytest
import torch

import oracle
from parity import LazyExperts, check_output_flips, check_routing, fp8_flip_model, set_equal
from sparse_moe_layer_wave_amd import inputs

pytestmark = pytest.mark.gpu
TOL_FP8 = 3e-2


def test_quantize_rows_bit_exact(gpu_lib):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    g = torch.Generator().manual_seed(30)
    x = (torch.randn((300, 512), generator=g) * 3).to(torch.bfloat16)
    x[7] = 0                                            # zero row: codes 0, scale 1
    x[8, :] = x[8, :] * 1e-30                           # tiny values: subnormal codes
    x[9, 5] = 1e30                                      # one huge outlier
    q, s = hy.quantize_rows_e4m3(x.cuda())
    q_ref, s_ref = oracle.quant_rows_e4m3(inputs.bits(x.float().contiguous()))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)


def _cpu_fp8_case(T, E, k, F, d=512, seed=40):
    c = dict(inputs.CONFIGS["hy3_fp8_T8192"], T=T, d=d, E=E, k=k, F=F, seed=seed)
    return inputs.make_inputs(c, device="cpu")


def _compare_cpu_case(inp, out, idx, w):
    """Routing and every output element of a CPU-drawn e4m3 case against the
    oracle (per-channel or block scales: the oracle's dequantisation reads
    the scale array's shape)."""
    c = inp["cfg"]
    args = (inputs.bits(inp["Wq_gu"]), inp["s_gu"].numpy(), inputs.bits(inp["Wq_dn"]), inp["s_dn"].numpy())
    x_bits = inputs.bits(inp["x"])
    ref, r = oracle.forward_fp8(x_bits, inp["W_gate"].numpy(), *args, c["k"], inp["scale"])
    idx = idx.cpu().numpy()
    stats = check_routing(idx, w.cpu().numpy(), r, inp["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, set_equal(idx, r), TOL_FP8,
                                    **fp8_flip_model(x_bits, r, *args)))
    return stats


def _run_fp8(inp):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = inp["cfg"]
    dev = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    out, idx, w = hy.forward_fp8(dev["x"], dev["W_gate"], dev["Wq_gu"], dev["s_gu"], dev["Wq_dn"],
                                 dev["s_dn"], c["k"], inp["scale"], bias=dev["bias"],
                                 return_routing=True)
    torch.cuda.synchronize()
    return out, idx, w


@pytest.mark.parametrize("T,E,k,F", [(128, 32, 8, 128), (37, 32, 8, 256), (1, 16, 4, 128),
                                     (700, 48, 8, 128)])
def test_fp8_small_full_parity(gpu_lib, T, E, k, F):
    inp = _cpu_fp8_case(T, E, k, F)
    out, idx, w = _run_fp8(inp)
    stats = _compare_cpu_case(inp, out, idx, w)
    print(T, E, k, F, stats)


@pytest.mark.parametrize("T,E,k,F,d", [(16, 64, 8, 256, 512), (64, 192, 8, 256, 256),
                                       (5, 24, 4, 512, 1024), (1, 8, 2, 256, 256),
                                       (12, 32, 8, 384, 512), (56, 24, 8, 256, 512)])
def test_fp8_decode_path_full_parity(gpu_lib, T, E, k, F, d):
    """T * k <= 11 E (20 E with two row groups) with d, d_ff multiples of 256: the e4m3 weight-streaming
    kernels (the fifth case, d_ff = 384, takes the grouped kernels instead;
    the last, 19 rows per expert, two 16-row groups per pass)."""
    inp = _cpu_fp8_case(T, E, k, F, d=d, seed=42 + T)
    out, idx, w = _run_fp8(inp)
    stats = _compare_cpu_case(inp, out, idx, w)
    print(T, E, k, F, d, stats)


@pytest.mark.parametrize("block128", [False, True], ids=["per_channel", "block128"])
@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (16, 1, 1), (300, 1, 1), (16, 4, 4), (500, 4, 4)])
def test_fp8_degenerate_expert_counts(gpu_lib, T, k, E, block128):
    """One expert and k = E with e4m3 experts, on the weight-streaming (T <= 16)
    and the grouped GEMMs, every token."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = dict(inputs.CONFIGS["hy3_fp8_block128_decode_T64" if block128 else "hy3_fp8_T8192"], T=T, d=512, E=E, k=k, F=256, seed=190 + T + E)
    inp = inputs.make_inputs(c, device="cpu")
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    out, idx, w = hy.forward_fp8(dev["x"], dev["W_gate"], dev["Wq_gu"], dev["s_gu"], dev["Wq_dn"], dev["s_dn"],
                                 k, inp["scale"], bias=dev["bias"], return_routing=True, block128=block128)
    torch.cuda.synchronize()
    assert all(sorted(row) == list(range(E)) for row in idx.cpu().numpy().tolist())
    print(T, k, E, block128, _compare_cpu_case(inp, out, idx, w))


def test_fp8_deterministic(gpu_lib):
    inp = _cpu_fp8_case(500, 32, 8, 128, seed=41)
    a = _run_fp8(inp)
    b = _run_fp8(inp)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("cfg", ["hy3_fp8_T8192", "hy3_fp8_decode_T64", "hy3_fp8_block128_decode_T64",
                                 "hy3_fp8_block128_T8192"])
def test_hy3_fp8(gpu_lib, cfg):
    """Per-channel and 128 x 128 block scales, at T=8192 and T=64,
    every token."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = inputs.make_inputs(cfg, device="cuda")
    c = inp["cfg"]
    out, idx, w = hy.forward_fp8(inp["x"], inp["W_gate"], inp["Wq_gu"], inp["s_gu"], inp["Wq_dn"],
                                 inp["s_dn"], c["k"], inp["scale"], return_routing=True,
                                 block128=c["weights"] == "fp8_block128")
    torch.cuda.synchronize()
    x_bits = inputs.bits(inp["x"])
    W = inputs.bits(inp["W_gate"])
    args = tuple(LazyExperts(inp[n]) for n in ("Wq_gu", "s_gu", "Wq_dn", "s_dn"))
    ref, r = oracle.forward_fp8(x_bits, W, *args, c["k"], inp["scale"])
    idx_np = idx.cpu().numpy()
    stats = check_routing(idx_np, w.cpu().numpy(), r, inp["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, set_equal(idx_np, r), TOL_FP8,
                                    **fp8_flip_model(x_bits, r, *args)))
    print("fp8", inp["cfg"]["name"], stats)


# ----------------------------------------------------------------------------- 128 x 128 block scales

def _cpu_fp8_block_case(T, E, k, F, d, seed):
    c = dict(inputs.CONFIGS["hy3_fp8_block128_decode_T64"], T=T, d=d, E=E, k=k, F=F, seed=seed)
    return inputs.make_inputs(c, device="cpu")


@pytest.mark.parametrize("T,E,k,F,d", [(16, 64, 8, 256, 512), (1, 8, 2, 256, 256), (56, 24, 8, 256, 512),
                                       (300, 32, 8, 256, 512), (700, 48, 4, 512, 768),
                                       (129, 16, 16, 256, 1024), (50, 1000, 4, 256, 256),
                                       (3000, 1000, 2, 256, 256)])
def test_fp8_block128_full_parity(gpu_lib, T, E, k, F, d):
    """hy3moe_forward_fp8_block128 on every token: decode-sized batches (the
    weight-streaming kernels, one and two row groups) and larger ones (the
    128 x 128 grouped kernels), d up to 8 k-blocks, k = 16, and 1000 experts
    on both paths."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = _cpu_fp8_block_case(T, E, k, F, d, seed=60 + T)
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    out, idx, w = hy.forward_fp8_block128(dev["x"], dev["W_gate"], dev["Wq_gu"], dev["s_gu"], dev["Wq_dn"],
                                          dev["s_dn"], k, inp["scale"], return_routing=True)
    torch.cuda.synchronize()
    stats = _compare_cpu_case(inp, out, idx, w)
    print(T, E, k, F, d, stats)


def test_fp8_block128_uses_the_block_scales(gpu_lib):
    """Scaling one 128 x 128 block of one expert's down matrix by 2 doubles
    exactly that block's contribution: with a power-of-two factor every
    product and partial sum scales exactly, so the output changes only in the
    block's 128 output channels, for the tokens routed to that expert."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = _cpu_fp8_block_case(40, 16, 4, 256, 512, seed=71)
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    args = (dev["x"], dev["W_gate"], dev["Wq_gu"], dev["s_gu"], dev["Wq_dn"])
    out, idx, _ = hy.forward_fp8_block128(*args, dev["s_dn"], 4, inp["scale"], return_routing=True)
    s2 = dev["s_dn"].clone()
    s2[3, 1, :] *= 2.0                                  # expert 3, output channels 128..255, all k
    out2 = hy.forward_fp8_block128(*args, s2, 4, inp["scale"])
    torch.cuda.synchronize()
    a, b = out.cpu().numpy(), out2.cpu().numpy()
    hit = (idx.cpu().numpy() == 3).any(axis=1)
    assert hit.any() and not hit.all()
    assert np.array_equal(a[~hit], b[~hit])
    assert np.array_equal(a[:, :128], b[:, :128]) and np.array_equal(a[:, 256:], b[:, 256:])
    assert np.any(a[hit, 128:256] != b[hit, 128:256])
