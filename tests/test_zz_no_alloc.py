"""hy3moe_forward_noalloc (the library's static scratch instead of a caller
workspace) against hy3moe_forward (a caller workspace), through the C ABI:
bit for bit, output and routing, on two calls in a row with the second on a
smaller batch (the scratch keeps the first call's contents), on the
weight-streaming path (Hy3 decode sizes) and on the grouped-GEMM path."""

import pytest
import torch

from sparse_moe_layer_wave_amd import inputs

pytestmark = pytest.mark.gpu


def _same(inp, T):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = inp["cfg"]
    x = inp["x"][:T].contiguous()
    args = (x, inp["W_gate"], inp["W_gu"], inp["W_dn"], c["k"], inp["scale"])
    ref = hy.forward(*args, bias=inp["bias"], return_routing=True)
    got = hy.forward_noalloc(*args, bias=inp["bias"], return_routing=True)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    return got[0]


@pytest.mark.parametrize("cfg,T1,T2", [("hy3_decode_T64", 64, 16),
                                       (dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=1000, seed=31), 1000, 300),
                                       ("hy3_skewed_decode_T64", 64, 40)],
                         ids=["hy3-decode", "grouped", "hy3-skewed-decode"])
def test_noalloc_matches_forward(gpu_lib, cfg, T1, T2):
    inp = inputs.make_inputs(cfg, device="cuda")
    big = _same(inp, T1)
    small = _same(inp, T2)
    assert big.shape[0] == T1 and small.shape[0] == T2
    assert torch.isfinite(small).all()


def test_noalloc_rejects_sizes_beyond_its_scratch(gpu_lib):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = inputs.make_inputs(dict(inputs.CONFIGS["hy3_decode_T64"], T=700), device="cuda")
    c = inp["cfg"]
    with pytest.raises(hy.Hy3MoeError, match="static scratch"):
        hy.forward_noalloc(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], c["k"], inp["scale"])
