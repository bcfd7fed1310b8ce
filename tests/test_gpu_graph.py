"""HIP graph capture of the forward entry points: the library only enqueues
kernels on the caller's stream (no allocation, no memset, no host sync), so a
captured forward replays like an eager one.  Each replay is compared with the
eager result, with eager work and synchronisations between the replays."""

import pytest
import torch

from sparse_moe_layer_wave_amd import hy3moe as hy
from sparse_moe_layer_wave_amd import inputs

pytestmark = pytest.mark.gpu


def _replays_match(run, n=3):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = run().clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = run()
    for i in range(n):
        captured.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(captured, eager), f"replay {i} differs"
        junk = torch.randn(1 << 20, device="cuda")   # eager work between replays
        junk.mul_(2.0)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T,E,k,F", [(64, 32, 8, 128), (1000, 32, 8, 128)])
def test_forward_bf16_graph(gpu_lib, T, E, k, F):
    c = dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=T, E=E, k=k, F=F, seed=400 + T)
    inp = inputs.make_inputs(c, device="cuda")
    ws = hy.alloc_workspace(T, c["d"], E, k, F, hy.WEIGHTS_BF16)
    out = torch.empty((T, c["d"]), dtype=torch.float32, device="cuda")
    _replays_match(lambda: hy.forward(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], k, inp["scale"],
                                      out=out, workspace=ws))


def test_forward_fp8_graph(gpu_lib):
    c = dict(inputs.CONFIGS["hy3_fp8_T8192"], T=300, d=512, E=32, F=256, seed=410)
    inp = inputs.make_inputs(c, device="cuda")
    ws = hy.alloc_workspace(300, 512, 32, 8, 256, hy.WEIGHTS_FP8_E4M3)
    out = torch.empty((300, 512), dtype=torch.float32, device="cuda")
    _replays_match(lambda: hy.forward_fp8(inp["x"], inp["W_gate"], inp["Wq_gu"], inp["s_gu"], inp["Wq_dn"],
                                          inp["s_dn"], 8, inp["scale"], out=out, workspace=ws))


def test_block_forward_graph(gpu_lib):
    c = dict(inputs.CONFIGS["hy3_block_decode_T64"], T=64, d=512, E=32, F=128, seed=420)
    inp = inputs.make_inputs(c, device="cuda")
    ws = torch.empty(hy.block_workspace_size(64, 512, 32, 8, 128), dtype=torch.uint8, device="cuda")
    out = torch.empty((64, 512), dtype=torch.float32, device="cuda")
    _replays_match(lambda: hy.block_forward(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], inp["Ws_gu"],
                                            inp["Ws_dn"], 8, inp["scale"], norm_weight=inp["norm_w"],
                                            norm_eps=1e-6, score_bias=inp["score_bias"], out=out,
                                            workspace=ws))


@pytest.mark.parametrize("T", [40, 600], ids=["decode-kernels", "grouped-kernels"])
def test_forward_fp8_block128_graph(gpu_lib, T):
    c = dict(inputs.CONFIGS["hy3_fp8_block128_decode_T64"], T=T, d=512, E=32, F=256, seed=430 + T)
    inp = inputs.make_inputs(c, device="cuda")
    ws = hy.alloc_workspace(T, 512, 32, 8, 256, hy.WEIGHTS_FP8_E4M3)
    out = torch.empty((T, 512), dtype=torch.float32, device="cuda")
    _replays_match(lambda: hy.forward_fp8_block128(inp["x"], inp["W_gate"], inp["Wq_gu"], inp["s_gu"],
                                                   inp["Wq_dn"], inp["s_dn"], 8, inp["scale"], out=out,
                                                   workspace=ws))


def test_block_forward_bf16_graph(gpu_lib):
    c = dict(inputs.CONFIGS["hy3_block_decode_T64"], T=64, d=512, E=32, F=128, seed=440)
    inp = inputs.make_inputs(c, device="cuda")
    res = inputs.make_residual(64, 512, 440, device="cuda")
    ws = torch.empty(hy.block_workspace_size(64, 512, 32, 8, 128), dtype=torch.uint8, device="cuda")
    out = torch.empty((64, 512), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: hy.block_forward_bf16(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], inp["Ws_gu"],
                                                 inp["Ws_dn"], 8, inp["scale"], residual=res,
                                                 norm_weight=inp["norm_w"], norm_eps=1e-6,
                                                 score_bias=inp["score_bias"], out=out, workspace=ws))
