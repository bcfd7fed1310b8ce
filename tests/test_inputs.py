"""Checks of the seeded input generator: shapes, dtypes, determinism and the
distributions the workloads specify; the skewed workload's load ratio under
the oracle's router."""

import numpy as np
import pytest
import torch

import oracle
from sparse_moe_layer_wave_amd import inputs


def test_tiny_config_shapes_and_determinism():
    a = inputs.make_inputs("tiny_T128_d512_E32_F128")
    b = inputs.make_inputs("tiny_T128_d512_E32_F128")
    c = a["cfg"]
    assert a["x"].shape == (c["T"], c["d"]) and a["x"].dtype == torch.bfloat16
    assert a["W_gate"].shape == (c["E"], c["d"]) and a["W_gate"].dtype == torch.float32
    assert a["W_gu"].shape == (c["E"], 2 * c["F"], c["d"])
    assert a["W_dn"].shape == (c["E"], c["d"], c["F"])
    for key in ("x", "W_gate", "W_gu", "W_dn"):
        assert torch.equal(a[key], b[key])
    assert a["bias"] is None


def test_workloads_are_looked_up_by_name():
    """Each workload's key is its name; seeds are distinct, so no two
    workloads draw the same inputs; a bare number is refused."""
    assert all(k == c["name"] for k, c in inputs.CONFIGS.items())
    seeds = [c["seed"] for c in inputs.CONFIGS.values()]
    assert len(set(seeds)) == len(seeds)
    with pytest.raises(TypeError):
        inputs.make_inputs(0)


def test_distributions():
    a = inputs.make_inputs("tiny_T128_d512_E32_F128")
    c = a["cfg"]
    assert abs(a["x"].float().std().item() - 1.0) < 0.02
    assert abs(a["W_gate"].std().item() * np.sqrt(c["d"]) - 1.0) < 0.03
    assert abs(a["W_gu"].float().std().item() - 0.02) < 0.001
    assert abs(a["W_dn"].float().std().item() - 0.02) < 0.001


def test_fp8_weights_have_per_row_scales():
    c = dict(inputs.CONFIGS["hy3_fp8_T8192"], T=8, d=128, E=4, F=64)
    a = inputs.make_inputs(c)
    q = a["Wq_gu"].view(torch.float8_e4m3fn).float()
    assert a["Wq_gu"].dtype == torch.uint8 and a["s_gu"].shape == (4, 128)
    assert torch.all(q.abs().amax(dim=2) == 448.0)
    assert abs((q * a["s_gu"][..., None]).std().item() - 0.02) < 0.002


def test_skew_bias_gives_about_15x_hottest_load():
    c = inputs.CONFIGS["hy3_long_skewed_T65536"]
    T = 2048
    x = inputs.bits(inputs.make_x(T, c["d"], c["seed"] + 100, "cpu"))
    W, b = inputs.make_router(c["E"], c["d"], c["seed"], "cpu", skew=True)
    r = oracle.route(x, W.numpy(), c["k"], inputs.ROUTER_SCALE, b.numpy())
    load = np.bincount(r.idx.reshape(-1), minlength=c["E"])
    ratio = load.max() / (T * c["k"] / c["E"])
    assert 12.5 < ratio < 17.5
