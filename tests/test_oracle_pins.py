"""Pins of the MoE oracle against what the pages print and what mathematics
fixes: printed parameter/FLOP counts, the weight-sum invariant, brute-force
subset enumeration, reductions to a dense MLP computed with torch, the tie
rule, monotonicity (sigmoid vs softmax vs logits) and symmetries."""

import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")
SCALE = float(np.float32(2.826))


def _rand_layer(rng, T, d, E, F, w_std=0.02):
    x = codecs.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    Wgu = codecs.f32_to_bf16_bits((rng.standard_normal((E, 2 * F, d)) * w_std).astype(np.float32))
    Wdn = codecs.f32_to_bf16_bits((rng.standard_normal((E, d, F)) * w_std).astype(np.float32))
    return x, Wg, Wgu, Wdn


def _torch_swiglu(x64, Wgu64, Wdn64):
    """Dense SwiGLU with torch's own silu and matmul, float64."""
    x = torch.from_numpy(x64)
    F = Wdn64.shape[1]
    g = x @ torch.from_numpy(Wgu64[:F]).T
    u = x @ torch.from_numpy(Wgu64[F:]).T
    return ((Fn.silu(g) * u) @ torch.from_numpy(Wdn64).T).numpy()


def _sig(printed_value, digits):
    return float(f"{printed_value:.{digits}g}")


# ----------------------------------------------------------------------------- printed figures

def test_page_printed_parameter_and_flop_counts():
    g = json.load(open(GOLDEN))
    d, F, E, k, L = 4096, 1536, 192, 8, 79
    per_expert = oracle.expert_param_count(d, F)
    assert per_expert == 18_874_368
    assert _sig(per_expert, g["expert_params"]["digits"]) == g["expert_params"]["value"]
    assert _sig(2 * F * d, 4) == g["expert_gate_up_params"]["value"]
    assert _sig(d * F, 3) == g["expert_down_params"]["value"]
    assert _sig(E * per_expert, 3) == g["routed_experts_per_layer_params"]["value"]
    assert _sig(E * d, 2) == g["router_params"]["value"]
    layer = (E + 1) * per_expert + E * d               # routed + shared expert + gate
    assert _sig(layer, 3) == g["moe_layer_params_with_shared"]["value"]
    # 79 layers of (192 routed + 1 shared expert + gate) = 287,839,617,024
    assert _sig(L * layer, g["moe_all_layers_params"]["digits"] + 1) == g["moe_all_layers_params"]["value"]
    # FLOPs: one expert per token, and nine experts (8 routed + 1 shared)
    per_expert_flops = oracle.flops_per_token(d, F, 1, E) - 2 * d * E
    assert per_expert_flops == 6 * d * F == 37_748_736
    assert _sig(per_expert_flops, 3) == g["flops_per_expert_per_token"]["value"]
    assert _sig(9 * per_expert_flops, 3) == g["flops_nine_experts_per_token"]["value"]
    assert oracle.flops_per_token(d, F, k, E) == 303_562_752


def test_weights_sum_to_scale_and_mean_weight():
    g = json.load(open(GOLDEN))
    rng = np.random.default_rng(3)
    x, Wg, _, _ = _rand_layer(rng, 512, 256, 192, 8)
    r = oracle.route(x, Wg, 8, SCALE)
    assert np.max(np.abs(r.w.sum(axis=1) - SCALE)) < 1e-12
    assert round(SCALE, 3) == g["routing_weight_sum"]["value"]
    assert round(SCALE / 8, 3) == g["mean_routing_weight"]["value"]
    assert np.all(r.w > 0)


def test_exactly_k_distinct_experts():
    rng = np.random.default_rng(4)
    x, Wg, _, _ = _rand_layer(rng, 300, 64, 40, 8)
    for k in (1, 2, 8, 39, 40):
        r = oracle.route(x, Wg, k, SCALE)
        assert r.idx.shape == (300, k)
        assert np.all((r.idx >= 0) & (r.idx < 40))
        assert all(len(set(row)) == k for row in r.idx.tolist())


# ----------------------------------------------------------------------------- brute force

def _brute_force_set(s32_row, k):
    """The subset of size k with the largest exact score sum; among equal
    sums, the lexicographically smallest index tuple."""
    fr = [Fraction(float(v)) for v in s32_row]
    best, best_set = None, None
    for sub in itertools.combinations(range(len(fr)), k):
        tot = sum(fr[i] for i in sub)
        if best is None or tot > best:
            best, best_set = tot, sub
    return best_set


@pytest.mark.parametrize("E,k,d,F,T", [(10, 3, 16, 8, 12), (16, 8, 16, 8, 6)])
def test_brute_force_subsets(E, k, d, F, T):
    rng = np.random.default_rng(5 + E)
    x, Wg, Wgu, Wdn = _rand_layer(rng, T, d, E, F, w_std=0.2)
    out, r = oracle.forward(x, Wg, Wgu, Wdn, k, SCALE, bf16_activations=False)
    x64 = codecs.bf16_bits_to_f64(x)
    logits = torch.from_numpy(x64) @ torch.from_numpy(Wg.astype(np.float64)).T
    s32 = torch.sigmoid(logits).numpy().astype(np.float32)
    assert np.array_equal(s32, r.scores)
    for t in range(T):
        best = _brute_force_set(s32[t], k)
        assert set(r.idx[t].tolist()) == set(best)
        # slot order: scores never increase along the slots
        sel = s32[t, r.idx[t]]
        assert np.all(sel[:-1] >= sel[1:])
        # output recomputed from the brute-force subset with torch's dense SwiGLU
        sel_sum = sum(float(s32[t, e]) for e in best)
        ref = np.zeros(d)
        for e in best:
            y = _torch_swiglu(x64[t:t + 1], codecs.bf16_bits_to_f64(Wgu[e]), codecs.bf16_bits_to_f64(Wdn[e]))
            ref += SCALE * float(s32[t, e]) / sel_sum * y[0]
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------- reductions

def test_identical_experts_reduce_to_dense_swiglu():
    rng = np.random.default_rng(6)
    T, d, E, F = 40, 64, 12, 16
    x, Wg, Wgu, Wdn = _rand_layer(rng, T, d, E, F)
    Wgu[:] = Wgu[0]
    Wdn[:] = Wdn[0]
    out, _ = oracle.forward(x, Wg, Wgu, Wdn, 4, SCALE, bf16_activations=False)
    x64 = codecs.bf16_bits_to_f64(x)
    Wgu0, Wdn0 = codecs.bf16_bits_to_f64(Wgu[0]), codecs.bf16_bits_to_f64(Wdn[0])
    ref = SCALE * _torch_swiglu(x64, Wgu0, Wdn0)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    # with bf16 activations: h and y rounded once, the weights still sum to scale
    out_b, _ = oracle.forward(x, Wg, Wgu, Wdn, 4, SCALE)
    F = Wdn0.shape[1]
    g = torch.from_numpy(x64) @ torch.from_numpy(Wgu0[:F]).T
    u = torch.from_numpy(x64) @ torch.from_numpy(Wgu0[F:]).T
    h = codecs.round_to_bf16((Fn.silu(g) * u).numpy())
    y = codecs.round_to_bf16((torch.from_numpy(h) @ torch.from_numpy(Wdn0).T).numpy())
    np.testing.assert_allclose(out_b, SCALE * y, rtol=1e-12, atol=1e-15)


def test_k1_is_scaled_argmax_expert():
    rng = np.random.default_rng(7)
    T, d, E, F = 30, 32, 9, 8
    x, Wg, Wgu, Wdn = _rand_layer(rng, T, d, E, F)
    out, r = oracle.forward(x, Wg, Wgu, Wdn, 1, SCALE, bf16_activations=False)
    x64 = codecs.bf16_bits_to_f64(x)
    logits = torch.from_numpy(x64) @ torch.from_numpy(Wg.astype(np.float64)).T
    top = torch.argmax(logits, dim=1).numpy()
    assert np.array_equal(r.idx[:, 0], top)
    assert np.allclose(r.w[:, 0], SCALE, rtol=0, atol=1e-15)
    for t in range(T):
        e = top[t]
        ref = SCALE * _torch_swiglu(x64[t:t + 1], codecs.bf16_bits_to_f64(Wgu[e]), codecs.bf16_bits_to_f64(Wdn[e]))
        np.testing.assert_allclose(out[t], ref[0], rtol=1e-12, atol=1e-15)


def test_k_equals_E_uses_every_expert():
    rng = np.random.default_rng(8)
    T, d, E, F = 10, 32, 6, 8
    x, Wg, Wgu, Wdn = _rand_layer(rng, T, d, E, F)
    out, r = oracle.forward(x, Wg, Wgu, Wdn, E, SCALE, bf16_activations=False)
    x64 = codecs.bf16_bits_to_f64(x)
    s = 1.0 / (1.0 + np.exp(-(x64 @ Wg.astype(np.float64).T)))
    s = s.astype(np.float32).astype(np.float64)
    ref = np.zeros((T, d))
    for e in range(E):
        ref += (SCALE * s[:, e] / s.sum(axis=1))[:, None] * _torch_swiglu(
            x64, codecs.bf16_bits_to_f64(Wgu[e]), codecs.bf16_bits_to_f64(Wdn[e]))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-15)
    assert not r.near_tie.any()


# ----------------------------------------------------------------------------- tie rule

def test_zero_token_ties_go_to_lower_index():
    rng = np.random.default_rng(9)
    T, d, E, F = 5, 32, 20, 8
    x, Wg, Wgu, Wdn = _rand_layer(rng, T, d, E, F)
    x[2] = 0                                   # every logit 0, every score exactly 0.5
    out, r = oracle.forward(x, Wg, Wgu, Wdn, 8, SCALE)
    assert r.idx[2].tolist() == list(range(8))
    assert np.all(r.w[2] == SCALE / 8)
    assert np.all(out[2] == 0)
    assert r.near_tie[2] and r.order_tie[2]


def test_duplicated_gate_rows_lower_index_wins():
    rng = np.random.default_rng(10)
    T, d, E = 50, 32, 16
    x, Wg, _, _ = _rand_layer(rng, T, d, E, 4)
    Wg[11] = Wg[3]                             # experts 3 and 11 always tie exactly
    r = oracle.route(x, Wg, 8, SCALE)
    for t in range(T):
        row = r.idx[t].tolist()
        if 11 in row:
            assert 3 in row and row.index(3) == row.index(11) - 1
        assert r.scores[t, 3] == r.scores[t, 11]


def test_near_tie_flag():
    x = codecs.f32_to_bf16_bits(np.float32([[1.0, 0.0]]))
    # experts 0..2 far apart; 3 and 4 differ by a hair at the k/k+1 boundary (k=4)
    Wg = np.float32([[5, 0], [4, 0], [3, 0], [0.25, 0], [0.25 - 1e-6, 0], [-3, 0]])
    r = oracle.route(x, Wg, 4, SCALE)
    assert r.idx[0].tolist() == [0, 1, 2, 3]
    assert r.near_tie[0] and 0 < r.gap[0] < oracle.NEAR_TIE
    r2 = oracle.route(x, Wg, 3, SCALE)
    assert not r2.near_tie[0] and not r2.order_tie[0]


# ----------------------------------------------------------------------------- monotonicity

def test_selection_matches_logit_and_softmax_topk_without_ties():
    rng = np.random.default_rng(11)
    x, Wg, _, _ = _rand_layer(rng, 400, 128, 48, 4)
    r = oracle.route(x, Wg, 8, SCALE)
    logits = torch.from_numpy(codecs.bf16_bits_to_f64(x)) @ torch.from_numpy(Wg.astype(np.float64)).T
    soft = torch.softmax(logits, dim=1)
    ok = ~r.order_tie
    assert ok.sum() > 390
    by_logit = torch.topk(logits, 8, dim=1).indices.numpy()
    by_soft = torch.topk(soft, 8, dim=1).indices.numpy()
    assert np.array_equal(r.idx[ok], by_logit[ok])
    assert np.array_equal(r.idx[ok], by_soft[ok])


def test_sigmoid_scores_match_library():
    from scipy.special import expit
    rng = np.random.default_rng(12)
    x, Wg, _, _ = _rand_layer(rng, 64, 64, 16, 4)
    b = rng.standard_normal(16).astype(np.float32)
    r = oracle.route(x, Wg, 4, SCALE, logit_bias=b)
    logits = codecs.bf16_bits_to_f64(x) @ Wg.astype(np.float64).T + b.astype(np.float64)
    assert np.array_equal(r.scores, expit(logits).astype(np.float32))


def test_logit_bias_shifts_selection():
    rng = np.random.default_rng(13)
    x, Wg, _, _ = _rand_layer(rng, 200, 64, 16, 4)
    b = np.zeros(16, np.float32)
    b[5] = 40.0                                # expert 5 wins everywhere
    r = oracle.route(x, Wg, 4, SCALE, logit_bias=b)
    assert np.all(r.idx[:, 0] == 5)


# ----------------------------------------------------------------------------- symmetries

def test_token_permutation_equivariance():
    rng = np.random.default_rng(14)
    T, d, E, F = 64, 64, 16, 16
    x, Wg, Wgu, Wdn = _rand_layer(rng, T, d, E, F)
    out, r = oracle.forward(x, Wg, Wgu, Wdn, 4, SCALE)
    perm = rng.permutation(T)
    out_p, r_p = oracle.forward(x[perm], Wg, Wgu, Wdn, 4, SCALE)
    assert np.array_equal(r_p.idx, r.idx[perm])
    np.testing.assert_array_equal(out_p, out[perm])


def test_expert_relabelling_invariance():
    rng = np.random.default_rng(15)
    T, d, E, F = 48, 64, 16, 16
    x, Wg, Wgu, Wdn = _rand_layer(rng, T, d, E, F)
    out, r = oracle.forward(x, Wg, Wgu, Wdn, 4, SCALE)
    perm = rng.permutation(E)                  # new expert i is old expert perm[i]
    inv = np.argsort(perm)
    out_p, r_p = oracle.forward(x, Wg[perm], Wgu[perm], Wdn[perm], 4, SCALE)
    ok = ~r.order_tie
    assert np.array_equal(r_p.idx[ok], inv[r.idx[ok]])
    np.testing.assert_allclose(out_p, out, rtol=1e-12, atol=1e-15)


def test_forward_tokens_equals_rows_of_forward():
    rng = np.random.default_rng(16)
    x, Wg, Wgu, Wdn = _rand_layer(rng, 40, 64, 16, 16)
    out, _ = oracle.forward(x, Wg, Wgu, Wdn, 4, SCALE)
    sub = np.array([3, 17, 0, 39])
    out_s, _ = oracle.forward_tokens(sub, x, Wg, Wgu, Wdn, 4, SCALE)
    np.testing.assert_allclose(out_s, out[sub], rtol=1e-13, atol=1e-16)


def test_empty_batch():
    rng = np.random.default_rng(17)
    x, Wg, Wgu, Wdn = _rand_layer(rng, 0, 32, 8, 8)
    out, r = oracle.forward(x, Wg, Wgu, Wdn, 4, SCALE)
    assert out.shape == (0, 32) and r.idx.shape == (0, 4)
