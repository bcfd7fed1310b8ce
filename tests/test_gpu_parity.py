"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small cases (the tiny workload and ragged/edge variants) are drawn on the CPU,
the Hy3-sized workloads on the GPU.  Routing is compared on every token, the
dispatch order against a stable sort of the GPU's own routing, and outputs
element by element on every token (check_output_flips) -- except the
65536-token skewed workload, whose outputs are compared on a stratified
sample: the first and last token of every 128-row block of every expert in
the GEMMs' row order."""

import numpy as np
import pytest
import torch

import oracle
from parity import (LazyExperts, bf16_flip_model, check_output_flips, check_permutation,
                    check_routing, set_equal, stratified_tokens)
from sparse_moe_layer_wave_amd import inputs

pytestmark = pytest.mark.gpu
TOL_BF16 = 1e-2


def _to(dev, d):
    return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in d.items()}


def _cpu_case(cfg, T=None, **over):
    c = dict(inputs.CONFIGS[cfg] if not isinstance(cfg, dict) else cfg)
    c.update(over)
    return inputs.make_inputs(c, device="cpu", T=T)


def _run_bf16(hy, inp):
    c = inp["cfg"]
    torch.cuda.synchronize()
    out, idx, w = hy.forward(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], c["k"], inp["scale"],
                             bias=inp["bias"], return_routing=True)
    torch.cuda.synchronize()
    return out, idx, w


def _oracle_bf16(inp_cpu):
    c = inp_cpu["cfg"]
    b = None if inp_cpu["bias"] is None else inp_cpu["bias"].numpy()
    return oracle.forward(inputs.bits(inp_cpu["x"]), inp_cpu["W_gate"].numpy(),
                          inputs.bits(inp_cpu["W_gu"]), inputs.bits(inp_cpu["W_dn"]), c["k"],
                          inp_cpu["scale"], b)


def _flip_model(inp_cpu, r):
    return bf16_flip_model(inputs.bits(inp_cpu["x"]), r, inputs.bits(inp_cpu["W_gu"]), inputs.bits(inp_cpu["W_dn"]))


def _full_compare(inp_cpu, tol=TOL_BF16):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = _to("cuda", inp_cpu)
    out, idx, w = _run_bf16(hy, inp)
    ref, r = _oracle_bf16(inp_cpu)
    stats = check_routing(idx.cpu().numpy(), w.cpu().numpy(), r, inp_cpu["scale"])
    stats.update(check_output_flips(out.cpu().numpy(), ref, set_equal(idx.cpu().numpy(), r), tol,
                                    **_flip_model(inp_cpu, r)))
    return stats, inp, idx


def test_tiny_workload_full_parity(gpu_lib):
    stats, inp, idx = _full_compare(_cpu_case("tiny_T128_d512_E32_F128"))
    print("tiny", stats)
    from sparse_moe_layer_wave_amd import hy3moe as hy
    counts, offsets, row_of, token_of = hy.permute(idx, inp["cfg"]["E"])
    check_permutation(idx.cpu().numpy(), inp["cfg"]["E"], counts.cpu().numpy(),
                      offsets.cpu().numpy(), row_of.cpu().numpy(), token_of.cpu().numpy())


@pytest.mark.parametrize("T,k,E,F", [(1, 8, 32, 128), (37, 8, 32, 128), (200, 1, 32, 128),
                                     (333, 4, 48, 192), (1000, 8, 32, 64), (130, 16, 64, 128)])
def test_ragged_and_small_shapes(gpu_lib, T, k, E, F):
    c = dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=T, k=k, E=E, F=F, seed=100 + T)
    stats, _, _ = _full_compare(_cpu_case(c))
    print(T, k, E, F, stats)


@pytest.mark.parametrize("T,k,E,F,d", [(300, 16, 1024, 64, 256), (64, 16, 1024, 128, 128),
                                       (70000, 2, 8, 64, 64)])
def test_maximum_sizes(gpu_lib, T, k, E, F, d):
    """The largest expert count and k the library takes (E = 1024, k = 16; the
    second case on the decode-path kernels), and more tokens than the largest
    workload with ~17,500 rows per expert (full 8-block chunks of the grouped
    GEMMs' work order).  Every token is compared; with k = 2 the weights are
    near 1.4, so a rounding-boundary flip of a large |y| is above 1e-2 * rms
    and the flip check has work to do there."""
    c = dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=T, k=k, E=E, F=F, d=d, seed=150 + k)
    stats, _, _ = _full_compare(_cpu_case(c))
    print(T, k, E, F, d, stats)


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (16, 1, 1), (300, 1, 1), (16, 4, 4), (500, 4, 4)])
def test_degenerate_expert_counts(gpu_lib, T, k, E):
    """One expert (every token's only slot, weight 2.826) and k = E (every
    token takes every expert, in score order), each on the weight-streaming
    (small T) and the grouped (larger T) GEMMs; every token compared."""
    c = dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=T, k=k, E=E, seed=170 + T + E)
    stats, _, idx = _full_compare(_cpu_case(c))
    idx = idx.cpu().numpy()
    assert all(sorted(row) == list(range(E)) for row in idx.tolist())
    print(T, k, E, stats)


def test_route_entry_matches_forward_routing(gpu_lib):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = _to("cuda", _cpu_case("tiny_T128_d512_E32_F128", T=300, seed=7))
    c = inp["cfg"]
    idx_r, w_r = hy.route(inp["x"], inp["W_gate"], c["k"], inp["scale"])
    _, idx_f, w_f = _run_bf16(hy, inp)
    assert torch.equal(idx_r, idx_f) and torch.equal(w_r, w_f)


@pytest.mark.parametrize("T,E,k,d", [(5000, 200, 8, 320), (4096, 1024, 16, 128), (4100, 7, 3, 64)])
def test_router_large_batch_shapes(gpu_lib, T, E, k, d):
    """Batches of 4096 tokens or more take the LDS-staged logits kernel:
    token tiles of 256 with a ragged last one, expert groups of 192 with a
    partial last one (E = 200, 1024) or a single short one (E = 7)."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=T, E=E, k=k, d=d, F=64, seed=300 + E)
    inp_cpu = _cpu_case(c)
    inp = _to("cuda", inp_cpu)
    idx, w = hy.route(inp["x"], inp["W_gate"], k, inp["scale"])
    torch.cuda.synchronize()
    r = oracle.route(inputs.bits(inp_cpu["x"]), inp_cpu["W_gate"].numpy(), k, inp_cpu["scale"], None)
    print(T, E, k, d, check_routing(idx.cpu().numpy(), w.cpu().numpy(), r, inp_cpu["scale"]))


def test_zero_tokens_tie_to_lowest_experts(gpu_lib):
    inp = _cpu_case("tiny_T128_d512_E32_F128", T=64, seed=8)
    inp["x"][5] = 0
    inp["x"][40] = 0
    stats, _, idx = _full_compare(inp)
    i = idx.cpu().numpy()
    assert i[5].tolist() == list(range(8)) and i[40].tolist() == list(range(8))


def test_duplicated_gate_rows_lower_index_wins(gpu_lib):
    inp = _cpu_case("tiny_T128_d512_E32_F128", T=256, seed=9)
    inp["W_gate"][17] = inp["W_gate"][4]
    stats, _, idx = _full_compare(inp)
    for row in idx.cpu().numpy().tolist():
        if 17 in row:
            assert 4 in row and row.index(4) == row.index(17) - 1


def test_all_tokens_one_expert(gpu_lib):
    """Maximum skew: a large logit bias sends every token to expert 5 first."""
    inp = _cpu_case("tiny_T128_d512_E32_F128", T=500, seed=10)
    b = torch.zeros(inp["cfg"]["E"], dtype=torch.float32)
    b[5] = 30.0
    inp["bias"] = b
    stats, _, idx = _full_compare(inp)
    assert torch.all(idx[:, 0] == 5)


@pytest.mark.parametrize("T,E,k,hot", [(64, 192, 8, True), (96, 192, 8, False), (16, 32, 8, True),
                                       (3, 40, 5, False), (56, 24, 8, False), (56, 24, 8, True),
                                       (40, 16, 4, False), (24, 32, 8, False)])
def test_decode_path_shapes(gpu_lib, T, E, k, hot):
    """Small batches take the weight-streaming kernels: T*k <= 11E with one
    16-row group per pass, and, where experts average 5 or more rows
    (T*k >= 5E with bf16 weights), T*k <= 20E with two groups (32-row slices;
    the last four cases, the second with a 56-row hot expert cut into two
    slices, the last at 6 rows per expert).  A hot expert with more rows than
    a slice is cut into several slices."""
    c = dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=T, E=E, k=k, F=128, seed=200 + T)
    inp = _cpu_case(c)
    if hot:
        b = torch.zeros(E, dtype=torch.float32)
        b[E - 1] = 30.0
        inp["bias"] = b
    stats, _, idx = _full_compare(inp)
    print(T, E, k, hot, stats)


def test_empty_batch(gpu_lib):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = _to("cuda", _cpu_case("tiny_T128_d512_E32_F128", T=0))
    out = hy.forward(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], 8, inp["scale"])
    assert out.shape == (0, 512)


def test_empty_batch_every_entry(gpu_lib):
    """T = 0 is a successful no-op on every entry point: nothing is launched and
    no output is written (outputs of fixed size, such as permute's counts, keep
    whatever they held), so only the shapes are checked."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    c = dict(inputs.CONFIGS["tiny_T128_d512_E32_F128"], T=0)
    inp = _to("cuda", _cpu_case(c))
    idx, w = hy.route(inp["x"], inp["W_gate"], 8, inp["scale"])
    assert idx.shape == (0, 8) and w.shape == (0, 8)
    counts, offsets, row_of, token_of = hy.permute(idx, c["E"])
    assert counts.shape == (c["E"],) and offsets.shape == (c["E"] + 1,)
    assert row_of.numel() == 0 and token_of.numel() == 0
    blk = inputs.make_inputs(dict(inputs.CONFIGS["hy3_block_decode_T64"], T=0, d=512, E=32, F=128), device="cuda")
    idx, w = hy.route_ex(blk["x"], blk["W_gate"], 8, blk["scale"], norm_weight=blk["norm_w"],
                         score_bias=blk["score_bias"])
    assert idx.shape == (0, 8)
    out = hy.block_forward(blk["x"], blk["W_gate"], blk["W_gu"], blk["W_dn"], blk["Ws_gu"], blk["Ws_dn"], 8,
                           blk["scale"], norm_weight=blk["norm_w"], score_bias=blk["score_bias"])
    assert out.shape == (0, 512)
    f8 = inputs.make_inputs(dict(inputs.CONFIGS["hy3_fp8_T8192"], T=0, d=512, E=32, F=256), device="cuda")
    out = hy.forward_fp8(f8["x"], f8["W_gate"], f8["Wq_gu"], f8["s_gu"], f8["Wq_dn"], f8["s_dn"], 8, f8["scale"])
    assert out.shape == (0, 512)
    torch.cuda.synchronize()


def test_deterministic(gpu_lib):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = _to("cuda", _cpu_case("tiny_T128_d512_E32_F128", T=777, seed=11))
    a = _run_bf16(hy, inp)
    b = _run_bf16(hy, inp)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("T,E,k", [(40, 24, 6), (700, 200, 8), (3000, 1024, 16)])
def test_permute_drops_bad_pairs(gpu_lib, T, E, k):
    """A caller's routing with entries outside [0, E) (negative, E, large) and
    experts repeated within a token's row: those pairs take no row, the rest
    keep the stable expert order (one routing block, and several)."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    bad = rng.random((T, k)) < 0.1
    idx[bad] = rng.choice(np.array([-1, -7, E, E + 5, 1 << 30, -(1 << 31)], np.int64), int(bad.sum()))
    rep = np.nonzero(rng.random(T) < 0.1)[0]
    idx[rep, k - 1] = idx[rep, 0]
    counts, offsets, row_of, token_of = hy.permute(torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    check_permutation(idx, E, counts.cpu().numpy(), offsets.cpu().numpy(), row_of.cpu().numpy(),
                      token_of.cpu().numpy())
    assert (row_of.cpu().numpy() < 0).sum() >= bad.sum()


def test_permute_entry_on_random_routing(gpu_lib):
    from sparse_moe_layer_wave_amd import hy3moe as hy
    rng = np.random.default_rng(12)
    for T, E, k in [(1, 8, 3), (64, 192, 8), (65, 192, 8), (5000, 192, 8), (3000, 1024, 16)]:
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, row_of, token_of = hy.permute(torch.from_numpy(idx).cuda(), E)
        check_permutation(idx, E, counts.cpu().numpy(), offsets.cpu().numpy(),
                          row_of.cpu().numpy(), token_of.cpu().numpy())


# ----------------------------------------------------------------------------- Hy3 sizes

def _hy3_case(cfg):
    """A Hy3-sized workload: routing and the dispatch order on every token;
    outputs on every token up to 8192 tokens, else on the stratified sample."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    inp = inputs.make_inputs(cfg, device="cuda")
    c = inp["cfg"]
    T = c["T"]
    out, idx, w = _run_bf16(hy, inp)
    x_bits = inputs.bits(inp["x"])
    W = inputs.bits(inp["W_gate"])
    b = None if inp["bias"] is None else inputs.bits(inp["bias"])
    r = oracle.route(x_bits, W, c["k"], inp["scale"], b)
    idx_np = idx.cpu().numpy()
    stats = check_routing(idx_np, w.cpu().numpy(), r, inp["scale"])
    counts, offsets, row_of, token_of = hy.permute(idx, c["E"])
    check_permutation(idx_np, c["E"], counts.cpu().numpy(), offsets.cpu().numpy(),
                      row_of.cpu().numpy(), token_of.cpu().numpy())
    sample = np.arange(T) if T <= 8192 else stratified_tokens(idx_np, c["E"])
    gu, dn = LazyExperts(inp["W_gu"]), LazyExperts(inp["W_dn"])
    xs = x_bits[sample]
    ref, rs = oracle.forward(xs, W, gu, dn, c["k"], inp["scale"], b)
    stats.update(check_output_flips(out.cpu().numpy()[sample], ref, set_equal(idx_np[sample], rs), TOL_BF16,
                                    **bf16_flip_model(xs, rs, gu, dn)))
    load = np.bincount(idx_np.reshape(-1), minlength=c["E"])
    stats.update(compared=int(len(sample)), experts_touched=int((load > 0).sum()),
                 hottest_over_mean=float(load.max() / load.mean()))
    return stats


def test_hy3_decode_T64(gpu_lib):
    print("decode", _hy3_case("hy3_decode_T64"))


def test_hy3_skewed_decode_T64(gpu_lib):
    """Decode batch with the skewed routing: hot experts get tens of rows,
    each cut into several 16-row slices of the weight-streaming kernels."""
    stats = _hy3_case("hy3_skewed_decode_T64")
    print("skewed decode", stats)
    assert stats["hottest_over_mean"] > 8


def test_hy3_prefill_T8192(gpu_lib):
    print("prefill", _hy3_case("hy3_prefill_T8192"))


def test_hy3_long_skewed_T65536(gpu_lib):
    stats = _hy3_case("hy3_long_skewed_T65536")
    print("skewed", stats)
    assert stats["hottest_over_mean"] > 10 and stats["compared"] > 4000
