"""Seeded synthetic inputs shaped like one Hy3 MoE layer.

This module only draws random tensors; it holds none of the layer's
arithmetic, and both the HIP path's tests/bench and the CPU oracle's checks
take their inputs from it.

Distributions (the second parameter of N(.,.) is a standard deviation):
  x       bf16  [T, d]        N(0, 1), rounded to bf16
  W_gate  fp32  [E, d]        N(0, 1/sqrt(d))  -> logits ~ N(0, 1)
  W_gu    bf16  [E, 2F, d]    N(0, 0.02)       (rows [0,F) gate, [F,2F) up)
  W_dn    bf16  [E, d, F]     N(0, 0.02)
  bias    fp32  [E]           skewed workload only: b_e = -tau * ln(rank_e), rank a
                              seeded permutation of 1..E, added to the logits
FP8 workload: W_gu / W_dn drawn as above in fp32, then per output row
(= per output channel) scale s = amax/448 and codes e4m3(w / s) via torch's
cast; the codes and the fp32 scales are the layer's inputs.
Block-128 FP8 workload: the same fp32 draws, one scale s = amax/448 per
128 x 128 block of each weight matrix instead of per row.
Full-block workloads add:
  norm_w      bf16  [d]       1 + N(0, 0.1)    route_norm weight
  score_bias  fp32  [E]       N(0, 0.05)       selection-only score bias (moves
                              a scale of score gaps, so it changes choices)
  Ws_gu       bf16  [2F, d]   N(0, 0.02)       shared expert
  Ws_dn       bf16  [d, F]    N(0, 0.02)
  residual    bf16  [T, d]    N(0, 1)          residual stream of the bf16-output
                              block (make_residual; drawn only when asked for)

Values depend on the device the generator runs on (torch's CPU and GPU
generators differ): tests draw small cases on the CPU and copy them over, and
draw the full-size workloads on the GPU and copy what the oracle needs back.
"""

import math

import numpy as np
import torch

ROUTER_SCALE = float(np.float32(2.826))   # router_scaling_factor, as a float32 value

# tau of the skewed workload's logit bias.  Fitted (bisection on the oracle's
# router over an 8192-token sample) so the most loaded expert receives about
# 15x the mean load; the fit is tests/golden/fit_skew_tau.py.
SKEW_TAU = 0.5467

# Seeded workloads by name: T, d, E, k, d_ff, seed, expert weight format,
# skewed routing.  The seed is a field of its own, so a workload's inputs do
# not depend on where it stands in this table.
_WORKLOADS = (
    dict(name="tiny_T128_d512_E32_F128", T=128, d=512, E=32, k=8, F=128, seed=0,
         weights="bf16", skew=False),
    dict(name="hy3_decode_T64", T=64, d=4096, E=192, k=8, F=1536, seed=1,
         weights="bf16", skew=False),
    dict(name="hy3_prefill_T8192", T=8192, d=4096, E=192, k=8, F=1536, seed=2,
         weights="bf16", skew=False),
    dict(name="hy3_long_skewed_T65536", T=65536, d=4096, E=192, k=8, F=1536, seed=3,
         weights="bf16", skew=True),
    dict(name="hy3_fp8_T8192", T=8192, d=4096, E=192, k=8, F=1536, seed=4,
         weights="fp8", skew=False),
    # the full block (shared expert, route_norm, selection-only score bias)
    dict(name="hy3_block_decode_T64", T=64, d=4096, E=192, k=8, F=1536, seed=5,
         weights="bf16", skew=False, block=True),
    dict(name="hy3_block_prefill_T8192", T=8192, d=4096, E=192, k=8, F=1536, seed=6,
         weights="bf16", skew=False, block=True),
    # e4m3 experts at the decode batch
    dict(name="hy3_fp8_decode_T64", T=64, d=4096, E=192, k=8, F=1536, seed=7,
         weights="fp8", skew=False),
    # the skewed routing of hy3_long_skewed_T65536 at the decode batch (hot experts get
    # tens of rows)
    dict(name="hy3_skewed_decode_T64", T=64, d=4096, E=192, k=8, F=1536, seed=8,
         weights="bf16", skew=True),
    # e4m3 experts with one scale per 128 x 128 weight block
    dict(name="hy3_fp8_block128_decode_T64", T=64, d=4096, E=192, k=8, F=1536, seed=9,
         weights="fp8_block128", skew=False),
    dict(name="hy3_fp8_block128_T8192", T=8192, d=4096, E=192, k=8, F=1536, seed=10,
         weights="fp8_block128", skew=False),
    # the full block ending the residual branch: bf16 output, residual added
    dict(name="hy3_block_residual_T8192", T=8192, d=4096, E=192, k=8, F=1536, seed=11,
         weights="bf16", skew=False, block=True, residual=True),
)
CONFIGS = {c["name"]: c for c in _WORKLOADS}

(_STREAM_X, _STREAM_WG, _STREAM_BIAS, _STREAM_WGU, _STREAM_WDN, _STREAM_NORM, _STREAM_SBIAS,
 _STREAM_SGU, _STREAM_SDN, _STREAM_RESID) = range(10)


def _gen(device, seed, stream):
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (seed + 1) + 7919 * stream)
    return g


def make_x(T, d, seed, device="cpu"):
    g = _gen(device, seed, _STREAM_X)
    return torch.randn((T, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_residual(T, d, seed, device="cpu"):
    """The decoder layer's residual stream for the bf16-output block."""
    g = _gen(device, seed, _STREAM_RESID)
    return torch.randn((T, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_router(E, d, seed, device="cpu", skew=False):
    g = _gen(device, seed, _STREAM_WG)
    W = torch.randn((E, d), generator=g, device=device, dtype=torch.float32) * (1.0 / math.sqrt(d))
    bias = None
    if skew:
        gb = _gen("cpu", seed, _STREAM_BIAS)
        rank = torch.randperm(E, generator=gb).to(torch.float64) + 1.0
        bias = (-SKEW_TAU * torch.log(rank)).to(torch.float32).to(device)
    return W.contiguous(), bias


def _expert_fp32(rows, cols, g, device):
    return torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * 0.02


def make_experts_bf16(E, d, F, seed, device="cpu"):
    gu = torch.empty((E, 2 * F, d), dtype=torch.bfloat16, device=device)
    dn = torch.empty((E, d, F), dtype=torch.bfloat16, device=device)
    g1 = _gen(device, seed, _STREAM_WGU)
    g2 = _gen(device, seed, _STREAM_WDN)
    for e in range(E):
        gu[e] = _expert_fp32(2 * F, d, g1, device).to(torch.bfloat16)
        dn[e] = _expert_fp32(d, F, g2, device).to(torch.bfloat16)
    return gu, dn


def _per_row_e4m3(w):
    amax = w.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (w / s[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s.to(torch.float32)


def make_experts_fp8(E, d, F, seed, device="cpu"):
    qgu = torch.empty((E, 2 * F, d), dtype=torch.uint8, device=device)
    sgu = torch.empty((E, 2 * F), dtype=torch.float32, device=device)
    qdn = torch.empty((E, d, F), dtype=torch.uint8, device=device)
    sdn = torch.empty((E, d), dtype=torch.float32, device=device)
    g1 = _gen(device, seed, _STREAM_WGU)
    g2 = _gen(device, seed, _STREAM_WDN)
    for e in range(E):
        qgu[e], sgu[e] = _per_row_e4m3(_expert_fp32(2 * F, d, g1, device))
        qdn[e], sdn[e] = _per_row_e4m3(_expert_fp32(d, F, g2, device))
    return qgu, sgu, qdn, sdn


def _block128_e4m3(w):
    """One fp32 scale per 128 x 128 block: s = amax / 448 (1 for an all-zero
    block), codes e4m3(w / s) via torch's cast."""
    R, C = w.shape
    b = w.reshape(R // 128, 128, C // 128, 128)
    amax = b.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (b / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.reshape(R, C).view(torch.uint8), s.to(torch.float32)


def make_experts_fp8_block128(E, d, F, seed, device="cpu"):
    """The fp8 workload's fp32 expert weights (same draws), quantised in
    128 x 128 blocks: codes [E,2F,d] / [E,d,F], scales [E,2F/128,d/128] /
    [E,d/128,F/128]."""
    qgu = torch.empty((E, 2 * F, d), dtype=torch.uint8, device=device)
    sgu = torch.empty((E, 2 * F // 128, d // 128), dtype=torch.float32, device=device)
    qdn = torch.empty((E, d, F), dtype=torch.uint8, device=device)
    sdn = torch.empty((E, d // 128, F // 128), dtype=torch.float32, device=device)
    g1 = _gen(device, seed, _STREAM_WGU)
    g2 = _gen(device, seed, _STREAM_WDN)
    for e in range(E):
        qgu[e], sgu[e] = _block128_e4m3(_expert_fp32(2 * F, d, g1, device))
        qdn[e], sdn[e] = _block128_e4m3(_expert_fp32(d, F, g2, device))
    return qgu, sgu, qdn, sdn


def make_block_extras(d, E, F, seed, device="cpu"):
    """route_norm weight, selection-only score bias and shared expert weights."""
    gn = _gen(device, seed, _STREAM_NORM)
    norm_w = (1.0 + 0.1 * torch.randn(d, generator=gn, device=device)).to(torch.bfloat16)
    gs = _gen(device, seed, _STREAM_SBIAS)
    score_bias = (0.05 * torch.randn(E, generator=gs, device=device)).to(torch.float32)
    g1 = _gen(device, seed, _STREAM_SGU)
    g2 = _gen(device, seed, _STREAM_SDN)
    Ws_gu = _expert_fp32(2 * F, d, g1, device).to(torch.bfloat16)
    Ws_dn = _expert_fp32(d, F, g2, device).to(torch.bfloat16)
    return dict(norm_w=norm_w.contiguous(), score_bias=score_bias.contiguous(),
                Ws_gu=Ws_gu.contiguous(), Ws_dn=Ws_dn.contiguous())


def make_inputs(cfg, device="cpu", T=None, with_experts=True):
    """All inputs of one workload as torch tensors on ``device``.

    ``cfg`` is a workload name (a CONFIGS key) or a dict with the same
    fields; ``T`` overrides
    the token count (the rows are the first T rows the seed would give only if
    the generator's draw order allows it -- treat each T as its own input)."""
    if not isinstance(cfg, (str, dict)):
        raise TypeError(f"workload must be a name or a dict, not {cfg!r}")
    c = dict(CONFIGS[cfg]) if isinstance(cfg, str) else dict(cfg)
    if T is not None:
        c["T"] = T
    out = dict(cfg=c, scale=ROUTER_SCALE)
    out["x"] = make_x(c["T"], c["d"], c["seed"], device)
    out["W_gate"], out["bias"] = make_router(c["E"], c["d"], c["seed"], device, c.get("skew", False))
    if with_experts:
        if c.get("weights", "bf16") == "fp8_block128":
            out["Wq_gu"], out["s_gu"], out["Wq_dn"], out["s_dn"] = make_experts_fp8_block128(
                c["E"], c["d"], c["F"], c["seed"], device)
        elif c.get("weights", "bf16") == "fp8":
            out["Wq_gu"], out["s_gu"], out["Wq_dn"], out["s_dn"] = make_experts_fp8(
                c["E"], c["d"], c["F"], c["seed"], device)
        else:
            out["W_gu"], out["W_dn"] = make_experts_bf16(c["E"], c["d"], c["F"], c["seed"], device)
    if c.get("block", False):
        out.update(make_block_extras(c["d"], c["E"], c["F"], c["seed"], device))
    if c.get("residual", False):
        out["residual"] = make_residual(c["T"], c["d"], c["seed"], device)
    return out


def bits(t):
    """A bf16/uint8 tensor's bit patterns as a host NumPy array (uint16/uint8);
    float tensors come back as float32 arrays."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.cpu().to(torch.float32).numpy()
