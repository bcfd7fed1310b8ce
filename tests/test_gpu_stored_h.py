"""The premises of the output check (parity.check_output_flips), on the
GPU's own intermediate values:
* the SwiGLU activation h the layer stores in bf16 lands on the other bf16
  neighbour than the oracle's rounding only where the oracle's h lies within
  the check's stated distance of a bf16 rounding boundary;
* with e4m3 experts, a stored activation code differs from the oracle's only
  where the check lets it flip, and a row scale only where the check lets
  the row's largest value flip;
* each stored expert output y differs from the oracle's bf16 rounding by no
  more than the check's per-slot y_allowance: nothing where y lies farther
  than D from a bf16 boundary, else D plus one bf16 step.
h, y and the row map are read back from the caller's workspace; the
workspace carving is mirrored here and must reproduce hy3moe_workspace_size,
so a change of the library's layout fails these tests instead of misreading
them."""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs
from parity import ETA_H, ETA_HA, ETA_HQ, bf16_boundary, e4m3_flip_flags, slot_flip_terms, y_allowance
from sparse_moe_layer_wave_amd import inputs

pytestmark = pytest.mark.gpu


def _align(v):
    return (v + 255) // 256 * 256


def _offsets(T, d, E, k, F, fp8, nsplit):
    """Byte offsets of the forward's workspace regions (routed experts only,
    no route_norm), in the order the library carves them."""
    R, nb = T * k, (T + 63) // 64
    regions = [("planes", 3 * E * d * 2), ("partial", nsplit * T * E * 4 if nsplit > 1 else 0),
               ("scores", T * E * 4), ("xn", 0), ("blk_counts", E * nb * 4), ("blk_base", E * nb * 4),
               ("counts", E * 4), ("offsets", (E + 2) * 4), ("tile_off", (E + 2) * 4), ("idx", R * 4),
               ("w", R * 4), ("row_of", R * 4), ("tok_of", R * 4)]
    if fp8:
        regions += [("h", R * F * 2), ("hq", R * F), ("hs", R * 4), ("amax", R * ((F + 127) // 128) * 4),
                    ("xq", T * d), ("xs", T * 4)]
    else:
        regions += [("h", R * F * 2)]
    regions += [("y", R * d * 2), ("sched", 16 * 4)]
    off, at = 0, {}
    for name, size in regions:
        at[name] = off
        off = _align(off + size)
    at["total"] = off
    return at


def _layout(T, d, E, k, F, fp8):
    from sparse_moe_layer_wave_amd import hy3moe
    total = hy3moe.workspace_size(T, d, E, k, F, hy3moe.WEIGHTS_FP8_E4M3 if fp8 else hy3moe.WEIGHTS_BF16)
    found = [_offsets(T, d, E, k, F, fp8, ns) for ns in (1, 2, 4, 8, 16, 32)]
    found = [L for L in found if L["total"] == total]
    assert len(found) == 1, "the mirrored workspace layout does not reproduce hy3moe_workspace_size"
    return found[0]


def _stored(ws, L, T, k, F, d):
    """The stored h [T, k, F] and y [T, k, d] of each (token, slot), as float64."""
    R = T * k
    row_of = ws[L["row_of"]:L["row_of"] + R * 4].cpu().numpy().view(np.int32).reshape(-1)
    h = ws[L["h"]:L["h"] + R * F * 2].cpu().numpy().view(np.uint16).reshape(R, F)
    y = ws[L["y"]:L["y"] + R * d * 2].cpu().numpy().view(np.uint16).reshape(R, d)
    return (codecs.bf16_bits_to_f64(h[row_of]).reshape(T, k, F),
            codecs.bf16_bits_to_f64(y[row_of]).reshape(T, k, d))


def _check_y(gpu_y, det, W_dn_of, fp8):
    """Each stored y element lies within the check's y_allowance of the
    oracle's bf16 rounding."""
    n_other = 0
    for ti, j, C, D in slot_flip_terms(det, W_dn_of, fp8):
        y = det.y[ti, j]
        diff = np.abs(gpu_y[ti, j] - codecs.round_to_bf16(y))
        allow = y_allowance(y, D)
        bad = diff > allow * (1 + 1e-9)
        assert not bad.any(), (f"{int(bad.sum())} stored y values beyond the per-slot allowance "
                               f"(worst excess {float((diff - allow)[bad].max()):.3e})")
        n_other += int((diff > 0).sum())
    return n_other


def _stored_codes(ws, L, T, k, F):
    """The stored e4m3 codes [T, k, F] and row scales [T, k] of h."""
    R = T * k
    row_of = ws[L["row_of"]:L["row_of"] + R * 4].cpu().numpy().view(np.int32).reshape(-1)
    q = ws[L["hq"]:L["hq"] + R * F].cpu().numpy().reshape(R, F)
    s = ws[L["hs"]:L["hs"] + R * 4].cpu().numpy().view(np.float32)
    return q[row_of].reshape(T, k, F), s[row_of].reshape(T, k)


def _check_codes(gpu_q, gpu_s, det):
    flag, rflag, _ = e4m3_flip_flags(det.h.reshape(-1, det.h.shape[2]), det.scaled.reshape(-1, det.h.shape[2]))
    q_ref = codecs.f32_to_e4m3_bits(det.scaled)
    other_q = (gpu_q != q_ref).reshape(flag.shape)
    other_s = (gpu_s != det.s_a).reshape(-1, 1)
    assert not (other_q & ~flag).any(), f"{int((other_q & ~flag).sum())} codes differ where no flip was allowed"
    assert not (other_s & ~rflag).any(), f"{int((other_s & ~rflag).sum())} row scales differ where none may"
    return int(other_q.sum()), int(other_s.sum())


def _check(gpu_h, det_h, fp8):
    """Every element whose stored bf16 value differs from the oracle's
    rounding lies within the check's margin of a bf16 boundary."""
    hmax = np.max(np.abs(det_h), axis=2, keepdims=True)
    dist, step = bf16_boundary(det_h)
    other = gpu_h != codecs.round_to_bf16(det_h)
    if fp8:
        inside = dist <= ETA_HQ * hmax
    else:
        inside = (dist <= ETA_H * step) | (dist <= ETA_HA * hmax)
    bad = other & ~inside
    assert not bad.any(), (f"{int(bad.sum())} stored h values on the other bf16 neighbour outside the margin "
                           f"(farthest {float(np.max((dist / hmax)[bad])):.3e} of the row's largest |h|)")
    return int(other.sum())


def test_stored_h_bf16_grouped(gpu_lib):
    """bf16 experts at Hy3 dims, T=512 (the grouped GEMMs)."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    T, d, E, k, F = 512, 4096, 192, 8, 1536
    c = dict(inputs.CONFIGS["hy3_prefill_T8192"], T=T, seed=4242)
    inp = inputs.make_inputs(c, device="cpu")
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    L = _layout(T, d, E, k, F, fp8=False)
    ws = hy.alloc_workspace(T, d, E, k, F, hy.WEIGHTS_BF16)
    _, idx, _ = hy.forward(dev["x"], dev["W_gate"], dev["W_gu"], dev["W_dn"], k, inp["scale"], bias=dev["bias"],
                           return_routing=True, workspace=ws)
    torch.cuda.synchronize()
    xb = inputs.bits(inp["x"])
    r = oracle.route(xb, inp["W_gate"].numpy(), k, inp["scale"],
                     None if inp["bias"] is None else inp["bias"].numpy())
    assert np.array_equal(idx.cpu().numpy(), r.idx)
    det = oracle.forward_detail(np.arange(T), xb, r, inputs.bits(inp["W_gu"]), inputs.bits(inp["W_dn"]))
    gh, gy = _stored(ws, L, T, k, F, d)
    n = _check(gh, det.h, fp8=False)
    W_dn = inputs.bits(inp["W_dn"])
    ny = _check_y(gy, det, lambda e: oracle.bf16_bits_to_f64(W_dn[e]), fp8=False)
    print("bf16: stored h on the other neighbour:", n, "; y off the oracle's rounding:", ny)


@pytest.mark.parametrize("case", ["per_channel_decode", "block128_grouped"])
def test_stored_h_e4m3(gpu_lib, case):
    """e4m3 experts: per-channel scales at Hy3 dims, T=128 (weight-streaming
    GEMMs), and 128 x 128 block scales on 393 tokens (grouped GEMMs)."""
    from sparse_moe_layer_wave_amd import hy3moe as hy
    if case == "per_channel_decode":
        T, d, E, k, F = 128, 4096, 192, 8, 1536
        c = dict(inputs.CONFIGS["hy3_fp8_T8192"], T=T, seed=4243)
    else:
        T, d, E, k, F = 393, 512, 31, 2, 256
        c = dict(inputs.CONFIGS["hy3_fp8_block128_decode_T64"], T=T, d=d, E=E, k=k, F=F, seed=800 + T)
    inp = inputs.make_inputs(c, device="cpu")
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    L = _layout(T, d, E, k, F, fp8=True)
    ws = hy.alloc_workspace(T, d, E, k, F, hy.WEIGHTS_FP8_E4M3)
    _, idx, _ = hy.forward_fp8(dev["x"], dev["W_gate"], dev["Wq_gu"], dev["s_gu"], dev["Wq_dn"], dev["s_dn"], k,
                               inp["scale"], bias=dev["bias"], return_routing=True, workspace=ws,
                               block128=case == "block128_grouped")
    torch.cuda.synchronize()
    xb = inputs.bits(inp["x"])
    r = oracle.route(xb, inp["W_gate"].numpy(), k, inp["scale"],
                     None if inp["bias"] is None else inp["bias"].numpy())
    assert np.array_equal(idx.cpu().numpy(), r.idx)
    qdn, sdn = inputs.bits(inp["Wq_dn"]), inp["s_dn"].numpy()
    det = oracle.forward_fp8_detail(np.arange(T), xb, r, inputs.bits(inp["Wq_gu"]), inp["s_gu"].numpy(), qdn, sdn)
    gh, gy = _stored(ws, L, T, k, F, d)
    n = _check(gh, det.h, fp8=True)
    nq, ns = _check_codes(*_stored_codes(ws, L, T, k, F), det)
    ny = _check_y(gy, det, lambda e: oracle.dequant_e4m3(qdn[e], sdn[e]), fp8=True)
    print(case, ": stored h on the other neighbour:", n, "; codes / row scales differing:", nq, ns,
          "; y off the oracle's rounding:", ny)
