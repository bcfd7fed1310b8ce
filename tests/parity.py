"""Comparison helpers shared by the GPU parity tests (routing, permutation,
outputs).  The tolerances and their reasons:

* routing indices: bit-exact, except tokens the oracle flags -- a k-th/(k+1)-th
  score gap below 1e-6 may change the chosen set, and any adjacent gap below
  1e-6 among the first k+1 may change the slot order.  The GPU's fp32 logits
  differ from the oracle's float64 ones by a few 1e-7 (fp32 accumulation over
  d terms), which moves a score by at most a quarter of that.
* routing weights: |dw| <= 1e-5 * scale (the same score error divided by a
  sum of k scores, plus fp32 rounding of the division and scaling).
* outputs: |out_gpu - out_ref| <= tol * rms(out_ref) element by element,
  tol = 1e-2 with bf16 experts and 3e-2 with e4m3 experts, over the tokens
  whose chosen expert set equals the oracle's -- except where a stored
  activation sits so close to a rounding boundary that the GPU's float32 value
  may round to the other neighbour (check_output_flips).
"""

import numpy as np


def check_routing(idx_gpu, w_gpu, r, scale):
    idx_gpu = np.asarray(idx_gpu, dtype=np.int64)
    w_gpu = np.asarray(w_gpu, dtype=np.float64)
    T = idx_gpu.shape[0]
    set_eq = np.array([set(a) == set(b) for a, b in zip(idx_gpu.tolist(), r.idx.tolist())],
                      dtype=bool) if T else np.zeros(0, bool)
    slot_eq = np.all(idx_gpu == r.idx, axis=1)
    bad_set = ~set_eq & ~r.near_tie
    bad_slot = ~slot_eq & ~r.order_tie
    assert not bad_set.any(), f"routing sets differ on unflagged tokens {np.nonzero(bad_set)[0][:10]}"
    assert not bad_slot.any(), f"slot order differs on unflagged tokens {np.nonzero(bad_slot)[0][:10]}"
    # every GPU row: k distinct experts in range, weights sum to scale
    assert np.all((idx_gpu >= 0) & (idx_gpu < r.scores.shape[1]))
    assert all(len(set(row)) == len(row) for row in idx_gpu.tolist())
    if T:
        assert np.max(np.abs(w_gpu.sum(axis=1) - scale)) < 1e-5 * scale
    dw = np.abs(w_gpu[slot_eq] - r.w[slot_eq])
    assert dw.size == 0 or dw.max() <= 1e-5 * scale, f"weights differ by {dw.max()}"
    return dict(tokens=T, near_tie=int(r.near_tie.sum()), set_diff=int((~set_eq).sum()),
                slot_diff=int((~slot_eq).sum()), max_dw=float(dw.max()) if dw.size else 0.0)


def expected_permutation(idx, E):
    """Stable counting sort of the (token, slot) pairs by expert, via NumPy's
    stable argsort: rows of one expert contiguous, ascending token inside.
    Pairs whose expert is outside [0, E) or repeats an expert earlier in the
    token's row are dropped (row -1, no token_of entry), as hy3moe_permute
    specifies for a caller's routing."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    ok = (idx >= 0) & (idx < E)
    for j in range(1, k):
        ok[:, j] &= ~np.any(idx[:, :j] == idx[:, j:j + 1], axis=1)
    flat = np.where(ok, idx, E).reshape(-1)
    n = int(ok.sum())
    order = np.argsort(flat, kind="stable")[:n]
    counts = np.bincount(flat[order], minlength=E)[:E]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    row_of = np.full(T * k, -1, dtype=np.int64)
    row_of[order] = np.arange(n)
    token_of = order // k
    return counts, offsets, row_of.reshape(T, k), token_of


def check_permutation(idx, E, counts, offsets, row_of, token_of):
    c, o, r, t = expected_permutation(idx, E)
    assert np.array_equal(np.asarray(counts), c)
    assert np.array_equal(np.asarray(offsets), o)
    assert np.array_equal(np.asarray(row_of), r)
    assert np.array_equal(np.asarray(token_of)[:len(t)], t)


class LazyExperts:
    """Expert weights left on the GPU; the oracle pulls each expert it needs
    (as host bit patterns) when it indexes this object."""

    def __init__(self, tensor):
        from sparse_moe_layer_wave_amd import inputs
        self._t = tensor
        self._bits = inputs.bits
        self.shape = tuple(tensor.shape)

    def __getitem__(self, e):
        return self._bits(self._t[int(e)])


# ----------------------------------------------------------------------------- rounding-boundary flips
#
# The layer stores three activations in narrow types, and the oracle rounds
# each where the layer does: h (bf16, or e4m3 with a row scale) and y (bf16).
# The GPU rounds its own float32 value of each, which differs from the
# oracle's float64 one in the last bits (other summation order, hardware
# exp2 / reciprocal).  Where the two fall on the two sides of a rounding
# boundary the stored values differ by one step, and with weights near 0.35
# one step of a large |y| is above 1e-2 * rms.  So an element may exceed the
# bound only by flips available to it, each predicted from the oracle's own
# pre-rounding values:
#
#   h (bf16 experts):  flippable if within ETA_H steps of a bf16 boundary, or
#       within ETA_HA * max|h of its row| (the float32 error of a small h
#       made of cancelling terms).  A flip moves y_c by |Wd[c, f]| * step.
#   h (e4m3):  h is rounded to bf16, and v = bf16(h) * r is quantised.  h's
#       bf16 rounding may flip within ETA_HQ * max|h of its row| of a bf16
#       boundary (the e4m3 path's error is absolute at its row's scale).  v
#       is flippable where h's bf16 rounding may flip and v lies within that
#       bf16 step (REL_BF16 * |v|) of an e4m3 boundary; every v of a row is,
#       where an element next to the row's maximum may flip (the row's scale
#       moves by up to REL_BF16, and y with it: REL_BF16 * |y_c|); and, for
#       the float32 arithmetic, within ETA_Q steps or ETA_QA * 448.  A code
#       flip moves y_c by |Wd[c, f]| * step * s_a.
#   y:  the GPU's float32 y may be off the oracle's pre-rounding y by D_c =
#       the h flips above + ETA_Y * sum_f |Wd[c, f] * h_f| (float32 sums of F
#       products and the scale multiplications).  Where y lies within D_c of
#       a bf16 boundary, the stored y may differ from the oracle's rounding by
#       up to D_c plus one bf16 step (D_c can span several steps when several
#       h values of the row may flip); elsewhere both round alike.  The
#       element may move by the weighted sum of that over its slots.
#
# The ETA values are chosen from the GPU's float32 error with margin: the
# gate and up sums over d terms carry about 2^-18 relative error, so h and v
# carry about 2^-17 relative, which is 2^-9 of a bf16 step (2^-8 relative)
# and 2^-13 of an e4m3 step (2^-4 relative) -- ETA_H and ETA_Q allow 2x and
# 8x that; the float32 sum of F exact products carries far less than
# ETA_Y = 2^-20 of the sum of the magnitudes of its terms.
ETA_H = 2.0 ** -8
ETA_HA = 2.0 ** -18
ETA_Q = 2.0 ** -10
ETA_QA = 2.0 ** -16
ETA_Y = 2.0 ** -20
REL_BF16 = 2.0 ** -7          # a bf16 step relative to the value, at most
ETA_HQ = ETA_Q * 32.0 / 448.0  # ETA_Q e4m3 steps at the row's largest v (448, step 32), relative to it


def bf16_boundary(v):
    """For float64 values: (distance to the nearest bf16 rounding boundary,
    the larger bf16 step on either side of that boundary)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    m, e = np.frexp(np.where(a > 0, a, 2.0 ** -126))
    step = np.ldexp(1.0, e - 8)                       # spacing of the binade [2^(e-1), 2^e)
    lo = np.floor(a / step) * step                    # the bf16 value at or below a
    at_pow2 = lo == np.ldexp(1.0, e - 1)
    below = np.where(at_pow2, step / 2, step)         # spacing just below lo
    dist = np.minimum(np.abs(a - (lo + step / 2)), np.abs(a - (lo - below / 2)))
    return dist, step


_E4M3_POS = None


def e4m3_boundary(v):
    """For float32 / float64 values on the e4m3 scale: (distance to the
    nearest e4m3 rounding boundary, the larger e4m3 step beside it).  Values
    beyond 448 saturate and have no boundary above."""
    global _E4M3_POS
    if _E4M3_POS is None:
        from oracle import codecs
        vals = codecs.e4m3_bits_to_f64(np.arange(0x7F, dtype=np.uint8))
        _E4M3_POS = np.unique(vals[np.isfinite(vals)])          # 0, 2^-9, ..., 448
    grid = _E4M3_POS
    a = np.abs(np.asarray(v, dtype=np.float64))
    i = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, len(grid) - 1)
    lo = grid[i]
    hi = grid[np.minimum(i + 1, len(grid) - 1)]
    prev = grid[np.maximum(i - 1, 0)]
    up = np.where(hi > lo, (lo + hi) / 2, np.inf)
    down = np.where(lo > prev, (prev + lo) / 2, -np.inf)
    dist = np.minimum(np.abs(a - up), np.abs(a - down))
    return dist, np.maximum(hi - lo, lo - prev)


def e4m3_flip_flags(h, scaled):
    """For e4m3 activation rows h [n, F] (the oracle's, before their bf16
    rounding) and the values the quantiser rounds, scaled [n, F]: (flag
    [n, F], where the GPU's code may differ from the oracle's; rflag [n, 1],
    where the GPU's row scale may differ; step [n, F], the e4m3 step beside
    each value)."""
    hd, _ = bf16_boundary(h)
    hmax = np.max(np.abs(h), axis=1, keepdims=True)
    hflag = hd <= ETA_HQ * hmax
    rflag = np.any(hflag & (np.abs(h) >= hmax * (1.0 - 2.0 ** -6)), axis=1, keepdims=True)
    v = np.asarray(scaled, dtype=np.float64)
    dist, step = e4m3_boundary(v)
    moved = (hflag.astype(np.float64) + rflag) * REL_BF16 * np.abs(v)
    flag = (dist <= ETA_Q * step) | (dist <= ETA_QA * 448.0) | (dist <= moved + ETA_Q * step)
    return flag, rflag, step


def slot_flip_terms(det, W_dn_of, fp8):
    """For each expert of the detail: (ti, j, C, D) with the (token, slot)
    pairs (ti, j) it serves, C [len(ti), d] the move of each expert output
    element through e4m3 code flips and row-scale moves (zero for bf16
    experts), and D [len(ti), d] how far the GPU's float32 y may lie from the
    oracle's before its bf16 rounding.  W_dn_of(e) gives expert e's down
    matrix as float64 [d, F] (e = -1: the shared expert)."""
    d = det.y.shape[2]
    for e in np.unique(det.expert):
        ti, j = np.nonzero(det.expert == e)
        Wd = np.abs(W_dn_of(int(e)))                  # [d, F]
        if fp8:
            # h is stored in bf16 and its bf16 values are quantised: where the
            # GPU's and the oracle's bf16(h) agree, and so do the row's
            # maxima, both compute v = float32(bf16(h) * r) with the same
            # float32 operations and get the same codes.  An element whose
            # bf16 rounding may flip moves its v by at most one bf16 step
            # (REL_BF16 of v); one next to the row's maximum moves the row's
            # scale by as much, hence every v of the row and the dequantised
            # row itself.
            # The e4m3 path's h carries an absolute error at the scale of its
            # row (fp8 MFMA sums): up to 2^-14.5 of the row's largest |h| was
            # measured.  ETA_HQ of the row's largest |h| -- the margin ETA_Q
            # gives v at the row's largest value (448, e4m3 step 32) --
            # decides where h's bf16 rounding may flip.
            flag, rflag, step = e4m3_flip_flags(det.h[ti, j], det.scaled[ti, j])
            ad = np.abs(det.a_deq[ti, j]) @ Wd.T
            # a row scale that moves by a factor (1 + delta) multiplies every
            # dequantised value of the row, so y moves by delta * y (code
            # flips are counted separately)
            C = (flag * step * det.s_a[ti, j].astype(np.float64)[:, None]) @ Wd.T + \
                rflag * REL_BF16 * np.abs(det.y[ti, j])
            D = C + ETA_Y * ad
        else:
            h = det.h[ti, j]
            dist, step = bf16_boundary(h)
            flag = (dist <= ETA_H * step) | (dist <= ETA_HA * np.max(np.abs(h), axis=1, keepdims=True))
            C = np.zeros((len(ti), d))
            from oracle import codecs
            D = (flag * step) @ Wd.T + ETA_Y * (np.abs(codecs.round_to_bf16(h)) @ Wd.T)
        yield ti, j, C, D


def y_allowance(y, D):
    """How far a stored bf16 expert output may lie from the oracle's rounding
    of y when the GPU's float32 y lies within D of the oracle's y: nothing
    where y is farther than D from a bf16 boundary (both round alike),
    otherwise D plus one bf16 step at |y| + D (each rounding moves a value by
    at most half a step)."""
    ydist, _ = bf16_boundary(y)
    _, step_hi = bf16_boundary(np.abs(y) + D)
    return (ydist <= D) * (D + step_hi)


def flip_allowance(det, W_dn_of, fp8):
    """Per element of the detail's tokens [n, d]: how far the GPU's output may
    move from the oracle's through predicted rounding-boundary flips: the
    weighted sum over the token's slots of y_allowance."""
    A = np.zeros((det.expert.shape[0], det.y.shape[2]))
    for ti, j, C, D in slot_flip_terms(det, W_dn_of, fp8):
        np.add.at(A, ti, det.w[ti, j][:, None] * y_allowance(det.y[ti, j], D))
    return A


def check_output_flips(out_gpu, out_ref, valid, tol, detail=None, W_dn_of=None, fp8=False,
                       out_bf16=False):
    """Every element of every valid token: |out_gpu - out_ref| <= tol * rms
    + A, where A is the flip allowance of the element (zero unless one of its
    stored activations lies at a rounding boundary) and, for a bf16 output
    (out_bf16), half a bf16 step of the output's own rounding.

    valid: tokens whose expert set equals the oracle's (None: all).
    detail(tokens): the oracle's per-slot parts of those tokens
    (oracle.forward_detail / forward_fp8_detail); only called for tokens with
    an element beyond the bound.  W_dn_of: as for flip_allowance."""
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    T = out_ref.shape[0]
    if valid is None:
        valid = np.ones(T, dtype=bool)
    assert np.all(np.isfinite(out_gpu))
    rms = float(np.sqrt(np.mean(out_ref ** 2))) if out_ref.size else 0.0
    diff = np.abs(out_gpu - out_ref)
    base = np.full(out_ref.shape, tol * rms)
    if out_bf16:
        base = base + 0.5 * bf16_boundary(np.maximum(np.abs(out_ref), np.abs(out_gpu)))[1]
    over = (diff > base) & valid[:, None]
    toks = np.nonzero(over.any(axis=1))[0]
    stats = dict(rms_ref=rms, max_ratio=float(diff[valid].max() / rms) if valid.any() and rms else 0.0,
                 elems_over_tol=int(over.sum()), tokens_over_tol=int(len(toks)), tokens=int(valid.sum()))
    if len(toks):
        assert detail is not None, f"{len(toks)} tokens beyond {tol} * rms and no flip model given"
        A = flip_allowance(detail(toks), W_dn_of, fp8)
        excess = diff[toks] - base[toks]
        bad = over[toks] & (excess > A)
        assert not bad.any(), (f"{int(bad.sum())} elements beyond {tol} * rms not explained by rounding "
                               f"flips (worst excess {float(excess[bad].max()):.3e}, rms {rms:.3e})")
        stats["max_excess_over_allowance"] = float(np.max(np.where(over[toks], excess / np.maximum(A, 1e-300), 0)))
    return stats


def bf16_flip_model(x_bits, r, W_gu, W_dn, Ws_gu=None, Ws_dn=None):
    """check_output_flips keywords for bf16 experts: the oracle's per-slot
    parts under its routing r (of the same token rows as x_bits), and the
    experts' down matrices.  W_gu / W_dn index by expert to bf16 bit patterns
    (arrays or LazyExperts); Ws_*: the shared expert, if any."""
    import oracle

    def W_dn_of(e):
        return oracle.bf16_bits_to_f64(Ws_dn if e < 0 else W_dn[e])

    return dict(detail=lambda toks: oracle.forward_detail(toks, x_bits, r, W_gu, W_dn, Ws_gu, Ws_dn),
                W_dn_of=W_dn_of)


def fp8_flip_model(x_bits, r, Wq_gu, s_gu, Wq_dn, s_dn):
    """check_output_flips keywords for e4m3 experts (per-channel or 128 x 128
    block scales)."""
    import oracle
    return dict(detail=lambda toks: oracle.forward_fp8_detail(toks, x_bits, r, Wq_gu, s_gu, Wq_dn, s_dn),
                W_dn_of=lambda e: oracle.dequant_e4m3(Wq_dn[e], s_dn[e]), fp8=True)


def set_equal(idx_gpu, r):
    """Tokens whose GPU expert set equals the oracle's."""
    return np.array([set(a) == set(b) for a, b in zip(np.asarray(idx_gpu).tolist(), r.idx.tolist())],
                    dtype=bool)


def stratified_tokens(idx, E, block=128):
    """Tokens covering every (expert, 128-row block) of the expert-contiguous
    row order the routing idx gives: the token of each block's first and last
    row (the last block of an expert may be partial), plus the batch's first
    and last token."""
    _, offsets, _, token_of = expected_permutation(idx, E)
    picks = [0, len(idx) - 1]
    for e in range(E):
        for b0 in range(offsets[e], offsets[e + 1], block):
            picks += [token_of[b0], token_of[min(b0 + block, offsets[e + 1]) - 1]]
    return np.unique(np.asarray(picks, dtype=np.int64))
