"""The Hy3 MoE layer forward pass, written out as its plain definition.

Test infrastructure only (see the package docstring).  Float64 throughout
except where the pages fix a precision:

* The router's scores are float32.  The Hy3 router casts hidden states and the
  gate weight to float before the linear map and the sigmoid ("Tencent
  Hy3-295B architecture teardown", section 4.1; "Tencent Hy3-Flash Q&A", Q6.2).
  The oracle computes the logit in float64 (closer to the exact value than any
  float32 summation order), applies the sigmoid in float64 and rounds the score
  once to float32.  Selection compares those float32 scores.
* The SwiGLU activation and each expert output are bf16 tensors in the model
  (its activations are bf16; the fp32 combine widens bf16 expert outputs:
  wmrh.cn Hy3 assembly blog, section 2.3), so ``bf16_activations=True`` (the
  default) rounds each once from float64 to bf16 where the layer stores it.
* The FP8 variant quantises activations to e4m3 with one float32 scale per row
  ("DeepSeek V4-Flash architecture Q&A", Q7.2 for the format, Q7.4 for
  per-channel scales), computing the scale and the scaled values in float32.
  The SwiGLU activation is a stored activation there too: it is rounded to
  bf16 (from float64, as above) and its bf16 values are quantised.
"""

from collections import namedtuple

import numpy as np

from .codecs import (bf16_bits_to_f64, e4m3_bits_to_f64, f32_to_bf16_bits, f32_to_e4m3_bits,
                     round_to_bf16, E4M3_MAX)

# Tokens whose k-th and (k+1)-th float32 scores differ by less than this are
# flagged: a float32 GPU router may legitimately pick either expert there.
NEAR_TIE = 1e-6

Route = namedtuple("Route", "idx w scores near_tie order_tie gap choice")


def _weights_f64(w):
    """An expert weight matrix as float64 values: bf16 bit patterns (uint16)
    are decoded; an array that is already float64 (the same values, decoded
    beforehand) is taken as it is."""
    w = np.asarray(w)
    return w if w.dtype == np.float64 else bf16_bits_to_f64(w)


def _sigmoid64(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def route(x_bits, W_gate, k, scale, logit_bias=None, block=4096, score_bias=None):
    """Sigmoid top-k router ("Tencent Hy3-295B architecture teardown", section
    4.1, router flow steps 1-5; "Tencent Hy3-Flash Q&A", Q4.2 and Q4.3).

    x_bits      uint16 [T, d]  bf16 hidden states
    W_gate      float32 [E, d] router weight
    k, scale    experts per token, router_scaling_factor (use float32(2.826))
    logit_bias  float32 [E] or None: added to each logit before the sigmoid
                (the gate linear map's per-expert bias term)
    score_bias  float32 [E] or None: e_score_correction_bias, added to the
                scores for the top-k choice only (step 2 of the router flow;
                Q4.3: it takes no part in the weights)

    Returns Route(idx int64 [T,k], w float64 [T,k], scores float32 [T,E],
    near_tie bool [T], order_tie bool [T], gap float64 [T], choice float32
    [T,E]).

    * scores = float32(sigmoid(x . W_gate^T + b)), logits summed in float64;
    * choice = scores + score_bias as a float32 addition (= scores without a
      score bias);
    * idx[t] = the first k experts when all E are ordered by choice
      descending, equal values by ascending expert index (slot j holds the
      j-th);
    * w[t, j] = scale * s[idx_j] / sum_j s[idx_j]  (float64, scores s);
    * near_tie: k < E and c_(k) - c_(k+1) < NEAR_TIE on the ranked choice
      values (the chosen set may differ on a float32 GPU router); order_tie:
      some adjacent pair among the first k+1 ranked values is that close (the
      slot order may differ).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    W = np.asarray(W_gate, dtype=np.float32).astype(np.float64)
    T = x_bits.shape[0]
    E = W.shape[0]
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    b = None if logit_bias is None else np.asarray(logit_bias, dtype=np.float32).astype(np.float64)
    scores = np.empty((T, E), dtype=np.float32)
    for t0 in range(0, T, block):
        xb = bf16_bits_to_f64(x_bits[t0:t0 + block])
        logits = xb @ W.T
        if b is not None:
            logits = logits + b
        scores[t0:t0 + block] = _sigmoid64(logits).astype(np.float32)
    if score_bias is None:
        choice = scores
    else:
        choice = scores + np.asarray(score_bias, dtype=np.float32)[None, :]   # float32 addition
    # stable sort on the negated value: equal values keep ascending expert order
    order = np.argsort(-choice.astype(np.float64), axis=1, kind="stable")
    idx = order[:, :k].astype(np.int64)
    ranked = np.take_along_axis(choice, order[:, :min(k + 1, E)], axis=1).astype(np.float64)
    sel = np.take_along_axis(scores, idx, axis=1).astype(np.float64)
    w = np.float64(np.float32(scale)) * sel / sel.sum(axis=1, keepdims=True) if T else sel.copy()
    if k < E:
        gap = ranked[:, k - 1] - ranked[:, k]
    else:
        gap = np.full(T, np.inf)
    near_tie = gap < NEAR_TIE
    adj = ranked[:, :-1] - ranked[:, 1:] if ranked.shape[1] > 1 else np.zeros((T, 0))
    order_tie = near_tie | (np.any(adj < NEAR_TIE, axis=1) if adj.shape[1] else np.zeros(T, bool))
    return Route(idx, w, scores, near_tie, order_tie, gap, choice)


def _swiglu_act(x, W_gu, F):
    """a = SiLU(x W_gate^T) * (x W_up^T) in float64, W_gu [2F, d] with the
    gate rows first."""
    g = x @ W_gu[:F].T
    u = x @ W_gu[F:].T
    return g * _sigmoid64(g) * u


def expert_swiglu_parts(x, W_gu, W_dn):
    """The two tensors a bf16 SwiGLU expert stores, each before its bf16
    rounding (float64): h_pre = a [n, F] and y_pre = bf16(h_pre) W_dn^T
    [n, d].  expert_swiglu's output is bf16(y_pre)."""
    h_pre = _swiglu_act(x, W_gu, W_dn.shape[1])
    return h_pre, round_to_bf16(h_pre) @ W_dn.T


def expert_swiglu(x, W_gu, W_dn, bf16_activations=True):
    """One SwiGLU expert on rows x [n, d] (float64).

    W_gu [2F, d]: rows [0, F) are the gate projection, rows [F, 2F) the up
    projection (the fused gate_up_proj of "Tencent Hy3-295B architecture
    teardown", section 2.3).  W_dn [d, F] is down_proj.  No bias.
    a = SiLU(x W_gate^T) * (x W_up^T), y = a W_dn^T ("DeepSeek V4-Flash
    architecture Q&A", Q4.5).  With bf16_activations, a and y are rounded to
    bf16 (the tensors a bf16 model stores); the products stay float64."""
    if bf16_activations:
        return round_to_bf16(expert_swiglu_parts(x, W_gu, W_dn)[1])
    return _swiglu_act(x, W_gu, W_dn.shape[1]) @ W_dn.T


def forward(x_bits, W_gate, W_gu_bits, W_dn_bits, k, scale, logit_bias=None,
            bf16_activations=True):
    """Routed MoE output with bf16 experts, float64 combine.

    x_bits uint16 [T,d]; W_gate float32 [E,d]; W_gu_bits uint16 [E,2F,d];
    W_dn_bits uint16 [E,d,F].  Returns (out float64 [T,d], Route).

    The combine is the per-expert loop of "DeepSeek V4-Flash architecture Q&A",
    Q8.4: for each expert, run it on the tokens that chose it and add
    weight * output into those tokens' rows.  The shared expert and the
    residual are not part of this output."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, d = x_bits.shape
    r = route(x_bits, W_gate, k, scale, logit_bias)
    out = np.zeros((T, d), dtype=np.float64)
    if T == 0:
        return out, r
    x = bf16_bits_to_f64(x_bits)
    for e in np.unique(r.idx):
        t, j = np.nonzero(r.idx == e)          # a token picks an expert at most once
        y = expert_swiglu(x[t], _weights_f64(W_gu_bits[e]), _weights_f64(W_dn_bits[e]),
                          bf16_activations)
        out[t] += r.w[t, j][:, None] * y
    return out, r


def forward_tokens(tokens, x_bits, W_gate, W_gu_bits, W_dn_bits, k, scale, logit_bias=None,
                   bf16_activations=True):
    """Output rows of ``forward`` for the listed tokens only.  Tokens are
    independent through the whole layer, so this is forward() on those rows."""
    tokens = np.asarray(tokens, dtype=np.int64)
    return forward(np.asarray(x_bits)[tokens], W_gate, W_gu_bits, W_dn_bits, k, scale, logit_bias,
                   bf16_activations)


# ----------------------------------------------------------------------------- full block

def rms_norm_bf16(x_bits, w_bits, eps):
    """route_norm: RMSNorm of bf16 rows with a bf16 weight, giving bf16 rows
    ("Tencent Hy3-Flash Q&A", Q4.9: the router scores an RMS-normalised copy
    of the hidden state).  The pages fix neither the precision nor eps; the
    reading (the usual bf16-model one) is:

    r = float32(1 / sqrt(sum(x^2) / d + eps))   (sum, division, sqrt in float64)
    a = bf16(float32(x * r))                     (normalised row, cast to bf16)
    y = bf16(a * w)                              (weight applied in bf16)

    x_bits uint16 [T, d]; w_bits uint16 [d]; returns uint16 [T, d]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, d = x_bits.shape
    if T == 0:
        return x_bits.copy()
    x = bf16_bits_to_f64(x_bits)
    v = np.sum(x * x, axis=1) / d + np.float64(eps)
    r = (1.0 / np.sqrt(v)).astype(np.float32)
    a = x.astype(np.float32) * r[:, None]                  # float32 products, rounded once
    a16 = f32_to_bf16_bits(a)
    prod = bf16_bits_to_f64(a16) * bf16_bits_to_f64(np.asarray(w_bits, dtype=np.uint16))[None, :]
    return f32_to_bf16_bits(prod.astype(np.float32))       # exact in float32, then one bf16 rounding


def forward_block(x_bits, W_gate, W_gu_bits, W_dn_bits, Ws_gu_bits, Ws_dn_bits, k, scale,
                  norm_w_bits=None, eps=1e-6, score_bias=None, logit_bias=None):
    """The Hy3 MoE block: shared expert plus routed experts.

    out = SharedExpert(x) + sum_j w[t, j] * Expert_idx[t, j](x)   ("Tencent
    Hy3-Flash Q&A", Q4.7), where the router scores route_norm(x) when
    norm_w_bits is given (Q4.9) and selects with score_bias when given (Q4.3).
    The experts, shared and routed, see x itself.  Ws_gu_bits [2F, d] and
    Ws_dn_bits [d, F] are the shared expert's SwiGLU weights; its activation
    and output are rounded to bf16 like a routed expert's.

    Returns (out float64 [T, d], Route)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, d = x_bits.shape
    xr = x_bits if norm_w_bits is None else rms_norm_bf16(x_bits, norm_w_bits, eps)
    r = route(xr, W_gate, k, scale, logit_bias, score_bias=score_bias)
    out = np.zeros((T, d), dtype=np.float64)
    if T == 0:
        return out, r
    x = bf16_bits_to_f64(x_bits)
    for e in np.unique(r.idx):
        t, j = np.nonzero(r.idx == e)
        y = expert_swiglu(x[t], _weights_f64(W_gu_bits[e]), _weights_f64(W_dn_bits[e]))
        out[t] += r.w[t, j][:, None] * y
    out += expert_swiglu(x, _weights_f64(Ws_gu_bits), _weights_f64(Ws_dn_bits))
    return out, r


def forward_block_tokens(tokens, x_bits, *args, **kwargs):
    """Output rows of ``forward_block`` for the listed tokens only (tokens are
    independent through the whole block)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    return forward_block(np.asarray(x_bits)[tokens], *args, **kwargs)


def forward_block_residual(x_bits, *args, residual_bits=None, **kwargs):
    """The decoder layer's residual branch ended in the block: the block output
    of ``forward_block`` plus the bf16 residual row (wmrh.cn Hy3 assembly blog,
    section 3.2, the residual add; section 2.3, the branches added in a wider
    type than bf16), in float64 and not rounded.  The library rounds this sum
    once to bf16; the tolerance of the comparison covers that rounding.

    residual_bits uint16 [T, d] or None (then the block output alone).
    Returns (out float64 [T, d], Route)."""
    out, r = forward_block(x_bits, *args, **kwargs)
    if residual_bits is not None:
        out = out + bf16_bits_to_f64(np.asarray(residual_bits, dtype=np.uint16))
    return out, r


# ----------------------------------------------------------------------------- FP8

def quant_row_e4m3(v):
    """Per-row e4m3 quantisation of a float32 vector.

    amax = max |v|.  amax = 0 gives codes 0 and scale 1.  Otherwise
    r = float32(448 / amax), codes = e4m3(float32(v * r)) (nearest, ties to
    even, saturating) and scale s = float32(amax / 448); the dequantised row is
    codes * s.  Returns (uint8 codes, float32 scale)."""
    q, s, _ = quant_row_e4m3_parts(v)
    return q, s


def quant_row_e4m3_parts(v):
    """quant_row_e4m3 with the float32 values it rounds: returns (codes,
    scale, scaled) where scaled = float32(v * r) (zeros for an all-zero
    row), so codes = e4m3(scaled)."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v)) if v.size else np.float32(0)
    if amax == 0:
        return np.zeros(v.shape, dtype=np.uint8), np.float32(1.0), np.zeros(v.shape, np.float32)
    r = np.float32(E4M3_MAX) / np.float32(amax)
    scaled = v * r
    return f32_to_e4m3_bits(scaled), np.float32(amax) / np.float32(E4M3_MAX), scaled


def quant_rows_e4m3(M):
    """quant_row_e4m3 applied to every row of a float32 matrix."""
    M = np.asarray(M, dtype=np.float32)
    q = np.empty(M.shape, dtype=np.uint8)
    s = np.empty(M.shape[0], dtype=np.float32)
    for i in range(M.shape[0]):
        q[i], s[i] = quant_row_e4m3(M[i])
    return q, s


def dequant_e4m3(q, s):
    """Dequantised float64 weight matrix from e4m3 codes q [R, C] and fp32
    scales: s [R] gives one scale per row (output channel); s [R/128, C/128]
    gives one per 128 x 128 block, element (n, i) taking s[n // 128, i // 128]
    ("DeepSeek V4-Flash architecture Q&A", Q7.2: block-wise quantisation)."""
    w = e4m3_bits_to_f64(np.asarray(q, dtype=np.uint8))
    s = np.asarray(s, dtype=np.float64)
    if s.ndim == 1:
        return w * s[:, None]
    R, C = w.shape
    assert s.shape == (R // 128, C // 128) and R % 128 == 0 and C % 128 == 0
    return w * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)


def forward_fp8(x_bits, W_gate, Wq_gu, s_gu, Wq_dn, s_dn, k, scale, logit_bias=None):
    """Routed MoE output with e4m3 experts.

    Wq_gu uint8 [E,2F,d] with float32 per-output-row scales s_gu [E,2F];
    Wq_dn uint8 [E,d,F] with s_dn [E,d].  Or block scales, one per 128 x 128
    block: s_gu [E,2F/128,d/128] and s_dn [E,d/128,F/128] (``dequant_e4m3``).
    Routing is the float32 router of
    ``route``.  Each token's bf16 row is quantised with quant_row_e4m3 before
    the gate_up product; each (token, slot) SwiGLU activation row, rounded to
    bf16 where the layer stores it, is quantised the same way before the down
    product.  Products use
    the dequantised operands in float64; each expert output row is rounded to
    bf16 (as in ``forward``) and the combine is as in ``forward``."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, d = x_bits.shape
    r = route(x_bits, W_gate, k, scale, logit_bias)
    out = np.zeros((T, d), dtype=np.float64)
    if T == 0:
        return out, r
    xd = _dequant_x_e4m3(x_bits)
    for e in np.unique(r.idx):
        t, j = np.nonzero(r.idx == e)
        y_pre = _fp8_expert_parts(xd[t], Wq_gu[e], s_gu[e], Wq_dn[e], s_dn[e])[4]
        out[t] += r.w[t, j][:, None] * round_to_bf16(y_pre)
    return out, r


def _dequant_x_e4m3(x_bits):
    """The bf16 rows quantised per row (quant_row_e4m3 of float32(x)) and
    dequantised, float64."""
    qx, sx = quant_rows_e4m3(bf16_bits_to_f64(x_bits).astype(np.float32))
    return e4m3_bits_to_f64(qx) * sx.astype(np.float64)[:, None]


def _fp8_expert_parts(xd, Wq_gu_e, s_gu_e, Wq_dn_e, s_dn_e):
    """One e4m3 expert on dequantised x rows xd [n, d] (float64).

    a = SiLU(xd Wg^T) * (xd Wu^T) with the dequantised weights, rounded to
    bf16 where the layer stores it; each row of bf16(a) (exact in float32) is
    quantised with quant_row_e4m3 and dequantised; the expert output before
    its bf16 rounding is y_pre = dequant(a) Wd^T.  Returns (a float64 [n, F]
    before its bf16 rounding; scaled float32 [n, F], the values
    quant_row_e4m3 rounds to e4m3; s_a float32 [n], the rows' scales; a_deq
    float64 [n, F]; y_pre float64 [n, d])."""
    Wdn = dequant_e4m3(Wq_dn_e, s_dn_e)
    a = _swiglu_act(xd, dequant_e4m3(Wq_gu_e, s_gu_e), Wdn.shape[1])
    a16 = round_to_bf16(a).astype(np.float32)
    n, F = a.shape
    qa = np.empty((n, F), np.uint8)
    sa = np.empty(n, np.float32)
    scaled = np.empty((n, F), np.float32)
    for i in range(n):
        qa[i], sa[i], scaled[i] = quant_row_e4m3_parts(a16[i])
    ad = e4m3_bits_to_f64(qa) * sa.astype(np.float64)[:, None]
    return a, scaled, sa, ad, ad @ Wdn.T


def forward_fp8_tokens(tokens, x_bits, W_gate, Wq_gu, s_gu, Wq_dn, s_dn, k, scale, logit_bias=None):
    """Output rows of ``forward_fp8`` for the listed tokens only."""
    tokens = np.asarray(tokens, dtype=np.int64)
    return forward_fp8(np.asarray(x_bits)[tokens], W_gate, Wq_gu, s_gu, Wq_dn, s_dn, k, scale,
                       logit_bias)


# ----------------------------------------------------------------------------- per-slot parts

Detail = namedtuple("Detail", "tokens expert w h y scaled s_a a_deq")


def forward_detail(tokens, x_bits, r, W_gu_bits, W_dn_bits, Ws_gu_bits=None, Ws_dn_bits=None):
    """The per-slot terms of ``forward`` (of ``forward_block`` when the shared
    expert's weights are given) for the listed tokens, each stored tensor
    before its bf16 rounding.

    r is ``route``'s result for the whole batch.  Slot j < k of token t is
    expert r.idx[t, j] with weight r.w[t, j]; with a shared expert, slot k is
    it, with weight 1 and expert id -1.  Returns Detail(tokens, expert int64
    [n, S], w float64 [n, S], h float64 [n, S, F], y float64 [n, S, d], None,
    None, None): h is the SwiGLU activation and y the expert output, both as
    ``expert_swiglu_parts`` gives them.  The layer's row is sum_j w * bf16(y)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)[tokens])
    idx = r.idx[tokens]
    n, k = idx.shape
    shared = Ws_gu_bits is not None
    S = k + (1 if shared else 0)
    F = np.asarray(W_dn_bits[int(idx[0, 0])]).shape[-1] if n else 0
    d = x.shape[1]
    h = np.zeros((n, S, F))
    y = np.zeros((n, S, d))
    expert = np.full((n, S), -1, dtype=np.int64)
    expert[:, :k] = idx
    w = np.ones((n, S))
    w[:, :k] = r.w[tokens]
    for e in np.unique(idx):
        ti, j = np.nonzero(idx == e)
        h[ti, j], y[ti, j] = expert_swiglu_parts(x[ti], _weights_f64(W_gu_bits[e]),
                                                 _weights_f64(W_dn_bits[e]))
    if shared and n:
        h[:, k], y[:, k] = expert_swiglu_parts(x, _weights_f64(Ws_gu_bits), _weights_f64(Ws_dn_bits))
    return Detail(tokens, expert, w, h, y, None, None, None)


def forward_fp8_detail(tokens, x_bits, r, Wq_gu, s_gu, Wq_dn, s_dn):
    """The per-slot terms of ``forward_fp8`` for the listed tokens (r:
    ``route``'s result for the whole batch; slot j is expert r.idx[t, j]).

    Returns Detail(tokens, expert [n, k], w [n, k], h float64 [n, k, F],
    y float64 [n, k, d], scaled float32 [n, k, F], s_a float32 [n, k], a_deq
    float64 [n, k, F]): h is the SwiGLU activation before its bf16 rounding,
    scaled holds the values the activation quantiser rounds to e4m3, s_a the
    activation rows' scales, a_deq the dequantised activations and y the
    expert outputs before their bf16 rounding."""
    tokens = np.asarray(tokens, dtype=np.int64)
    xd = _dequant_x_e4m3(np.asarray(x_bits, dtype=np.uint16)[tokens])
    idx = r.idx[tokens]
    n, k = idx.shape
    F = np.asarray(Wq_dn[int(idx[0, 0])]).shape[-1] if n else 0
    d = xd.shape[1]
    y = np.zeros((n, k, d))
    h = np.zeros((n, k, F))
    scaled = np.zeros((n, k, F), np.float32)
    s_a = np.zeros((n, k), np.float32)
    a_deq = np.zeros((n, k, F))
    for e in np.unique(idx):
        ti, j = np.nonzero(idx == e)
        h[ti, j], scaled[ti, j], s_a[ti, j], a_deq[ti, j], y[ti, j] = _fp8_expert_parts(
            xd[ti], Wq_gu[e], s_gu[e], Wq_dn[e], s_dn[e])
    return Detail(tokens, idx.astype(np.int64), r.w[tokens].copy(), h, y, scaled, s_a, a_deq)


# ----------------------------------------------------------------------------- accounting

def expert_param_count(d, d_ff):
    """Parameters of one routed expert: the fused gate_up matrix [2*d_ff, d]
    plus the down matrix [d, d_ff] (no bias)."""
    gate_up = (2 * d_ff) * d
    down = d * d_ff
    return gate_up + down


def flops_per_token(d, d_ff, k, E):
    """Useful FLOPs per token of the routed layer: for each of the k experts a
    [1,d]x[d,2F] and a [1,F]x[F,d] product (2 FLOPs per multiply-add), plus
    the [1,d]x[d,E] router product.  The sigmoid, SiLU and combine are not
    counted."""
    per_expert = 2 * (d * 2 * d_ff) + 2 * (d_ff * d)
    return k * per_expert + 2 * d * E
