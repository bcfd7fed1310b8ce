"""ctypes binding of libhy3moe (include/hy3moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch tensors supply device memory and the current HIP stream; the
functions check dtype, shape, device and contiguity, pass raw pointers, and
raise Hy3MoeError on a negative status.  There is no fallback: if the library
is not built, lib() raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# HY3MOE_LIBRARY names another build of the same library (the sanitized one
# the C ABI's CPU tests load); by default the in-tree build.
LIB_PATH = os.environ.get("HY3MOE_LIBRARY") or os.path.join(_PKG, "libhy3moe.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_ALIGN, ERR_HIP, ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
NOALLOC_SCRATCH_BYTES = 64 << 20
WEIGHTS_BF16, WEIGHTS_FP8_E4M3 = 0, 1

EXPORTS = (
    "hy3moe_workspace_size", "hy3moe_route", "hy3moe_permute", "hy3moe_forward",
    "hy3moe_forward_timed", "hy3moe_forward_noalloc", "hy3moe_forward_fp8", "hy3moe_forward_fp8_timed",
    "hy3moe_forward_fp8_block128", "hy3moe_forward_fp8_block128_timed",
    "hy3moe_block_workspace_size", "hy3moe_route_ex", "hy3moe_block_forward",
    "hy3moe_block_forward_timed", "hy3moe_block_forward_bf16", "hy3moe_block_forward_bf16_timed",
    "hy3moe_quantize_rows_e4m3", "hy3moe_status_string",
    "hy3moe_last_hip_error",
)

_lib = None


class Hy3MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().hy3moe_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {lib().hy3moe_last_hip_error()})"
        super().__init__(f"{where}: status {status}: {msg}")


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(python -m sparse_moe_layer_wave_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, S, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    L.hy3moe_workspace_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(Z)]
    L.hy3moe_route.argtypes = [P, P, P, I, I, I, I, F, P, P, P, Z, S]
    L.hy3moe_permute.argtypes = [P, I, I, I, P, P, P, P, P, Z, S]
    L.hy3moe_forward.argtypes = [P, P, P, P, P, I, I, I, I, I, F, S, P, P, P, P, Z]
    L.hy3moe_forward_timed.argtypes = [P, P, P, P, P, I, I, I, I, I, F, S, P, P, P, P, Z, P]
    L.hy3moe_forward_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, S, P, P, P]
    L.hy3moe_forward_fp8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, S, P, P, P, P, Z]
    L.hy3moe_forward_fp8_timed.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, S, P, P, P, P, Z, P]
    L.hy3moe_forward_fp8_block128.argtypes = L.hy3moe_forward_fp8.argtypes
    L.hy3moe_forward_fp8_block128_timed.argtypes = L.hy3moe_forward_fp8_timed.argtypes
    L.hy3moe_block_workspace_size.argtypes = [I, I, I, I, I, ctypes.POINTER(Z)]
    L.hy3moe_route_ex.argtypes = [P, P, F, P, P, P, I, I, I, I, F, P, P, P, Z, S]
    L.hy3moe_block_forward.argtypes = [P, P, F, P, P, P, P, P, P, P, I, I, I, I, I, F, S, P, P, P, Z]
    L.hy3moe_block_forward_timed.argtypes = [P, P, F, P, P, P, P, P, P, P, I, I, I, I, I, F, S, P, P,
                                             P, Z, P]
    L.hy3moe_block_forward_bf16.argtypes = [P, P, F, P, P, P, P, P, P, P, P, I, I, I, I, I, F, S, P,
                                            P, P, Z]
    L.hy3moe_block_forward_bf16_timed.argtypes = L.hy3moe_block_forward_bf16.argtypes + [P]
    L.hy3moe_quantize_rows_e4m3.argtypes = [P, I, I, P, P, S]
    L.hy3moe_status_string.argtypes = [I]
    L.hy3moe_status_string.restype = ctypes.c_char_p
    L.hy3moe_last_hip_error.argtypes = []
    for name in EXPORTS:
        if name not in ("hy3moe_status_string",):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status, where):
    if status != OK:
        raise Hy3MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def workspace_size(T, d, E, k, d_ff, weight_dtype=WEIGHTS_BF16):
    n = ctypes.c_size_t(0)
    _check(lib().hy3moe_workspace_size(T, d, E, k, d_ff, weight_dtype, ctypes.byref(n)),
           "hy3moe_workspace_size")
    return n.value


def alloc_workspace(T, d, E, k, d_ff, weight_dtype=WEIGHTS_BF16, device="cuda"):
    return torch.empty(max(workspace_size(T, d, E, k, d_ff, weight_dtype), 1), dtype=torch.uint8,
                       device=device)


def route(x, W_gate, k, scale, bias=None, workspace=None):
    """hy3moe_route: returns (topk_idx int32 [T,k], topk_w fp32 [T,k])."""
    T, d = x.shape
    E = W_gate.shape[0]
    _need(x, torch.bfloat16, (T, d), "x")
    _need(W_gate, torch.float32, (E, d), "W_gate")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, d, E, k, 64, device=x.device) if T else None
    _check(lib().hy3moe_route(_ptr(x), _ptr(W_gate), _ptr(bias), T, d, E, k, float(scale),
                              _ptr(idx), _ptr(w), _ptr(workspace),
                              0 if workspace is None else workspace.numel(), _stream()),
           "hy3moe_route")
    return idx, w


def permute(topk_idx, E, workspace=None):
    """hy3moe_permute: returns (counts [E], offsets [E+1], row_of [T,k], token_of [T*k])."""
    T, k = topk_idx.shape
    _need(topk_idx, torch.int32, (T, k), "topk_idx")
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_of = torch.empty((T, k), dtype=torch.int32, device=dev)
    token_of = torch.empty(T * k, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(T, 64, E, k, 64, device=dev) if T else None
    _check(lib().hy3moe_permute(_ptr(topk_idx), T, E, k, _ptr(counts), _ptr(offsets), _ptr(row_of),
                                _ptr(token_of), _ptr(workspace),
                                0 if workspace is None else workspace.numel(), _stream()),
           "hy3moe_permute")
    return counts, offsets, row_of, token_of


STAGES = ("router", "dispatch", "gate_up", "down", "combine")


def forward(x, W_gate, W_gate_up, W_down, k, scale, bias=None, out=None, workspace=None,
            return_routing=False, stage_events=None):
    """hy3moe_forward: returns out fp32 [T,d] (and (idx, w) if return_routing).

    stage_events: optional list of 6 torch.cuda.Event (enable_timing=True);
    hy3moe_forward_timed records them around the five stages (STAGES)."""
    T, d = x.shape
    E = W_gate.shape[0]
    F = W_down.shape[2]
    _need(x, torch.bfloat16, (T, d), "x")
    _need(W_gate, torch.float32, (E, d), "W_gate")
    _need(W_gate_up, torch.bfloat16, (E, 2 * F, d), "W_gate_up")
    _need(W_down, torch.bfloat16, (E, d, F), "W_down")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, (T, d), "out")
    idx = w = None
    if return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, d, E, k, F, device=x.device) if T else None
    args = (_ptr(x), _ptr(W_gate), _ptr(W_gate_up), _ptr(W_down), _ptr(out), T, d, E, k, F,
            float(scale), _stream(), _ptr(bias), _ptr(idx), _ptr(w), _ptr(workspace),
            0 if workspace is None else workspace.numel())
    if stage_events is None:
        _check(lib().hy3moe_forward(*args), "hy3moe_forward")
    else:
        _check(lib().hy3moe_forward_timed(*args, _event_array(stage_events)), "hy3moe_forward_timed")
    return (out, idx, w) if return_routing else out


def forward_noalloc(x, W_gate, W_gate_up, W_down, k, scale, bias=None, out=None, return_routing=False):
    """hy3moe_forward_noalloc: hy3moe_forward with the library's static
    scratch instead of a workspace (allocates nothing in the library; this
    wrapper allocates out / the routing outputs only when not given)."""
    T, d = x.shape
    E = W_gate.shape[0]
    F = W_down.shape[2]
    _need(x, torch.bfloat16, (T, d), "x")
    _need(W_gate, torch.float32, (E, d), "W_gate")
    _need(W_gate_up, torch.bfloat16, (E, 2 * F, d), "W_gate_up")
    _need(W_down, torch.bfloat16, (E, d, F), "W_down")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, (T, d), "out")
    idx = w = None
    if return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check(lib().hy3moe_forward_noalloc(_ptr(x), _ptr(W_gate), _ptr(W_gate_up), _ptr(W_down), _ptr(out), T, d,
                                        E, k, F, float(scale), _stream(), _ptr(bias), _ptr(idx), _ptr(w)),
           "hy3moe_forward_noalloc")
    return (out, idx, w) if return_routing else out


def _event_array(stage_events):
    if len(stage_events) != 6:
        raise ValueError("stage_events: need 6 events")
    for ev in stage_events:
        if not ev.cuda_event:           # torch creates the hipEvent on first record
            ev.record()
    return (ctypes.c_void_p * 6)(*[ctypes.c_void_p(ev.cuda_event) for ev in stage_events])


def forward_fp8(x, W_gate, Wq_gate_up, s_gate_up, Wq_down, s_down, k, scale, bias=None, out=None,
                workspace=None, return_routing=False, stage_events=None, block128=False):
    """hy3moe_forward_fp8: e4m3 experts (uint8 codes) with fp32 per-channel
    scales; with block128=True, hy3moe_forward_fp8_block128: one fp32 scale
    per 128 x 128 weight block, s_gate_up [E, 2F/128, d/128] and s_down
    [E, d/128, F/128]."""
    T, d = x.shape
    E = W_gate.shape[0]
    F = Wq_down.shape[2]
    _need(x, torch.bfloat16, (T, d), "x")
    _need(W_gate, torch.float32, (E, d), "W_gate")
    _need(Wq_gate_up, torch.uint8, (E, 2 * F, d), "Wq_gate_up")
    _need(Wq_down, torch.uint8, (E, d, F), "Wq_down")
    if block128:
        _need(s_gate_up, torch.float32, (E, 2 * F // 128, d // 128), "s_gate_up")
        _need(s_down, torch.float32, (E, d // 128, F // 128), "s_down")
    else:
        _need(s_gate_up, torch.float32, (E, 2 * F), "s_gate_up")
        _need(s_down, torch.float32, (E, d), "s_down")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, (T, d), "out")
    idx = w = None
    if return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, d, E, k, F, WEIGHTS_FP8_E4M3, device=x.device) if T else None
    args = (_ptr(x), _ptr(W_gate), _ptr(Wq_gate_up), _ptr(s_gate_up), _ptr(Wq_down), _ptr(s_down),
            _ptr(out), T, d, E, k, F, float(scale), _stream(), _ptr(bias), _ptr(idx), _ptr(w),
            _ptr(workspace), 0 if workspace is None else workspace.numel())
    name = "hy3moe_forward_fp8_block128" if block128 else "hy3moe_forward_fp8"
    if stage_events is None:
        _check(getattr(lib(), name)(*args), name)
    else:
        _check(getattr(lib(), name + "_timed")(*args, _event_array(stage_events)), name + "_timed")
    return (out, idx, w) if return_routing else out


def forward_fp8_block128(x, W_gate, Wq_gate_up, sb_gate_up, Wq_down, sb_down, k, scale, **kw):
    """hy3moe_forward_fp8_block128 (forward_fp8 with block128=True)."""
    return forward_fp8(x, W_gate, Wq_gate_up, sb_gate_up, Wq_down, sb_down, k, scale, block128=True, **kw)


def block_workspace_size(T, d, E, k, d_ff):
    n = ctypes.c_size_t(0)
    _check(lib().hy3moe_block_workspace_size(T, d, E, k, d_ff, ctypes.byref(n)),
           "hy3moe_block_workspace_size")
    return n.value


def route_ex(x, W_gate, k, scale, norm_weight=None, norm_eps=1e-6, bias=None, score_bias=None,
             workspace=None):
    """hy3moe_route_ex: the full block's router (optional route_norm weight,
    pre-sigmoid logit bias and selection-only score bias).  Returns
    (topk_idx int32 [T,k], topk_w fp32 [T,k])."""
    T, d = x.shape
    E = W_gate.shape[0]
    _need(x, torch.bfloat16, (T, d), "x")
    _need(W_gate, torch.float32, (E, d), "W_gate")
    if norm_weight is not None:
        _need(norm_weight, torch.bfloat16, (d,), "norm_weight")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    if score_bias is not None:
        _need(score_bias, torch.float32, (E,), "score_bias")
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None and T:
        n = block_workspace_size(T, d, E, k, 64) if norm_weight is not None else workspace_size(T, d, E, k, 64)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
    _check(lib().hy3moe_route_ex(_ptr(x), _ptr(norm_weight), float(norm_eps), _ptr(W_gate),
                                 _ptr(bias), _ptr(score_bias), T, d, E, k, float(scale), _ptr(idx),
                                 _ptr(w), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), _stream()),
           "hy3moe_route_ex")
    return idx, w


def block_forward(x, W_gate, W_gate_up, W_down, Ws_gate_up, Ws_down, k, scale, norm_weight=None,
                  norm_eps=1e-6, score_bias=None, out=None, workspace=None, return_routing=False,
                  stage_events=None):
    """hy3moe_block_forward: shared expert + routed experts, with optional
    route_norm and selection-only score bias.  Returns out fp32 [T,d] (and
    (idx, w) if return_routing)."""
    T, d = x.shape
    E = W_gate.shape[0]
    F = W_down.shape[2]
    _need(x, torch.bfloat16, (T, d), "x")
    _need(W_gate, torch.float32, (E, d), "W_gate")
    _need(W_gate_up, torch.bfloat16, (E, 2 * F, d), "W_gate_up")
    _need(W_down, torch.bfloat16, (E, d, F), "W_down")
    if Ws_gate_up is not None or Ws_down is not None:
        _need(Ws_gate_up, torch.bfloat16, (2 * F, d), "Ws_gate_up")
        _need(Ws_down, torch.bfloat16, (d, F), "Ws_down")
    if norm_weight is not None:
        _need(norm_weight, torch.bfloat16, (d,), "norm_weight")
    if score_bias is not None:
        _need(score_bias, torch.float32, (E,), "score_bias")
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, (T, d), "out")
    idx = w = None
    if return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None and T:
        workspace = torch.empty(max(block_workspace_size(T, d, E, k, F), 1), dtype=torch.uint8,
                                device=x.device)
    args = (_ptr(x), _ptr(norm_weight), float(norm_eps), _ptr(W_gate), _ptr(score_bias),
            _ptr(W_gate_up), _ptr(W_down), _ptr(Ws_gate_up), _ptr(Ws_down), _ptr(out), T, d, E, k, F,
            float(scale), _stream(), _ptr(idx), _ptr(w), _ptr(workspace),
            0 if workspace is None else workspace.numel())
    if stage_events is None:
        _check(lib().hy3moe_block_forward(*args), "hy3moe_block_forward")
    else:
        _check(lib().hy3moe_block_forward_timed(*args, _event_array(stage_events)),
               "hy3moe_block_forward_timed")
    return (out, idx, w) if return_routing else out


def block_forward_bf16(x, W_gate, W_gate_up, W_down, Ws_gate_up, Ws_down, k, scale, residual=None,
                       norm_weight=None, norm_eps=1e-6, score_bias=None, out=None, workspace=None,
                       return_routing=False, stage_events=None):
    """hy3moe_block_forward_bf16: the block's output plus the bf16 residual
    (if given), summed in fp32 and rounded once to bf16.  Returns out bf16
    [T,d] (and (idx, w) if return_routing); out may be the residual tensor."""
    T, d = x.shape
    E = W_gate.shape[0]
    F = W_down.shape[2]
    _need(x, torch.bfloat16, (T, d), "x")
    _need(W_gate, torch.float32, (E, d), "W_gate")
    _need(W_gate_up, torch.bfloat16, (E, 2 * F, d), "W_gate_up")
    _need(W_down, torch.bfloat16, (E, d, F), "W_down")
    if Ws_gate_up is not None or Ws_down is not None:
        _need(Ws_gate_up, torch.bfloat16, (2 * F, d), "Ws_gate_up")
        _need(Ws_down, torch.bfloat16, (d, F), "Ws_down")
    if norm_weight is not None:
        _need(norm_weight, torch.bfloat16, (d,), "norm_weight")
    if score_bias is not None:
        _need(score_bias, torch.float32, (E,), "score_bias")
    if residual is not None:
        _need(residual, torch.bfloat16, (T, d), "residual")
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (T, d), "out")
    idx = w = None
    if return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None and T:
        workspace = torch.empty(max(block_workspace_size(T, d, E, k, F), 1), dtype=torch.uint8,
                                device=x.device)
    args = (_ptr(x), _ptr(norm_weight), float(norm_eps), _ptr(W_gate), _ptr(score_bias), _ptr(W_gate_up),
            _ptr(W_down), _ptr(Ws_gate_up), _ptr(Ws_down), _ptr(residual), _ptr(out), T, d, E, k, F,
            float(scale), _stream(), _ptr(idx), _ptr(w), _ptr(workspace),
            0 if workspace is None else workspace.numel())
    if stage_events is None:
        _check(lib().hy3moe_block_forward_bf16(*args), "hy3moe_block_forward_bf16")
    else:
        _check(lib().hy3moe_block_forward_bf16_timed(*args, _event_array(stage_events)),
               "hy3moe_block_forward_bf16_timed")
    return (out, idx, w) if return_routing else out


def quantize_rows_e4m3(x):
    """hy3moe_quantize_rows_e4m3: returns (codes uint8 [rows, cols], scales fp32 [rows])."""
    rows, cols = x.shape
    _need(x, torch.bfloat16, (rows, cols), "x")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(lib().hy3moe_quantize_rows_e4m3(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream()),
           "hy3moe_quantize_rows_e4m3")
    return q, s
