"""Thin ctypes binding of libxmod.so (the C ABI declared in include/xmod.h).

Argument marshalling only: every step of the layer runs in the HIP kernels behind the C ABI.
Tensors are torch tensors on a ROCm device; their data pointers and the current stream are
passed through. Importing this module fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxmod.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m sparse_depth_token_amd.build`")
lib = ctypes.CDLL(_LIB_PATH)

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
WS_ROUTE_TOPK, WS_SPARSE_LAYER, WS_DENSE_LAYER, WS_BLOCK, WS_SPARSE_THRESHOLD = 0, 1, 2, 3, 4
WS_ROUTED_FFN, WS_ATTN_LAYER, WS_SPARSE_FULLKV = 5, 6, 7
WS_TRAIN_SAVED, WS_BACKWARD = 8, 9
NOALLOC_SCRATCH_BYTES = 64 << 20   # XMOD_NOALLOC_SCRATCH_BYTES
GEMM_NT, GEMM_NN, GEMM_TN = 0, 1, 2

# Every symbol include/xmod.h declares, in declaration order.
EXPORTED = ["xmod_workspace_bytes", "xmod_route_topk", "xmod_topk_workspace_bytes",
            "xmod_topk_from_logits", "xmod_pack",
            "xmod_scatter_gated", "xmod_sparse_layer_fwd", "xmod_sparse_layer_fwd_noalloc",
            "xmod_threshold_select",
            "xmod_sparse_layer_fwd_threshold", "xmod_mask_agreement", "xmod_routed_ffn_fwd",
            "xmod_attention_layer_fwd", "xmod_sparse_layer_fwd_fullkv", "xmod_dense_layer_fwd",
            "xmod_block_fwd", "xmod_sparse_layer_fwd_train", "xmod_sparse_layer_bwd",
            "xmod_rmsnorm_rows", "xmod_gemm_bf16_nt", "xmod_gemm_bf16", "xmod_attention_fwd",
            "xmod_attention_fwd_lse", "xmod_attention_bwd",
            "xmod_phase_timing_enable", "xmod_phase_timing_slots", "xmod_phase_times",
            "xmod_probe_mfma", "xmod_probe_read", "xmod_probe_read_chunked",
            "xmod_status_string",
            "xmod_last_hip_error"]


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("d", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_hidden", ctypes.c_int32),
                ("rms_eps", ctypes.c_float)]


class Layer(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("router_bias", ctypes.c_float),
                ("varsigma", ctypes.c_float), ("g_attn", ctypes.c_void_p),
                ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("g_ffn", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("residual", ctypes.c_int32),
                ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p),
                ("rope_theta", ctypes.c_float)]


GRAD_FIELDS = ("w_router", "router_bias", "varsigma", "g_attn", "w_qkv", "w_o", "g_ffn",
               "w_gate", "w_up", "w_down")


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_P = ctypes.POINTER
_sig = {
    "xmod_workspace_bytes": (_sz, [_P(Dims), _i32, _i32]),
    "xmod_route_topk": (_i32, [_vp, _vp, _f32, _vp, _f32, _i32, _P(Dims), _vp, _vp, _vp, _vp, _sz, _vp]),
    "xmod_topk_workspace_bytes": (_sz, [_i32, _i32]),
    "xmod_topk_from_logits": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _f32, _vp, _sz, _vp]),
    "xmod_pack": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "xmod_scatter_gated": (_i32, [_vp, _vp, _vp, _f32, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "xmod_sparse_layer_fwd_train": (_i32, [_vp, _P(Layer), _P(Dims), _i32, _vp, _f32, _f32, _vp,
                                           _vp, _vp, _sz, _vp]),
    "xmod_sparse_layer_bwd": (_i32, [_vp, _vp, _vp, _P(Layer), _P(Dims), _i32, _f32, _vp, _sz,
                                     _P(Grads), _vp, _vp, _sz, _vp]),
    "xmod_sparse_layer_fwd": (_i32, [_vp, _P(Layer), _P(Dims), _i32, _vp, _f32, _f32, _vp, _vp,
                                     _vp, _sz, _vp]),
    "xmod_sparse_layer_fwd_noalloc": (_i32, [_vp, _P(Layer), _P(Dims), _i32, _vp, _f32, _f32,
                                             _vp, _vp, _vp]),
    "xmod_threshold_select": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp]),
    "xmod_sparse_layer_fwd_threshold": (_i32, [_vp, _P(Layer), _P(Dims), _vp, _f32, _f32, _vp,
                                               _vp, _vp, _vp, _sz, _vp]),
    "xmod_mask_agreement": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "xmod_routed_ffn_fwd": (_i32, [_vp, _P(Layer), _P(Dims), _i32, _vp, _f32, _f32, _vp, _vp,
                                   _vp, _sz, _vp]),
    "xmod_attention_layer_fwd": (_i32, [_vp, _P(Layer), _P(Dims), _vp, _sz, _vp]),
    "xmod_sparse_layer_fwd_fullkv": (_i32, [_vp, _P(Layer), _P(Dims), _i32, _vp, _f32, _f32, _vp,
                                            _vp, _vp, _sz, _vp]),
    "xmod_dense_layer_fwd": (_i32, [_vp, _P(Layer), _P(Dims), _vp, _sz, _vp]),
    "xmod_block_fwd": (_i32, [_vp, _P(Layer), _i32, _P(Dims), _i32, _i32, _f32, _i32, _vp, _f32,
                              _f32, _vp, _sz, _vp]),
    "xmod_rmsnorm_rows": (_i32, [_vp, _vp, _vp, _f32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "xmod_gemm_bf16_nt": (_i32, [_vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp]),
    "xmod_attention_fwd_lse": (_i32, [_vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                      _vp]),
    "xmod_attention_bwd": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                  _i32, _i32, _i32, _i32, _vp]),
    "xmod_gemm_bf16": (_i32, [_i32, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                              _vp]),
    "xmod_attention_fwd": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "xmod_probe_read": (_i32, [_vp, _sz, _i32, _vp, _vp]),
    "xmod_probe_read_chunked": (_i32, [_vp, _sz, _vp, _vp]),
    "xmod_phase_timing_enable": (None, [_i32]),
    "xmod_phase_timing_slots": (None, [ctypes.c_uint32]),
    "xmod_phase_times": (_i32, [_P(_f32), _i32, _P(_i32)]),
    "xmod_status_string": (ctypes.c_char_p, [_i32]),
    "xmod_last_hip_error": (_i32, []),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(lib, _name)
    _fn.restype, _fn.argtypes = _res, _args


class XmodError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib.xmod_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {lib.xmod_last_hip_error()})"
        super().__init__(f"{what}: {msg}")
        self.status = status


def _check(status: int, what: str):
    if status != OK:
        raise XmodError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# Every tensor handed to the library lives on the ROCm device ("cuda" in torch's naming).
_DEVICE_TYPE = "cuda"
_BF16, _F32, _I32, _U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


def _arg(t, name, dtype, n=None, at_least=None, optional=False):
    """Raw device pointer of tensor t, after the host checks the C ABI cannot make behind a bare
    pointer: a device tensor of the expected dtype, contiguous, with exactly n (or at least
    at_least) elements. A wrong buffer raises here, before any kernel is launched."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name}: expected a {_DEVICE_TYPE} tensor, got {t.device}")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name}: expected dtype {' or '.join(map(str, dts))}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")
    if at_least is not None and t.numel() < at_least:
        raise ValueError(f"{name}: expected at least {at_least} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _mat(t, name, dtype, rows, cols):
    """A 2-D row-major operand with unit column stride and at least rows x cols elements;
    returns (pointer, leading dimension in elements)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name}: expected a {_DEVICE_TYPE} tensor, got {t.device}")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name}: expected dtype {' or '.join(map(str, dts))}, got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) < t.shape[1]):
        raise ValueError(f"{name}: expected a 2-D row-major matrix with unit column stride")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name}: expected at least {rows} x {cols}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr()), int(t.stride(0))


def _ws(ws, name="ws"):
    _arg(ws, name, _U8)
    return ctypes.c_void_p(ws.data_ptr()), ws.numel()


def _bt(dims):
    return dims.B * dims.T


def _x(x, dims, name="x"):
    return _arg(x, name, _BF16, n=dims.B * dims.T * dims.d)


def _check_layer(layer, dims, sparse=True, fields=None):
    """The weights a layer struct points to: bf16 device tensors of the shapes dims implies."""
    w = getattr(layer, "_tensors", None)
    if w is None:
        raise ValueError("layer: build it with make_layer (it keeps the weight tensors)")
    d, F = dims.d, dims.ffn_hidden
    dq, dkv = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    sizes = {"w_router": d, "g_attn": d, "w_qkv": (dq + 2 * dkv) * d, "w_o": d * dq, "g_ffn": d,
             "w_gate": F * d, "w_up": F * d, "w_down": d * F}
    need = fields if fields is not None else [n for n in sizes if sparse or n != "w_router"]
    for n in sizes:
        _arg(w.get(n), f"layer.{n}", _BF16, n=sizes[n], optional=n not in need)
    for n in ("q_norm", "k_norm"):
        _arg(w.get(n), f"layer.{n}", _BF16, n=dims.head_dim, optional=True)


def _k(dims, K):
    if K < 1 or dims.T // K < 1:
        raise ValueError(f"K = {K}: floor(T/K) must be at least 1")
    return dims.T // K


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_dims(B, T, d, n_q_heads, n_kv_heads, head_dim, ffn_hidden, rms_eps=1e-6) -> Dims:
    return Dims(B, T, d, n_q_heads, n_kv_heads, head_dim, ffn_hidden, rms_eps)


def make_layer(w: dict) -> Layer:
    """w: dict of device tensors (bf16) w_router, g_attn, w_qkv, w_o, g_ffn, w_gate, w_up,
    w_down, optional q_norm / k_norm, and host values router_bias, varsigma, optional residual
    (0 or 1) and rope_theta. The returned struct holds raw device pointers; it keeps a
    reference to the tensors so that they outlive it (a caller passing a temporary dict would
    otherwise hand the library freed memory that the allocator gives to the next tensor).
    The entry points check the tensors' dtype, device and sizes against their dims."""
    L = Layer(_ptr(w.get("w_router")), float(w.get("router_bias", 0.0)),
              float(w.get("varsigma", 1.0)), _ptr(w["g_attn"]), _ptr(w["w_qkv"]),
              _ptr(w["w_o"]), _ptr(w["g_ffn"]), _ptr(w["w_gate"]), _ptr(w["w_up"]),
              _ptr(w["w_down"]), int(w.get("residual", 0)), _ptr(w.get("q_norm")),
              _ptr(w.get("k_norm")), float(w.get("rope_theta", 0.0) or 0.0))
    L._tensors = dict(w)
    return L


def workspace_bytes(dims: Dims, K: int, entry: int) -> int:
    return int(lib.xmod_workspace_bytes(ctypes.byref(dims), K, entry))


def alloc_workspace(dims: Dims, K: int, entry: int, device="cuda"):
    n = workspace_bytes(dims, K, entry)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def route_topk(x, w_router, router_bias, bias, tau, K, dims, logits, idx, gate, ws=None,
               stream=None):
    """ws: None (one workgroup per sequence) or alloc_workspace(dims, K, WS_ROUTE_TOPK)."""
    k = _k(dims, K)
    args = (_x(x, dims), _arg(w_router, "w_router", _BF16, n=dims.d))
    bias_p = _arg(bias, "bias", _F32, n=_bt(dims), optional=True)
    outs = (_arg(logits, "logits", _F32, n=_bt(dims)), _arg(idx, "idx", _I32, at_least=dims.B * k),
            _arg(gate, "gate", _F32, at_least=dims.B * k))
    wp, wn = _ws(ws) if ws is not None else (None, 0)
    _check(lib.xmod_route_topk(args[0], args[1], router_bias, bias_p, tau, K, ctypes.byref(dims),
                               *outs, wp, wn, _stream(stream)), "xmod_route_topk")


def topk_workspace_bytes(B, T):
    return int(lib.xmod_topk_workspace_bytes(B, T))


def topk_from_logits(logits, k, idx, gate=None, bias=None, delta=0.0, ws=None, stream=None):
    """ws: None (one workgroup per sequence) or a uint8 device tensor of at least
    topk_workspace_bytes(B, T) bytes (long sequences split over several workgroups)."""
    if logits.dim() != 2:
        raise ValueError("logits: expected [B, T]")
    B, T = logits.shape
    lp = _arg(logits, "logits", _F32)
    ip = _arg(idx, "idx", _I32, at_least=B * k)
    gp = _arg(gate, "gate", _F32, at_least=B * k, optional=True)
    bp = _arg(bias, "bias", _F32, n=B * T, optional=True)
    wp, wn = _ws(ws) if ws is not None else (None, 0)
    _check(lib.xmod_topk_from_logits(lp, B, T, k, ip, gp, bp, delta, wp, wn, _stream(stream)),
           "xmod_topk_from_logits")


def pack(x, idx, x_packed, stream=None):
    if x.dim() != 3 or idx.dim() != 2 or idx.shape[0] != x.shape[0]:
        raise ValueError("pack: x [B, T, d] and idx [B, k] expected")
    B, T, d = x.shape
    k = idx.shape[1]
    xp, ip = _arg(x, "x", _BF16), _arg(idx, "idx", _I32)
    op = _arg(x_packed, "x_packed", _BF16, at_least=B * k * d)
    _check(lib.xmod_pack(xp, ip, B, T, d, k, op, _stream(stream)), "xmod_pack")


def scatter_gated(x, idx, gate, varsigma, a_packed, f_packed, stream=None):
    if x.dim() != 3 or idx.dim() != 2 or idx.shape[0] != x.shape[0]:
        raise ValueError("scatter_gated: x [B, T, d] and idx [B, k] expected")
    B, T, d = x.shape
    k = idx.shape[1]
    ptrs = (_arg(x, "x", _BF16), _arg(idx, "idx", _I32), _arg(gate, "gate", _F32, n=B * k))
    ap = _arg(a_packed, "a_packed", _BF16, at_least=B * k * d)
    fp = _arg(f_packed, "f_packed", _BF16, at_least=B * k * d)
    _check(lib.xmod_scatter_gated(ptrs[0], ptrs[1], ptrs[2], varsigma, ap, fp, B, T, d, k,
                                  _stream(stream)), "xmod_scatter_gated")


def _routed_args(x, layer, dims, K, bias, ws, idx_out, gate_out, fields=None):
    k = _k(dims, K)
    _check_layer(layer, dims, True, fields)
    return (_x(x, dims), _arg(bias, "bias", _F32, n=_bt(dims), optional=True),
            _arg(idx_out, "idx_out", _I32, at_least=dims.B * k, optional=True),
            _arg(gate_out, "gate_out", _F32, at_least=dims.B * k, optional=True), *_ws(ws))


def sparse_layer_fwd(x, layer: Layer, dims: Dims, K, bias, tau, delta, ws, idx_out=None,
                     gate_out=None, stream=None):
    xp, bp, ip, gp, wp, wn = _routed_args(x, layer, dims, K, bias, ws, idx_out, gate_out)
    _check(lib.xmod_sparse_layer_fwd(xp, ctypes.byref(layer), ctypes.byref(dims), K, bp, tau,
                                     delta, ip, gp, wp, wn, _stream(stream)),
           "xmod_sparse_layer_fwd")


def sparse_layer_fwd_noalloc(x, layer: Layer, dims: Dims, K, bias, tau, delta, idx_out=None,
                             gate_out=None, stream=None):
    """xmod_sparse_layer_fwd with the library's static per-GPU workspace (no allocation; calls
    that overlap on one GPU race)."""
    k = _k(dims, K)
    _check_layer(layer, dims, True)
    xp = _x(x, dims)
    bp = _arg(bias, "bias", _F32, n=_bt(dims), optional=True)
    ip = _arg(idx_out, "idx_out", _I32, at_least=dims.B * k, optional=True)
    gp = _arg(gate_out, "gate_out", _F32, at_least=dims.B * k, optional=True)
    _check(lib.xmod_sparse_layer_fwd_noalloc(xp, ctypes.byref(layer), ctypes.byref(dims), K, bp,
                                             tau, delta, ip, gp, _stream(stream)),
           "xmod_sparse_layer_fwd_noalloc")


def make_grads(g: dict) -> Grads:
    """g: dict of fp32 device tensors named as GRAD_FIELDS (the shapes of the weights;
    router_bias and varsigma one element each). Keeps a reference to the tensors."""
    G = Grads(*[_ptr(g[n]) for n in GRAD_FIELDS])
    G._tensors = dict(g)
    return G


def alloc_grads(dims: Dims, device="cuda") -> dict:
    d, F = dims.d, dims.ffn_hidden
    dq, dkv = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    shapes = {"w_router": (d,), "router_bias": (1,), "varsigma": (1,), "g_attn": (d,),
              "w_qkv": (dq + 2 * dkv, d), "w_o": (d, dq), "g_ffn": (d,), "w_gate": (F, d),
              "w_up": (F, d), "w_down": (d, F)}
    return {n: torch.empty(sh, dtype=torch.float32, device=device) for n, sh in shapes.items()}


def sparse_layer_fwd_train(x, layer: Layer, dims: Dims, K, bias, tau, delta, saved, idx_out=None,
                           gate_out=None, stream=None):
    xp, bp, ip, gp, wp, wn = _routed_args(x, layer, dims, K, bias, saved, idx_out, gate_out)
    _check(lib.xmod_sparse_layer_fwd_train(xp, ctypes.byref(layer), ctypes.byref(dims), K, bp,
                                           tau, delta, ip, gp, wp, wn, _stream(stream)),
           "xmod_sparse_layer_fwd_train")


def sparse_layer_bwd(x, dy, dx, layer: Layer, dims: Dims, K, route_coef, saved, grads: Grads,
                     ws, loss_route=None, stream=None):
    _k(dims, K)
    _check_layer(layer, dims, True)
    ptrs = (_x(x, dims), _x(dy, dims, "dy"), _x(dx, dims, "dx"))
    sp, sn = _ws(saved, "saved")
    wp, wn = _ws(ws)
    d, F = dims.d, dims.ffn_hidden
    dq, dkv = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    sizes = {"w_router": d, "router_bias": 1, "varsigma": 1, "g_attn": d,
             "w_qkv": (dq + 2 * dkv) * d, "w_o": d * dq, "g_ffn": d, "w_gate": F * d,
             "w_up": F * d, "w_down": d * F}
    gt = getattr(grads, "_tensors", None)
    if gt is None:
        raise ValueError("grads: build it with make_grads (it keeps the gradient tensors)")
    for n in GRAD_FIELDS:
        _arg(gt.get(n), f"grads.{n}", _F32, n=sizes[n])
    lp = _arg(loss_route, "loss_route", _F32, at_least=1, optional=True)
    _check(lib.xmod_sparse_layer_bwd(ptrs[0], ptrs[1], ptrs[2], ctypes.byref(layer),
                                     ctypes.byref(dims), K, route_coef, sp, sn,
                                     ctypes.byref(grads), lp, wp, wn, _stream(stream)),
           "xmod_sparse_layer_bwd")


def threshold_select(logits, counts, offsets, src, n_total, gate=None, bias=None, delta=0.0,
                     stream=None):
    if logits.dim() != 2:
        raise ValueError("logits: expected [B, T]")
    B, T = logits.shape
    ptrs = (_arg(logits, "logits", _F32), _arg(counts, "counts", _I32, at_least=B),
            _arg(offsets, "offsets", _I32, at_least=B), _arg(src, "src", _I32, at_least=B * T))
    gp = _arg(gate, "gate", _F32, at_least=B * T, optional=True)
    np_ = _arg(n_total, "n_total", _I32, at_least=1)
    bp = _arg(bias, "bias", _F32, n=B * T, optional=True)
    _check(lib.xmod_threshold_select(ptrs[0], B, T, ptrs[1], ptrs[2], ptrs[3], gp, np_, bp, delta,
                                     _stream(stream)), "xmod_threshold_select")


def sparse_layer_fwd_threshold(x, layer: Layer, dims: Dims, bias, tau, delta, ws, src_out=None,
                               counts_out=None, n_total_out=None, stream=None):
    _check_layer(layer, dims, True)
    xp = _x(x, dims)
    bp = _arg(bias, "bias", _F32, n=_bt(dims), optional=True)
    sp = _arg(src_out, "src_out", _I32, at_least=_bt(dims), optional=True)
    cp = _arg(counts_out, "counts_out", _I32, at_least=dims.B, optional=True)
    tp = _arg(n_total_out, "n_total_out", _I32, at_least=1, optional=True)
    wp, wn = _ws(ws)
    _check(lib.xmod_sparse_layer_fwd_threshold(xp, ctypes.byref(layer), ctypes.byref(dims), bp,
                                               tau, delta, sp, cp, tp, wp, wn, _stream(stream)),
           "xmod_sparse_layer_fwd_threshold")


def mask_agreement(logits, idx, agree, stream=None):
    if logits.dim() != 2 or idx.dim() != 2 or idx.shape[0] != logits.shape[0]:
        raise ValueError("mask_agreement: logits [B, T] and idx [B, k] expected")
    B, T = logits.shape
    ptrs = (_arg(logits, "logits", _F32), _arg(idx, "idx", _I32),
            _arg(agree, "agree", (_I32, torch.uint32) if hasattr(torch, "uint32") else _I32,
                 at_least=1))
    _check(lib.xmod_mask_agreement(ptrs[0], ptrs[1], B, T, idx.shape[1], ptrs[2],
                                   _stream(stream)), "xmod_mask_agreement")


def routed_ffn_fwd(x, layer: Layer, dims: Dims, K, bias, tau, delta, ws, idx_out=None,
                   gate_out=None, stream=None):
    xp, bp, ip, gp, wp, wn = _routed_args(
        x, layer, dims, K, bias, ws, idx_out, gate_out,
        fields=["w_router", "g_ffn", "w_gate", "w_up", "w_down"])
    _check(lib.xmod_routed_ffn_fwd(xp, ctypes.byref(layer), ctypes.byref(dims), K, bp, tau, delta,
                                   ip, gp, wp, wn, _stream(stream)), "xmod_routed_ffn_fwd")


def attention_layer_fwd(x, layer: Layer, dims: Dims, ws, stream=None):
    _check_layer(layer, dims, False, fields=["g_attn", "w_qkv", "w_o"])
    xp = _x(x, dims)
    wp, wn = _ws(ws)
    _check(lib.xmod_attention_layer_fwd(xp, ctypes.byref(layer), ctypes.byref(dims), wp, wn,
                                        _stream(stream)), "xmod_attention_layer_fwd")


def sparse_layer_fwd_fullkv(x, layer: Layer, dims: Dims, K, bias, tau, delta, ws, idx_out=None,
                            gate_out=None, stream=None):
    xp, bp, ip, gp, wp, wn = _routed_args(x, layer, dims, K, bias, ws, idx_out, gate_out)
    _check(lib.xmod_sparse_layer_fwd_fullkv(xp, ctypes.byref(layer), ctypes.byref(dims), K, bp,
                                            tau, delta, ip, gp, wp, wn, _stream(stream)),
           "xmod_sparse_layer_fwd_fullkv")


def dense_layer_fwd(x, layer: Layer, dims: Dims, ws, stream=None):
    _check_layer(layer, dims, False)
    xp = _x(x, dims)
    wp, wn = _ws(ws)
    _check(lib.xmod_dense_layer_fwd(xp, ctypes.byref(layer), ctypes.byref(dims), wp, wn,
                                    _stream(stream)), "xmod_dense_layer_fwd")


def block_fwd(x, layers: list, dims: Dims, N0, N1, A, K, bias, tau, delta, ws, stream=None):
    ak = int(round(A * K))
    _k(dims, K)
    for i, L in enumerate(layers):
        sparse = i >= N0 and (i - N0) % (ak + 1) < ak
        _check_layer(L, dims, sparse)
    xp = _x(x, dims)
    bp = _arg(bias, "bias", _F32, n=_bt(dims))
    wp, wn = _ws(ws)
    arr = (Layer * len(layers))(*layers)
    _check(lib.xmod_block_fwd(xp, arr, len(layers), ctypes.byref(dims), N0, N1, A, K, bp, tau,
                              delta, wp, wn, _stream(stream)), "xmod_block_fwd")


def rmsnorm_rows(x, idx, gain, eps, k, out, stream=None):
    if x.dim() != 3:
        raise ValueError("rmsnorm_rows: x [B, T, d] expected")
    B, T, d = x.shape
    xp = _arg(x, "x", _BF16)
    ip = _arg(idx, "idx", _I32, n=B * k, optional=True)
    gp = _arg(gain, "gain", _BF16, n=d)
    op = _arg(out, "out", _BF16, at_least=B * k * d)
    _check(lib.xmod_rmsnorm_rows(xp, ip, gp, eps, B, T, d, k, op, _stream(stream)),
           "xmod_rmsnorm_rows")


def gemm_bf16_nt(A, Bm, C, stream=None):
    M, K = A.shape
    N = Bm.shape[0]
    ap, lda = _mat(A, "A", _BF16, M, K)
    bp, ldb = _mat(Bm, "B", _BF16, N, K)
    cp, ldc = _mat(C, "C", _BF16, M, N)
    _check(lib.xmod_gemm_bf16_nt(ap, lda, bp, ldb, cp, ldc, M, N, K, _stream(stream)),
           "xmod_gemm_bf16_nt")


def gemm_bf16(layout, A, Bm, C, stream=None):
    """C = A(m, k) B(n, k) summed over k; layouts as xmod_gemm_bf16 (NT: A [M,K], B [N,K];
    NN: A [M,K], B [K,N]; TN: A [K,M], B [K,N]); C bf16 or fp32 [M, N]."""
    if layout == GEMM_TN:
        K, M = A.shape
    else:
        M, K = A.shape
    N = Bm.shape[0] if layout == GEMM_NT else Bm.shape[1]
    ap, lda = _mat(A, "A", _BF16, *A.shape)
    bp, ldb = _mat(Bm, "B", _BF16, *Bm.shape)
    cp, ldc = _mat(C, "C", (_BF16, _F32), M, N)
    out_f32 = 1 if C.dtype == torch.float32 else 0
    _check(lib.xmod_gemm_bf16(layout, ap, lda, bp, ldb, cp, ldc, out_f32, M, N, K,
                              _stream(stream)), "xmod_gemm_bf16")


def _attn_mats(qkv, o, B, k, Hq, Hkv, hd):
    qp, ldq = _mat(qkv, "qkv", _BF16, B * k, (Hq + 2 * Hkv) * hd)
    op, ldo = _mat(o, "o", _BF16, B * k, Hq * hd)
    return qp, ldq, op, ldo


def attention_fwd_lse(qkv, o, lse, B, k, Hq, Hkv, hd, stream=None):
    qp, ldq, op, ldo = _attn_mats(qkv, o, B, k, Hq, Hkv, hd)
    lp = _arg(lse, "lse", _F32, at_least=B * k * Hq)
    _check(lib.xmod_attention_fwd_lse(qp, ldq, op, ldo, lp, B, k, Hq, Hkv, hd, _stream(stream)),
           "xmod_attention_fwd_lse")


def attention_bwd(qkv, o, lse, dO, D, dqkv, B, k, Hq, Hkv, hd, stream=None):
    qp, ldq, op, ldo = _attn_mats(qkv, o, B, k, Hq, Hkv, hd)
    lp = _arg(lse, "lse", _F32, at_least=B * k * Hq)
    dop, ldd = _mat(dO, "dO", _BF16, B * k, Hq * hd)
    Dp = _arg(D, "D", _F32, at_least=B * k * Hq)
    gp, ldg = _mat(dqkv, "dqkv", _BF16, B * k, (Hq + 2 * Hkv) * hd)
    _check(lib.xmod_attention_bwd(qp, ldq, op, ldo, lp, dop, ldd, Dp, gp, ldg, B, k, Hq, Hkv, hd,
                                  _stream(stream)), "xmod_attention_bwd")


def attention_fwd(qkv, o, B, k, Hq, Hkv, hd, stream=None):
    qp, ldq, op, ldo = _attn_mats(qkv, o, B, k, Hq, Hkv, hd)
    _check(lib.xmod_attention_fwd(qp, ldq, op, ldo, B, k, Hq, Hkv, hd, _stream(stream)),
           "xmod_attention_fwd")


PHASES = ["router", "topk", "gather_rmsnorm", "qkv_gemm", "attention", "o_gemm",
          "residual_rmsnorm", "gateup_swiglu_gemm", "down_scatter_gemm",
          # backward (xmod_sparse_layer_bwd)
          "bwd_resid", "bwd_dg_gemm", "bwd_dw_down_gemm", "bwd_dv_gemm", "bwd_dw_gateup_gemm",
          "bwd_rmsnorm2", "bwd_do_gemm", "bwd_dw_o_gemm", "bwd_attention", "bwd_du_gemm",
          "bwd_dw_qkv_gemm", "bwd_rmsnorm1", "bwd_router", "bwd_sums"]
FWD_PHASES = PHASES[:9]


PROBE_THREADS = 1024 * 256  # values the ceiling probes write (one per thread)


def probe_mfma(out, iters, stream=None):
    """Back-to-back bf16 MFMAs on every SIMD (4 * iters per wave, 4096 waves); out: fp32
    tensor of PROBE_THREADS, each set to 64 * iters. Returns the flops enqueued."""
    op = _arg(out, "out", _F32, at_least=PROBE_THREADS)
    _check(lib.xmod_probe_mfma(op, int(iters), _stream(stream)), "xmod_probe_mfma")
    return 4096 * 4 * int(iters) * 32768


def probe_read(src, out, loads_in_flight=4, stream=None):
    """Streaming read of every byte of the contiguous tensor src, loads_in_flight (4, 8 or 16)
    16-byte loads outstanding per thread; out: int32 tensor of PROBE_THREADS whose 32-bit
    wrap-around sum equals that of src's 32-bit words. Returns the bytes read."""
    nbytes = src.numel() * src.element_size()
    sp = _arg(src, "src", src.dtype)
    op = _arg(out, "out", _I32, at_least=PROBE_THREADS)
    _check(lib.xmod_probe_read(sp, nbytes, int(loads_in_flight), op, _stream(stream)),
           "xmod_probe_read")
    return nbytes


def probe_read_chunked(src, out, stream=None):
    """The same read as probe_read (same sums in out), each workgroup streaming its own
    contiguous share of src with non-temporal loads. Returns the bytes read."""
    nbytes = src.numel() * src.element_size()
    sp = _arg(src, "src", src.dtype)
    op = _arg(out, "out", _I32, at_least=PROBE_THREADS)
    _check(lib.xmod_probe_read_chunked(sp, nbytes, op, _stream(stream)),
           "xmod_probe_read_chunked")
    return nbytes


def phase_timing(on: bool, slots=None):
    """Enable / disable the per-kernel events; slots: names (PHASES) of the kernels to bracket
    with events, None for every kernel."""
    mask = 0xFFFFFFFF if slots is None else sum(1 << PHASES.index(n) for n in slots)
    lib.xmod_phase_timing_slots(mask)
    lib.xmod_phase_timing_enable(1 if on else 0)


def phase_times():
    """Milliseconds per kernel slot summed over the recorded calls, and the number of calls."""
    ms = (ctypes.c_float * len(PHASES))()
    n = ctypes.c_int32(0)
    _check(lib.xmod_phase_times(ms, len(PHASES), ctypes.byref(n)), "xmod_phase_times")
    return {p: float(ms[i]) for i, p in enumerate(PHASES)}, int(n.value)
