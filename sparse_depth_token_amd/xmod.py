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
GEMM_NT, GEMM_NN, GEMM_TN = 0, 1, 2

# Every symbol include/xmod.h declares, in declaration order.
EXPORTED = ["xmod_workspace_bytes", "xmod_route_topk", "xmod_topk_from_logits", "xmod_pack",
            "xmod_scatter_gated", "xmod_sparse_layer_fwd", "xmod_threshold_select",
            "xmod_sparse_layer_fwd_threshold", "xmod_mask_agreement", "xmod_routed_ffn_fwd",
            "xmod_attention_layer_fwd", "xmod_sparse_layer_fwd_fullkv", "xmod_dense_layer_fwd",
            "xmod_block_fwd", "xmod_sparse_layer_fwd_train", "xmod_sparse_layer_bwd",
            "xmod_rmsnorm_rows", "xmod_gemm_bf16_nt", "xmod_gemm_bf16", "xmod_attention_fwd",
            "xmod_attention_fwd_lse", "xmod_attention_bwd",
            "xmod_phase_timing_enable", "xmod_phase_timing_slots", "xmod_phase_times",
            "xmod_probe_mfma", "xmod_probe_read",
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
    "xmod_topk_from_logits": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _f32, _vp]),
    "xmod_pack": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "xmod_scatter_gated": (_i32, [_vp, _vp, _vp, _f32, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "xmod_sparse_layer_fwd_train": (_i32, [_vp, _P(Layer), _P(Dims), _i32, _vp, _f32, _f32, _vp,
                                           _vp, _vp, _sz, _vp]),
    "xmod_sparse_layer_bwd": (_i32, [_vp, _vp, _vp, _P(Layer), _P(Dims), _i32, _f32, _vp, _sz,
                                     _P(Grads), _vp, _vp, _sz, _vp]),
    "xmod_sparse_layer_fwd": (_i32, [_vp, _P(Layer), _P(Dims), _i32, _vp, _f32, _f32, _vp, _vp,
                                     _vp, _sz, _vp]),
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
    otherwise hand the library freed memory that the allocator gives to the next tensor)."""
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


def route_topk(x, w_router, router_bias, bias, tau, K, dims, logits, idx, gate, stream=None):
    _check(lib.xmod_route_topk(_ptr(x), _ptr(w_router), router_bias, _ptr(bias), tau, K,
                               ctypes.byref(dims), _ptr(logits), _ptr(idx), _ptr(gate), None, 0,
                               _stream(stream)), "xmod_route_topk")


def topk_from_logits(logits, k, idx, gate=None, bias=None, delta=0.0, stream=None):
    B, T = logits.shape
    _check(lib.xmod_topk_from_logits(_ptr(logits), B, T, k, _ptr(idx), _ptr(gate), _ptr(bias),
                                     delta, _stream(stream)), "xmod_topk_from_logits")


def pack(x, idx, x_packed, stream=None):
    B, T, d = x.shape
    _check(lib.xmod_pack(_ptr(x), _ptr(idx), B, T, d, idx.shape[1], _ptr(x_packed),
                         _stream(stream)), "xmod_pack")


def scatter_gated(x, idx, gate, varsigma, a_packed, f_packed, stream=None):
    B, T, d = x.shape
    _check(lib.xmod_scatter_gated(_ptr(x), _ptr(idx), _ptr(gate), varsigma, _ptr(a_packed),
                                  _ptr(f_packed), B, T, d, idx.shape[1], _stream(stream)),
           "xmod_scatter_gated")


def sparse_layer_fwd(x, layer: Layer, dims: Dims, K, bias, tau, delta, ws, idx_out=None,
                     gate_out=None, stream=None):
    _check(lib.xmod_sparse_layer_fwd(_ptr(x), ctypes.byref(layer), ctypes.byref(dims), K,
                                     _ptr(bias), tau, delta, _ptr(idx_out), _ptr(gate_out),
                                     _ptr(ws), ws.numel(), _stream(stream)),
           "xmod_sparse_layer_fwd")


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
    _check(lib.xmod_sparse_layer_fwd_train(_ptr(x), ctypes.byref(layer), ctypes.byref(dims), K,
                                           _ptr(bias), tau, delta, _ptr(idx_out), _ptr(gate_out),
                                           _ptr(saved), saved.numel(), _stream(stream)),
           "xmod_sparse_layer_fwd_train")


def sparse_layer_bwd(x, dy, dx, layer: Layer, dims: Dims, K, route_coef, saved, grads: Grads,
                     ws, loss_route=None, stream=None):
    _check(lib.xmod_sparse_layer_bwd(_ptr(x), _ptr(dy), _ptr(dx), ctypes.byref(layer),
                                     ctypes.byref(dims), K, route_coef, _ptr(saved), saved.numel(),
                                     ctypes.byref(grads), _ptr(loss_route), _ptr(ws), ws.numel(),
                                     _stream(stream)), "xmod_sparse_layer_bwd")


def threshold_select(logits, counts, offsets, src, n_total, gate=None, bias=None, delta=0.0,
                     stream=None):
    B, T = logits.shape
    _check(lib.xmod_threshold_select(_ptr(logits), B, T, _ptr(counts), _ptr(offsets), _ptr(src),
                                     _ptr(gate), _ptr(n_total), _ptr(bias), delta,
                                     _stream(stream)), "xmod_threshold_select")


def sparse_layer_fwd_threshold(x, layer: Layer, dims: Dims, bias, tau, delta, ws, src_out=None,
                               counts_out=None, n_total_out=None, stream=None):
    _check(lib.xmod_sparse_layer_fwd_threshold(_ptr(x), ctypes.byref(layer), ctypes.byref(dims),
                                               _ptr(bias), tau, delta, _ptr(src_out),
                                               _ptr(counts_out), _ptr(n_total_out), _ptr(ws),
                                               ws.numel(), _stream(stream)),
           "xmod_sparse_layer_fwd_threshold")


def mask_agreement(logits, idx, agree, stream=None):
    B, T = logits.shape
    _check(lib.xmod_mask_agreement(_ptr(logits), _ptr(idx), B, T, idx.shape[1], _ptr(agree),
                                   _stream(stream)), "xmod_mask_agreement")


def routed_ffn_fwd(x, layer: Layer, dims: Dims, K, bias, tau, delta, ws, idx_out=None,
                   gate_out=None, stream=None):
    _check(lib.xmod_routed_ffn_fwd(_ptr(x), ctypes.byref(layer), ctypes.byref(dims), K,
                                   _ptr(bias), tau, delta, _ptr(idx_out), _ptr(gate_out),
                                   _ptr(ws), ws.numel(), _stream(stream)), "xmod_routed_ffn_fwd")


def attention_layer_fwd(x, layer: Layer, dims: Dims, ws, stream=None):
    _check(lib.xmod_attention_layer_fwd(_ptr(x), ctypes.byref(layer), ctypes.byref(dims),
                                        _ptr(ws), ws.numel(), _stream(stream)),
           "xmod_attention_layer_fwd")


def sparse_layer_fwd_fullkv(x, layer: Layer, dims: Dims, K, bias, tau, delta, ws, idx_out=None,
                            gate_out=None, stream=None):
    _check(lib.xmod_sparse_layer_fwd_fullkv(_ptr(x), ctypes.byref(layer), ctypes.byref(dims), K,
                                            _ptr(bias), tau, delta, _ptr(idx_out),
                                            _ptr(gate_out), _ptr(ws), ws.numel(),
                                            _stream(stream)), "xmod_sparse_layer_fwd_fullkv")


def dense_layer_fwd(x, layer: Layer, dims: Dims, ws, stream=None):
    _check(lib.xmod_dense_layer_fwd(_ptr(x), ctypes.byref(layer), ctypes.byref(dims), _ptr(ws),
                                    ws.numel(), _stream(stream)), "xmod_dense_layer_fwd")


def block_fwd(x, layers: list, dims: Dims, N0, N1, A, K, bias, tau, delta, ws, stream=None):
    arr = (Layer * len(layers))(*layers)
    _check(lib.xmod_block_fwd(_ptr(x), arr, len(layers), ctypes.byref(dims), N0, N1, A, K,
                              _ptr(bias), tau, delta, _ptr(ws), ws.numel(), _stream(stream)),
           "xmod_block_fwd")


def rmsnorm_rows(x, idx, gain, eps, k, out, stream=None):
    B, T, d = x.shape
    _check(lib.xmod_rmsnorm_rows(_ptr(x), _ptr(idx), _ptr(gain), eps, B, T, d, k, _ptr(out),
                                 _stream(stream)), "xmod_rmsnorm_rows")


def gemm_bf16_nt(A, Bm, C, stream=None):
    M, K = A.shape
    N = Bm.shape[0]
    _check(lib.xmod_gemm_bf16_nt(_ptr(A), A.stride(0), _ptr(Bm), Bm.stride(0), _ptr(C),
                                 C.stride(0), M, N, K, _stream(stream)), "xmod_gemm_bf16_nt")


def gemm_bf16(layout, A, Bm, C, stream=None):
    """C = A(m, k) B(n, k) summed over k; layouts as xmod_gemm_bf16 (NT: A [M,K], B [N,K];
    NN: A [M,K], B [K,N]; TN: A [K,M], B [K,N]); C bf16 or fp32 [M, N]."""
    if layout == GEMM_TN:
        K, M = A.shape
    else:
        M, K = A.shape
    N = Bm.shape[0] if layout == GEMM_NT else Bm.shape[1]
    out_f32 = 1 if C.dtype == torch.float32 else 0
    _check(lib.xmod_gemm_bf16(layout, _ptr(A), A.stride(0), _ptr(Bm), Bm.stride(0), _ptr(C),
                              C.stride(0), out_f32, M, N, K, _stream(stream)), "xmod_gemm_bf16")


def attention_fwd_lse(qkv, o, lse, B, k, Hq, Hkv, hd, stream=None):
    _check(lib.xmod_attention_fwd_lse(_ptr(qkv), qkv.stride(0), _ptr(o), o.stride(0), _ptr(lse),
                                      B, k, Hq, Hkv, hd, _stream(stream)), "xmod_attention_fwd_lse")


def attention_bwd(qkv, o, lse, dO, D, dqkv, B, k, Hq, Hkv, hd, stream=None):
    _check(lib.xmod_attention_bwd(_ptr(qkv), qkv.stride(0), _ptr(o), o.stride(0), _ptr(lse),
                                  _ptr(dO), dO.stride(0), _ptr(D), _ptr(dqkv), dqkv.stride(0), B,
                                  k, Hq, Hkv, hd, _stream(stream)), "xmod_attention_bwd")


def attention_fwd(qkv, o, B, k, Hq, Hkv, hd, stream=None):
    _check(lib.xmod_attention_fwd(_ptr(qkv), qkv.stride(0), _ptr(o), o.stride(0), B, k, Hq, Hkv,
                                  hd, _stream(stream)), "xmod_attention_fwd")


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
    _check(lib.xmod_probe_mfma(_ptr(out), int(iters), _stream(stream)), "xmod_probe_mfma")
    return 4096 * 4 * int(iters) * 32768


def probe_read(src, out, stream=None):
    """Streaming read of every byte of the contiguous tensor src; out: int32 tensor of
    PROBE_THREADS whose 32-bit wrap-around sum equals that of src's 32-bit words. Returns the
    bytes read."""
    nbytes = src.numel() * src.element_size()
    lib.xmod_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_void_p]
    _check(lib.xmod_probe_read(_ptr(src), nbytes, _ptr(out), _stream(stream)), "xmod_probe_read")
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
