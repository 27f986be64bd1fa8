"""Throughput of one X-MoD Sparse(K) layer forward on one MI355X.

Headline workload: the long-context Sparse(K=4) layer with grouped-query attention, B=1 x
T=32768, d=4096, 32 query / 8 key-value heads x 128, SwiGLU hidden 14336, bf16; 8192 of the
32768 tokens are routed (8192 routed rows per step). Weights N(0, 0.02), activations N(0, 1)
with 1 % of the rows scaled x8 (a skewed router distribution), all seeded and synthetic. A step
is one xmod_sparse_layer_fwd call (router, top-k, gather + RMSNorm, QKV GEMM, attention over the
routed subset, O GEMM, residual + RMSNorm, gate/up GEMM with SwiGLU, down GEMM with the gated
scatter back into x).

Protocol of the timed steps: before every step, outside its events, x and the carried bias are
restored from pristine device copies and a 512 MiB scratch buffer is read (the 256 MB
last-level cache then holds no part of the layer's inputs), so each step starts from the same state
with its inputs resident in HBM. Each step is bracketed by HIP events on the launch stream;
ms_per_step is the median. Untimed steps run for at least 0.2 s first (the clocks settle), then
the W warm-up steps.

Prints one JSON line: routed tokens/s; the roofline of the dominant kernel (the gate/up GEMM),
timed by HIP events the library records around that kernel in every timed step; a per-kernel
breakdown from further steps with events around every kernel (cold, as the timed steps, and
warm, back to back); the same for the other single-layer workloads (the small K=2 layer and the
K=8 layer at B8 x T4096); the two stack workloads through the block entry point; informational
lines for the eval-time threshold rule and one training step on the K=8 layer; the copy and
read bandwidth, MFMA rate and vendor-library GEMM rates this GPU sustains; and the CPU oracle
timed on a bounded sample of the headline workload on this host.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline] [--no-threshold]
                      [--no-train] [--no-blocks] [--no-ceilings] [--no-configs] [--copy-probe]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workload as wl  # noqa: E402

METRIC = "routed tokens/s per sparse layer (bf16, 1 GPU); % MFMA peak; route/pack GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def algorithmic_work(w):
    """Per-step algorithmic FLOPs and bytes of each kernel (what the method must do)."""
    B, T, d, k = w.B, w.T, w.d, w.k
    M = B * k
    dq, dkv, F = w.d_q, w.d_kv, w.ffn_hidden
    nqkv = dq + 2 * dkv
    att_flops = 2.0 * B * w.n_q_heads * w.head_dim * k * (k + 1)   # causal QK^T and PV
    return {
        "router": {"bytes": 2.0 * B * T * d + 2 * d + 8.0 * B * T, "flops": 2.0 * B * T * d},
        "topk": {"bytes": 4.0 * B * T + 8.0 * M + 8.0 * M, "flops": 0.0},
        "gather_rmsnorm": {"bytes": 4.0 * M * d, "flops": 3.0 * M * d},
        "qkv_gemm": {"flops": 2.0 * M * d * nqkv, "bytes": 2.0 * (M * d + nqkv * d + M * nqkv)},
        "attention": {"flops": att_flops, "bytes": 2.0 * (M * nqkv + M * dq)},
        # a is written in fp32
        "o_gemm": {"flops": 2.0 * M * dq * d, "bytes": 2.0 * (M * dq + d * dq) + 4.0 * M * d},
        # X (bf16) and a (fp32) read, v (bf16) written
        "residual_rmsnorm": {"bytes": 8.0 * M * d, "flops": 4.0 * M * d},
        "gateup_swiglu_gemm": {"flops": 4.0 * M * d * F, "bytes": 2.0 * (M * d + 2 * F * d + M * F)},
        # g, W_down, X (bf16) and a (fp32) read, the selected rows of x (bf16) written
        "down_scatter_gemm": {"flops": 2.0 * M * F * d,
                              "bytes": 2.0 * (M * F + d * F) + 8.0 * M * d},
    }


def algorithmic_work_bwd(w):
    """Per-step algorithmic FLOPs and bytes of each kernel slot of the backward."""
    B, T, d, k = w.B, w.T, w.d, w.k
    M = B * k
    dq, dkv, F = w.d_q, w.d_kv, w.ffn_hidden
    nqkv = dq + 2 * dkv
    att = 2.0 * B * w.n_q_heads * w.head_dim * k * (k + 1)
    g = lambda m, n, kk: {"flops": 2.0 * m * n * kk, "bytes": 2.0 * (m * kk + n * kk) + 4.0 * m * n}
    return {
        "bwd_resid": {"flops": 0.0, "bytes": 12.0 * M * d},
        "bwd_dg_gemm": dict(g(M, F, d), bytes=2.0 * (M * d + F * d) + 8.0 * M * F),
        "bwd_dw_down_gemm": g(d, F, M),
        "bwd_dv_gemm": g(M, d, 2 * F),
        "bwd_dw_gateup_gemm": g(2 * F, d, M),
        "bwd_rmsnorm2": {"flops": 0.0, "bytes": 20.0 * M * d},
        "bwd_do_gemm": dict(g(M, dq, d), bytes=2.0 * (M * d + dq * d + M * dq)),
        "bwd_dw_o_gemm": g(d, dq, M),
        "bwd_attention": {"flops": 2.5 * att, "bytes": 2.0 * (M * nqkv * 2 + 2 * M * dq)},
        "bwd_du_gemm": g(M, d, nqkv),
        "bwd_dw_qkv_gemm": g(nqkv, d, M),
        "bwd_rmsnorm1": {"flops": 0.0, "bytes": 12.0 * M * d},
        "bwd_router": {"flops": 0.0, "bytes": 6.0 * (B * T - M) * d + 13.0 * B * T},
        "bwd_sums": {"flops": 0.0, "bytes": 0.0},
    }


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` at `workload` from the committed rocprofv3 counter
    summary, or None if there is none or the kernel's sources changed since the counters were
    taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    return int(rec["traffic_bytes_per_launch"])


FLUSH_BYTES = 512 << 20   # read before each cold step: twice the 256 MB last-level cache


class LayerRun:
    """One single-layer workload on the device: seeded inputs (workload.py), pristine copies of
    x and the carried bias, the layer's weights and workspace."""

    def __init__(self, xmod, w):
        import torch
        self.xmod, self.w = xmod, w
        self.xb = wl.make_x(w)
        self.lay = wl.make_layer(w, 0)
        self.bias_np = wl.make_bias(w)
        up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()
        self.dl = {k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in self.lay.items()}
        self.L = xmod.make_layer(self.dl)
        self.dims = xmod.make_dims(w.B, w.T, w.d, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                   w.ffn_hidden, w.rms_eps)
        self.x0 = up(self.xb)
        self.x = self.x0.clone()
        self.b0 = torch.from_numpy(self.bias_np).cuda()
        self.bias = self.b0.clone()
        self.ws = xmod.alloc_workspace(self.dims, w.K, xmod.WS_SPARSE_LAYER)
        self.stream = torch.cuda.current_stream()
        # the flush reads a buffer twice the size of the last-level cache (reads leave no dirty
        # lines behind, whose write-back would slow the next kernel's reads)
        self.flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.flush_sums = torch.empty(xmod.PROBE_THREADS, dtype=torch.int32, device="cuda")

    def step(self):
        w = self.w
        self.xmod.sparse_layer_fwd(self.x, self.L, self.dims, w.K, self.bias, w.tau, w.delta,
                                   self.ws, stream=self.stream)

    def restore(self, cold=True):
        self.x.copy_(self.x0)
        self.bias.copy_(self.b0)
        if cold:
            self.xmod.probe_read(self.flush, self.flush_sums, stream=self.stream)

    def settle(self, warmup):
        """Untimed steps for at least 0.2 s (clocks settle), then the warm-up steps."""
        import torch
        t_end = time.perf_counter() + 0.2
        for _ in range(400):
            self.step()
            torch.cuda.synchronize()
            if time.perf_counter() > t_end:
                break
        for _ in range(warmup):
            self.restore()
            self.step()
        self.restore(cold=False)
        torch.cuda.synchronize()

    def timed(self, steps, slots=None, cold=True):
        """Per-step event times (ms) of `steps` steps, each from the pristine state (and, cold,
        after the cache flush), with the library's events on the kernels of `slots` (None: no
        kernel events; "all": every kernel). Returns (step times, kernel ms sums, calls)."""
        import torch
        xm = self.xmod
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        if slots is not None:
            xm.phase_timing(True, slots=None if slots == "all" else slots)
        for i in range(steps):
            self.restore(cold)
            ev[i][0].record(self.stream)
            self.step()
            ev[i][1].record(self.stream)
        torch.cuda.synchronize()
        ph, n = (xm.phase_times() if slots is not None else ({}, 0))
        if slots is not None:
            xm.phase_timing(False)
        return [a.elapsed_time(b) for a, b in ev], ph, n

    def back_to_back(self, steps, slots="all"):
        """`steps` steps back to back on the evolving state (warm caches), kernel events on."""
        import torch
        self.restore(cold=False)
        self.xmod.phase_timing(True, slots=None if slots == "all" else slots)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        ph, n = self.xmod.phase_times()
        self.xmod.phase_timing(False)
        return ph, n


def phase_table(w, phase_ms, steps):
    work = algorithmic_work(w)
    out = {}
    for name in work:
        avg = phase_ms[name] / steps
        e = {"ms": round(avg, 5)}
        if work[name]["flops"] > 0 and name.endswith(("gemm", "attention")):
            e["tflops"] = round(work[name]["flops"] / (avg * 1e-3) / 1e12, 1)
            e["frac_mfma_peak"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4)
        else:
            e["gbs"] = round(work[name]["bytes"] / (avg * 1e-3) / 1e9, 1)
            e["frac_hbm_peak"] = round(e["gbs"] / PEAK_HBM_GBS, 4)
        out[name] = e
    return out


def layer_line(run, steps, warmup):
    """Timed steps of one single-layer workload (cold, from the pristine state, the dominant
    kernel bracketed by the library's events), then the per-kernel breakdown cold and warm."""
    import statistics
    w = run.w
    run.settle(warmup)
    work = algorithmic_work(w)
    dom = max(work, key=lambda n: work[n]["flops"])
    times, dom_ms, n = run.timed(steps, slots=[dom])
    assert n == steps
    med = statistics.median(times)
    M = w.B * w.k
    dom_s = dom_ms[dom] / steps * 1e-3
    achieved = work[dom]["flops"] / dom_s / 1e12
    layer_fl = sum(v["flops"] for v in work.values())
    _, ph_cold, _ = run.timed(steps, slots="all")
    ph_warm, _ = run.back_to_back(steps)
    return {
        "ms_per_step": round(med, 5), "ms_mean": round(sum(times) / steps, 5),
        "ms_min": round(min(times), 5), "routed_tokens_per_s": round(M / (med * 1e-3), 1),
        "layer_tflops": round(layer_fl / (med * 1e-3) / 1e12, 1),
        "layer_frac_mfma_peak": round(layer_fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom, w.name),
                     "flops_per_launch": work[dom]["flops"],
                     "ms_per_launch": round(dom_s * 1e3, 5)},
        "phases_cold": phase_table(w, ph_cold, steps),
        "phases_warm": phase_table(w, ph_warm, steps),
    }


def threshold_layer(xmod, w, xb, dl, dims, steps, warmup, time_oracle=True):
    """The same layer with the eval-time causal threshold rule (ell >= 0 enters). An untrained
    router would pass half of the tokens; here its bias beta_r is set so that the expected
    share of tokens with s >= 0 is 1/K, as the rule is meant to route (s ~ N(beta_r, sigma^2),
    sigma = 0.02 * sqrt(d) for N(0, 1) activations and N(0, 0.02) router weights), and no
    carried bias is used, so every call routes about B*T/K tokens. Reports the time per call
    and routed tokens/s at the number the last call routed. Informational; the headline is the
    training-time top-k layer."""
    import statistics
    import torch
    sigma = 0.02 * math.sqrt(w.d)
    beta = -sigma * statistics.NormalDist().inv_cdf(1.0 - 1.0 / w.K)
    L = xmod.make_layer(dict(dl, router_bias=beta))
    x0 = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).cuda()
    x = x0.clone()
    n_total = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = xmod.alloc_workspace(dims, 1, xmod.WS_SPARSE_THRESHOLD)
    stream = torch.cuda.current_stream()

    # every call starts from the same hidden state (restored outside the timed calls), so the
    # routed count does not drift as in-place updates accumulate
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    for i in range(warmup + steps):
        x.copy_(x0)
        if i >= warmup:
            events[i - warmup][0].record(stream)
        xmod.sparse_layer_fwd_threshold(x, L, dims, None, w.tau, w.delta, ws, n_total_out=n_total,
                                        stream=stream)
        if i >= warmup:
            events[i - warmup][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in events) / steps
    routed = int(n_total.item())   # the same for every call
    out = {"ms_per_call": round(ms, 5), "routed_tokens": routed,
           "routed_tokens_per_s": round(routed / (ms * 1e-3), 1),
           "rule": "ell >= 0 (routing probability >= 1/2)", "router_bias": round(beta, 4),
           "timing": "each call on the same input, events around each call"}
    if time_oracle:
        import oracle
        lay = dict(wl.make_layer(w, 0), router_bias=beta)
        t0 = time.perf_counter()
        res = oracle.sparse_layer_threshold(xb[:1], lay, w, tau=w.tau, delta=w.delta)
        t1 = time.perf_counter() - t0
        n = int(np.sum(res["counts"]))
        out["cpu_baseline"] = {"value": round(n / t1, 1), "unit": "routed tokens/s",
                               "kind": "oracle", "seconds": round(t1, 3),
                               "sample": f"1 of the {w.B} sequences ({n} routed tokens), float64"}
    return out


def train_step(xmod, w, xb, dl, dims, steps, warmup, route_coef=1e-4, oracle_budget_s=6.0):
    """One training step of the same layer: xmod_sparse_layer_fwd_train (the forward that keeps
    what the backward reads) then xmod_sparse_layer_bwd (gradients of the hidden state and of
    every parameter, with the routing loss of Eq. (9) at the page's coefficient 1e-4). Each step
    starts from the same hidden state and bias (restored outside the events). In the timed steps
    the library brackets only the backward's largest product with events (its roofline); a
    further pass with events around every kernel gives the per-kernel breakdown; the backward
    oracle is timed on one sequence. Informational."""
    import torch
    L = xmod.make_layer(dl)
    x0 = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).cuda()
    bias_np = wl.make_bias(w)
    b0 = torch.from_numpy(bias_np).cuda()
    x, bias = x0.clone(), b0.clone()
    dy_np = wl.make_dy(w)
    dy = torch.from_numpy(np.ascontiguousarray(dy_np).view(np.int16)).view(torch.bfloat16).cuda()
    dx = torch.empty_like(dy)
    saved = xmod.alloc_workspace(dims, w.K, xmod.WS_TRAIN_SAVED)
    ws = xmod.alloc_workspace(dims, w.K, xmod.WS_BACKWARD)
    grads = xmod.make_grads(xmod.alloc_grads(dims))
    stream = torch.cuda.current_stream()
    work = algorithmic_work_bwd(w)
    dom = max(work, key=lambda n: work[n]["flops"])

    def one(e=None):
        x.copy_(x0)
        bias.copy_(b0)
        if e:
            e[0].record(stream)
        xmod.sparse_layer_fwd_train(x, L, dims, w.K, bias, w.tau, w.delta, saved, stream=stream)
        if e:
            e[1].record(stream)
        xmod.sparse_layer_bwd(x, dy, dx, L, dims, w.K, route_coef, saved, grads, ws,
                              stream=stream)
        if e:
            e[2].record(stream)

    for _ in range(warmup):
        one()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    xmod.phase_timing(True, slots=[dom])
    for i in range(steps):
        one(ev[i])
    torch.cuda.synchronize()
    dom_ms, _ = xmod.phase_times()
    xmod.phase_timing(False)
    fwd = sum(a.elapsed_time(b) for a, b, _ in ev) / steps
    bwd = sum(b.elapsed_time(c) for _, b, c in ev) / steps
    # breakdown
    xmod.phase_timing(True)
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    ph, _ = xmod.phase_times()
    xmod.phase_timing(False)
    phases = {}
    for name, v in work.items():
        avg = ph[name] / steps
        e = {"ms": round(avg, 5)}
        if v["flops"] > 0:
            e["tflops"] = round(v["flops"] / (avg * 1e-3) / 1e12, 1)
        if v["bytes"] > 0 and v["flops"] == 0:
            e["gbs"] = round(v["bytes"] / (avg * 1e-3) / 1e9, 1)
        phases[name] = e
    M = w.B * w.k
    fwork = algorithmic_work(w)
    f_fwd = sum(v["flops"] for k2, v in fwork.items() if k2.endswith(("gemm", "attention")))
    f_bwd = sum(v["flops"] for v in work.values())
    dom_s = dom_ms[dom] / steps * 1e-3
    ach = work[dom]["flops"] / dom_s / 1e12
    out = {"fwd_train_ms": round(fwd, 5), "bwd_ms": round(bwd, 5),
           "routed_tokens_per_s": round(M / ((fwd + bwd) * 1e-3), 1),
           "bwd_tflops": round(f_bwd / (bwd * 1e-3) / 1e12, 1),
           "step_frac_mfma_peak": round((f_fwd + f_bwd) / ((fwd + bwd) * 1e-3) / 1e12
                                        / PEAK_BF16_TFLOPS, 4),
           "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_BF16_TFLOPS, 4)},
           "phases": phases, "route_coef": route_coef,
           "timing": "each step on the same input, events around the forward and the backward"}
    if oracle_budget_s > 0:
        import oracle
        t0 = time.perf_counter()
        oracle.sparse_layer_grad(xb[:1], {k2: v for k2, v in wl.make_layer(w, 0).items()}, w,
                                 w.K, dy_np[:1], bias=bias_np[:1], tau=w.tau,
                                 route_coef=route_coef)
        t1 = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(w.k / t1, 1), "unit": "routed tokens/s",
                               "kind": "oracle", "seconds": round(t1, 3),
                               "sample": "forward and backward of 1 of the 8 sequences, float64"}
    return out


def layer_flops(w, sparse):
    """Algorithmic matrix-core flops of one layer: the projections on its rows and the causal
    attention over them (a sparse layer: the B*k routed rows; a dense layer: all B*T)."""
    P = w.d * (w.d_q + 2 * w.d_kv) + w.d_q * w.d + 3 * w.d * w.ffn_hidden
    n = w.k if sparse else w.T
    return 2.0 * w.B * n * P + 2.0 * w.B * w.n_q_heads * w.head_dim * n * (n + 1)


def blocks(xmod, steps=5, warmup=2, seed=7):
    """The two stack workloads through xmod_block_fwd: the original MoD alternation
    ([Sparse(8)] + [Dense]) x 4 at B4 x T4096, d 1536, and the X-MoD A3K16 block (one dense
    prefix layer, 48 Sparse(16) layers, one dense anchor) at B4 x T4096, d 1024. Weights are
    drawn on the device (N(0, 0.02), gains 1), activations N(0, 1); each timed call starts from
    the same hidden state. Reports the block's time and flop rate, the same block captured once
    as a HIP graph and replayed (the host launch cost of its kernels removed), and one sparse
    and one dense layer of the same shapes timed alone (routed tokens/s of the sparse layer; the
    ratio of the two layers' times; their sum over the block's layers), and for the A3K16 block
    which tokens its sparse layers route (`routing_diagnostics`). Informational."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    bf = torch.bfloat16
    out = {}
    for name in ("mod_pairs_k8_b4x4096_d1536", "a3k16_block_b4x4096_d1024"):
        w = wl.WORKLOADS[name]
        n_layers = w.N0 + w.N1 * (w.AK + 1)
        rnd = lambda *shape: (torch.randn(*shape, device="cuda", generator=g) * 0.02).to(bf)
        one = lambda *shape: torch.ones(*shape, device="cuda", dtype=bf)
        Ls = [xmod.make_layer({"w_router": rnd(w.d), "g_attn": one(w.d),
                               "w_qkv": rnd(w.d_q + 2 * w.d_kv, w.d), "w_o": rnd(w.d, w.d_q),
                               "g_ffn": one(w.d), "w_gate": rnd(w.ffn_hidden, w.d),
                               "w_up": rnd(w.ffn_hidden, w.d), "w_down": rnd(w.d, w.ffn_hidden)})
              for _ in range(n_layers)]
        dims = xmod.make_dims(w.B, w.T, w.d, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ffn_hidden,
                              w.rms_eps)
        x0 = torch.randn(w.B, w.T, w.d, device="cuda", generator=g).to(bf)
        x = x0.clone()
        bias = torch.zeros(w.B, w.T, device="cuda")
        ws = xmod.alloc_workspace(dims, w.K, xmod.WS_BLOCK)
        A = w.AK / w.K

        def timed(fn):
            for _ in range(warmup):
                x.copy_(x0)
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for e0, e1 in ev:
                x.copy_(x0)
                e0.record()
                fn()
                e1.record()
            torch.cuda.synchronize()
            return sum(a.elapsed_time(b) for a, b in ev) / steps

        t_block = timed(lambda: xmod.block_fwd(x, Ls, dims, w.N0, w.N1, A, w.K, bias, w.tau,
                                               w.delta, ws))
        # the same block captured once as a HIP graph and replayed: the launches of its
        # kernels (about nine per layer) no longer go through the host one by one
        x.copy_(x0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            xmod.block_fwd(x, Ls, dims, w.N0, w.N1, A, w.K, bias, w.tau, w.delta, ws)
        t_graph = timed(graph.replay)
        del graph
        t_sparse = timed(lambda: xmod.sparse_layer_fwd(x, Ls[w.N0], dims, w.K, bias, w.tau,
                                                       w.delta, ws))
        t_dense = timed(lambda: xmod.dense_layer_fwd(x, Ls[0], dims, ws))
        n_sparse = w.N1 * w.AK
        n_dense = n_layers - n_sparse
        routing = routing_diagnostics(xmod, w, Ls, dims, x, x0, bias, ws) if w.AK > 1 else None
        f_block = n_sparse * layer_flops(w, True) + n_dense * layer_flops(w, False)
        out[name] = {"layers": n_layers, "sparse_layers": n_sparse, "block_ms": round(t_block, 4),
                     "block_tflops": round(f_block / (t_block * 1e-3) / 1e12, 1),
                     "block_graph_replay_ms": round(t_graph, 4),
                     "layers_alone_ms": round(n_sparse * t_sparse + n_dense * t_dense, 4),
                     "sparse_layer_ms": round(t_sparse, 5), "dense_layer_ms": round(t_dense, 5),
                     "sparse_routed_tokens_per_s": round(w.B * w.k / (t_sparse * 1e-3), 1),
                     "sparse_layer_tflops": round(layer_flops(w, True) / (t_sparse * 1e-3) / 1e12, 1),
                     "dense_layer_tflops": round(layer_flops(w, False) / (t_dense * 1e-3) / 1e12, 1),
                     "sparse_over_dense_time": round(t_sparse / t_dense, 4)}
        if routing:
            out[name]["routing"] = routing
        del Ls, ws, x, x0
        torch.cuda.empty_cache()
    out["timing"] = ("events around each call (or graph replay), each from the same hidden "
                     "state")
    return out


def routing_diagnostics(xmod, w, Ls, dims, x, x0, bias, ws):
    """Which tokens the stack's sparse layers route (random-initialised weights, synthetic
    input): the stack walked layer by layer through the single-layer entry points (the same
    results as the block entry point) with each sparse layer's selection kept. coverage: the
    share of tokens routed by at least one sparse layer; adjacent_jaccard: the mean, over
    sequences and adjacent sparse layers, of |S_l & S_l+1| / |S_l | S_l+1|. Beside them the
    values for independent random choices of a 1/K share per layer, 1 - (1 - 1/K)^n and
    p / (2 - p), the references the X-MoD review's routing-diagnostics table prints."""
    import torch
    x.copy_(x0)
    idx = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
    masks = []
    n_in_block = w.AK + 1
    for i, L in enumerate(Ls):
        sparse = i >= w.N0 and (i - w.N0) % n_in_block < w.AK
        if i >= w.N0 and (i - w.N0) % n_in_block == 0:
            bias.zero_()                                  # the block start's reset
        if sparse:
            xmod.sparse_layer_fwd(x, L, dims, w.K, bias, w.tau, w.delta, ws, idx)
            m = torch.zeros((w.B, w.T), dtype=torch.bool, device="cuda")
            m.scatter_(1, idx.long(), True)
            masks.append(m)
        else:
            xmod.dense_layer_fwd(x, L, dims, ws)
    sel = torch.stack(masks)                              # [layers, B, T]
    coverage = sel.any(0).float().mean().item()
    inter = (sel[1:] & sel[:-1]).sum(-1).float()
    union = (sel[1:] | sel[:-1]).sum(-1).float()
    jac = (inter / union).mean().item()
    p = 1.0 / w.K
    n = sel.shape[0]
    return {"sparse_layers": n, "coverage": round(coverage, 5),
            "adjacent_jaccard": round(jac, 5),
            "independent_coverage": round(1.0 - (1.0 - p) ** n, 5),
            "independent_jaccard": round(p / (2.0 - p), 5),
            "bias_step": w.delta}


def measured_ceilings(w, reps=10):
    """What this GPU sustains on plain work, beside the vendor peaks the fractions use: HBM copy
    bandwidth (read + write of a 1 GiB buffer by torch's copy kernel), the library's ceiling
    probes (a streaming read of the same 1 GiB, grid-stride and in per-workgroup chunks with
    non-temporal loads; back-to-back bf16 MFMAs on every SIMD, no memory
    traffic) and the vendor GEMM library
    (torch.matmul, i.e. hipBLASLt) on the layer's gate/up shape and on 8192^3, bf16. Context
    for the roofline fractions; no part of the layer runs here."""
    import torch

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    from sparse_depth_token_amd import xmod
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del dst
    # the library's own probes: a streaming read of the same 1 GiB, back-to-back MFMAs
    sums = torch.empty(xmod.PROBE_THREADS, dtype=torch.int32, device="cuda")
    t_reads = {dep: timed(lambda: xmod.probe_read(src, sums, dep)) for dep in (4, 8, 16)}
    t_chunked = timed(lambda: xmod.probe_read_chunked(src, sums))
    del src
    # the same chunked read over a buffer of the layer's hidden-state size, each rep after the
    # cold-step flush: the bare-read time of exactly the bytes the router streams
    xb = w.B * w.T * w.d * 2
    xsrc = torch.ones(xb, dtype=torch.uint8, device="cuda")
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    t_x = []
    for _ in range(reps + 1):
        xmod.probe_read(flush, sums)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        xmod.probe_read_chunked(xsrc, sums)
        e1.record()
        torch.cuda.synchronize()
        t_x.append(e0.elapsed_time(e1) * 1e-3)
    t_x = sorted(t_x[1:])[reps // 2]
    del xsrc, flush
    acc = torch.empty(xmod.PROBE_THREADS, dtype=torch.float32, device="cuda")
    iters = 4096
    t_mfma = timed(lambda: xmod.probe_mfma(acc, iters))
    mfma_flops = 4096 * 4 * iters * 32768
    M = w.B * w.k
    out = {"hbm_copy_gbs": round(2 * n / t_copy / 1e9, 1),
           "hbm_read_gbs": round(n / min(t_reads.values()) / 1e9, 1),
           "hbm_read_gbs_by_loads_in_flight": {str(dep): round(n / t / 1e9, 1)
                                               for dep, t in t_reads.items()},
           "hbm_read_chunked_nt_gbs": round(n / t_chunked / 1e9, 1),
           "hbm_read_chunked_nt_x_bytes": {"bytes": xb, "us": round(t_x * 1e6, 1),
                                           "gbs": round(xb / t_x / 1e9, 1)},
           "mfma_bf16_tflops": round(mfma_flops / t_mfma / 1e12, 1)}
    # the same products by the vendor library and by this library's GEMM (xmod_gemm_bf16_nt,
    # plain bf16 store), one after the other on the same operands (N(0, 1), so the matrix
    # cores draw the power of random data), after a warm-up of a second each
    gemms, ours = {}, {}
    for name, (m, nn, kk) in {"gateup_shape": (M, 2 * w.ffn_hidden, w.d),
                              "square_8192": (8192, 8192, 8192)}.items():
        a = torch.randn(m, kk, device="cuda").to(torch.bfloat16)
        bw = torch.randn(nn, kk, device="cuda").to(torch.bfloat16)
        c = torch.empty(m, nn, device="cuda", dtype=torch.bfloat16)
        for label, fn in (("vendor", lambda: torch.matmul(a, bw.t(), out=c)),
                          ("ours", lambda: xmod.gemm_bf16_nt(a, bw, c))):
            t_one = timed(fn)
            for _ in range(max(1, int(1.0 / t_one))):
                fn()
            t = min(timed(fn) for _ in range(3))
            (gemms if label == "vendor" else ours)[name] = round(2.0 * m * nn * kk / t / 1e12, 1)
        del a, bw, c
    out["library_gemm_tflops"] = gemms
    out["this_library_gemm_tflops"] = ours
    out["note"] = ("torch copy (read + write), the library's streaming-read probe (4, 8 or 16 "
                   "16-byte loads in flight per thread, 1024 threads per CU; the best is "
                   "hbm_read_gbs), the chunked non-temporal read of 1 GiB and of the hidden "
                   "state's bytes after the cold-step flush (hbm_read_chunked_nt_*), the "
                   "back-to-back MFMA probe, and torch.matmul (vendor library) "
                   "beside this library's plain GEMM on the same operands, on this GPU; the "
                   "roofline fractions use the vendor peaks (8 TB/s, 2.5 PFLOP/s)")
    return out


def cpu_baseline(w, xb, lay, bias, budget_s=12.0):
    """The oracle (float64 NumPy, oracle/) on a bounded sample of the same workload on this
    host: the router and top-k over every token and, per sequence, RMSNorm, keys and values of
    the routed rows up to the last sampled one, then queries, attention, O, RMSNorm and SwiGLU
    for evenly spaced sampled rows. Passes on more rows per sequence until one takes at least
    half of budget_s (or covers every routed row); routed tokens/s = sampled rows / time of
    that pass."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def sample(n):
        n = max(1, min(w.k, n))
        rows = np.unique(np.linspace(0, w.k - 1, n).round().astype(np.int64))
        return {b: rows for b in range(w.B)}, len(rows)

    rows = 64
    while True:
        smp, n = sample(rows)
        t0 = time.perf_counter()
        oracle.sparse_layer(xb, lay, w, w.K, bias=bias, tau=w.tau, delta=w.delta, sample=smp)
        t1 = time.perf_counter() - t0
        if t1 >= 0.5 * budget_s or n >= w.k:
            break
        rows = min(w.k, int(rows * max(2.0, 0.8 * budget_s / max(t1, 1e-3))))
    routed = n * w.B
    return {"value": round(routed / t1, 1), "unit": "routed tokens/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(t1, 3),
            "sample": f"{n} of the {w.k} routed rows of each of the {w.B} sequence(s), evenly "
                      f"spaced ({routed} routed tokens; router and top-k over all {w.B * w.T} "
                      f"tokens, keys and values of the routed rows up to the last sampled one), "
                      f"float64"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-threshold", action="store_true",
                    help="skip the informational threshold-routing line")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the informational training-step (forward + backward) object")
    ap.add_argument("--no-blocks", action="store_true",
                    help="skip the informational stack workloads (MoD pairs, A3K16 block)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured bandwidth, MFMA and library GEMM ceilings")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other single-layer workloads (K=2 small layer, K=8 layer)")
    ap.add_argument("--workload", default=wl.BENCH_WORKLOAD, choices=sorted(wl.WORKLOADS),
        help="the single-layer workload of the headline (default: the long-context GQA layer); "
             "a stack workload gives one sparse layer of the stack's shape")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 256 MiB device copy first (a known-size reference for "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_depth_token_amd import xmod

    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = wl.WORKLOADS[args.workload]
    print(f"[bench] {w.name}: drawing inputs", file=sys.stderr, flush=True)
    run = LayerRun(xmod, w)
    print(f"[bench] {w.name}: timing", file=sys.stderr, flush=True)
    head = layer_line(run, args.steps, args.warmup)
    assert torch.isfinite(run.x.float()).all().item(), "non-finite hidden state"
    M = w.B * w.k
    out = {
        "metric": METRIC, "value": head["routed_tokens_per_s"], "unit": "routed tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "d": w.d, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "ffn_hidden": w.ffn_hidden,
                   "K": w.K, "routed_tokens_per_step": M, "parallelism": "none (1 GPU)"},
        "timing": "median of per-step events; each step from pristine x and bias after a "
                  "512 MiB cache flush by a streaming read (outside the events)",
        "ms_mean": head["ms_mean"], "ms_min": head["ms_min"],
        "layer_tflops": head["layer_tflops"], "layer_frac_mfma_peak": head["layer_frac_mfma_peak"],
        "roofline": head["roofline"],
        "phases_cold": head["phases_cold"], "phases_warm": head["phases_warm"],
    }
    xb, lay, bias_np = run.xb, run.lay, run.bias_np
    del run
    torch.cuda.empty_cache()
    if not args.no_configs:
        cfgs = {}
        for name in ("sparse_k2_b2x512_d256", "sparse_k8_b8x4096_d2048"):
            if name == w.name:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            r = LayerRun(xmod, wl.WORKLOADS[name])
            cfgs[name] = layer_line(r, args.steps, args.warmup)
            if not args.no_cpu_baseline:  # the oracle on this workload, a few seconds' sample
                cfgs[name]["cpu_baseline"] = cpu_baseline(r.w, r.xb, r.lay, r.bias_np,
                                                          budget_s=4.0)
            del r
            torch.cuda.empty_cache()
        out["configs"] = cfgs
    k8 = wl.WORKLOADS["sparse_k8_b8x4096_d2048"]
    if not (args.no_threshold and args.no_train):
        r = LayerRun(xmod, k8)
        if not args.no_threshold:
            print("[bench] threshold layer", file=sys.stderr, flush=True)
            out["threshold_layer"] = threshold_layer(xmod, k8, r.xb, r.dl, r.dims, args.steps,
                                                     args.warmup,
                                                     time_oracle=not args.no_cpu_baseline)
        if not args.no_train:
            print("[bench] training step", file=sys.stderr, flush=True)
            out["train_step"] = train_step(xmod, k8, r.xb, r.dl, r.dims, args.steps, args.warmup,
                                           oracle_budget_s=0.0 if args.no_cpu_baseline else 6.0)
        del r
        torch.cuda.empty_cache()
    if not args.no_blocks:
        print("[bench] stacks", file=sys.stderr, flush=True)
        out["blocks"] = blocks(xmod)
    if not args.no_ceilings:
        print("[bench] ceilings", file=sys.stderr, flush=True)
        out["measured_ceilings"] = measured_ceilings(w)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, xb, lay, bias_np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
