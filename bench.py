#!/usr/bin/env python3
"""Benchmark of the TwELL sparse-FFN forward on one MI355X.

One step = one call of twell_ffn_forward (gate matmul + TwELL epilogue,
sparse up projection, which also finds the overflow rows, sparse down
projection, overflow-row list, dense fallback) over the whole token batch of
the workload, with inputs resident in HBM.

Timing protocol (HIP events on the launch stream, W untimed warm-up calls
first, then exactly K timed calls; median, min and p90 reported beside the
mean):
  cold (primary)  a 1 GiB buffer is rewritten before every timed call,
                  outside its events, so weights and activations come from
                  HBM (L2 and the 256 MB Infinity Cache evicted), as for a
                  layer whose weights another layer has just displaced;
  warm            K calls back to back, everything the previous call left in
                  the caches.
Before any timed loop the dense layer runs untimed for 50 ms, past the clock
dip of a freshly loaded GPU.  Prints ONE JSON line on stdout:

  value        tokens/s of the sparse forward, cold (T * K / sum of the K times)
  roofline     the dominant kernel (the gate matmul with the TwELL epilogue)
               against the bf16 matrix-core peak, duration measured live
  cpu_baseline the float64 CPU oracle, three passes over the batch (median)
  workloads    the skewed and larger-layer workloads (forward, own dense and
               torch dense FFN, cold and warm) and the density sweep
  speedups, stage times, gather byte rates, training formats, backward, the
               fused up+down kernel, the HBM and matrix-core probes

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
                       [--no-cpu-baseline] [--no-extra] [--no-torch] [--no-cold]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-FFN tokens/s at 99% sparsity; achieved HBM GB/s vs peak; speedup vs dense"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
# L2 read bandwidth from the unit counts: 8 XCDs x 16 L2 channels x 128 bytes
# per clock at the 2.4 GHz peak clock (the CDNA L2 organisation)
L2_PEAK_GBS = 8 * 16 * 128 * 2.4
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3
HYBRID_WIDTH = 256           # ELL slots per row for the TwELL -> hybrid timing
L1_LAMBDA = 2e-5             # L1 coefficient of the training recipe


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="layer_1p5b_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work to aim for per pass")
    p.add_argument("--cpu-reps", type=int, default=3, help="oracle passes (the median is reported)")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the skewed / larger-layer workloads and the density sweep")
    p.add_argument("--no-torch", action="store_true", help="skip the torch (hipBLASLt) dense FFN")
    p.add_argument("--no-cold", action="store_true", help="time warm only (profiling runs)")
    return p.parse_args()


def to_dev(a, dtype, dev):
    import numpy as np
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def event_time(fn, steps, warmup):
    """Average ms per call over exactly `steps` calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall


def split_time(first, second, steps, warmup):
    """Run `steps` steps of first(); second() with events around each part, all on
    the current stream: the same launch sequence as the fused entry point, with
    each kernel's average duration measured in that sequence."""
    import torch
    for _ in range(warmup):
        first()
        second()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
    for i in range(steps):
        ev[2 * i].record(s)
        first()
        ev[2 * i + 1].record(s)
        second()
    ev[2 * steps].record(s)
    torch.cuda.synchronize()
    a = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)) / steps
    b = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(steps)) / steps
    return a, b


def stats_us(times_ms):
    """mean / median / min / p90 (microseconds) of a list of per-call times."""
    t = sorted(times_ms)
    n = len(t)
    if n == 0:
        return None
    p90 = t[min(n - 1, int(round(0.9 * (n - 1))))]
    return {"mean_us": 1e3 * sum(t) / n, "median_us": 1e3 * t[n // 2], "min_us": 1e3 * t[0],
            "p90_us": 1e3 * p90, "n": n}


def cold_times(fn, reps, warmup, flush_buf):
    """Per-call ms of `reps` calls, each after rewriting a 1 GiB buffer (evicts L2
    and the Infinity Cache) outside its events; `warmup` untimed calls first."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = []
    for _ in range(reps):
        flush_buf.add_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def warm_times(fn, reps, warmup):
    """Per-call ms of `reps` back-to-back calls (one event between consecutive
    calls) and the mean over the whole run (events only at its ends)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(s)
    for i in range(reps):
        fn()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return per, ev[0].elapsed_time(ev[reps]) / reps


def n_dense_rows_bytes(packed, F, s):
    """Bytes of the dense backup rows a TwELL matrix holds."""
    return min(int(packed.n_ovf.item()), packed.ovf_cap) * F * s


def gather_bytes(T, d, F, tile, cap, s, nnz_kept, rows_sparse):
    """Algorithmic bytes of the up + down stages: one W_u^T row and one W_d row per
    active entry of the non-overflow rows, the x row read and y row written per
    such token, and the TwELL row (counts, values, indices) it reads."""
    nt = F // tile
    return (nnz_kept * 2 * d * s + rows_sparse * d * (s + s)
            + rows_sparse * nt * (2 + cap * (s + 1)))


def settle(fn, settle_ms=50.0):
    """Run fn untimed for settle_ms: under sustained load the clocks of a fresh
    GPU dip for some milliseconds before they settle."""
    import torch
    t_end = time.perf_counter() + settle_ms * 1e-3
    while time.perf_counter() < t_end:
        fn()
        torch.cuda.synchronize()


def forward_timings(w, x, wg, wu, wd, b, steps, warmup, flush, want_torch=True, want_split=True):
    """The sparse forward, the library's dense FFN and a torch (hipBLASLt) dense
    FFN on the same device inputs: cold and warm per-call statistics, the gate
    kernel back to back, and the gate / rest split inside the sequence."""
    import numpy as np
    import torch
    import activation_sparse_transformer_bf16_amd as tw

    dev = x.device
    T, d, F = w.T, w.d, w.F
    packed = tw.TwellMatrix.empty(T, F, w.tile, w.cap, x.dtype, dev, T, dense=False)
    y = torch.empty((T, d), dtype=x.dtype, device=dev)
    ws = torch.empty((tw.twell_ffn_workspace_size(T, d, F, w.tile, w.cap, x.dtype),), dtype=torch.uint8,
                     device=dev)
    yd = torch.empty_like(y)
    wsd = torch.empty((tw.dense_ffn_workspace_size(T, d, F, x.dtype),), dtype=torch.uint8, device=dev)
    sparse = lambda: tw.twell_ffn_forward(x, wg, wu, wd, b, packed=packed, y=y, workspace=ws)
    gate = lambda: tw.twell_gate_pack(x, wg, b, packed=packed, scan=False)
    rest = lambda: tw.twell_sparse_ffn(packed, x, wg, wu, wd, b, y=y, workspace=ws)
    dense = lambda: tw.dense_ffn_forward(x, wg, wu, wd, b, y=yd, workspace=wsd)
    settle(dense)

    r = {"workload": w.name}
    # the headline protocol: exactly `steps` timed calls after `warmup`
    if flush is not None:
        t = cold_times(sparse, steps, warmup, flush)
        r["sparse_cold"] = stats_us(t)
        r["sparse_cold_ms_list"] = t
        r["dense_cold"] = stats_us(cold_times(dense, steps, warmup, flush))
    per, mean = warm_times(sparse, steps, warmup)
    r["sparse_warm"] = {**stats_us(per), "back_to_back_mean_us": mean * 1e3}
    per, mean = warm_times(dense, steps, warmup)
    r["dense_warm"] = {**stats_us(per), "back_to_back_mean_us": mean * 1e3}
    # The gate kernel's average launch duration: the same launch back to back,
    # events only around the whole run, which is what a kernel trace's
    # per-launch average measures.
    _, ms_gate_b2b = warm_times(gate, steps, warmup)
    r["gate_back_to_back_us"] = ms_gate_b2b * 1e3
    if want_split:
        ms_gate, ms_rest = split_time(gate, rest, steps, warmup)
        r["gate_in_sequence_us"], r["rest_in_sequence_us"] = ms_gate * 1e3, ms_rest * 1e3
    if want_torch:
        import torch.nn.functional as Fn

        def torch_dense():
            pre = torch.addmm(b[:, None].to(x.dtype), x, wg.t())  # bias in the activation dtype
            a = torch.relu(pre) * Fn.linear(x, wu)
            return a @ wd

        per, mean = warm_times(torch_dense, steps, warmup)
        r["torch_dense_warm"] = {**stats_us(per), "back_to_back_mean_us": mean * 1e3}
        if flush is not None:
            r["torch_dense_cold"] = stats_us(cold_times(torch_dense, steps, warmup, flush))
    sparse()
    torch.cuda.synchronize()
    cnt = packed.cnt.cpu().numpy().view(np.uint16).astype(np.int64)
    r["n_ovf"] = int(packed.n_ovf.item())
    r["density"] = float(cnt.sum()) / (T * F)
    ovf = (cnt > w.cap).any(axis=1)
    r["nnz"], r["nnz_kept"], r["rows_sparse"] = int(cnt.sum()), int(cnt[~ovf].sum()), int((~ovf).sum())
    r["gate_tflops"] = 2.0 * T * d * F / (ms_gate_b2b * 1e-3) / 1e12
    key = "sparse_cold" if flush is not None else "sparse_warm"
    dkey = "dense_cold" if flush is not None else "dense_warm"
    r["speedup_vs_dense"] = r[dkey]["mean_us"] / r[key]["mean_us"]
    if want_torch:
        tkey = "torch_dense_cold" if flush is not None else "torch_dense_warm"
        r["speedup_vs_torch_dense"] = r[tkey]["mean_us"] / r[key]["mean_us"]
    r["tokens_per_s"] = T / (r[key]["mean_us"] * 1e-6)
    r["tokens_per_s_warm"] = T / (r["sparse_warm"]["back_to_back_mean_us"] * 1e-6)
    r["speedup_vs_dense_warm"] = r["dense_warm"]["back_to_back_mean_us"] / r["sparse_warm"]["back_to_back_mean_us"]
    log(f"[bench] {w.name}: forward {r[key]['mean_us']:.1f} us ({key}), warm "
        f"{r['sparse_warm']['back_to_back_mean_us']:.1f} us; own dense {r[dkey]['mean_us']:.1f} us; gate "
        f"{r['gate_back_to_back_us']:.1f} us; n_ovf {r['n_ovf']}; speedup {r['speedup_vs_dense']:.2f}x")
    bufs = (packed, y, ws, yd, wsd)
    return r, bufs


def backward_timing(w, hy, x, wg, wu, wd, b, nnz_all, steps, warmup, want_torch):
    """twell_ffn_backward from the hybrid activations hy (every dense row kept):
    dx and the three weight gradients with the L1 term, for a seeded dy; and
    torch's dense backward beside it."""
    import torch

    import activation_sparse_transformer_bf16_amd as tw
    from workloads.synth import grad_output
    dev = x.device
    T, d, F = w.T, w.d, w.F
    s = 2 if w.dtype == "bf16" else 4
    n_dense = int(hy.n_dense.item())
    dy = to_dev(grad_output(T, d, w.dtype, seed=0), w.dtype, dev)
    bw_ws = torch.empty((tw.twell_ffn_backward_workspace_size(T, d, F, HYBRID_WIDTH, hy.dense_cap, x.dtype),),
                        dtype=torch.uint8, device=dev)
    dxb = torch.empty_like(x)
    dwb = [torch.empty((F, d), dtype=torch.float32, device=dev) for _ in range(3)]
    bw = lambda: tw.twell_ffn_backward(hy, x, wg, wu, wd, dy, L1_LAMBDA, dxb, *dwb, workspace=bw_ws)
    ms_bw, _ = event_time(bw, steps, warmup)
    # the same without the forward's saved u (the backward gathers W_u rows
    # again to recompute it)
    ms_bw_recompute = None
    if hy.u is not None:
        saved_u, hy.u = hy.u, None
        ms_bw_recompute, _ = event_time(bw, steps, warmup)
        hy.u = saved_u
    # gathered per active entry: W_u and W_d rows (entry gradients), W_u and
    # W_g rows (dx), x and dy rows (weight gradients); plus the weight
    # gradients written once and the x / dy / dx rows
    bw_bytes = nnz_all * 6 * d * s + 3 * F * d * 4 + 3 * T * d * s
    # compulsory: every weight row once, x and dy read, dx and the fp32
    # weight gradients written once
    bw_comp = 3 * F * d * s + 3 * T * d * s + 3 * F * d * 4
    backward = {"us": ms_bw * 1e3, "tokens_per_s": T / (ms_bw * 1e-3), "hybrid_width": HYBRID_WIDTH,
                "saved_u": hy.u is not None,
                "us_recomputing_u": ms_bw_recompute * 1e3 if ms_bw_recompute is not None else None,
                "n_dense": n_dense, "entries": nnz_all, "bytes_alg": bw_bytes,
                "effective_GBps": bw_bytes / (ms_bw * 1e-3) / 1e9,
                "compulsory_bytes": bw_comp,
                "compulsory_frac_of_hbm_peak": bw_comp / (ms_bw * 1e-3) / 1e9 / HBM_PEAK_GBS, "lam": L1_LAMBDA,
                "note": "twell_ffn_backward: dx (activation dtype) and fp32 dW_g, dW_u, dW_d from the hybrid "
                        "activations; bytes_alg = 6 rows of d per active entry + weight gradients + x, dy, dx "
                        "(an effective rate: L2-served re-reads counted, not a roofline fraction); "
                        "compulsory = each weight row, x, dy, dx and the weight gradients once"}
    log(f"[bench] {w.name} backward {ms_bw * 1e3:.1f} us ({n_dense} dense rows; "
        f"{backward['effective_GBps']:.0f} GB/s effective)"
        + (f"; recomputing u {ms_bw_recompute * 1e3:.1f} us" if ms_bw_recompute is not None else ""))
    if want_torch:
        import torch.nn.functional as Fn
        hd = torch.relu(torch.addmm(b[:, None].to(x.dtype), x, wg.t()))
        ud = Fn.linear(x, wu)

        def torch_backward():  # dense, with h and u saved by the forward (bf16 outputs)
            da = dy @ wd.t()
            du = da * hd
            dp = (da * ud + L1_LAMBDA) * (hd > 0)
            return du @ wu + dp @ wg, du.t() @ x, dp.t() @ x, (hd * ud).t() @ dy

        ms_tbw, _ = event_time(torch_backward, steps, warmup)
        backward["torch_dense_backward_us"] = ms_tbw * 1e3
        backward["speedup_vs_torch_dense_backward"] = ms_tbw / ms_bw
        log(f"[bench] torch (hipBLASLt) dense backward {ms_tbw * 1e3:.1f} us")
        del hd, ud
    del dy, bw_ws, dxb, dwb
    return backward


def training_step_timing(w, x, wg, wu, wd, b, ws, y, packed_tr, hy, steps, warmup, want_torch):
    """One training step of the layer on this batch, timed as one sequence:
    the forward that saves u (twell_ffn_forward with packed.u), the TwELL ->
    hybrid conversion, the L1 norm of h and the backward (dx and the three
    weight gradients with the L1 term); beside it torch's dense forward and
    backward of the same layer (bf16 matmuls, h and u kept)."""
    import torch

    import activation_sparse_transformer_bf16_amd as tw
    from workloads.synth import grad_output
    dev = x.device
    T, d, F = w.T, w.d, w.F
    dy = to_dev(grad_output(T, d, w.dtype, seed=0), w.dtype, dev)
    bw_ws = torch.empty((tw.twell_ffn_backward_workspace_size(T, d, F, HYBRID_WIDTH, hy.dense_cap, x.dtype),),
                        dtype=torch.uint8, device=dev)
    l1_out = torch.empty((1,), dtype=torch.float64, device=dev)
    l1_ws = torch.empty((tw.twell_l1_workspace_size(),), dtype=torch.uint8, device=dev)
    dxb = torch.empty_like(x)
    dwb = [torch.empty((F, d), dtype=torch.float32, device=dev) for _ in range(3)]

    def step():
        tw.twell_ffn_forward(x, wg, wu, wd, b, packed=packed_tr, y=y, workspace=ws)
        tw.twell_to_hybrid(packed_tr, HYBRID_WIDTH, out=hy)
        tw.twell_l1_norm(packed_tr, out=l1_out, workspace=l1_ws)
        tw.twell_ffn_backward(hy, x, wg, wu, wd, dy, L1_LAMBDA, dxb, *dwb, workspace=bw_ws)

    ms_step, _ = event_time(step, steps, warmup)
    out = {"us": ms_step * 1e3, "tokens_per_s": T / (ms_step * 1e-3),
           "note": "forward saving u + TwELL->hybrid + L1 norm + backward (dx, dW_g, dW_u, dW_d with the L1 term), "
                   "one sequence on the launch stream, warm"}
    log(f"[bench] {w.name} training step (forward + hybrid + L1 + backward) {ms_step * 1e3:.1f} us")
    if want_torch:
        bcol = b[:, None].to(x.dtype)

        def torch_step():  # dense forward keeping h and u, then the dense backward
            hd = torch.relu(torch.addmm(bcol, x, wg.t()))
            ud = x @ wu.t()
            a = hd * ud
            yt = a @ wd
            da = dy @ wd.t()
            du = da * hd
            dp = (da * ud + L1_LAMBDA) * (hd > 0)
            return yt, du @ wu + dp @ wg, du.t() @ x, dp.t() @ x, a.t() @ dy

        ms_t, _ = event_time(torch_step, steps, warmup)
        out["torch_dense_step_us"] = ms_t * 1e3
        out["speedup_vs_torch_dense_step"] = ms_t / ms_step
        log(f"[bench] torch (hipBLASLt) dense training step {ms_t * 1e3:.1f} us")
    del dy, bw_ws, l1_out, l1_ws, dxb, dwb
    return out


def measure(w, steps, warmup, want_torch=True, want_cold=True):
    import numpy as np
    import torch
    import activation_sparse_transformer_bf16_amd as tw

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    inp = w.inputs()
    log(f"[bench] inputs for {w.name} generated in {time.perf_counter() - t0:.1f}s")
    x, wg, wu, wd = (to_dev(a, w.dtype, dev) for a in (inp.x, inp.w_gate, inp.w_up, inp.w_down))
    b = torch.from_numpy(inp.gate_bias).to(dev)
    T, d, F = w.T, w.d, w.F
    s = 2 if w.dtype == "bf16" else 4
    flush = torch.empty((1 << 28,), dtype=torch.float32, device=dev) if want_cold else None

    fw, (packed, y, ws, yd, wsd) = forward_timings(w, x, wg, wu, wd, b, steps, warmup, flush, want_torch)
    gate = lambda: tw.twell_gate_pack(x, wg, b, packed=packed, scan=False)

    # The fused up+down kernel (one wave per token, both gathers in one flow)
    # in place of the two XCD-placed gather kernels, same gate and fallback.
    fused_rest = lambda: tw.twell_sparse_ffn_fused(packed, x, wg, wu, wd, b, y=y, workspace=ws)
    _, ms_fused_rest = split_time(gate, fused_rest, steps, warmup)
    ms_fused, _ = event_time(lambda: (gate(), fused_rest()), steps, warmup)
    log(f"[bench] fused up+down: {ms_fused_rest * 1e3:.1f} us in sequence, forward {ms_fused * 1e3:.1f} us")
    # The hidden-group-major fused prototype (fp32 partial output rows per
    # group, added in group order by a second kernel).
    grouped = None
    if w.d <= (4096 if w.dtype == "bf16" else 2048):
        ws_g = torch.empty((tw.twell_sparse_ffn_grouped_workspace_size(T, d, F, w.tile, w.cap, x.dtype),),
                           dtype=torch.uint8, device=dev)
        grouped_rest = lambda: tw.twell_sparse_ffn_grouped(packed, x, wg, wu, wd, b, y=y, workspace=ws_g)
        ms_gate_r, ms_grouped_rest = split_time(gate, grouped_rest, steps, warmup)
        ms_grouped, _ = event_time(lambda: (gate(), grouped_rest()), steps, warmup)
        grouped = {"forward_us": ms_grouped * 1e3, "gate_us": ms_gate_r * 1e3, "up_down_fallback_us": ms_grouped_rest * 1e3,
                   "partial_bytes": ws_g.numel() - tw.twell_ffn_workspace_size(T, d, F, w.tile, w.cap, x.dtype)}
        log(f"[bench] grouped fused up+down: gate {ms_gate_r * 1e3:.1f} us, {ms_grouped_rest * 1e3:.1f} us in "
            f"sequence, forward {ms_grouped * 1e3:.1f} us")
        # the same over the tile-major TwELL layout written by the gate (a
        # tile's records of consecutive tokens contiguous)
        packed_t = tw.TwellMatrix.empty(T, F, w.tile, w.cap, x.dtype, dev, T, dense=True, layout="tiles")
        gate_t = lambda: tw.twell_gate_pack(x, wg, b, packed=packed_t, scan=False)
        grouped_t_rest = lambda: tw.twell_sparse_ffn_grouped(packed_t, x, wg, wu, wd, b, y=y, workspace=ws_g)
        ms_gate_t, ms_grouped_t_rest = split_time(gate_t, grouped_t_rest, steps, warmup)
        ms_grouped_t, _ = event_time(lambda: (gate_t(), grouped_t_rest()), steps, warmup)
        grouped["tile_major"] = {"forward_us": ms_grouped_t * 1e3, "gate_us": ms_gate_t * 1e3,
                                 "up_down_fallback_us": ms_grouped_t_rest * 1e3}
        log(f"[bench] grouped fused up+down over tile-major TwELL: gate {ms_gate_t * 1e3:.1f} us, "
            f"{ms_grouped_t_rest * 1e3:.1f} us in sequence, forward {ms_grouped_t * 1e3:.1f} us")
        del ws_g, packed_t

    # Training-format kernels on this batch's TwELL matrix (with its dense
    # backup rows): TwELL -> hybrid at an ELL width of 256, the L1 norm and the
    # L1 gradient.
    packed_tr = tw.TwellMatrix.empty(T, F, w.tile, w.cap, x.dtype, dev, T, dense=True, u=True)
    tw.twell_ffn_forward(x, wg, wu, wd, b, packed=packed_tr, y=y, workspace=ws)
    hy = tw.TwellHybrid.empty(T, F, HYBRID_WIDTH, x.dtype, dev, u=True)
    l1_out = torch.empty((1,), dtype=torch.float64, device=dev)
    l1_ws = torch.empty((tw.twell_l1_workspace_size(),), dtype=torch.uint8, device=dev)
    gval, gdense = torch.empty_like(packed_tr.val), torch.empty_like(packed_tr.dense)
    ms_hybrid, _ = event_time(lambda: tw.twell_to_hybrid(packed_tr, HYBRID_WIDTH, out=hy), steps, warmup)
    ms_l1, _ = event_time(lambda: tw.twell_l1_norm(packed_tr, out=l1_out, workspace=l1_ws), steps, warmup)
    ms_l1g, _ = event_time(lambda: tw.twell_l1_grad(packed_tr, L1_LAMBDA, gval, gdense), steps, warmup)
    torch.cuda.synchronize()
    n_dense = int(hy.n_dense.item())
    nnz_all = int(packed_tr.cnt.cpu().numpy().view(np.uint16).astype(np.int64).sum())
    nt = F // w.tile
    # bytes the conversion must move: counts and used slots read, ELL rows
    # (values + int32 columns) and counts written, dense rows copied
    hybrid_bytes = (T * nt * 2 + nnz_all * (s + 1) + T * 4 + T * HYBRID_WIDTH * (s + 4)
                    + n_dense * F * s * 2)
    # Activation memory kept for back-propagation: the dense h, the TwELL
    # matrix (cnt, val, idx and its dense backup rows), and the hybrid
    # format (cnt, ELL values and int32 columns, the dense row list and rows).
    n_ovf_tr = int(packed_tr.n_ovf.item())
    # The saved u (fp32 per TwELL slot, then per ELL entry) is counted apart:
    # it trades memory for the backward's W_u gather.
    mem = {"dense_h_bytes": T * F * s,
           "twell_bytes": T * nt * (2 + w.cap * (s + 1)) + n_ovf_tr * (4 + F * s),
           "hybrid_bytes": T * 4 + T * HYBRID_WIDTH * (s + 4) + n_dense * (4 + F * s),
           "twell_saved_u_bytes": T * nt * w.cap * 4,
           "hybrid_saved_u_bytes": T * HYBRID_WIDTH * 4}
    mem["twell_over_dense"] = mem["twell_bytes"] / mem["dense_h_bytes"]
    mem["hybrid_over_dense"] = mem["hybrid_bytes"] / mem["dense_h_bytes"]
    log(f"[bench] activation memory: dense {mem['dense_h_bytes'] / 2**20:.0f} MiB, TwELL "
        f"{mem['twell_bytes'] / 2**20:.1f} MiB, hybrid {mem['hybrid_bytes'] / 2**20:.1f} MiB")
    training = {"hybrid_width": HYBRID_WIDTH, "n_dense": n_dense, "activation_memory": mem,
                "to_hybrid_us": ms_hybrid * 1e3, "to_hybrid_GBps": hybrid_bytes / (ms_hybrid * 1e-3) / 1e9,
                "l1_norm_us": ms_l1 * 1e3, "l1_grad_us": ms_l1g * 1e3,
                "note": "TwELL -> hybrid conversion, ||h||_1 and its gradient on this batch; GBps over the "
                        "bytes the conversion must move; twell_pack of the batch's rounded gate "
                        "pre-activations (read T*F values, write the TwELL matrix)"}
    log(f"[bench] training formats: to_hybrid {ms_hybrid * 1e3:.1f} us, l1 norm {ms_l1 * 1e3:.1f} us, "
        f"l1 grad {ms_l1g * 1e3:.1f} us")
    del l1_out, l1_ws, gval, gdense

    # Backward from these hybrid activations (every dense row kept): dx and
    # the three weight gradients with the L1 term, for a seeded dy.
    backward = backward_timing(w, hy, x, wg, wu, wd, b, nnz_all, steps, warmup, want_torch)
    backward["training_step"] = training_step_timing(w, x, wg, wu, wd, b, ws, y, packed_tr, hy, steps, warmup,
                                                     want_torch)
    del packed_tr, hy

    # Standalone twell_pack of this batch's rounded gate pre-activations
    # (dumped once by the gate kernel): HBM-bound, T*F*s bytes read plus the
    # TwELL matrix written.
    packed_p = tw.TwellMatrix.empty(T, F, w.tile, w.cap, x.dtype, dev, T, dense=True)
    _, pre = tw.twell_gate_pack(x, wg, b, packed=packed_p, pre_out=True, scan=False)
    ms_pack, _ = event_time(lambda: tw.twell_pack(pre, w.tile, w.cap, out=packed_p), steps, warmup)
    pack_bytes = T * F * s + T * nt * (2 + w.cap * (s + 1)) + n_dense_rows_bytes(packed_p, F, s)
    training["twell_pack_us"] = ms_pack * 1e3
    training["twell_pack_GBps"] = pack_bytes / (ms_pack * 1e-3) / 1e9
    training["twell_pack_frac_of_hbm_peak"] = pack_bytes / (ms_pack * 1e-3) / 1e9 / HBM_PEAK_GBS
    log(f"[bench] twell_pack {ms_pack * 1e3:.1f} us ({training['twell_pack_GBps']:.0f} GB/s)")
    del pre, packed_p

    # A plain device copy of known size (256 MiB read + 256 MiB written): the
    # measured HBM copy bandwidth beside the 8 TB/s spec; in rocprofv3 counter
    # runs its FETCH_SIZE / WRITE_SIZE readings also calibrate the byte counters.
    src = torch.empty((1 << 26,), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms_copy, _ = event_time(lambda: dst.copy_(src), steps, warmup)
    copy_gbs = 2 * src.numel() * 4 / (ms_copy * 1e-3) / 1e9
    log(f"[bench] device copy of 256 MiB: {copy_gbs:.0f} GB/s")
    training["twell_pack_frac_of_measured_copy"] = training["twell_pack_GBps"] / copy_gbs
    del src, dst

    # The library's own streaming probe: 1 GiB read, and 512 MiB copied into
    # 512 MiB (both well beyond the 256 MB Infinity Cache).
    big = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
    sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    ms_read, _ = event_time(lambda: tw.twell_stream_probe(big, sink, 0), steps, warmup)
    half = big.numel() // 2
    lo, hi = big[:half], big[half:]
    ms_pcopy, _ = event_time(lambda: tw.twell_stream_probe(lo, hi, 1), steps, warmup)
    probe = {"read_GBps": big.numel() / (ms_read * 1e-3) / 1e9,
             "copy_GBps": 2 * half / (ms_pcopy * 1e-3) / 1e9}
    probe["read_frac_of_spec"] = probe["read_GBps"] / HBM_PEAK_GBS
    probe["copy_frac_of_spec"] = probe["copy_GBps"] / HBM_PEAK_GBS
    probe["note"] = ("twell_stream_probe: one 16-byte chunk per thread; read 1 GiB, copy 512 MiB -> 512 MiB "
                     "(bytes read + written); twell_mfma_probe: 32x32x16 bf16 MFMAs on registers; the measured "
                     "denominators beside the 8 TB/s and 2.5 PFLOP/s specs")
    training["twell_pack_frac_of_measured_read"] = training["twell_pack_GBps"] / probe["read_GBps"]
    # The library's matrix-core probe: the sustained bf16 MFMA rate of this
    # device (1024 workgroups of 8 waves, 8 independent MFMAs per round).
    mfma_flops = [0.0]

    def mfma_run():
        mfma_flops[0] = tw.twell_mfma_probe(sink, 2000, 1024)
    ms_mfma, _ = event_time(mfma_run, steps, warmup)
    probe["mfma_bf16_TFLOPs"] = mfma_flops[0] / (ms_mfma * 1e-3) / 1e12
    probe["mfma_frac_of_spec"] = probe["mfma_bf16_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
    log(f"[bench] mfma probe: {probe['mfma_bf16_TFLOPs']:.0f} TFLOP/s bf16")
    log(f"[bench] stream probe: read {probe['read_GBps']:.0f} GB/s, copy {probe['copy_GBps']:.0f} GB/s")
    del big, lo, hi, sink

    B_alg = gather_bytes(T, d, F, w.tile, w.cap, s, fw["nnz_kept"], fw["rows_sparse"])
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    res = {
        "T": T, "forward": fw, "gather_bytes": B_alg, "peak": peak,
        "training": training, "backward": backward, "copy_gbs": copy_gbs, "probe": probe,
        "fused": {"forward_us": ms_fused * 1e3, "up_down_fallback_us": ms_fused_rest * 1e3,
                  "two_kernel_up_down_fallback_us": fw["rest_in_sequence_us"],
                  "grouped": grouped,
                  "note": "gate then twell_sparse_ffn_fused (up and down in one kernel, one wave per token), and "
                          "gate then twell_sparse_ffn_grouped (hidden-group-major fused kernel with per-group fp32 "
                          "partial output rows), warm, back to back; the headline uses the two XCD-placed "
                          "gather kernels"},
    }
    del x, wg, wu, wd, b, packed, y, ws, yd, wsd, flush
    torch.cuda.empty_cache()
    return res, inp


def extra_workloads(args, base_inp):
    """The skewed and larger-layer workloads and the density sweep: forward, own
    dense FFN and torch dense FFN, cold and warm, with the same protocol."""
    import numpy as np
    import torch

    import activation_sparse_transformer_bf16_amd as tw
    from workloads import CONFIGS, workload
    from workloads.configs import SWEEP_DENSITIES

    dev = torch.device("cuda:0")
    flush = torch.empty((1 << 28,), dtype=torch.float32, device=dev) if not args.no_cold else None
    out = {}
    for name in ("skewed_bf16", "large_bf16"):
        w = CONFIGS[name]
        t0 = time.perf_counter()
        inp = w.inputs()
        log(f"[bench] inputs for {name} generated in {time.perf_counter() - t0:.1f}s")
        x, wg, wu, wd = (to_dev(a, w.dtype, dev) for a in (inp.x, inp.w_gate, inp.w_up, inp.w_down))
        b = torch.from_numpy(inp.gate_bias).to(dev)
        r, bufs = forward_timings(w, x, wg, wu, wd, b, args.steps, args.warmup, flush, not args.no_torch)
        r.pop("sparse_cold_ms_list", None)
        r["config"] = w.summary()
        if name == "skewed_bf16":
            # the backward on the skewed batch: its hot rows are the hybrid's
            # dense backup rows
            ws = bufs[2]
            packed_tr = tw.TwellMatrix.empty(w.T, w.F, w.tile, w.cap, x.dtype, dev, w.T, dense=True, u=True)
            tw.twell_ffn_forward(x, wg, wu, wd, b, packed=packed_tr, y=bufs[1], workspace=ws)
            hy = tw.TwellHybrid.empty(w.T, w.F, HYBRID_WIDTH, x.dtype, dev, u=True)
            tw.twell_to_hybrid(packed_tr, HYBRID_WIDTH, out=hy)
            torch.cuda.synchronize()
            nnz_all = int(packed_tr.cnt.cpu().numpy().view(np.uint16).astype(np.int64).sum())
            r["backward"] = backward_timing(w, hy, x, wg, wu, wd, b, nnz_all, args.steps, args.warmup,
                                            not args.no_torch)
            del packed_tr, hy
        out[name] = r
        del x, wg, wu, wd, b, bufs, inp
        torch.cuda.empty_cache()
    # the sweep reuses the 1.5B-class x and weights; only the gate bias changes
    base = CONFIGS["layer_1p5b_bf16"]
    x, wg, wu, wd = (to_dev(a, base.dtype, dev) for a in (base_inp.x, base_inp.w_gate, base_inp.w_up,
                                                          base_inp.w_down))
    sweep = []
    for rho in SWEEP_DENSITIES:
        w = workload(f"sweep@{rho}")
        b = torch.from_numpy(w.bias_vector()).to(dev)
        r, bufs = forward_timings(w, x, wg, wu, wd, b, args.steps, args.warmup, flush, False, want_split=False)
        rec = {"density_target": rho, "density": r["density"], "n_ovf": r["n_ovf"],
               "forward_cold": r.get("sparse_cold"), "dense_cold": r.get("dense_cold"),
               "forward_warm_us": r["sparse_warm"]["back_to_back_mean_us"],
               "dense_warm_us": r["dense_warm"]["back_to_back_mean_us"],
               "sparse_tokens_per_s": r["tokens_per_s"],
               "dense_tokens_per_s": r["tokens_per_s"] / r["speedup_vs_dense"],
               "speedup_vs_dense": r["speedup_vs_dense"], "speedup_vs_dense_warm": r["speedup_vs_dense_warm"],
               "gate_tflops": r["gate_tflops"]}
        sweep.append(rec)
        del bufs
    out["density_sweep"] = sweep
    del x, wg, wu, wd, flush
    torch.cuda.empty_cache()
    return out


GATE_SOURCES = ("gate_twell.hip", "gemm.hpp", "common.hpp")
SPARSE_SOURCES = ("sparse.hip", "gather.hpp", "common.hpp")
COUNTER_FILE = os.path.join(ROOT, "profiles", "forward.layer_1p5b_bf16.counters.txt")


def source_hash(files):
    """Hash of a kernel's sources with comments and blank space removed (a
    comment edit does not change the kernel the counters were taken on)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "activation_sparse_transformer_bf16_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_summary(workload_name):
    """Per-kernel figures of the committed rocprofv3 summary for this workload:
    {'gate': {...}, 'up': {...}, 'down': {...}}, each kept only while the
    kernel's sources hash to the value recorded with the counters."""
    if workload_name != "layer_1p5b_bf16" or not os.path.exists(COUNTER_FILE):
        return {}
    kv = {}
    with open(COUNTER_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith(("#", "|")):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    out = {}
    for part, files in (("gate", GATE_SOURCES), ("up", SPARSE_SOURCES), ("down", SPARSE_SOURCES)):
        rec = {k.split(".", 1)[1]: v for k, v in kv.items() if k.startswith(part + ".")}
        if rec.get("source_hash") != source_hash(files):
            continue
        for k, v in list(rec.items()):
            try:
                rec[k] = float(v)
            except ValueError:
                pass
        out[part] = rec
    return out


def cpu_baseline(w, inp, budget_s, reps=3):
    """The float64 oracle (gate, TwELL pack, dense FFN) on the first n tokens of
    the batch, `reps` passes; the median pass time is reported."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import ffn, gate_pre, pack, round_to_storage

    cores = len(os.sched_getaffinity(0))

    def run(n):
        r = slice(0, n)
        t0 = time.perf_counter()
        pre = gate_pre(inp.x[r], inp.w_gate, inp.gate_bias[r], w.dtype)
        pack(round_to_storage(pre, w.dtype), w.dtype, w.tile, w.cap)
        ffn(inp.x[r], inp.w_gate, inp.w_up, inp.w_down, inp.gate_bias[r], w.dtype)
        return time.perf_counter() - t0

    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        run(min(w.T, 64))                       # warm up numpy / BLAS
        n0 = min(w.T, 512)
        t_cal = run(n0)
        # the per-call cost is part fixed (weight decoding), so the linear
        # estimate is pessimistic: take the whole batch unless it would
        # clearly exceed the budget
        n = w.T if t_cal * w.T / n0 <= 3 * budget_s else \
            int(max(n0, n0 * budget_s / max(t_cal, 1e-6)) // 256 * 256)
        times = sorted(run(n) for _ in range(max(1, reps)))
    t = times[len(times) // 2]
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": n / t, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "cpu_model": cpu_model, "reps": len(times), "pass_seconds": times,
            "sample": f"first {n} of {w.T} tokens of the same batch, float64 (gate, TwELL pack, dense FFN); "
                      f"median of {len(times)} passes, {t:.1f}s; cpu threads available {cores}"}


def gather_record(w, r):
    """Byte rates of the two gather stages (sparse up and down).

    effective_GBps counts the algorithmic bytes (one W_u^T row and one W_d row
    per active entry, x, y and TwELL) over the in-sequence time of up + down +
    fallback; most weight rows are served from L2, so it is an effective rate
    and no roofline fraction.  The physical figures come from the committed
    rocprofv3 summary of the same kernels: bytes between L2 and the memory
    fabric per launch (FETCH_SIZE + WRITE_SIZE, Infinity Cache hits included,
    so an upper bound on HBM bytes) over the kernel-trace duration, against
    the 8 TB/s HBM spec, and their ratio to the compulsory bytes (each weight
    row once, x, y and TwELL once)."""
    fw = r["forward"]
    t = fw["rest_in_sequence_us"] * 1e-6
    s = 2 if w.dtype == "bf16" else 4
    twell_bytes = w.T * w.n_tiles * (2 + w.cap * (s + 1))
    rec = {"bytes_alg": r["gather_bytes"], "effective_GBps": r["gather_bytes"] / t / 1e9,
           "time_in_sequence_us": t * 1e6,
           "compulsory_bytes": {"up": w.F * w.d * s + w.T * w.d * s + twell_bytes,
                                "down": w.F * w.d * s + w.T * w.d * s}}
    cs = counter_summary(w.name)
    for part in ("up", "down"):
        c = cs.get(part)
        if not c:
            rec[part] = None
            continue
        b, us = c["fabric_bytes"], c["trace_us"]
        rec[part] = {"kernel": c.get("kernel"), "trace_us": us, "fabric_bytes": b,
                     "fabric_GBps": b / (us * 1e-6) / 1e9,
                     "fabric_frac_of_hbm_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "fabric_over_compulsory": b / rec["compulsory_bytes"][part],
                     "ta_busy": c.get("ta_busy"), "valu_busy": c.get("valu_busy")}
        # the weight rows the kernel gathers (one d-row per kept entry) all
        # pass through L2: a lower bound on its L2 bytes, against the L2 peak
        l2 = fw["nnz_kept"] * w.d * s
        rec[part].update({"l2_gathered_bytes": l2, "l2_GBps": l2 / (us * 1e-6) / 1e9,
                          "l2_frac_of_peak": l2 / (us * 1e-6) / 1e9 / L2_PEAK_GBS})
    # compulsory bytes (each weight row, x, y and TwELL once) over the same
    # time, against the spec and the measured streaming read; and the reuse
    # factor of the algorithmic bytes over the counted fabric bytes
    comp = rec["compulsory_bytes"]["up"] + rec["compulsory_bytes"]["down"]
    rec["compulsory_frac_of_hbm_peak"] = comp / t / 1e9 / HBM_PEAK_GBS
    probe_read = (r.get("probe") or {}).get("read_GBps")
    rec["compulsory_frac_of_measured_read"] = comp / t / 1e9 / probe_read if probe_read else None
    if rec.get("up") and rec.get("down"):
        fab = rec["up"]["fabric_bytes"] + rec["down"]["fabric_bytes"]
        rec["reuse_factor"] = r["gather_bytes"] / fab
        # both gather kernels together: counted fabric bytes over their
        # summed kernel-trace durations (Infinity Cache hits included)
        both_s = (rec["up"]["trace_us"] + rec["down"]["trace_us"]) * 1e-6
        rec["fabric_GBps_up_down"] = fab / both_s / 1e9
        rec["fabric_frac_of_hbm_peak_up_down"] = fab / both_s / 1e9 / HBM_PEAK_GBS
    rec["note"] = ("effective_GBps: algorithmic bytes / in-sequence time (L2-served re-reads counted; not a "
                   "roofline fraction). up/down: rocprofv3 FETCH_SIZE + WRITE_SIZE per launch (scaled by a plain "
                   "copy; Infinity Cache hits included) over the kernel-trace average duration, from the committed "
                   "summary of these sources; ta_busy / valu_busy: TA_TA_BUSY and SQ_INSTS_VALU x 4 cycles over "
                   "the elapsed cycles; l2_*: the gathered weight rows (one d-row per kept entry, a lower bound on "
                   "the kernel's L2 traffic) over the kernel-trace duration, against the L2 peak of 8 XCDs x 16 "
                   "channels x 128 B per clock at 2.4 GHz")
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: --gpus {args.gpus} is not supported "
              "(the TwELL forward shards by tokens: each GPU runs the layer on its own rows with its own copy of the weights, with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from workloads import workload

    w = workload(args.workload)
    r, inp = measure(w, args.steps, args.warmup, want_torch=not args.no_torch, want_cold=not args.no_cold)
    fw = r["forward"]
    extra = None
    if not args.no_extra and w.name == "layer_1p5b_bf16":
        extra = extra_workloads(args, inp)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, inp, args.cpu_budget, args.cpu_reps)

    cold = "sparse_cold" in fw
    head = fw["sparse_cold"] if cold else fw["sparse_warm"]
    ms_step = head["mean_us"] * 1e-3
    ach = fw["gate_tflops"]
    cs = counter_summary(w.name).get("gate", {})
    record = {
        "metric": METRIC,
        "value": w.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded Gaussian x and weights (var 1/fan_in), per-token gate bias for the density",
        "config": {**w.summary(), "parallelism": "single GPU",
                   "timing": "cold: 1 GiB rewritten before every timed step, outside its HIP events" if cold
                   else "warm: back-to-back steps"},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": r["peak"], "unit": "TFLOP/s",
                     "frac": ach / r["peak"], "traffic": cs.get("fabric_bytes"),
                     "measured_peak": r["probe"]["mfma_bf16_TFLOPs"] if w.dtype == "bf16" else None,
                     "frac_of_measured_peak": ach / r["probe"]["mfma_bf16_TFLOPs"] if w.dtype == "bf16" else None,
                     "mfma_busy_counter": cs.get("mfma_busy"),
                     "kernel": "k_gate_twell (gate matmul + TwELL epilogue)",
                     "duration_us": fw["gate_back_to_back_us"],
                     "timing": "HIP events around back-to-back launches on the launch stream"},
        "cpu_baseline": cpu,
        "timing_us": {"forward_cold": fw.get("sparse_cold"), "forward_warm": fw["sparse_warm"],
                      "dense_cold": fw.get("dense_cold"), "dense_warm": fw["dense_warm"],
                      "torch_dense_cold": fw.get("torch_dense_cold"), "torch_dense_warm": fw.get("torch_dense_warm")},
        "speedup_vs_dense": fw["speedup_vs_dense"],
        "speedup_vs_torch_dense": fw.get("speedup_vs_torch_dense"),
        "speedup_vs_dense_warm": fw["speedup_vs_dense_warm"],
        "tokens_per_s_warm": fw["tokens_per_s_warm"],
        "stages_us": {"gate_twell_in_sequence": fw["gate_in_sequence_us"],
                      "gate_twell_back_to_back": fw["gate_back_to_back_us"],
                      "up_down_fallback_in_sequence": fw["rest_in_sequence_us"]},
        "gather": gather_record(w, r),
        "dense_mfma_tflops_warm": 3 * 2.0 * w.T * w.d * w.F / (fw["dense_warm"]["back_to_back_mean_us"] * 1e-6) / 1e12,
        "dense_mfma_frac_of_peak": 3 * 2.0 * w.T * w.d * w.F / (fw["dense_warm"]["back_to_back_mean_us"] * 1e-6)
        / 1e12 / MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else None,
        "hbm_copy_GBps": r["copy_gbs"],
        "hbm_probe": r["probe"],
        "workloads": extra,
        "training_formats": r["training"],
        "backward": r["backward"],
        "fused_up_down": r["fused"],
        "density": fw["density"],
        "n_ovf": fw["n_ovf"],
    }
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
