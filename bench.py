#!/usr/bin/env python3
"""Throughput of the sparse MoE layer forward on one MI355X.

One step = one moe_forward call (router, dispatch plan, grouped expert FFN,
combine) over one batch of seeded synthetic tokens already resident in HBM.
Default workload: the fine-grained many-expert layer, the largest of the
layer shapes (8192 tokens, d=7168, E=256, k=8, d_ff=2048, bf16, capacity
factor 1.5); --workload selects another.

With --pass backward, one step is one moe_backward call instead (the
forward state recomputed, then the gradients of x, W_g, W_up and W_down for
a seeded output gradient); with --pass train, one training step of the
layer (moe_forward_train, which keeps the forward state, then
moe_backward_after_forward). Both are reported in the same JSON form;
--dropout P adds the training-mode dropout on the expert outputs to either.

Prints ONE JSON line on stdout. Besides the contract fields it carries:
  roofline      the dominant kernel (the slower of the two expert products)
                against its binding roofline: HBM when its arithmetic
                intensity (flops per algorithmic byte) is below the bf16
                ridge 2.5 PFLOP/s / 8 TB/s, else the bf16 MFMA peak; both
                fractions are given. Its duration is timed with HIP events
                on the stream it runs on, each repetition after a 1 GiB
                write and read that flush the L2 caches and the 256 MB MALL;
  cpu_baseline  the CPU oracle timed on this host on a bounded sample;
  secondary     per-stage average durations (flushed and back to back) and
                derived rates.
Diagnostics go to stderr.

Measurement helpers (not timed runs):
  --probe             a 1 GiB device copy (the counter calibration), then
                      --steps forwards: the program rocprofv3 --pmc runs;
  --traffic-summary   turns two such counter runs (FETCH_SIZE, WRITE_SIZE)
                      into HBM bytes per launch in profiles/traffic.json.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 MI355X; expert-GEMM % MFMA peak; router HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SRC = os.path.join(ROOT, "sparse_mixture_experts_20_amd", "csrc", "experts.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(path):
    """Hash of a kernel source with its comments and spacing removed (an edit
    of comments alone does not change the kernel the counters measured)."""
    with open(path) as f:
        t = f.read()
    t = re.sub(r"//[^\n]*", "", t)
    t = re.sub(r"/\*.*?\*/", "", t, flags=re.S)
    t = re.sub(r"\s+", " ", t).strip()
    return hashlib.sha256(t.encode()).hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(f"{kernel}/{workload}")
    if not e or e.get("source_sha") != source_sha(GEMM_SRC):
        return None
    return e.get("bytes_per_launch")


def gemm_kernel_name(wl, mode):
    """Name of the expert-product kernel the library launches for this
    workload (mode 0: up, 1: down), from the library's own query."""
    import torch
    from sparse_mixture_experts_20_amd import binding as B
    dt = torch.bfloat16 if wl.cfg.dtype == "bf16" else torch.float32
    return B.expert_kernel_name(wl.N, wl.d, wl.E, wl.d_ff, wl.k, wl.cfg.cf, dt, mode)


def cpu_baseline(wl, target_s=15.0):
    """The oracle as it stands: routing and slots for all N tokens, expert FFN
    and combine for a seeded sample of S tokens sized for ~target_s of work."""
    import numpy as np
    import oracle

    x64 = wl.x64()
    t0 = time.perf_counter()
    _, idx, gate = oracle.router(x64, wl.wg64(), wl.noise64(), wl.k)
    C = oracle.capacity(wl.N, wl.E, wl.k, wl.cfg.cf)
    slot, used = oracle.assign(idx, wl.E, C)
    t_route = time.perf_counter() - t0

    rng = np.random.default_rng(0)
    bup, bdown = wl.b_up(), wl.b_down()
    # experts' weights as float64, regenerated once and excluded from timing
    def ffn(rows):
        y = np.zeros((len(rows), wl.k, wl.d))
        sel_i, sel_s = idx[rows], slot[rows]
        t = 0.0
        for e in np.unique(sel_i[sel_s >= 0]):
            r_pos, j_pos = np.nonzero((sel_i == e) & (sel_s >= 0))
            wu, wd = wl.as_f64(wl.w_up(int(e))), wl.as_f64(wl.w_down(int(e)))
            a = time.perf_counter()
            bu = None if bup is None else bup[int(e)].astype(np.float64)
            bd = None if bdown is None else bdown[int(e)].astype(np.float64)
            y[r_pos, j_pos] = oracle.expert_rows(x64, rows[r_pos], wu, wd, wl.cfg.act, bu, bd)
            t += time.perf_counter() - a
        a = time.perf_counter()
        oracle.combine(gate[rows], slot[rows], y)
        return t + time.perf_counter() - a

    probe = np.sort(rng.choice(wl.N, size=min(wl.N, 16), replace=False))
    t_probe = ffn(probe)
    per_tok = t_probe / len(probe)
    S = int(min(wl.N, max(16, target_s / max(per_tok, 1e-9))))
    rows = np.sort(rng.choice(wl.N, size=S, replace=False))
    t_ffn = ffn(rows)
    if t_ffn < 0.5 * target_s and S < wl.N:
        # a probe of 16 tokens over many experts overstates the cost per
        # token (an expert's call has a fixed part): size the sample again
        S = int(min(wl.N, S * target_s / max(t_ffn, 1e-9)))
        rows = np.sort(rng.choice(wl.N, size=S, replace=False))
        t_ffn = ffn(rows)
    est_full = t_route + t_ffn * wl.N / S
    return {
        "value": wl.N / est_full,
        "unit": "tokens/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": (f"routing+slots for all {wl.N} tokens ({t_route:.2f} s); expert FFN+combine "
                   f"for {S} seeded tokens ({t_ffn:.2f} s); tokens/s = N / (t_route + "
                   f"t_ffn*N/S), float64 C loops with OpenMP"),
    }


def cpu_baseline_backward(wl, target_s=15.0, dropout=None):
    """The oracle's backward as it stands, on the first S tokens of the
    workload (same weights; capacity recomputed for S tokens), S sized for
    ~target_s of work."""
    import numpy as np
    import oracle

    x64, wg64 = wl.x64(), wl.wg64()
    nz = wl.noise64()
    dout = wl.as_f64(wl.dout())
    wu = np.stack([wl.as_f64(wl.w_up(e)) for e in range(wl.E)])
    wd = np.stack([wl.as_f64(wl.w_down(e)) for e in range(wl.E)])

    bu, bd = wl.b_up(), wl.b_down()

    def run(S):
        a = time.perf_counter()
        oracle.backward(x64[:S], wg64, None if nz is None else nz[:S], wu, wd, wl.k, wl.cfg.cf,
                        dout[:S], act=wl.cfg.act, bup64=bu, bdown64=bd,
                        **({} if dropout is None else
                           dict(dropout=dropout[0], seed=dropout[1], offset=dropout[2])))
        return time.perf_counter() - a

    S = min(wl.N, 8)
    t = run(S)
    S = int(min(wl.N, max(8, target_s * S / max(t, 1e-9))))
    t = run(S)
    return {
        "value": S / t,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"full backward (all four gradients) of the first {S} tokens with the "
                   f"workload's weights, capacity recomputed for {S} tokens ({t:.2f} s); "
                   f"tokens/s = S / t, serial float64 C loops"),
    }


def _dropout(args):
    """(p, seed, offset) of the expert-output dropout asked for, or None."""
    return (args.dropout, 1, 0) if args.dropout > 0 else None


def _dropout_note(args):
    return f"; expert-output dropout p={args.dropout}" if args.dropout > 0 else ""


def bench_backward(args, wl, dev, train=False):
    """One step = one moe_backward call (forward state recomputed, then every
    gradient) over the workload, with a seeded output gradient; with
    ``train``, one moe_forward_train + moe_backward_after_forward pair (a
    training step's layer work: the forward keeps its state for the
    backward)."""
    import numpy as np
    import torch
    from sparse_mixture_experts_20_amd import binding as B

    cfg = wl.cfg
    if cfg.dtype != "bf16":
        print("the backward pass runs on bf16 layers", file=sys.stderr)
        sys.exit(2)
    dout = torch.from_numpy(wl.dout().view(np.int16)).view(torch.bfloat16).to("cuda")
    if train:
        ts = B.TrainStep(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                         cfg.cf, act=dev["act"], b_up=dev["b_up"], b_down=dev["b_down"],
                         dropout=_dropout(args))

        def bwd():
            ts.forward()
            return ts.backward(dout)
    else:
        bwd = B.Backward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                         cfg.cf, dout, act=dev["act"], b_up=dev["b_up"], b_down=dev["b_down"],
                         dropout=_dropout(args))
    for _ in range(args.warmup):
        bwd()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        bwd()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = max(wall_ms, ev_ms)
    _, st = B.forward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                      cfg.cf, export=True, act=dev["act"], b_up=dev["b_up"],
                      b_down=dev["b_down"])
    kept = int(st.used.sum().item())
    C = st.capacity
    prod = 2.0 * kept * wl.d * wl.d_ff
    flops = 6 * prod + 2 * 2.0 * wl.N * wl.k * wl.d
    achieved = flops / (ms_per_step * 1e-3) / 1e12
    what = "train step" if train else "backward"
    log(f"[bench] {what} {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall "
        f"{wall_ms * 1e3:.1f}, events {ev_ms * 1e3:.1f}); {achieved:.0f} TFLOP/s over the pass")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle's backward on a bounded sample ...")
        cpu = cpu_baseline_backward(wl, dropout=_dropout(args))
        log(f"[bench] cpu_baseline {cpu['value']:.1f} tokens/s")
    line = {
        "metric": ("MoE-layer training step (forward + backward) tokens/sec at 1 MI355X"
                   if train else "MoE-layer backward tokens/sec at 1 MI355X"),
        "value": round(wl.N / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian inputs, output gradient and random-init weights)",
        "config": {
            "workload": (cfg.description or cfg.name) + _dropout_note(args) + (
                "; training step: forward keeping its state, then backward" if train
                else "; backward pass"),
            "tokens": wl.N, "d": wl.d, "experts": wl.E, "top_k": wl.k, "d_ff": wl.d_ff,
            "capacity_factor": cfg.cf, "capacity": C, "noise_sigma": cfg.sigma,
            "seed": cfg.seed, "kept_assignments": kept, "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": ("forward + backward (2 forward and 4 gradient expert products on the "
                       "expert GEMM kernel + router gradient)" if train else
                       "moe_backward pass (6 expert products on the expert GEMM kernel + "
                       "router gradient)"),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "algorithmic_per_launch": (f"6*2*kept*d*d_ff + 4*N*k*d = {flops:.4g} flop "
                                       f"(kept={kept}; " + ("2 forward + 4 gradient products)"
                                                            if train else
                                                            "forward recomputed: 2 of the 6)")),
            "avg_launch_us": round(ms_per_step * 1e3, 2),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


FLUSH_BYTES = 1 << 30     # more than the L2 caches and the 256 MB MALL together


class Flusher:
    """Writes, then reads, a 1 GiB device buffer on the current stream (torch's
    fill and sum kernels), evicting every operand of the previous launch from
    the L2 caches and the 256 MB MALL before a timed repetition; the read pass
    leaves the caches holding clean lines, so that the timed kernel does not
    pay for writing the flush's own data back."""

    def __init__(self):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(self.i)
        self.sink = self.buf.sum()


def time_stage(fn, reps, flush=None):
    """Average duration (ms) of fn() from HIP events on torch's current
    stream (the stream the library launches on). Without `flush`: reps
    back-to-back calls between one pair of events. With `flush`: a cache
    flush precedes every rep outside its own pair of events (the event pair
    adds a few microseconds, which matters only for the smallest stages)."""
    import torch
    for _ in range(3):
        if fn() != 0:
            raise RuntimeError("stage failed")
    torch.cuda.synchronize()
    if flush is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    evs = []
    for _ in range(reps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def algorithmic(wl, kept):
    """Bytes and flops a launch of each stage must move or compute at least
    (the layer's own arithmetic, not the kernels'): per stage (bytes, flops)."""
    xb = 2 if wl.cfg.dtype == "bf16" else 4
    N, d, E, k, dff = wl.N, wl.d, wl.E, wl.k, wl.d_ff
    noise = N * E * 4 if wl.noise is not None else 0
    w = E * dff * d * xb                       # one expert weight tensor
    prod = 2.0 * kept * d * dff                # one expert product
    yb = y_row_bytes(wl.cfg.dtype, d)          # one expert output row
    return {
        "router": (N * d * xb + E * d * 4 + noise + N * k * 8, 2.0 * N * d * E),
        "dispatch": (N * k * 8 + kept * 4, 0.0),
        "expert_up": (N * d * xb + w + kept * dff * xb, prod),
        "expert_down": (kept * dff * xb + w + kept * yb, prod),
        "combine": (kept * yb + N * k * 8 + N * d * xb, 2.0 * kept * d),
    }


def y_row_bytes(dtype, d):
    """Bytes of one expert output row as the layer stores it: fp32 for an
    fp32 layer; for a bf16 layer fp16 values plus one shift byte per 32
    columns."""
    return d * 2 + (d + 31) // 32 if dtype == "bf16" else d * 4


def bench_forward(args, wl, dev):
    import ctypes

    import torch
    from sparse_mixture_experts_20_amd import binding as B

    cfg = wl.cfg
    fwd = B.Forward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                    cfg.cf, export=True, act=dev["act"],
                    b_up=dev["b_up"], b_down=dev["b_down"])

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        fwd()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = max(wall_ms, ev_ms)
    used = fwd.used.cpu().numpy()
    kept = int(used.sum())
    C = int(fwd.stats.capacity)
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall_ms * 1e3:.1f}, "
        f"events {ev_ms * 1e3:.1f}); kept {kept}/{wl.N * wl.k}, C={C}")

    # ---- per-stage timing through the stage entry points (HIP events) ----
    x, wg, nz, wu, wd = dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"]
    idx, gate = B.router(x, wg, nz, wl.k)
    slot, usedt, slot_token, tiles = B.dispatch(idx, wl.E, C)
    ceff = min(C, wl.N)
    H = torch.empty((wl.E, max(ceff, 1), wl.d_ff), dtype=x.dtype, device="cuda")
    # expert output rows in the layer's own form: compact for a bf16 layer
    # (fp16 values and one shift per 32 columns), fp32 otherwise
    compact = x.dtype == torch.bfloat16
    Y = torch.empty((wl.N * wl.k, wl.d), dtype=torch.float16 if compact else torch.float32,
                    device="cuda")
    Ysh = torch.empty((wl.N, B.y_groups(wl.d), wl.k), dtype=torch.int8, device="cuda")
    out = torch.empty_like(x)
    # each stage's C entry point with its arguments marshalled once, so the
    # timed loop is not bound by Python-side argument handling
    L = B.lib()
    r = ctypes.byref
    dx, dg, dn, du, dd, do, dy = (B.desc(x), B.desc(wg), B.desc(nz), B.desc(wu), B.desc(wd),
                                  B.desc(out), None if compact else B.desc(Y))
    s_ = B._stream()
    p = B._ptr
    rws = B.alloc_workspace(B.router_workspace_size(wl.N, wl.d, wl.E, x.dtype))
    ews = B.alloc_workspace(B.expert_workspace_size(x.dtype))
    dws = B.alloc_workspace(B.dispatch_workspace_size(wl.N, wl.E, wl.k))
    eo = B.ExpertOpts(dev["act"], dev["b_up"], dev["b_down"])   # the workload's expert
    opts = eo.ref()
    stages = {
        "router": lambda: L.moe_router(r(dx), r(dg), r(dn) if dn else None, wl.k, p(idx),
                                       p(gate), p(rws), rws.numel(), s_),
        "dispatch": lambda: L.moe_dispatch(wl.N, wl.E, wl.k, C, p(idx), p(gate), p(slot),
                                           p(usedt), p(slot_token), p(tiles), None, None, None,
                                           p(dws), dws.numel(), s_),
        "expert_up": lambda: L.moe_expert_up_ex(r(dx), r(du), opts, wl.k, C, p(usedt),
                                                p(slot_token), p(tiles), p(H), p(ews),
                                                ews.numel(), s_),
        "expert_down": (
            (lambda: L.moe_expert_down_compact(wl.N, r(dd), opts, wl.k, C, p(usedt),
                                               p(slot_token), p(tiles), p(H), p(Y), p(Ysh),
                                               p(ews), ews.numel(), s_)) if compact else
            (lambda: L.moe_expert_down_ex(wl.N, r(dd), opts, wl.k, C, p(usedt), p(slot_token),
                                          p(tiles), p(H), p(Y), p(ews), ews.numel(), s_))),
        "combine": (
            (lambda: L.moe_combine_compact(wl.N, wl.d, wl.k, p(Y), p(Ysh), p(gate), p(slot),
                                           r(do), s_)) if compact else
            (lambda: L.moe_combine(wl.N, wl.d, wl.k, r(dy), p(gate), p(slot), r(do), s_))),
    }
    flush = Flusher()
    warm = {n: time_stage(fn, 5 * args.stage_reps) for n, fn in stages.items()}
    cold = {n: time_stage(fn, args.stage_reps, flush) for n, fn in stages.items()}
    del flush
    alg = algorithmic(wl, kept)
    for n in stages:
        gbps = alg[n][0] / (cold[n] * 1e-3) / 1e9
        tf = alg[n][1] / (cold[n] * 1e-3) / 1e12
        log(f"[bench] stage {n:12s} flushed {cold[n] * 1e3:9.2f} us ({gbps:7.0f} GB/s, "
            f"{tf:6.1f} TFLOP/s); back to back {warm[n] * 1e3:9.2f} us")

    dom = "expert_up" if cold["expert_up"] >= cold["expert_down"] else "expert_down"
    dom_kernel = gemm_kernel_name(wl, 0 if dom == "expert_up" else 1)
    nbytes, flops = alg[dom]
    t = cold[dom] * 1e-3
    intensity = flops / nbytes
    hbm_bound = intensity < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    mfma_frac = flops / t / 1e12 / PEAK_BF16_TFLOPS
    hbm_frac = nbytes / t / 1e9 / PEAK_HBM_GBPS
    roofline = {
        "kernel": dom_kernel,
        "bound": "hbm" if hbm_bound else "mfma",
        "achieved": round(nbytes / t / 1e9 if hbm_bound else flops / t / 1e12, 2),
        "peak": PEAK_HBM_GBPS if hbm_bound else PEAK_BF16_TFLOPS,
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "frac": round(hbm_frac if hbm_bound else mfma_frac, 4),
        "traffic": traffic_for(dom_kernel, cfg.name),
        "mfma_frac": round(mfma_frac, 4),
        "hbm_frac": round(hbm_frac, 4),
        "algorithmic_per_launch": (f"{nbytes:.4g} B (x + weights + output rows) and "
                                   f"2*kept*d*d_ff = {flops:.4g} flop (kept={kept}); "
                                   f"{intensity:.0f} flop/B against the bf16 ridge "
                                   f"{PEAK_BF16_TFLOPS / PEAK_HBM_GBPS * 1e3:.0f} flop/B"),
        "avg_launch_us": round(cold[dom] * 1e3, 2),
        "timing": "HIP events on the launch stream, L2 and MALL flushed before each rep",
    }

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(wl)
        log(f"[bench] cpu_baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    ffn_frac = (2 * alg["expert_up"][1]) / ((cold["expert_up"] + cold["expert_down"]) * 1e-3) \
        / 1e12 / PEAK_BF16_TFLOPS
    value = wl.N / (ms_per_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian inputs and random-init weights)",
        "config": {
            "workload": cfg.description or cfg.name,
            "tokens": wl.N, "d": wl.d, "experts": wl.E, "top_k": wl.k, "d_ff": wl.d_ff,
            "capacity_factor": cfg.cf, "capacity": C, "noise_sigma": cfg.sigma,
            "seed": cfg.seed, "kept_assignments": kept, "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": {
            "expert_gemm_pct_mfma_peak": round(100 * ffn_frac, 2),
            "router_hbm_GBps": round(alg["router"][0] / (cold["router"] * 1e-3) / 1e9, 1),
            "combine_hbm_GBps": round(alg["combine"][0] / (cold["combine"] * 1e-3) / 1e9, 1),
            "expert_tflops": round(2 * alg["expert_up"][1] /
                                   ((cold["expert_up"] + cold["expert_down"]) * 1e-3) / 1e12, 1),
            "stage_us_flushed": {k: round(v * 1e3, 2) for k, v in cold.items()},
            "stage_us_back_to_back": {k: round(v * 1e3, 2) for k, v in warm.items()},
        },
    }
    print(json.dumps(line), flush=True)


def probe(args, wl, dev):
    """The program the HBM-traffic counter runs profile: a plain 1 GiB device
    copy of known size (its counter readings against 1 GiB read and 1 GiB
    written give the counter-to-bytes factors), then --steps forwards."""
    import torch
    from sparse_mixture_experts_20_amd import binding as B

    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    fwd = B.Forward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                    wl.cfg.cf, export=True, act=dev["act"],
                    b_up=dev["b_up"], b_down=dev["b_down"])
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    if args.probe_info:
        # sizes and kept assignments, for the algorithmic byte counts
        info = {"workload": wl.cfg.name, "N": wl.N, "d": wl.d, "E": wl.E, "k": wl.k,
                "d_ff": wl.d_ff, "dtype": wl.cfg.dtype, "noise": dev["noise"] is not None,
                "kept": int(fwd.used.sum().item()), "steps": args.steps}
        with open(args.probe_info, "w") as f:
            json.dump(info, f)
    log(f"[bench] probe done: {wl.cfg.name}, {args.steps} forwards")


# ---- HBM traffic from two rocprofv3 --pmc runs of --probe ------------------
COPY = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30
CSRC = os.path.join(ROOT, "sparse_mixture_experts_20_amd", "csrc")


def _short(name):
    n = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].strip()


def _per_dispatch(run_dir, counter):
    """Average counter value per dispatch, by kernel; for the calibration
    copy, the largest dispatch (small copies of other data may share its
    kernel name)."""
    import collections
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    vals = collections.defaultdict(list)
    for fn in files:
        with open(fn) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (max(v) if k == COPY else sum(v) / len(v)) for k, v in vals.items()}


def _algorithmic_bytes(kernel, p):
    """Bytes a launch must move at least, from the probe's sizes and counts."""
    N, d, E, k, dff, kept = p["N"], p["d"], p["E"], p["k"], p["d_ff"], p["kept"]
    sx = 2 if p["dtype"] == "bf16" else 4
    noise = N * E * 4 if p["noise"] else 0
    m = re.search(r"expert_gemm_kernel<[^>]*, (\d)>", kernel)
    if m and m.group(1) == "0":       # x (whole), W_up, H rows written
        return N * d * sx + E * dff * d * sx + kept * dff * sx, "x + W_up + H"
    yb = y_row_bytes(p["dtype"], d)
    if m and m.group(1) == "1":       # H rows read, W_down, Y rows written
        return kept * dff * sx + E * d * dff * sx + kept * yb, "H + W_down + Y"
    if kernel.startswith("router"):
        return N * d * sx + E * d * 4 + noise + N * k * 8, "x + W_g + noise + ids/gates"
    if kernel.startswith("combine"):
        return kept * yb + N * k * 8 + N * d * sx, "Y + ids/gates + out"
    return None, ""


# source file of each kernel family of the library (by name prefix)
KERNEL_SOURCES = (("expert_gemm", "experts.hip"), ("split_fixup", "experts.hip"),
                  ("experts_f32", "experts.hip"), ("router_", "router.hip"),
                  ("rank_scores", "router.hip"), ("split_router", "router.hip"),
                  ("dispatch", "dispatch.hip"), ("chunk_hist", "dispatch.hip"),
                  ("chunk_scan", "dispatch.hip"), ("combine_backward", "backward.hip"),
                  ("combine", "combine.hip"))


def kernel_source(kern):
    """The csrc file that defines a library kernel (by its name)."""
    for prefix, src in KERNEL_SOURCES:
        if kern.startswith(prefix):
            return src
    return kern.split("_")[0] + ".hip"


def traffic_summary(workload, fetch_dir, write_dir, probe_json, out_json=TRAFFIC_FILE):
    """Counter readings (KiB per dispatch) to bytes per launch: writes
    profiles/traffic.json entries keyed "<kernel>/<workload>" (with the hash of
    the kernel's source, so that stale entries are recognisable) and prints a
    markdown table."""
    with open(probe_json) as f:
        pr = json.load(f)
    fetch = _per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _per_dispatch(write_dir, "WRITE_SIZE")
    ff = COPY_BYTES / (fetch[COPY] * 1024.0)
    wf = COPY_BYTES / (write[COPY] * 1024.0)
    try:
        with open(out_json) as f:
            out = json.load(f)
    except (OSError, ValueError):
        out = {}
    out["_calibration"] = {
        "copy_bytes": COPY_BYTES, "fetch_size_kib": fetch[COPY], "write_size_kib": write[COPY],
        "fetch_factor": ff, "write_factor": wf,
        "note": "bytes = counter_KiB * 1024 * factor, factors from a 1 GiB device copy"}
    print("| kernel | fetch MB | write MB | total MB | algorithmic MB | total / algorithmic |")
    print("|---|---|---|---|---|---|")
    for kern in sorted(set(fetch) & set(write)):
        if kern == COPY or kern.startswith("at::") or kern.startswith("void at::"):
            continue   # the calibration copy and torch's own set-up kernels
        fb = fetch[kern] * 1024.0 * ff
        wb = write[kern] * 1024.0 * wf
        alg, what = _algorithmic_bytes(kern, pr)
        ratio = f"{(fb + wb) / alg:.2f}" if alg else "-"
        algs = f"{alg / 1e6:.2f}" if alg else "-"
        print(f"| `{kern}` | {fb / 1e6:.2f} | {wb / 1e6:.2f} | {(fb + wb) / 1e6:.2f} | {algs} "
              f"| {ratio} |")
        path = os.path.join(CSRC, kernel_source(kern))
        out[f"{kern}/{workload}"] = {
            "bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
            "write_bytes": int(round(wb)), "algorithmic_bytes": alg, "algorithmic": what,
            "source_sha": source_sha(path) if os.path.exists(path) else None}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


WORKLOADS = ["finegrained", "mixtral", "skew", "nanomoe", "nanomoe_gelu", "tiny"]


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="finegrained", choices=WORKLOADS)
    ap.add_argument("--stage-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "train"],
                    default="forward",
                    help="time the layer's forward (default), its backward pass, or a "
                         "training step (forward keeping its state + backward)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="training-mode dropout probability on the expert outputs "
                         "(generator seed 1, offset 0); 0 = none")
    ap.add_argument("--probe", action="store_true",
                    help="run the counter-calibration copy and --steps forwards, no timing")
    ap.add_argument("--probe-info", default="",
                    help="with --probe: write the workload's sizes and kept count here")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "PROBE_JSON"),
                    help="summarise two rocprofv3 --pmc runs of --probe for --workload (host)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.workload, *args.traffic_summary)
        return
    if not 0.0 <= args.dropout < 1.0:
        ap.error("--dropout must be in [0, 1)")
    if args.dropout > 0 and args.which == "forward":
        ap.error("--dropout is training-mode: use it with --pass backward or --pass train")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the layer has no multi-GPU path in this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_mixture_experts_20_amd import binding as B
    from sparse_mixture_experts_20_amd import device as D
    from sparse_mixture_experts_20_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    B.lib()
    wl = W.make(args.workload)
    cfg = wl.cfg
    log(f"[bench] workload {cfg.name}: N={wl.N} d={wl.d} E={wl.E} k={wl.k} d_ff={wl.d_ff} "
        f"{cfg.dtype} cf={cfg.cf}")
    dev = D.upload(wl, keep_host=not args.no_cpu_baseline and not args.probe)
    if args.probe:
        probe(args, wl, dev)
    elif args.which in ("backward", "train"):
        bench_backward(args, wl, dev, train=args.which == "train")
    else:
        bench_forward(args, wl, dev)


if __name__ == "__main__":
    main()
