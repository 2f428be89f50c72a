#!/usr/bin/env python3
"""Throughput of the sparse MoE layer forward on one MI355X.

One step = one moe_forward call (router, dispatch plan, grouped expert FFN,
combine) over one batch of seeded synthetic tokens already resident in HBM.
Default workload: the nanoMoE-shaped layer (2048 tokens, d=768, E=8, k=2,
d_ff=3072, bf16, capacity factor 1.25, noise sigma 1.0).

With --pass backward, one step is one moe_backward call instead (the
forward state recomputed, then the gradients of x, W_g, W_up and W_down for
a seeded output gradient); with --pass train, one training step of the
layer (moe_forward_train, which keeps the forward state, then
moe_backward_after_forward). Both are reported in the same JSON form;
--dropout P adds the training-mode dropout on the expert outputs to either.

Prints ONE JSON line on stdout. Besides the contract fields it carries:
  roofline      the dominant kernel (the larger of the two expert GEMMs)
                against bf16 MFMA peak, its duration timed with HIP events on
                the stream it runs on;
  cpu_baseline  the CPU oracle timed on this host on a bounded sample;
  stages        per-stage average durations (HIP events) and derived rates.
Diagnostics go to stderr.
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


def gemm_kernel_name(wl, C, mode):
    """Name of the expert-GEMM instantiation the library launches for this
    workload (mirrors the library's tile choice: 256x256 when experts hold
    >= 256 rows on average and that gives >= 256 tiles or a wide product;
    128x128 in two K sets when 128x128 gives 192 to 383 tiles; 128x64 below
    that; else 128x128). Template arguments: tile rows, columns, waves along
    rows, columns and K, K-step, LDS stages, mode."""
    rpe = min(C, -(-wl.N * wl.k // wl.E))
    nout = wl.d_ff if mode == 0 else wl.d
    t256 = wl.E * -(-rpe // 256) * -(-nout // 256)
    if rpe >= 256 and (t256 >= 256 or nout >= 2048):
        return f"expert_gemm_kernel<256, 256, 4, 4, 1, 64, 2, {mode}>"
    t128 = wl.E * -(-rpe // 128) * -(-nout // 128)
    if t128 < 192:
        return f"expert_gemm_kernel<128, 64, 2, 2, 1, 64, 2, {mode}>"
    if t128 < 384:
        return f"expert_gemm_kernel<128, 128, 2, 4, 2, 128, 2, {mode}>"
    return f"expert_gemm_kernel<128, 128, 2, 2, 1, 64, 2, {mode}>"


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


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="nanomoe",
                    choices=["nanomoe", "mixtral", "skew", "finegrained", "tiny", "nanomoe_gelu"])
    ap.add_argument("--stage-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "train"],
                    default="forward",
                    help="time the layer's forward (default), its backward pass, or a "
                         "training step (forward keeping its state + backward)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="training-mode dropout probability on the expert outputs "
                         "(generator seed 1, offset 0); 0 = none")
    args = ap.parse_args()
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
    dev = D.upload(wl, keep_host=not args.no_cpu_baseline)
    if args.which in ("backward", "train"):
        bench_backward(args, wl, dev, train=args.which == "train")
        return
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
    Y = torch.empty((wl.N * wl.k, wl.d), dtype=x.dtype, device="cuda")
    out = torch.empty_like(x)
    # each stage's C entry point with its arguments marshalled once, so the
    # timed loop is not bound by Python-side argument handling
    import ctypes
    L = B.lib()
    r = ctypes.byref
    dx, dg, dn, du, dd, do, dy = (B.desc(x), B.desc(wg), B.desc(nz), B.desc(wu), B.desc(wd),
                                  B.desc(out), B.desc(Y))
    s_ = B._stream()
    p = B._ptr
    rws = B.alloc_workspace(B.router_workspace_size(wl.N, wl.d, wl.E, x.dtype))
    ews = B.alloc_workspace(B.expert_workspace_size(x.dtype))
    eo = B.ExpertOpts(dev["act"], dev["b_up"], dev["b_down"])   # the workload's expert
    opts = eo.ref()
    stages = {
        "router": lambda: L.moe_router(r(dx), r(dg), r(dn) if dn else None, wl.k, p(idx),
                                       p(gate), p(rws), rws.numel(), s_),
        "dispatch": lambda: L.moe_dispatch(wl.N, wl.E, wl.k, C, p(idx), p(slot), p(usedt),
                                           p(slot_token), p(tiles), s_),
        "expert_up": lambda: L.moe_expert_up_ex(r(dx), r(du), opts, wl.k, C, p(usedt),
                                                p(slot_token), p(tiles), p(H), p(ews),
                                                ews.numel(), s_),
        "expert_down": lambda: L.moe_expert_down_ex(wl.N, r(dd), opts, wl.k, C, p(usedt),
                                                    p(slot_token), p(tiles), p(H), p(Y), p(ews),
                                                    ews.numel(), s_),
        "combine": lambda: L.moe_combine(wl.N, wl.d, wl.k, r(dy), p(gate), p(slot), r(do), s_),
    }
    st_ms = {}
    for name, fn in stages.items():
        for _ in range(3):
            if fn() != 0:
                raise RuntimeError(f"stage {name} failed")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.stage_reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        st_ms[name] = e0.elapsed_time(e1) / args.stage_reps
    gemm_flops = 2.0 * kept * wl.d * wl.d_ff          # one of the two products
    s = dict(st_ms)
    xbytes = 2 if cfg.dtype == "bf16" else 4
    router_bytes = wl.N * wl.d * xbytes + wl.E * wl.d * 4 + wl.N * wl.k * 8 + (
        wl.N * wl.E * 4 if wl.noise is not None else 0)
    combine_bytes = kept * wl.d * xbytes + wl.N * wl.k * 8 + wl.N * wl.d * xbytes
    up_tflops = gemm_flops / (s["expert_up"] * 1e-3) / 1e12
    down_tflops = gemm_flops / (s["expert_down"] * 1e-3) / 1e12
    ffn_frac = (2 * gemm_flops) / ((s["expert_up"] + s["expert_down"]) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    router_gbps = router_bytes / (s["router"] * 1e-3) / 1e9
    combine_gbps = combine_bytes / (s["combine"] * 1e-3) / 1e9
    for n, v in s.items():
        log(f"[bench] stage {n:12s} {v * 1e3:9.2f} us")
    log(f"[bench] expert_up {up_tflops:.0f} TFLOP/s, expert_down {down_tflops:.0f} TFLOP/s, "
        f"FFN {100 * ffn_frac:.1f}% of bf16 peak; router {router_gbps:.0f} GB/s; "
        f"combine {combine_gbps:.0f} GB/s")

    dom = "expert_up" if s["expert_up"] >= s["expert_down"] else "expert_down"
    dom_kernel = gemm_kernel_name(wl, C, 0 if dom == "expert_up" else 1)
    achieved = gemm_flops / (s[dom] * 1e-3) / 1e12
    roofline = {
        "kernel": dom_kernel,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic_for(dom_kernel, cfg.name),
        "algorithmic_per_launch": f"2*kept*d*d_ff = {gemm_flops:.4g} flop (kept={kept})",
        "avg_launch_us": round(s[dom] * 1e3, 2),
    }

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(wl)
        log(f"[bench] cpu_baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

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
            "router_hbm_GBps": round(router_gbps, 1),
            "combine_hbm_GBps": round(combine_gbps, 1),
            "expert_tflops": round(2 * gemm_flops / ((s["expert_up"] + s["expert_down"]) * 1e-3)
                                   / 1e12, 1),
            "stage_us": {k: round(v * 1e3, 2) for k, v in s.items()},
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
