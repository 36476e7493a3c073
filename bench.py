"""Benchmark of the MoE FFN hot path on one MI355X.

A step is one full moe_ffn_forward call (router -> top-k -> expert grouping
-> gate/up -> down -> combine) over one batch of synthetic tokens whose
inputs are already resident in HBM.  The default workload is single-token
decode with GELU-GLU experts (T=1, H=2816, I=704, E=128, top-8, bf16
weights, f32 activations); --workload selects another.

Decode steps rotate over a pool of distinct token vectors, so consecutive
steps select different experts and the weights stream from HBM rather than
from the 256 MB Infinity Cache (the full expert set is 1.5 GB).

Prints one JSON line.  Fields beyond the common contract:
  roofline      dominant kernel: algorithmic bytes (decode) or flops or
                bytes (prefill: whichever its arithmetic intensity makes
                binding against the MI355X ridge point, both fractions
                reported) per launch over its average launch time, measured
                with hipEvents recorded on the launch stream around every
                launch, in a second (eager) pass over the same K steps;
                traffic = HBM bytes per launch (FETCH_SIZE + WRITE_SIZE,
                scaled by a plain copy of known size) from the committed
                counter record, null when the kernel sources have changed
                since the counters were taken
  cpu_baseline  the float64 CPU oracle timed on a bounded sample of tokens
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE FFN tokens/s; HBM GB/s at T=1, MFMA TFLOP/s at T=4096"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode_geglu_t1")
    ap.add_argument("--pool", type=int, default=64, help="distinct token batches to rotate")
    ap.add_argument("--eager", action="store_true", help="no HIP graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gating", choices=["softmax", "sigmoid"], default="softmax",
                    help="routing scores (the workloads are quoted with softmax)")
    ap.add_argument("--routed-scale", type=float, default=1.0)
    ap.add_argument("--pre-norm", type=float, default=None, metavar="EPS",
                    help="run the layer on RMSNorm(x) with this epsilon")
    ap.add_argument("--residual", action="store_true", help="add a residual to out")
    ap.add_argument("--op", choices=["forward", "backward"], default="forward",
                    help="backward: the weighted-combine and gated-activation backward kernels "
                         "at the workload's shape")
    ap.add_argument("--weight-layout", choices=["auto", "rowmajor", "packed"], default="auto",
                    help="packed: prepare the bf16 expert weights in the prefill GEMMs' packed "
                         "layout once, before timing (auto: for bf16 prefill workloads whose "
                         "routes fill whole 256-route tiles, where it measured faster)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a kernel of known "
                         "traffic, to scale hardware byte counters)")
    return ap.parse_args()


def bytes_per_weight(wf):
    return {0: 4.0, 1: 2.0, 2: 0.5 + 4.0 / 32}[wf]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.op == "backward":
        return bench_backward(args)
    import numpy as np
    import torch

    import mixture_experts_ffn_gemv_amd as M
    from mixture_experts_ffn_gemv_amd.profiling import recorded_traffic
    from moe_synth import CONFIGS, generate, WF_U4
    from moe_synth.generator import x_rows
    from moe_synth.device import desc_kwargs, weights_kwargs

    cfg = CONFIGS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calib_copy_mb:
        n = args.calib_copy_mb << 18  # float32 elements
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp = generate(cfg, backend="torch", device=dev)
    gating = {"softmax": M.GATING_SOFTMAX, "sigmoid": M.GATING_SIGMOID}[args.gating]
    desc = M.make_desc(**desc_kwargs(cfg, gating=gating, routed_scale=args.routed_scale),
                       norm_eps=args.pre_norm)
    wkw = weights_kwargs(inp)
    if args.pre_norm is not None:
        from moe_synth import norm_weight_values
        wkw["norm_weight"] = torch.from_numpy(norm_weight_values(cfg)).to(dev)
    w = M.make_weights(**wkw)
    layout = args.weight_layout
    if layout == "auto":
        layout = "packed" if (cfg.weight_format == 1 and cfg.act_dtype == 1 and cfg.T > 32
                              and cfg.T * cfg.k >= 256 * cfg.E) else "rowmajor"
    packed_bufs = M.pack_weights(desc, w, device=dev) if layout == "packed" else None
    res = None
    if args.residual:
        from moe_synth import residual_values
        res = torch.from_numpy(residual_values(cfg)).to(dev)
    T = cfg.T
    decode = T <= 32
    P = args.pool if decode else 1
    # token pool: pool[0] is the generated x, the rest are fresh draws
    xs = [inp.x]
    for a in range(1, P):
        xs.append(x_rows(cfg, range(T), 1000 + a, backend="torch", device=dev))
    ws = M.alloc_workspace(desc, T, dev)
    out = torch.empty((T, cfg.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        M.moe_ffn_forward(desc, xs[i % P], w, out=out, workspace=ws, residual=res)

    # realized expert load of pool[0] (for the algorithmic byte / flop counts)
    r = M.moe_route(desc, xs[0], w, workspace=ws)
    torch.cuda.synchronize()
    counts = r.counts.cpu().numpy()
    touched = int((counts > 0).sum())

    # HIP graph of the whole pool rotation (P consecutive steps): one replay
    # runs P steps back to back, so the per-replay launch cost is amortised
    graph = None
    if not args.eager:
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            for i in range(3):
                step(i)
        stream.wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(P):
                step(i)
        torch.cuda.synchronize()

    def run_steps(n):
        """n consecutive steps: whole-pool graph replays, then single eager steps."""
        i = 0
        if graph is not None:
            while n - i >= P:
                graph.replay()
                i += P
        while i < n:
            step(i)
            i += 1

    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed

    # ---- per-kernel durations: hipEvents around each launch, eager pass ------
    M.timing_reset()
    M.timing_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kt = M.timing_read()
    M.timing_enable(False)
    kernel_ms = {k: v[1] / v[0] for k, v in kt.items()}

    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    bpw = bytes_per_weight(cfg.weight_format)
    if decode:
        # selected-expert gate+up weight bytes streamed by one gate/up launch
        dom = "gemv_gateup"
        alg = touched * 2 * I * H * bpw + (2 * cfg.Is * H * bpw if cfg.shared else 0)
    if decode:
        achieved = alg / (kernel_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(cfg.name, dom), "algorithmic_bytes_per_launch": alg,
                "avg_launch_us": round(kernel_ms[dom] * 1e3, 2)}
        step_bytes = touched * 3 * I * H * bpw + (3 * cfg.Is * H * bpw if cfg.shared else 0)
        extra = {"path_weight_bytes": step_bytes,
                 "path_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1)}
    else:
        # gate/up grouped GEMM: flops, and the bytes it must move at least
        # (touched experts' gate+up weights, x, h written; shared expert alike)
        dom = "gemm_gateup"
        R = T * k
        Is = cfg.Is if cfg.shared else 0
        fl = 2.0 * (R * 2 * I * H + T * 2 * Is * H)
        by = (touched * 2 * I * H + 2 * Is * H) * bpw + T * H * 2 + (R * I + T * Is) * 2
        sec = kernel_ms[dom] * 1e-3
        tflops, gbs = fl / sec / 1e12, by / sec / 1e9
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        f_mfma, f_hbm = tflops / MFMA_BF16_PEAK_TFLOPS, gbs / HBM_PEAK_GBS
        if fl / by >= ridge:   # arithmetic intensity above the ridge: bound by MFMA
            roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(f_mfma, 4)}
        else:
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(f_hbm, 4)}
        roof.update({"kernel": dom, "traffic": recorded_traffic(cfg.name, dom),
                     "algorithmic_flops_per_launch": fl, "algorithmic_bytes_per_launch": by,
                     "arithmetic_intensity": round(fl / by, 1), "ridge": round(ridge, 1),
                     "frac_mfma": round(f_mfma, 4), "frac_hbm": round(f_hbm, 4),
                     "avg_launch_us": round(kernel_ms[dom] * 1e3, 2)})
        tot = 2.0 * T * (k * 3 * I * H + (3 * cfg.Is * H if cfg.shared else 0) + (E + 1) * H)
        extra = {"path_flops": tot, "path_tflops": round(tot / (ms_per_step * 1e-3) / 1e12, 1)}

    cpu = None
    if not args.no_cpu_baseline:
        pn = None
        if args.pre_norm is not None:
            from moe_synth import norm_weight_values
            pn = (norm_weight_values(cfg), args.pre_norm)
        cpu = cpu_baseline(cfg, inp, xs, args.cpu_seconds, gating, args.routed_scale, pn,
                           None if res is None else res.cpu().numpy())

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.weight_format == 1 and cfg.act_dtype == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": H, "I": I, "E": E, "top_k": k,
                   "activation": ["silu", "gelu_tanh"][cfg.act],
                   "weights": ["f32", "bf16", "u4_g32"][cfg.weight_format],
                   "weight_layout": layout,
                   "activations": ["f32", "bf16"][cfg.act_dtype],
                   "shared_expert": cfg.Is if cfg.shared else 0,
                   "gating": args.gating, "routed_scale": args.routed_scale,
                   "pre_norm_eps": args.pre_norm, "residual": args.residual,
                   "touched_experts": touched, "token_pool": P,
                   "launch": "eager" if graph is None else f"hipgraph x{P} steps",
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "kernels_us": {k2: round(v * 1e3, 2) for k2, v in kernel_ms.items()},
        **extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _host_copy(inp):
    """numpy copy (storage format) of every input tensor, made before timing."""
    from moe_synth.device import host_views
    from moe_synth import U4Weights
    hv = host_views(inp)
    for name in ("x", "router", "router_bias", "gate", "up", "down", "shared_gate_inp",
                 "shared_gate", "shared_up", "shared_down"):
        v = getattr(hv, name)
        if v is None:
            continue
        if isinstance(v, U4Weights):
            setattr(hv, name, U4Weights(v.codes[:], v.scales[:], v.mins[:], v.K, v.group))
        else:
            setattr(hv, name, v[:])
    return hv


def bench_backward(args):
    """Both backward kernels at the workload's shape (f32 inputs resident in
    HBM), timed together as one step; roofline of the combine backward."""
    import torch
    import mixture_experts_ffn_gemv_amd as M
    from mixture_experts_ffn_gemv_amd.profiling import recorded_traffic
    from moe_synth import CONFIGS, grad_inputs
    cfg = CONFIGS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calib_copy_mb:
        src = torch.ones(args.calib_copy_mb << 18, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    g = grad_inputs(cfg)
    d = {k: torch.from_numpy(v).to(dev) for k, v in g.items()}
    T, k, H, I = cfg.T, cfg.k, cfg.H, cfg.I
    R = T * k
    dy = torch.empty((T, k, H), dtype=torch.float32, device=dev)
    dw = torch.empty((T, k), dtype=torch.float32, device=dev)
    dgu = torch.empty((R, 2 * I), dtype=torch.float32, device=dev)
    lib = M.load()
    stream = torch.cuda.current_stream().cuda_stream

    def step(_=0):
        M._check(lib.moe_weighted_sum_backward(T, k, H, d["w"].data_ptr(), d["y"].data_ptr(),
                                               d["dout"].data_ptr(), dy.data_ptr(),
                                               dw.data_ptr(), stream))
        M._check(lib.moe_glu_backward(R, I, cfg.act, d["gate_up"].data_ptr(), d["dh"].data_ptr(),
                                      dgu.data_ptr(), stream))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    M.timing_reset()
    M.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = M.timing_read()
    M.timing_enable(False)
    kernel_ms = {n: v[1] / v[0] for n, v in kt.items()}
    wsum_bytes = 4 * (2 * R * H + T * H + 2 * R)        # y, dy, dout, w, dw
    glu_bytes = 4 * (2 * R * 2 * I + R * I)             # gate_up, d_gate_up, dh
    dom = "wsum_backward"
    achieved = wsum_bytes / (kernel_ms[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(cfg.name, dom), "algorithmic_bytes_per_launch": wsum_bytes,
            "avg_launch_us": round(kernel_ms[dom] * 1e3, 2),
            "glu_backward": {"algorithmic_bytes_per_launch": glu_bytes,
                             "avg_launch_us": round(kernel_ms["glu_backward"] * 1e3, 2),
                             "achieved_gbs": round(glu_bytes / (kernel_ms["glu_backward"] * 1e-3)
                                                   / 1e9, 1)}}
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        from oracle import weighted_sum_backward, glu_backward
        n, tcpu, t = 0, 0.0, 0
        while tcpu < args.cpu_seconds:
            t0c = time.perf_counter()
            weighted_sum_backward(g["w"][t:t + 1], g["y"][t:t + 1], g["dout"][t:t + 1])
            glu_backward(g["gate_up"][t * k:(t + 1) * k], g["dh"][t * k:(t + 1) * k], cfg.act)
            tcpu += time.perf_counter() - t0c
            n += 1
            t = (t + 1) % T
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        cpu = {"value": round(n / tcpu, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} tokens of {cfg.name}: both float64 backward steps per token"}
    ms = elapsed * 1e3 / args.steps
    print(json.dumps({
        "metric": "MoE FFN backward tokens/s (routing-weighted combine + gated activation)",
        "value": round(T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "op": "backward", "T": T, "H": H, "I": I, "top_k": k,
                   "activation": ["silu", "gelu_tanh"][cfg.act], "parallelism": "single-gpu"},
        "roofline": roof, "kernels_us": {n: round(v * 1e3, 2) for n, v in kernel_ms.items()},
        "cpu_baseline": cpu}), flush=True)


def cpu_baseline(cfg, inp, xs, seconds, gating=0, scale=1.0, pre_norm=None, residual=None):
    """The float64 CPU oracle, as it stands, on a bounded sample of tokens."""
    from threadpoolctl import threadpool_info
    from moe_synth.device import HostView
    from oracle import moe_ffn, WeightSource

    host = _host_copy(inp) if cfg.E * cfg.I * cfg.H * 3 <= (1 << 31) else None
    if host is None:
        from moe_synth.device import host_views
        host = host_views(inp)     # too large to copy whole: slices are read on demand
    n_done = 0
    t_total = 0.0
    j = 0
    while t_total < seconds:
        host.x = HostView(xs[j % len(xs)])[:]
        for tok in range(cfg.T):
            src = WeightSource(host, cache=False)
            t0 = time.perf_counter()
            moe_ffn(host, tokens=[tok], src=src, gating=gating, scale=scale, pre_norm=pre_norm,
                    residual=residual)
            t_total += time.perf_counter() - t0
            n_done += 1
            if t_total >= seconds:
                break
        j += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(n_done / t_total, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_done} tokens of {cfg.name} (drawn from the benchmark's token pool), "
                      f"one float64 oracle call per token with its experts decoded per call; "
                      f"inputs copied to host memory before timing"}


if __name__ == "__main__":
    main()
