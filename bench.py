"""Benchmark of the MoE FFN hot path on one MI355X.

A step is one full moe_ffn_forward call (router -> top-k -> expert grouping
-> gate/up -> down -> combine) over one batch of synthetic tokens whose
inputs are already resident in HBM.  The default workload is single-token
decode with GELU-GLU experts (T=1, H=2816, I=704, E=128, top-8, bf16
weights, f32 activations); --workload selects another.

Decode steps rotate over a pool of token vectors chosen so that no expert
is used twice within 3 consecutive steps (at the one-token shape that is
285 MB of other weights in between, more than the 256 MB Infinity Cache
holds), so each step's weights stream from HBM.  The timed steps run as
HIP-graph replays (a graph of min(steps, pool) steps, plus one graph for
the remainder), captured before the timed region; config.launch says what
ran.

Prints one JSON line.  Fields beyond the common contract:
  roofline      dominant kernel: algorithmic bytes (decode) or flops or
                bytes (prefill: whichever its arithmetic intensity makes
                binding against the MI355X ridge point, both fractions
                reported) per launch over its average launch time, measured
                with hipEvents recorded on the launch stream around every
                launch, in a second (eager) pass over the same steps; the
                *_cold figures come from a third eager pass with a 512 MiB
                copy between steps (outside the brackets), which leaves
                nothing of the step's own data in L2 or the Infinity Cache;
                traffic = HBM bytes per launch (FETCH_SIZE + WRITE_SIZE,
                scaled by a plain copy of known size) from the committed
                counter record, null when the kernel sources have changed
                since the counters were taken
  cold_mall     that cold pass: event-bracketed step and kernel times
  prefill_t4096, prefill_t16384
                the prefill workloads (T=4096 shared-expert, T=16384
                skewed) timed in the same run: ms per step over graph
                replays, the gate/up GEMM's TFLOP/s and the fractions of
                the bf16 MFMA and HBM peaks, for the GEMM and the step
  cpu_baseline  the float64 CPU oracle timed on a bounded sample of tokens
  measured_peaks
                what this GPU sustains with library routines, as context for
                the fractions (which use the published peaks): a 1 GiB
                device copy (GB/s, bytes read plus written) and a bf16
                8192^3 matrix product through torch (TFLOP/s)
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
    ap.add_argument("--expert-scale", action="store_true",
                    help="apply the generator's per-expert routing scale")
    ap.add_argument("--host-inputs", action="store_true",
                    help="generate inputs on the host (numpy) and copy them: no generator "
                         "kernels run on the GPU (for profiled runs)")
    ap.add_argument("--inputs-dir", default=None,
                    help="copy the inputs from .npy files in this directory when it has them, "
                         "else generate them on the GPU and save them there (so that a "
                         "profiled run can launch no generator kernels)")
    ap.add_argument("--cold-mib", type=int, default=512,
                    help="MiB copied between the steps of the cold-cache kernel pass "
                         "(0: no such pass)")
    ap.add_argument("--prefill", default="prefill_shared_t4096,prefill_skew_t16384",
                    help="prefill workloads timed after the main one, reported under "
                         "prefill_t<T> keys ('none': skip)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the copy and bf16 matrix product peak measurements")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a kernel of known "
                         "traffic, to scale hardware byte counters)")
    return ap.parse_args()


def measured_peaks(dev, iters=20):
    """Sustained bandwidth and bf16 matrix throughput of this GPU measured
    with library routines (a device copy, a matrix product), each the mean
    over `iters` back-to-back calls bracketed by events."""
    import torch

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / iters

    nb = 1 << 30
    a = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    copy_s = timed(lambda: b.copy_(a))
    del a, b
    m = 8192
    x = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    y = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    z = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    mm_s = timed(lambda: torch.matmul(x, y, out=z))
    del x, y, z
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * nb / copy_s / 1e9, 1),
            "bf16_gemm_tflops": round(2 * m ** 3 / mm_s / 1e12, 1),
            "how": "1 GiB f32 device copy (bytes read + written) and bf16 8192x8192x8192 "
                   "torch.matmul, mean of 20 back-to-back calls each"}


def bytes_per_weight(wf):
    return {0: 4.0, 1: 2.0, 2: 0.5 + 4.0 / 32}[wf]


def _nproc():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def _blas_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


_INPUT_FIELDS = ("x", "router", "router_bias", "gate", "up", "down", "shared_gate_inp",
                 "shared_gate", "shared_up", "shared_down")


def _save_inputs(inp, d):
    """Storage-format copies of every input tensor, one .npy per array."""
    import numpy as np
    import torch
    from moe_synth import U4Weights
    os.makedirs(d, exist_ok=True)

    def host(t):
        if t.dtype in (torch.bfloat16, torch.float16):
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.contiguous().cpu().numpy()
    for name in _INPUT_FIELDS:
        v = getattr(inp, name)
        if v is None:
            continue
        if isinstance(v, U4Weights):
            for part in ("codes", "scales", "mins"):
                np.save(os.path.join(d, f"{name}.{part}.npy"), host(getattr(v, part)))
        else:
            np.save(os.path.join(d, f"{name}.npy"), host(v))


def _load_inputs(cfg, d):
    """A host MoeInputs read back from _save_inputs' files (memory-mapped)."""
    import numpy as np
    from moe_synth import MoeInputs, U4Weights, WF_U4

    def ld(name):
        f = os.path.join(d, f"{name}.npy")
        return np.load(f, mmap_mode="r") if os.path.exists(f) else None
    vals = {}
    for name in _INPUT_FIELDS:
        if cfg.weight_format == WF_U4 and name in ("gate", "up", "down"):
            K = cfg.I if name == "down" else cfg.H
            vals[name] = U4Weights(ld(f"{name}.codes"), ld(f"{name}.scales"),
                                   ld(f"{name}.mins"), K, cfg.group_size)
        else:
            vals[name] = ld(name)
    inp = MoeInputs(cfg, vals["x"], vals["router"], vals["router_bias"], vals["gate"],
                    vals["up"], vals["down"], backend="numpy")
    for name in _INPUT_FIELDS[6:]:
        setattr(inp, name, vals[name])
    return inp


def make_inputs_on_device(cfg, dev, host_inputs, inputs_dir=None):
    """The workload's inputs resident in HBM.  host_inputs: generated with
    the numpy generator and copied (no generator kernels run on the GPU).
    inputs_dir: when it holds this workload's arrays, they are copied from
    there (again no generator kernels); else they are generated on the GPU
    and saved there, for a later (profiled) run."""
    from moe_synth import generate
    from moe_synth.device import to_device
    if inputs_dir and os.path.exists(os.path.join(inputs_dir, "x.npy")):
        return to_device(_load_inputs(cfg, inputs_dir), dev)
    if host_inputs:
        return to_device(generate(cfg, backend="numpy"), dev)
    inp = generate(cfg, backend="torch", device=dev)
    if inputs_dir:
        _save_inputs(inp, inputs_dir)
    return inp


def token_pool(M, cfg, desc, w, inp, P, dev, host_inputs, window=3):
    """P token batches to rotate through.  pool[0] is the generated x.  For
    decode batches whose experts can be kept apart (T*k*(window+1) <= E),
    the others are drawn so that no expert is used by two batches within
    `window` steps of each other (cyclically): each step's weights then
    come from HBM, not from what earlier steps left in the 256 MB Infinity
    Cache (window 3: at least 3 steps of weights, 285 MB at the one-token
    decode shape, between two uses of an expert)."""
    import numpy as np
    import torch
    from moe_synth.generator import x_rows
    from moe_synth.device import _t
    T = cfg.T
    if P == 1:
        return [inp.x], None

    def rows(rr, attempt):
        if host_inputs:
            return _t(x_rows(cfg, rr, attempt, backend="numpy"), dev,
                      bf16=cfg.act_dtype == 1)
        return x_rows(cfg, rr, attempt, backend="torch", device=dev)

    if T * cfg.k * (window + 1) > cfg.E:
        # every batch touches most experts: plain distinct draws
        return [inp.x] + [rows(range(T), 1000 + a) for a in range(1, P)], None
    # candidates: one batch of C*T rows, routed once by the library
    C = 64 * P
    cand = rows(range(C * T), 1000)
    ws = M.alloc_workspace(desc, C * T, dev)
    r = M.moe_route(desc, cand, w, workspace=ws)
    torch.cuda.synchronize()
    ids = r.ids.cpu().numpy().reshape(C, T * cfg.k)
    r0 = M.moe_route(desc, inp.x, w)
    torch.cuda.synchronize()
    sets = [set(r0.ids.cpu().numpy().ravel().tolist())]
    chosen = [None]
    used = np.zeros(C, dtype=bool)
    for a in range(1, P):
        near = [sets[i] for i in range(max(0, a - window), a)]
        # the last batches also come within `window` of the first ones
        near += [sets[i] for i in range(0, max(0, a + window - P + 1))]
        avoid = set().union(*near)
        pick = next((c for c in range(C) if not used[c] and avoid.isdisjoint(ids[c])), None)
        if pick is None:
            raise RuntimeError("no candidate token batch keeps the experts apart")
        used[pick] = True
        chosen.append(pick)
        sets.append(set(ids[pick].tolist()))
    pool = [inp.x] + [cand[c * T:(c + 1) * T].clone() for c in chosen[1:]]
    return pool, window


class Stepper:
    """K consecutive steps as HIP-graph replays: a graph of G = min(K, pool)
    steps replayed K // G times, then a graph of the K % G remaining steps.
    prepare(K) captures those graphs (outside any timed region); warm(W)
    replays the G-step graph until at least W steps have run.  Records what
    ran for the JSON line."""

    def __init__(self, step, P, eager):
        self.step, self.P, self.eager = step, P, eager
        self.graphs = {}
        self.ran = []

    def prepare(self, n):
        if self.eager or n == 0:
            return
        G = min(n, self.P)
        self._graph(G)
        if n % G:
            self._graph(n % G)

    def warm(self, n, steps):
        """At least n warm-up steps, as replays of the timed run's main graph."""
        if self.eager or steps == 0:
            for i in range(n):
                self.step(i)
            return
        g = self._graph(min(steps, self.P))
        for _ in range((n + min(steps, self.P) - 1) // min(steps, self.P)):
            g.replay()

    def _graph(self, n):
        import torch
        if n not in self.graphs:
            stream = torch.cuda.current_stream()
            s = torch.cuda.Stream()
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                for i in range(min(n, 3)):
                    self.step(i)
            stream.wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    self.step(i)
            torch.cuda.synchronize()
            self.graphs[n] = g
        return self.graphs[n]

    def run(self, n):
        if self.eager or n == 0:
            for i in range(n):
                self.step(i)
            self.ran = [("eager", n, 1)]
            return
        G = min(n, self.P)
        full, rem = divmod(n, G)
        g = self._graph(G)
        rg = self._graph(rem) if rem else None
        for _ in range(full):
            g.replay()
        if rg is not None:
            rg.replay()
        self.ran = [("graph", G, full)] + ([("graph", rem, 1)] if rem else [])

    def label(self):
        parts = []
        for kind, size, reps in self.ran:
            parts.append(f"{kind} {size} steps" if kind == "eager"
                         else f"hipgraph of {size} steps x{reps}")
        return " + ".join(parts)


def kernel_times(M, step, n, scrub=None):
    """Average event-bracketed duration per kernel (ms) over n eager steps;
    with `scrub`, a 512 MiB copy runs before every step, outside the
    brackets, so the step starts with nothing of its own in the caches.
    Also returns the average event-bracketed step (ms)."""
    import torch
    M.timing_reset()
    M.timing_enable(True)
    ev = []
    for i in range(n):
        if scrub is not None:
            scrub[1].copy_(scrub[0])
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step(i)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    st = sum(a.elapsed_time(b) for a, b in ev)
    kt = M.timing_read()
    M.timing_enable(False)
    return {k: v[1] / v[0] for k, v in kt.items()}, st / max(n, 1)


def prefill_figures(cfg, touched, sec_gateup, sec_step):
    """Flops and bytes the prefill path must do at least, and the fractions
    of the MI355X peaks they reach in the given times."""
    T, k, H, I, E = cfg.T, cfg.k, cfg.H, cfg.I, cfg.E
    R = T * k
    Is = cfg.Is if cfg.shared else 0
    fl = 2.0 * (R * 2 * I * H + T * 2 * Is * H)
    by = (touched * 2 * I * H + 2 * Is * H) * 2 + T * H * 2 + (R * I + T * Is) * 2
    tot = 2.0 * T * (k * 3 * I * H + 3 * Is * H + (E + 1) * H)
    tot_by = (touched * 3 * I * H + 3 * Is * H + (E + 1) * H) * 2 + T * H * 2 + T * H * 4
    tf, gbs = fl / sec_gateup / 1e12, by / sec_gateup / 1e9
    return {
        "gateup_flops": fl, "gateup_bytes": by, "gateup_tflops": round(tf, 1),
        "gateup_frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "gateup_frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
        "path_flops": tot, "path_bytes": tot_by,
        "path_tflops": round(tot / sec_step / 1e12, 1),
        "frac_mfma": round(tot / sec_step / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "frac_hbm": round(tot_by / sec_step / 1e9 / HBM_PEAK_GBS, 4),
    }


def bench_prefill(M, name, steps, warmup, dev):
    """One prefill workload (inputs resident in HBM): ms per step over
    graph replays, the gate/up GEMM's event-bracketed time, and the
    fractions of the bf16 MFMA and HBM peaks."""
    import torch
    from moe_synth import CONFIGS
    from moe_synth.device import desc_kwargs, weights_kwargs
    cfg = CONFIGS[name]
    inp = make_inputs_on_device(cfg, dev, False)
    desc = M.make_desc(**desc_kwargs(cfg))
    w = M.make_weights(**weights_kwargs(inp))
    packed = None
    if cfg.T * cfg.k >= 256 * cfg.E:
        packed = M.pack_weights(desc, w, device=dev)
    ws = M.alloc_workspace(desc, cfg.T, dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev)
    r = M.moe_route(desc, inp.x, w, workspace=ws)
    torch.cuda.synchronize()
    touched = int((r.counts.cpu().numpy() > 0).sum())

    def step(i):
        M.moe_ffn_forward(desc, inp.x, w, out=out, workspace=ws)

    st = Stepper(step, steps, False)
    st.prepare(steps)
    st.warm(warmup, steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st.run(steps)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    km, _ = kernel_times(M, step, max(3, min(steps, 10)))
    fig = prefill_figures(cfg, touched, km["gemm_gateup"] * 1e-3, sec)
    res = {"workload": name, "T": cfg.T, "ms_per_step": round(sec * 1e3, 4),
           "tokens_per_s": round(cfg.T / sec, 1), "launch": st.label(),
           "weight_layout": "packed" if packed else "rowmajor", "touched_experts": touched,
           "gateup_us": round(km["gemm_gateup"] * 1e3, 1),
           "kernels_us": {k2: round(v * 1e3, 1) for k2, v in km.items()}, **fig}
    del inp, w, ws, out, packed
    torch.cuda.empty_cache()
    return res


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
    from moe_synth import CONFIGS, expert_scale_values
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
    loaded = bool(args.inputs_dir) and os.path.exists(os.path.join(args.inputs_dir, "x.npy"))
    inp = make_inputs_on_device(cfg, dev, args.host_inputs, args.inputs_dir)
    host_side = args.host_inputs or loaded    # the token pool is drawn on the host too
    gating = {"softmax": M.GATING_SOFTMAX, "sigmoid": M.GATING_SIGMOID}[args.gating]
    desc = M.make_desc(**desc_kwargs(cfg, gating=gating, routed_scale=args.routed_scale),
                       norm_eps=args.pre_norm)
    wkw = weights_kwargs(inp)
    if args.pre_norm is not None:
        from moe_synth import norm_weight_values
        wkw["norm_weight"] = torch.from_numpy(norm_weight_values(cfg)).to(dev)
    escale = expert_scale_values(cfg) if args.expert_scale else None
    if escale is not None:
        wkw["expert_scale"] = torch.from_numpy(escale).to(dev)
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
    xs, window = token_pool(M, cfg, desc, w, inp, P, dev, host_side)
    ws = M.alloc_workspace(desc, T, dev)
    out = torch.empty((T, cfg.H), dtype=torch.float32, device=dev)

    def step(i):
        M.moe_ffn_forward(desc, xs[i % P], w, out=out, workspace=ws, residual=res)

    # realized expert load of pool[0] (for the algorithmic byte / flop counts)
    r = M.moe_route(desc, xs[0], w, workspace=ws)
    torch.cuda.synchronize()
    counts = r.counts.cpu().numpy()
    touched = int((counts > 0).sum())

    stepper = Stepper(step, P, args.eager)
    stepper.prepare(args.steps)        # graph capture stays outside the timed region
    stepper.warm(args.warmup, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    stepper.run(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed

    # ---- per-kernel durations: hipEvents around each launch, eager passes ---
    nk = max(1, min(args.steps, 400))
    kernel_ms, _ = kernel_times(M, step, nk)
    cold_ms = cold_step_ms = None
    if args.cold_mib:
        n = args.cold_mib << 18   # float32 elements
        scrub = (torch.ones(n, device=dev), torch.empty(n, device=dev))
        cold_ms, cold_step_ms = kernel_times(M, step, nk, scrub)
        del scrub

    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    bpw = bytes_per_weight(cfg.weight_format)
    if decode:
        # selected-expert gate+up weight bytes streamed by one gate/up launch
        dom = "gemv_gateup"
        alg = touched * 2 * I * H * bpw + (2 * cfg.Is * H * bpw if cfg.shared else 0)
        achieved = alg / (kernel_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(cfg.name, dom), "algorithmic_bytes_per_launch": alg,
                "avg_launch_us": round(kernel_ms[dom] * 1e3, 2)}
        if cold_ms:
            ac = alg / (cold_ms[dom] * 1e-3) / 1e9
            roof.update({"achieved_cold": round(ac, 1), "frac_cold": round(ac / HBM_PEAK_GBS, 4),
                         "avg_launch_us_cold": round(cold_ms[dom] * 1e3, 2)})
        step_bytes = touched * 3 * I * H * bpw + (3 * cfg.Is * H * bpw if cfg.shared else 0)
        extra = {"path_weight_bytes": step_bytes,
                 "path_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                 "path_frac_hbm": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        # gate/up grouped GEMM: flops, and the bytes it must move at least
        # (touched experts' gate+up weights, x, h written; shared expert alike)
        dom = "gemm_gateup"
        fig = prefill_figures(cfg, touched, kernel_ms[dom] * 1e-3, ms_per_step * 1e-3)
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        fl, by = fig["gateup_flops"], fig["gateup_bytes"]
        if fl / by >= ridge:   # arithmetic intensity above the ridge: bound by MFMA
            roof = {"bound": "mfma", "achieved": fig["gateup_tflops"],
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": fig["gateup_frac_mfma"]}
        else:
            roof = {"bound": "hbm", "achieved": round(by / (kernel_ms[dom] * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": fig["gateup_frac_hbm"]}
        roof.update({"kernel": dom, "traffic": recorded_traffic(cfg.name, dom),
                     "algorithmic_flops_per_launch": fl, "algorithmic_bytes_per_launch": by,
                     "arithmetic_intensity": round(fl / by, 1), "ridge": round(ridge, 1),
                     "frac_mfma": fig["gateup_frac_mfma"], "frac_hbm": fig["gateup_frac_hbm"],
                     "avg_launch_us": round(kernel_ms[dom] * 1e3, 2)})
        extra = {"path_flops": fig["path_flops"], "path_tflops": fig["path_tflops"],
                 "path_frac_mfma": fig["frac_mfma"]}
    if cold_ms:
        extra["cold_mall"] = {
            "scrub_mib": args.cold_mib, "steps": nk,
            "step_us": round(cold_step_ms * 1e3, 2),
            "kernels_us": {k2: round(v * 1e3, 2) for k2, v in cold_ms.items()}}

    cpu = None
    if not args.no_cpu_baseline:
        pn = None
        if args.pre_norm is not None:
            from moe_synth import norm_weight_values
            pn = (norm_weight_values(cfg), args.pre_norm)
        cpu = cpu_baseline(cfg, inp, xs, args.cpu_seconds, gating, args.routed_scale, pn,
                           None if res is None else res.cpu().numpy(), escale)

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
                   "expert_scale": bool(args.expert_scale),
                   "pre_norm_eps": args.pre_norm, "residual": args.residual,
                   "touched_experts": touched, "token_pool": P,
                   "expert_reuse_window": window,
                   "launch": stepper.label(),
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "kernels_us": {k2: round(v * 1e3, 2) for k2, v in kernel_ms.items()},
        **extra,
        "cpu_baseline": cpu,
    }
    del packed_bufs
    # the T=4096 (and T=16384) half of the metric: prefill workloads, same run
    if args.prefill and args.prefill != "none":
        del inp, w, ws, xs, out
        torch.cuda.empty_cache()
        for name in args.prefill.split(","):
            pf = bench_prefill(M, name, args.prefill_steps, 2, dev)
            line[f"prefill_t{CONFIGS[name].T}"] = pf
    if not args.no_peaks:
        line["measured_peaks"] = measured_peaks(dev)
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
        from oracle import weighted_sum_backward, glu_backward
        n, tcpu, t = 0, 0.0, 0
        while tcpu < args.cpu_seconds:
            t0c = time.perf_counter()
            weighted_sum_backward(g["w"][t:t + 1], g["y"][t:t + 1], g["dout"][t:t + 1])
            glu_backward(g["gate_up"][t * k:(t + 1) * k], g["dh"][t * k:(t + 1) * k], cfg.act)
            tcpu += time.perf_counter() - t0c
            n += 1
            t = (t + 1) % T
        cpu = {"value": round(n / tcpu, 3), "unit": "tokens/s", "cores": _blas_threads(),
               "host_cores": _nproc(), "kind": "oracle",
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


def cpu_baseline(cfg, inp, xs, seconds, gating=0, scale=1.0, pre_norm=None, residual=None,
                 expert_scale=None):
    """The float64 CPU oracle, as it stands, on a bounded sample of tokens."""
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
                    residual=residual, expert_scale=expert_scale)
            t_total += time.perf_counter() - t0
            n_done += 1
            if t_total >= seconds:
                break
        j += 1
    return {"value": round(n_done / t_total, 3), "unit": "tokens/s", "cores": _blas_threads(),
            "host_cores": _nproc(), "kind": "oracle",
            "sample": f"{n_done} tokens of {cfg.name} (drawn from the benchmark's token pool), "
                      f"one float64 oracle call per token with its experts decoded per call; "
                      f"inputs copied to host memory before timing; cores = the BLAS threads "
                      f"of its matrix products (the per-token loop is one Python thread), "
                      f"host_cores = the cores this process may use"}


if __name__ == "__main__":
    main()
