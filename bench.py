#!/usr/bin/env python3
"""Throughput of the MoE FFN layer on one MI355X; prints one JSON line.

A step is one forward pass of the whole layer (router, permutation, routed
and shared experts, combine) over one batch of synthetic tokens, with inputs
resident in HBM.  Successive steps cycle through several independently drawn
weight sets (as successive layers of a model would), so that the 256 MB
last-level cache cannot hold the weights a step streams.

The headline workload (`--workload`, default the full-size one-token decode:
hidden 5120, 384 MXFP4 experts of width 2304, top-6, one bf16 shared expert)
gives `value`, `ms_per_step` and `roofline`.  The same run also times the
other shapes the metric names (`--also`: 64-token decode, 4096-token prefill
and the 16384-token skewed layer by default); each gets its own entry under
`workloads` with its time, tokens/s, the layer's HBM and MFMA fractions and
the roofline of its dominant kernel.  A workload is bound by HBM or by the
matrix units, whichever its algorithmic bytes and flops take longer on at the
published peaks.  Kernel durations come from HIP events on the library's
stream around every kernel.  `cpu_baseline` times the CPU oracle on a few
tokens of the headline workload, with its weights already in host memory.
Timed steps are plain launches on one HIP stream by default (`--launch graph`
replays HIP graphs; the other form is timed after for reference).  Before
its W warm-up steps each workload runs untimed for `--settle-s` seconds, so
that the clock has left its idle level when the K timed steps start.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec on 1 MI355X (decode B=1/64, prefill 4K); % HBM/MFMA roofline"
# MI355X published peaks (dense)
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP4_PEAK_TFLOPS = 10100.0  # MXFP4 / MXFP6
FP8_PEAK_TFLOPS = 5000.0
PROFILES = os.path.join(ROOT, "profiles")
DEFAULT_ALSO = "decode_t64_h5120_e384,prefill_t4096_h5120_e384,skew_t16384_h5120_e128"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the clock ramps over the first ~0.1 s of work; --settle-s covers that, whatever the warm-up count
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_t1_h5120_e384")
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="comma-separated workloads timed in the same run ('' for none); each runs "
                         "min(steps, 200) timed steps after min(warmup, 20) untimed ones")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed seconds of steps before the warm-up steps, for the clock to reach its busy level")
    ap.add_argument("--weight-sets", type=int, default=0, help="0: enough to exceed the last-level cache")
    ap.add_argument("--launch", choices=["stream", "graph"], default="stream",
                    help="timed steps as plain launches on one HIP stream or as replays of HIP graphs (one per "
                         "cycle over the weight sets, as a serving loop replays its captured step over a model's "
                         "layers); the other form is timed afterwards for reference")
    ap.add_argument("--kernel-reps", type=int, default=5, help="timed forwards per weight set for kernel times")
    ap.add_argument("--cpu-sample", type=int, default=16, help="decode tokens the CPU oracle runs (0: skip)")
    ap.add_argument("--json-out", default="")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy 3x (reference for hardware byte counters)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_ffn_07_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str, digest: str):
    """HBM bytes per launch of `kernel` from a committed PMC summary, if taken on this kernel source."""
    path = os.path.join(PROFILES, f"pmc_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel source digest:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != digest:
        return None
    m = re.search(rf"^\|\s*{re.escape(kernel)}\s*\|[^|]*\|[^|]*\|\s*([0-9.eE+]+)\s*\|", text, flags=re.M)
    return float(m.group(1)) if m else None


def code_bytes(cfg) -> float:
    """Bytes per routed-expert weight element: MXFP4 codes are half a byte, MXFP8 codes one byte."""
    return 1.0 if cfg.expert_format == "mxfp8" else 0.5


def algorithmic_bytes(cfg, touched: float) -> dict:
    """Bytes each kernel must move at least: weights it reads once, inputs once, outputs once."""
    t, h, e, k, i = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.inter
    i_s = cfg.shared_inter if cfg.n_shared else 0
    n = t * k
    cb = code_bytes(cfg)
    gu_expert = 2 * i * (h * cb + h // 32)
    dn_expert = h * (i * cb + i // 32)
    return {
        "router_logits": e * h * 4 + t * h * 2 + t * e * 4,
        "router_topk": t * e * 4 + n * 8,
        "permute": n * 4 * 3 + (e + 1) * 4,
        "routed_gate_up": touched * gu_expert + t * h * 2 + n * i * 2,
        "routed_down": touched * dn_expert + n * i * 2 + n * h * 2,
        "shared_gate_up": 2 * i_s * h * 2 + t * h * 2 + t * i_s * 2,
        "shared_down": h * i_s * 2 + t * i_s * 2 + t * h * 2,
        "combine": n * h * 2 + t * h * 2 * 2 + n * 8,
        # few tokens: routed down projection with the weighted combine and the shared output folded in
        "routed_down_combine": touched * dn_expert + n * i * 2 + n * 8 + t * h * 2 * 2,
        # few tokens: the shared expert's projections run inside the router and routing launches
        "router_shared_gate_up": e * h * 4 + t * h * 2 + t * e * 4 + 2 * i_s * h * 2 + t * i_s * 2,
        "route_shared_down": t * e * 4 + n * 8 + n * 4 * 2 + h * i_s * 2 + t * i_s * 2 + t * h * 2,
        # one or two tokens, streaming form: router scores alone, routing beside the shared gate/up,
        # the shared down projection beside the routed gate/up
        "router_scores": e * h * 4 + t * h * 2 + 2 * t * e * 4,
        # pre-FFN RMSNorm: inside the router launch (x, gain, normalised rows out), or a launch of its own
        "norm_router_scores": e * h * 4 + t * h * 2 + h * 2 + t * h * 2 + 2 * t * e * 4,
        "rmsnorm": 2 * t * h * 2 + h * 2,
        "route_shared_gate_up": 2 * t * e * 4 + n * 8 + n * 4 * 2 + 2 * i_s * h * 2 + t * h * 2 + t * i_s * 2,
        "routed_gate_up_shared_down": touched * gu_expert + t * h * 2 + n * i * 2 + h * i_s * 2 + t * i_s * 2
        + t * h * 2,
        # one or two tokens, three launches: routed gate/up (every wave routing from the scores) beside the
        # shared gate/up; routed down with the shared down and the combine
        "route_gate_up_shared_gate_up": touched * gu_expert + 2 * i_s * h * 2 + t * h * 2 + 2 * t * e * 4
        + n * i * 2 + t * i_s * 2 + n * 16,
        "routed_down_shared_down_combine": touched * dn_expert + h * i_s * 2 + n * i * 2 + t * i_s * 2 + n * 12
        + t * h * 2,
        # one or two tokens without the pre-FFN norm: router scores beside the shared gate/up; routed gate/up
        # (every wave routing from the scores) beside the shared down; routed down with the combine
        "router_scores_shared_gate_up": e * h * 4 + t * h * 2 + 2 * t * e * 4 + 2 * i_s * h * 2 + t * i_s * 2,
        "route_gate_up_shared_down": touched * gu_expert + t * h * 2 + 2 * t * e * 4 + n * i * 2 + n * 16
        + h * i_s * 2 + t * i_s * 2 + t * h * 2,
        # few-token path: routed and shared experts share a launch, routing is one fused kernel
        "route_permute": t * e * 4 + n * 8 + n * 4 * 2 + (e + 1) * 4,
        "gate_up": touched * gu_expert + 2 * i_s * h * 2 + t * h * 2 + n * i * 2 + t * i_s * 2,
        "down": touched * dn_expert + h * i_s * 2 + n * i * 2 + t * i_s * 2 + n * h * 2 + t * h * 2,
        # many tokens: x and h rows to two-term MXFP6 records (208 bytes per 128 values)
        "mx6_x": t * h * 2 + t * h * 208 / 128,
        "mx6_h": n * i * 2 + n * i * 208 / 128,
    }


def kernel_flops(cfg) -> dict:
    """Flops each matrix kernel must do (the selected experts' products only)."""
    t, h, e, k, i = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.inter
    i_s = cfg.shared_inter if cfg.n_shared else 0
    n = t * k
    return {"routed_gate_up": 2.0 * n * h * 2 * i, "routed_down": 2.0 * n * i * h,
            "shared_gate_up": 2.0 * t * h * 2 * i_s, "shared_down": 2.0 * t * i_s * h,
            "router_logits": 2.0 * t * e * h}


# the arithmetic each matrix kernel runs in, and that type's published dense peak (TFLOP/s); the routed GEMMs
# for many tokens with MXFP4 experts run on two-term MXFP6 activations (the x and h records, kernels mx6_x and
# mx6_h): two FP4-rate block-scaled MFMAs per step, so they reach at most half the FP4 peak in algorithmic flops
KERNEL_DTYPE_MX6 = {"routed_gate_up": ("two-term MXFP6 x MXFP4 block-scaled MFMA", FP4_PEAK_TFLOPS),
                    "routed_down": ("two-term MXFP6 x MXFP4 block-scaled MFMA", FP4_PEAK_TFLOPS)}
KERNEL_DTYPE = {"routed_gate_up": ("bf16 MFMA on exactly dequantised expert weights", BF16_PEAK_TFLOPS),
                "routed_down": ("bf16 MFMA on exactly dequantised expert weights", BF16_PEAK_TFLOPS),
                "shared_gate_up": ("bf16 MFMA", BF16_PEAK_TFLOPS), "shared_down": ("bf16 MFMA", BF16_PEAK_TFLOPS),
                "router_logits": ("bf16 MFMA on three exact bf16 terms of the fp32 weights", BF16_PEAK_TFLOPS)}


def layer_bytes(cfg, touched: float) -> float:
    """Algorithmic bytes of the whole layer: touched experts' and shared weights, router, x and y once."""
    t, h, e, i = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.inter
    i_s = cfg.shared_inter if cfg.n_shared else 0
    cb = code_bytes(cfg)
    per_expert = 2 * i * (h * cb + h // 32) + h * (i * cb + i // 32)
    return touched * per_expert + 3 * i_s * h * 2 + e * h * 4 + 2 * t * h * 2


def layer_flops(cfg) -> dict:
    """Algorithmic flops of the layer: routed (selected experts), shared, router."""
    t, h, e, k, i = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.inter
    i_s = cfg.shared_inter if cfg.n_shared else 0
    return {"routed": 2.0 * t * 3 * h * i * k, "shared": 2.0 * t * 3 * h * i_s, "router": 2.0 * t * e * h}


def layer_roofline(cfg, touched: float, ms: float) -> dict:
    """Time the layer needs at the published peaks, its bound, and the fractions a measured time reaches.

    Matrix time: routed flops at the FP4 (MXFP4/MXFP6) peak, shared flops at the bf16 peak, router flops as three
    exact bf16 terms at the bf16 peak."""
    lb = layer_bytes(cfg, touched)
    f = layer_flops(cfg)
    t_hbm = lb / (HBM_PEAK_GBS * 1e9)
    fp4_peak = FP8_PEAK_TFLOPS if cfg.expert_format == "mxfp8" else FP4_PEAK_TFLOPS
    t_mfma = f["routed"] / (fp4_peak * 1e12) + (f["shared"] + 3 * f["router"]) / (BF16_PEAK_TFLOPS * 1e12)
    s = ms * 1e-3
    return {"bound": "mfma" if t_mfma > t_hbm else "hbm", "algorithmic_bytes": lb, "flops": f,
            "t_hbm_us": t_hbm * 1e6, "t_mfma_us": t_mfma * 1e6,
            "hbm_frac": lb / s / (HBM_PEAK_GBS * 1e9),
            "routed_fp4_frac": f["routed"] / s / (fp4_peak * 1e12),
            "mfma_frac": t_mfma / s,
            "roofline_frac": max(t_hbm, t_mfma) / s}


def kernel_roofline(cfg, touched: float, kernel: str, kernel_ms: float, bound: str, digest: str,
                    mx6: bool = False) -> dict:
    """Roofline entry of one kernel: algorithmic bytes (HBM-bound layer) or flops (MFMA-bound layer) over its
    event-timed duration, against the published peak of that resource (for flops, of the kernel's own dtype)."""
    algo = algorithmic_bytes(cfg, touched)
    flops = kernel_flops(cfg)
    s = kernel_ms * 1e-3
    if bound == "mfma" and kernel in flops:
        dtype, peak = (KERNEL_DTYPE_MX6 if mx6 and kernel in KERNEL_DTYPE_MX6 else KERNEL_DTYPE)[kernel]
        ach = flops[kernel] / s / 1e12
        out = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
               "dtype": dtype, "flops": flops[kernel], "fp4_peak_frac": ach / FP4_PEAK_TFLOPS}
    else:
        ach = algo.get(kernel, 0.0) / s / 1e9
        out = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
               "algorithmic_bytes": algo.get(kernel, 0.0)}
        if kernel in flops:
            out["mfma_tflops"] = flops[kernel] / s / 1e12
    out.update({"traffic": traffic_from_profile(kernel, cfg.name, digest), "kernel": kernel, "kernel_ms": kernel_ms})
    return out


def cpu_baseline(cfg, inp, sample: int) -> dict:
    """The oracle, untuned, on `sample` decode tokens of this workload (one call per token), its inputs in host
    memory before the timed region starts."""
    import numpy as np

    import oracle
    from moe_synth import make_router_inputs

    try:
        from threadpoolctl import threadpool_info
        blas = [(p.get("internal_api"), p.get("num_threads", 1)) for p in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []
    threads = max([n for _, n in blas] + [1])
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    xs, _, _ = make_router_inputs(cfg.with_(tokens=sample), seed=0, device="cpu", x_seed=1234)
    host = inp.to("cpu")  # every weight copied to host memory before timing
    args = host.oracle_args()
    args.pop("x_bits")
    t0 = time.perf_counter()
    for t in range(sample):
        oracle.layer_forward(x_bits=xs[t:t + 1].numpy().view(np.uint16), **args)
    dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{sample} decode tokens of {cfg.name}, one oracle call per token (float64 numpy, weights in "
                      f"host memory), {dt:.1f} s",
            "host": {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
                     "blas": blas}}


def run_workload(name: str, steps: int, warmup: int, launch: str, weight_sets: int, kernel_reps: int, dev: str,
                 keep_inputs: bool = False, settle_s: float = 0.0) -> dict:
    import torch

    import mixture_experts_ffn_07_amd as moe
    from moe_synth import CONFIGS, make_inputs

    cfg = CONFIGS[name]
    c = moe.config_from(cfg)
    # enough weight sets that one pass over them exceeds the 256 MB last-level cache 4x over
    per_step = layer_bytes(cfg, min(cfg.n_experts, cfg.tokens * cfg.top_k))
    sets = weight_sets or max(2, min(16, int(4 * 256e6 / per_step) + 1))
    t0 = time.time()
    inputs = [make_inputs(cfg, seed=0, device=dev, weight_set=s) for s in range(sets)]
    for s in range(1, sets):  # one batch of tokens, every weight set
        inputs[s].x = inputs[0].x
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    weights = [moe.weights_from(inp) for inp in inputs]
    t = cfg.tokens
    x = inputs[0].x
    y = torch.empty((t, cfg.hidden), dtype=torch.int16, device=dev)
    ws = moe.workspace(c, t, device=dev)

    # routing of every set: distinct experts each step touches
    idx = torch.empty((t, cfg.top_k), dtype=torch.int32, device=dev)
    wt = torch.empty((t, cfg.top_k), dtype=torch.float32, device=dev)
    touched = []
    for w in weights:
        moe.moe_layer_forward(c, w, x, t, y, idx, wt, ws)
        touched.append(int(torch.unique(idx).numel()))
    torch.cuda.synchronize()
    touched_avg = sum(touched) / len(touched)

    def step_eager(s):
        moe.moe_layer_forward(c, weights[s], x, t, y, None, None, ws)

    # HIP graphs: one graph per weight set (one step) and one graph of a whole
    # cycle over the sets, replayed back to back as a model-level graph would
    # run consecutive layers; a step is still one whole layer forward
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_eager(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for s in range(sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_eager(s)
        graphs.append(g)
    cycle = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cycle):
        for s in range(sets):
            step_eager(s)
    torch.cuda.synchronize()

    def run(n_steps, offset=0, graph=True):
        i = 0
        while i < n_steps:
            s = (i + offset) % sets
            if graph and s == 0 and n_steps - i >= sets:
                cycle.replay()
                i += sets
            elif graph:
                graphs[s].replay()
                i += 1
            else:
                step_eager(s)
                i += 1

    use_graph = launch == "graph"
    # clock settle: the chip's clock ramps up over the first ~0.1 s of steady work after idle, so the step
    # runs untimed for a fixed wall time before the W warm-up steps, as it would in a serving loop that is
    # already busy (a handful of warm-up steps alone still measures the ramp)
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle_s:
        run(sets * 8, graph=use_graph)
        settle_steps += sets * 8
        torch.cuda.synchronize()
    run(warmup, graph=use_graph)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record()
    run(steps, offset=warmup, graph=use_graph)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / steps

    # the other launch form for reference (same steps, from the same weight-set position)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n_other = min(steps, 200) // sets * sets or sets
    run(sets, graph=not use_graph)
    e0.record()
    run(n_other, graph=not use_graph)
    e1.record()
    torch.cuda.synchronize()
    other_ms = e0.elapsed_time(e1) / n_other

    # per-kernel durations, HIP events on the library's stream around each kernel
    sums, counts = {}, {}
    for rep in range(kernel_reps):
        for s in range(sets):
            for kname, ms in moe.moe_layer_forward_timed(c, weights[s], x, t, y, ws):
                sums[kname] = sums.get(kname, 0.0) + ms
                counts[kname] = counts.get(kname, 0) + 1
    kernel_ms = {k: sums[k] / counts[k] for k in sums}
    dominant = max(kernel_ms, key=kernel_ms.get)
    digest = kernel_source_digest()
    layer = layer_roofline(cfg, touched_avg, ms_per_step)
    roof = kernel_roofline(cfg, touched_avg, dominant, kernel_ms[dominant], layer["bound"], digest,
                           mx6="mx6_x" in kernel_ms)
    out = {
        "workload": cfg.name, "tokens": t, "ms_per_step": ms_per_step, "tokens_per_s": t / (ms_per_step * 1e-3),
        "steps": steps, "warmup": warmup, "clock_settle": {"seconds": settle_s, "steps": settle_steps},
        "config": {"workload": cfg.name, "tokens": t, "hidden": cfg.hidden, "n_experts": cfg.n_experts,
                   "top_k": cfg.top_k, "inter": cfg.inter, "shared_inter": cfg.shared_inter,
                   "expert_weights": ("mxfp8 (e4m3 + e8m0 per 32)" if cfg.expert_format == "mxfp8"
                                      else "mxfp4 (e2m1 + e8m0 per 32)"), "router_weights": "fp32",
                   "router_bias": "zipf(1.2)" if cfg.bias == "zipf" else "none",
                   "pre_ffn_rmsnorm": bool(cfg.norm), "weight_sets_cycled": sets,
                   "launch": ("hipgraph (one graph per cycle over the weight sets)" if use_graph
                              else "stream (plain launches on the caller's HIP stream; from 17 to 512 tokens the "
                                    "library forks the shared expert onto its side stream and joins it before the "
                                    "combine)"),
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "layer": dict(layer, experts_touched_per_step=touched_avg, kernel_ms=kernel_ms,
                      kernel_source_digest=digest, timed_wall_s=wall, input_gen_s=gen_s,
                      **{("stream_ms_per_step" if use_graph else "graph_ms_per_step"): other_ms}),
    }
    if keep_inputs:
        out["_inputs"] = inputs[0]
    del graphs, cycle, inputs, weights, ws, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this layer is measured on one MI355X and has no multi-GPU "
              "path here. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_ffn_07_amd as moe
    from moe_synth import CONFIGS

    moe.load()  # raises if the HIP library is missing: there is no other path
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    head = run_workload(args.workload, args.steps, args.warmup, args.launch, args.weight_sets, args.kernel_reps, dev,
                        keep_inputs=args.cpu_sample > 0, settle_s=args.settle_s)
    print(f"# {head['workload']}: {head['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    head_inputs = head.pop("_inputs", None)
    others = []
    for name in [n for n in args.also.split(",") if n and n != args.workload]:
        if name not in CONFIGS:
            raise SystemExit(f"unknown workload {name}")
        r = run_workload(name, min(args.steps, 200), min(args.warmup, 20), args.launch, args.weight_sets,
                         min(args.kernel_reps, 3), dev, settle_s=args.settle_s)
        print(f"# {name}: {r['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        others.append(r)

    cfg = CONFIGS[args.workload]
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": head["clock_settle"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "layer": head["layer"],
        "workloads": [{k: v for k, v in r.items()} for r in [head] + others],
        "cpu_baseline": None,
    }
    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(cfg, head_inputs, args.cpu_sample)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 1 << 30
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
