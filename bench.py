#!/usr/bin/env python3
"""Throughput of the MoE FFN layer on one MI355X; prints one JSON line.

A step is one forward pass of the whole layer (router, permutation, routed
and shared experts, combine) over one batch of synthetic tokens, with inputs
resident in HBM.  Successive steps cycle through several independently drawn
weight sets (as successive layers of a model would), so that the 256 MB
last-level cache cannot hold the weights a step streams.

Default workload: full-size decode, 1 token (hidden 5120, 384 MXFP4 experts
of width 2304, top-6, one bf16 shared expert).  `roofline` describes the
kernel that takes the most time, measured with HIP events on the stream it
runs on; `cpu_baseline` times the CPU oracle on a few tokens of the same
workload.  Timed steps are plain launches on one HIP stream by default
(`--launch graph` replays HIP graphs instead; the other form is timed after
for reference).
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
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode_t1_h5120_e384")
    ap.add_argument("--weight-sets", type=int, default=0, help="0: enough to exceed the last-level cache")
    ap.add_argument("--launch", choices=["stream", "graph"], default="stream",
                    help="timed steps as plain launches on one HIP stream (measured ~2 us/step faster at one "
                         "token) or as replays of HIP graphs (one per cycle over the weight sets); the other "
                         "form is timed afterwards for reference")
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
        # few-token path: routed and shared experts share a launch, routing is one fused kernel
        "route_permute": t * e * 4 + n * 8 + n * 4 * 2 + (e + 1) * 4,
        "gate_up": touched * gu_expert + 2 * i_s * h * 2 + t * h * 2 + n * i * 2 + t * i_s * 2,
        "down": touched * dn_expert + h * i_s * 2 + n * i * 2 + t * i_s * 2 + n * h * 2 + t * h * 2,
    }


def layer_bytes(cfg, touched: float) -> float:
    """Algorithmic bytes of the whole layer: touched experts' and shared weights, router, x and y once."""
    t, h, e, i = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.inter
    i_s = cfg.shared_inter if cfg.n_shared else 0
    cb = code_bytes(cfg)
    per_expert = 2 * i * (h * cb + h // 32) + h * (i * cb + i // 32)
    return touched * per_expert + 3 * i_s * h * 2 + e * h * 4 + 2 * t * h * 2


def layer_flops(cfg) -> float:
    t, h, e, k, i = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.inter
    i_s = cfg.shared_inter if cfg.n_shared else 0
    return 2.0 * t * (3 * h * i * k + 3 * h * i_s + e * h)


def cpu_baseline(cfg, inp, sample: int) -> dict:
    """The oracle, untuned, on `sample` decode tokens of this workload (one call per token)."""
    import numpy as np

    import oracle
    from moe_synth import make_router_inputs

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    xs, _, _ = make_router_inputs(cfg.with_(tokens=sample), seed=0, device="cpu", x_seed=1234)
    args = inp.oracle_args()
    args.pop("x_bits")
    t0 = time.perf_counter()
    for t in range(sample):
        oracle.layer_forward(x_bits=xs[t:t + 1].numpy().view(np.uint16), **args)
    dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{sample} decode tokens of {cfg.name}, one oracle call per token (float64 numpy; "
                      f"expert weights copied from the GPU per expert inside the timed region), {dt:.1f} s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this layer is measured on one MI355X and has no multi-GPU "
              "path here. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_ffn_07_amd as moe
    from moe_synth import CONFIGS, make_inputs

    moe.load()  # raises if the HIP library is missing: there is no other path
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    cfg = CONFIGS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    c = moe.config_from(cfg)
    # enough weight sets that one pass over them exceeds the 256 MB last-level cache 4x over
    per_step = layer_bytes(cfg, min(cfg.n_experts, cfg.tokens * cfg.top_k))
    sets = args.weight_sets or max(2, min(16, int(4 * 256e6 / per_step) + 1))
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

    use_graph = args.launch == "graph"
    run(args.warmup, graph=use_graph)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record()
    run(args.steps, offset=args.warmup, graph=use_graph)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # the other launch form for reference (same steps, from the same weight-set position)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n_other = min(args.steps, 200) // sets * sets or sets
    run(sets, graph=not use_graph)
    e0.record()
    run(n_other, graph=not use_graph)
    e1.record()
    torch.cuda.synchronize()
    other_ms = e0.elapsed_time(e1) / n_other

    # per-kernel durations, HIP events on the library's stream around each kernel
    sums, counts = {}, {}
    for rep in range(args.kernel_reps):
        for s in range(sets):
            for name, ms in moe.moe_layer_forward_timed(c, weights[s], x, t, y, ws):
                sums[name] = sums.get(name, 0.0) + ms
                counts[name] = counts.get(name, 0) + 1
    kernel_ms = {k: sums[k] / counts[k] for k in sums}
    dominant = max(kernel_ms, key=kernel_ms.get)
    algo = algorithmic_bytes(cfg, touched_avg)
    achieved = algo[dominant] / (kernel_ms[dominant] * 1e-3) / 1e9
    digest = kernel_source_digest()
    traffic = traffic_from_profile(dominant, cfg.name, digest)

    tokens_per_s = t / (ms_per_step * 1e-3)
    lb = layer_bytes(cfg, touched_avg)
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": t, "hidden": cfg.hidden, "n_experts": cfg.n_experts,
                   "top_k": cfg.top_k, "inter": cfg.inter, "shared_inter": cfg.shared_inter,
                   "expert_weights": ("mxfp8 (e4m3 + e8m0 per 32)" if cfg.expert_format == "mxfp8"
                                      else "mxfp4 (e2m1 + e8m0 per 32)"), "router_weights": "fp32",
                   "pre_ffn_rmsnorm": bool(cfg.norm),
                   "weight_sets_cycled": sets, "launch": ("hipgraph (one graph per cycle over the weight sets)" if use_graph
                                                       else "stream (plain launches on one HIP stream)"),
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dominant,
                     "kernel_ms": kernel_ms[dominant], "algorithmic_bytes": algo[dominant]},
        "layer": {"algorithmic_bytes": lb, "hbm_frac": lb / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                  "flops": layer_flops(cfg), "experts_touched_per_step": touched_avg,
                  ("stream_ms_per_step" if use_graph else "graph_ms_per_step"): other_ms, "kernel_ms": kernel_ms,
                  "kernel_source_digest": digest, "timed_wall_s": wall, "input_gen_s": gen_s},
        "cpu_baseline": None,
    }
    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(cfg, inputs[0], args.cpu_sample)
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
