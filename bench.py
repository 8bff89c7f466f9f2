"""Benchmark of the Nemotron-H MoE layer forward on one MI355X.

One step = one ``moe_forward`` call (route -> permute -> routed expert MLPs ->
shared expert -> combine) over one batch of seeded synthetic tokens that are
already resident in HBM; for the block workloads one ``moe_block_forward``
(RMSNorm first, the residual added in combine).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is the largest one-GPU configuration: the
load-imbalanced prefill of the Nemotron-H layer (T=16384, d=2688, 128 experts
in 8 groups, top-6 from one group, I=1856, shared 3712, bf16, eight experts'
correction bias raised by 2.0).  Besides tokens/s the line carries the
roofline of the dominant kernel, timed live with per-kernel HIP events on the
stream the kernels run on, and the fp64 CPU oracle timed on a bounded sample
of the same workload (its first 1024 tokens at most).  After the default
workload, the line's ``other_workloads`` gives the same timing, in short, for
the decode step (T=32, bf16 and 4-bit experts), the balanced prefill chunk
(T=4096) and the fp8 experts (T=8192); ``--no-others`` skips them.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; TFLOP/s and HBM GB/s as % of MI355X peak"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
DEFAULT_WORKLOAD = "skew-bf16-T16384"
DEFAULT_STEPS = {"tiny-f32-T64": 200, "decode-bf16-T32": 200, "prefill-bf16-T4096": 50,
                 "skew-bf16-T16384": 20, "fp8-T8192": 30, "decode-fp4-T32": 200,
                 "block-decode-bf16-T32": 200}
# configurations timed after the default one (steps each), reported in short
OTHER_WORKLOADS = ["decode-bf16-T32", "prefill-bf16-T4096", "fp8-T8192", "decode-fp4-T32"]
OTHER_STEPS = {"decode-bf16-T32": 100, "prefill-bf16-T4096": 30, "fp8-T8192": 20,
               "decode-fp4-T32": 100}
# tokens of the oracle's timed sample (about 12 s of fp64 work on 16 host threads)
CPU_SAMPLE_TOKENS = 1024
# kernels whose counter readings are reported as "traffic"
TRAFFIC_SOURCES = ["non_gated_relu_amd/csrc/gemm.hip", "non_gated_relu_amd/csrc/common.hpp",
                   "non_gated_relu_amd/csrc/internal.hpp"]


def esize(dt):
    return {"f32": 4, "bf16": 2, "fp8": 1}[dt]


def wbytes(dt, rows: int, cols: int) -> int:
    """Stored bytes of one [rows, cols] weight matrix: its elements, plus the
    fp32 row scales (fp8) or the E8M0 scale of every 32 elements (fp4)."""
    if dt == "fp4":
        return rows * cols // 2 + rows * cols // 32
    return rows * cols * esize(dt) + (rows * 4 if dt == "fp8" else 0)


def mfma_dtype(dt):
    """Operand type of the MFMA a weight type runs on (fp4 is widened to bf16)."""
    return "bf16" if dt == "fp4" else dt


def add_flops(stage, dtype, flops):
    """Record the MFMA work of a launch by operand type (a launch with fp8
    routed experts and a bf16 shared expert holds both)."""
    by = stage.setdefault("flops_by_dtype", {stage["dtype"]: stage["flops"] - flops})
    by[dtype] = by.get(dtype, 0) + flops


def stage_work(wl, active: int, stages):
    """Algorithmic bytes and flops of each stage's launch(es) for one step,
    for the stages the library runs (binding.stages_of).

    ``bytes`` counts only what the method itself must move through the
    launch: the weights of the active experts (one unit = one expert
    projection of I*d elements with its scales: fp32 per row for fp8, E8M0
    per 32 elements for fp4), the shared expert's weights in the launches
    that run it, the layer input x read by the up projections, and the layer
    output y written by whichever launch combines.  Traffic that exists only
    because the layer is split into launches (h written and read back, the
    fp32 per-slot rows written by the down projection and read by the
    combine, the shared expert's fp32 rows, the routing indices) is
    ``implementation_bytes``, reported beside it and never credited.
    """
    T, d, E, k, I, Is = wl.tokens, wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter
    S = T * k
    ae = esize(wl.act_dtype)
    edt, sdt = wl.expert_dtype, wl.shared_weight_dtype
    fp8 = edt == "fp8"
    a_in = 1 if fp8 else ae              # the routed GEMMs read x (fp8: its e4m3 codes)
    h_out = 4 if fp8 or edt == "f32" else 2  # h as written by the up GEMM (bf16 for bf16, fp4)
    h_in = 1 if fp8 else h_out
    up_u, dn_u = wbytes(edt, I, d), wbytes(edt, d, I)
    combined = "combine" not in stages   # the shared down projection combines
    block = bool(getattr(wl, "block", False))
    y_bytes = T * d * ae * (2 if block else 1)  # y written (+ the residual x read)
    comb_impl = S * d * 4 + S * 8          # slot rows and routing weights read
    w = {
        "route": dict(bytes=T * d * ae + E * d * ae + E * 4, flops=2 * T * d * E,
                      implementation_bytes=S * 8, dtype=wl.act_dtype),
        "routed_up": dict(bytes=active * up_u + T * d * a_in, flops=2 * S * d * I,
                          implementation_bytes=S * I * h_out, dtype=mfma_dtype(edt),
                          unit_bytes=up_u, units=active),
        "routed_down": dict(bytes=active * dn_u, flops=2 * S * I * d,
                            implementation_bytes=S * I * h_in + S * d * 4,
                            dtype=mfma_dtype(edt), unit_bytes=dn_u, units=active),
    }
    if Is:
        sh_h = 4 if sdt == "f32" else 2
        su, sd = wbytes(sdt, Is, d), wbytes(sdt, d, Is)
        sh_out = 0 if combined else T * d * 4      # the shared rows, unless combined
        shared_down = dict(bytes=sd + (y_bytes if combined else 0), flops=2 * T * Is * d,
                           implementation_bytes=T * Is * sh_h + sh_out +
                           (comb_impl if combined else 0),
                           dtype=mfma_dtype(sdt), unit_bytes=sd, units=1)
        if "shared_up" in stages:
            w["shared_up"] = dict(bytes=su + T * d * ae, flops=2 * T * d * Is,
                                  implementation_bytes=T * Is * sh_h, dtype=mfma_dtype(sdt),
                                  unit_bytes=su, units=1)
        else:  # one more group of the routed up launch (x is already counted)
            w["routed_up"]["bytes"] += su
            w["routed_up"]["flops"] += 2 * T * d * Is
            w["routed_up"]["implementation_bytes"] += T * Is * sh_h
            w["routed_up"]["shared_weight_bytes"] = su
            add_flops(w["routed_up"], mfma_dtype(sdt), 2 * T * d * Is)
        if "shared_down" in stages:
            w["shared_down"] = shared_down
        else:  # one more group of the routed down launch
            for key in ("bytes", "flops", "implementation_bytes"):
                w["routed_down"][key] += shared_down[key]
            w["routed_down"]["shared_weight_bytes"] = sd
            add_flops(w["routed_down"], mfma_dtype(sdt), shared_down["flops"])
    if not combined:
        w["combine"] = dict(bytes=y_bytes, flops=0, dtype="f32",
                            implementation_bytes=comb_impl + (T * d * 4 if Is else 0))
    if fp8:
        w["quant_x"] = dict(bytes=0, flops=0, dtype="f32", implementation_bytes=T * d * (ae + 1) + T * 4)
        w["quant_h"] = dict(bytes=0, flops=0, dtype="f32", implementation_bytes=S * I * 5 + S * 4)
    if block:
        # the norm reads x and writes x_norm
        w["norm"] = dict(bytes=T * d * ae + d * ae, flops=0, dtype="f32",
                         implementation_bytes=T * d * ae)
    return w


def layer_work(wl, active: int):
    """Algorithmic flops and bytes of one whole layer step."""
    T, d, E, k, I, Is = wl.tokens, wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter
    ae = esize(wl.act_dtype)
    edt, sdt = wl.expert_dtype, wl.shared_weight_dtype
    flops = T * (2 * d * E + k * 4 * d * I + 4 * d * Is)
    byts = (active * (wbytes(edt, I, d) + wbytes(edt, d, I)) + wbytes(sdt, Is, d) +
            wbytes(sdt, d, Is) + E * d * ae + E * 4 + 2 * T * d * ae)
    if getattr(wl, "block", False):
        byts += d * ae  # the norm weight (x is read once and y written once either way)
    return flops, byts


def source_hash():
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str, kernel_stage: str):
    """HBM bytes per launch from committed counter readings, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(workload, {}).get(kernel_stage)
    if not entry or entry.get("source_sha256") != source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(wl, inp, y_gpu, idx_gpu, budget_s: float):
    """The oracle on the first min(T, CPU_SAMPLE_TOKENS) tokens of the bench's
    own input, repeated until about budget_s seconds have passed (at least
    once); tokens are independent, so tokens/s over the sample is the
    oracle's rate on the whole workload."""
    import numpy as np

    import oracle

    T = wl.tokens
    n = min(T, CPU_SAMPLE_TOKENS)
    tokens = np.arange(n)
    reps, elapsed, out = 0, 0.0, None
    t0 = time.perf_counter()
    while reps == 0 or (elapsed < budget_s and reps < 1000):
        out = (oracle.block_forward(wl, inp, tokens=tokens) if getattr(wl, "block", False)
               else oracle.forward(wl, inp, tokens=tokens))
        reps += 1
        elapsed = time.perf_counter() - t0
    R = float(np.sqrt(np.mean(out["y"] ** 2)))
    err = np.abs(y_gpu[:n].astype(np.float64) - out["y"])
    parity = {"tokens_checked": n, "max_over_rms": float(err.max() / R),
              "mean_over_rms": float(err.mean() / R),
              "routing_exact": bool(np.array_equal(idx_gpu[:n], out["topk_idx"]))}
    base = {"value": n * reps / elapsed, "unit": "tokens/s",
            "cores": int(oracle.lib().orc_num_threads()), "kind": "oracle",
            "sample": f"fp64 oracle on the first {n} tokens of this workload, "
                      f"{reps} repetition(s), {elapsed:.1f} s wall"}
    return base, parity


def measure(wl, steps: int, warmup: int, graph: bool, evict_mb: int):
    """Time `steps` layer steps of workload `wl` (after `warmup` untimed ones):
    per-kernel HIP events on the eager steps, then the whole step replayed
    from a HIP graph.  Returns the figures, and the layer, its input and its
    output for the oracle check."""
    import numpy as np
    import torch

    from non_gated_relu_amd import binding
    from non_gated_relu_amd.synthetic import make_inputs

    dev = torch.device("cuda:0")
    print(f"bench: generating {wl.name}", file=sys.stderr, flush=True)
    inp = make_inputs(wl)
    layer = binding.MoELayer(wl, inp, device=dev)
    x = binding.to_device(inp["x"], dev, "x", wl)
    y = torch.empty((wl.tokens, wl.hidden), dtype=x.dtype, device=dev)
    block = bool(getattr(wl, "block", False))
    stages = binding.stages_of(wl, block=block)

    def run(ev):
        if block:
            layer.block(x, out=y, stage_events=ev)
        else:
            layer(x, y=y, stage_events=ev)
    # one set of kernel timestamp events per timed step, read after the region
    evs = [binding.StageEvents() for _ in range(steps)]

    print(f"bench: warmup {warmup}, timing {steps} steps", file=sys.stderr, flush=True)
    for i in range(warmup):
        run(evs[i % steps])
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(steps):
        run(evs[i])
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t0

    per_stage = {s: 0.0 for s in stages}
    step_sums = []
    for e in evs:
        ms_e = e.elapsed_ms(stages)
        step_sums.append(sum(ms_e.values()))
        for s, ms in ms_e.items():
            per_stage[s] += ms
    stage_ms = {s: per_stage[s] / steps for s in stages}
    q10, q50, q90 = np.percentile(step_sums, [10, 50, 90])
    eager_s = total_s

    # the same step replayed from a HIP graph: no per-kernel launch gaps
    graph_s = None
    if graph:
        gstep = binding.GraphStep(layer, x, y, block=block)
        for _ in range(warmup):
            gstep.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            gstep.replay()
        torch.cuda.synchronize()
        graph_s = time.perf_counter() - t0
        total_s = graph_s

    # cache check: the eager steps again, each after reading a buffer larger than
    # the Infinity Cache (a read, so no dirty lines are left to write back)
    cache_check = None
    if evict_mb > 0:
        big = torch.ones(evict_mb * (1 << 20) // 4, dtype=torch.float32, device=dev)
        sink = torch.zeros((), dtype=torch.float32, device=dev)
        evs2 = [binding.StageEvents() for _ in range(steps)]
        for i in range(steps):
            sink += big.sum()
            run(evs2[i])
        torch.cuda.synchronize()
        ev_stage = {s: 0.0 for s in stages}
        for e in evs2:
            for s, ms in e.elapsed_ms(stages).items():
                ev_stage[s] += ms / steps
        cache_check = {"evict": f"{evict_mb} MB read before each eager step",
                       "stages_ms_sum": round(sum(stage_ms.values()), 5),
                       "stages_ms_sum_after_evict": round(sum(ev_stage.values()), 5)}
        del big

    counts = layer.expert_counts.cpu().numpy()
    active = int((counts > 0).sum())
    work = stage_work(wl, active, stages)
    ms_per_step = 1e3 * total_s / steps
    tokens_per_s = wl.tokens * steps / total_s

    # dominant kernel: the GEMM stage with the largest device time
    gemm_stages = [s for s in stages if s in work and work[s]["flops"] > 0 and s != "route"]
    dom = max(gemm_stages, key=lambda s: stage_ms[s])
    dw = work[dom]
    t_s = stage_ms[dom] / 1e3
    peak_t = PEAK_TFLOPS[dw["dtype"]]
    if len(dw.get("flops_by_dtype", {})) > 1:
        # mixed MFMA types: the rate at which the launch's work would run at each type's peak
        peak_t = dw["flops"] / sum(f / PEAK_TFLOPS[t] for t, f in dw["flops_by_dtype"].items())
    hbm_bound = dw["bytes"] / (PEAK_HBM_GBS * 1e9) >= dw["flops"] / (peak_t * 1e12)
    if hbm_bound:
        achieved, peak, unit = dw["bytes"] / t_s / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = dw["flops"] / t_s / 1e12, peak_t, "TFLOP/s"
    roofline = {"bound": "hbm" if hbm_bound else "mfma", "achieved": achieved, "peak": peak,
                "unit": unit, "frac": achieved / peak, "traffic": load_traffic(wl.name, dom),
                "kernel": dom, "kernel_ms": stage_ms[dom],
                "algorithmic_bytes_per_launch": dw["bytes"],
                "algorithmic_flops_per_launch": dw["flops"],
                "implementation_bytes_per_launch": dw["implementation_bytes"]}
    if "unit_bytes" in dw:
        roofline["units_per_launch"] = dw["units"]
        roofline["unit_bytes"] = dw["unit_bytes"]
    if "shared_weight_bytes" in dw:
        roofline["shared_weight_bytes_per_launch"] = dw["shared_weight_bytes"]
    if len(dw.get("flops_by_dtype", {})) > 1:
        roofline["flops_by_dtype"] = dw["flops_by_dtype"]
        roofline["peak_note"] = "time-weighted peak of the launch's fp8 and bf16 MFMA work"

    flops, byts = layer_work(wl, active)
    layer_fig = {"tflops": flops / total_s * steps / 1e12,
                 "tflops_frac_bf16_peak": flops / total_s * steps / 1e12 / PEAK_TFLOPS["bf16"],
                 "hbm_gbs": byts / total_s * steps / 1e9,
                 "hbm_frac": byts / total_s * steps / 1e9 / PEAK_HBM_GBS,
                 "algorithmic_flops_per_step": flops, "algorithmic_bytes_per_step": byts,
                 "active_experts": active}

    fig = {"value": tokens_per_s, "ms_per_step": ms_per_step,
           "launch": ("hipGraph replay of " if graph_s else "eager ") +
                     ("moe_block_forward" if block else "moe_forward"),
           "eager_ms_per_step": 1e3 * eager_s / steps,
           "eager_kernel_ms_per_step": {"p10": round(float(q10), 5),
                                        "median": round(float(q50), 5),
                                        "p90": round(float(q90), 5)},
           "roofline": roofline, "layer": layer_fig,
           "stages_ms": {s: round(v, 5) for s, v in stage_ms.items()}}
    if cache_check:
        fig["cache_check"] = cache_check
    return fig, layer, inp, y


def wl_dtype(wl):
    return {"fp8": "fp8+bf16", "fp4": "bf16 (fp4 weights)"}.get(wl.expert_dtype, wl.act_dtype)


def brief(wl, fig, steps: int):
    """A workload's figures in short, for the line's `other_workloads`."""
    r = fig["roofline"]
    lay = fig["layer"]
    return {"tokens": wl.tokens, "expert_dtype": wl.expert_dtype, "steps": steps,
            "ms_per_step": round(fig["ms_per_step"], 5),
            "tokens_per_s": round(fig["value"], 1), "launch": fig["launch"],
            "layer_tflops_frac_bf16_peak": round(lay["tflops_frac_bf16_peak"], 4),
            "layer_hbm_frac": round(lay["hbm_frac"], 4),
            "roofline": {"bound": r["bound"], "kernel": r["kernel"],
                         "kernel_ms": round(r["kernel_ms"], 5),
                         "achieved": round(r["achieved"], 1), "peak": r["peak"],
                         "unit": r["unit"], "frac": round(r["frac"], 4),
                         "traffic": r["traffic"]},
            "stages_ms": fig["stages_ms"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload at this many tokens instead (a prefix of its rows)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (default: the step replayed from a HIP graph)")
    ap.add_argument("--evict-mb", type=int, default=512,
                    help="after the timed region, repeat the eager steps with a read of this "
                         "many MB between them (outside their events), so that nothing of one "
                         "step stays in the 256 MB Infinity Cache for the next (0 = skip)")
    ap.add_argument("--no-others", dest="others", action="store_false",
                    help="with the default workload, skip timing the other configurations "
                         "after it")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 10 device-to-device copies of this many bytes (a "
                         "reference kernel for calibrating HBM byte counters)")
    args = ap.parse_args()
    if args.copy_bytes:
        import torch
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "copies": 10}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from non_gated_relu_amd.synthetic import WORKLOADS

    wl = WORKLOADS[args.workload]
    steps = args.steps or DEFAULT_STEPS.get(args.workload, 50)
    if args.tokens > 0:
        wl = dataclasses.replace(wl, tokens=args.tokens,
                                 name=re.sub(r"T\d+$", f"T{args.tokens}", wl.name))
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fig, layer, inp, y = measure(wl, steps, args.warmup, not args.no_graph, args.evict_mb)

    line = {"metric": METRIC, "value": fig["value"], "unit": "tokens/s", "n_gpus": 1,
            "steps": steps, "warmup": args.warmup, "ms_per_step": fig["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": wl_dtype(wl),
            "data": "synthetic (seeded Gaussian inputs and weights)",
            "config": {"workload": wl.name, "tokens": wl.tokens, "hidden": wl.hidden,
                       "experts": wl.n_experts, "groups": wl.n_group,
                       "topk_group": wl.topk_group, "top_k": wl.top_k, "inter": wl.inter,
                       "shared_inter": wl.shared_inter, "expert_dtype": wl.expert_dtype,
                       "parallelism": "single GPU"}}
    line.update({k: v for k, v in fig.items() if k not in ("value", "ms_per_step")})
    if args.cpu_seconds > 0:
        y_np = y.float().cpu().numpy()
        idx_np = layer.topk_idx[:wl.tokens].cpu().numpy()
        line["cpu_baseline"], line["parity"] = cpu_baseline(wl, inp, y_np, idx_np,
                                                            args.cpu_seconds)
    if args.others and args.workload == DEFAULT_WORKLOAD and args.tokens == 0:
        # the other one-GPU configurations, timed the same way after the
        # headline (their oracle parity is in the tests): the decode steps
        # that stream the expert weights, the balanced prefill chunk, the fp8
        # experts and the 4-bit decode step
        del layer, inp, y
        torch.cuda.empty_cache()
        line["other_workloads"] = {}
        for name in OTHER_WORKLOADS:
            owl = WORKLOADS[name]
            ost = OTHER_STEPS[name]
            ofig, olayer, _, _ = measure(owl, ost, min(args.warmup, 5), not args.no_graph, 0)
            line["other_workloads"][name] = brief(owl, ofig, ost)
            del olayer
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
