"""Benchmark: one MoE layer forward per step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--backward]

A step is the whole forward -- gate + softmax + top-k, dispatch (index build +
permute), grouped expert FFN (up-projection + GELU, down-projection), weighted
combine, aux loss -- over one batch of synthetic tokens already resident in
HBM. Default workload: large-experts-e8 (T=8192 tokens, d=4096,
d_ff=16384, E=8, top-2, capacity factor 1.25, bf16).

Prints ONE JSON line: tokens/s, ms per step, the roofline of the dominant
kernel (timed live with HIP events on the launch stream), a per-call
breakdown, and the CPU oracle timed on this host as a baseline.

With --backward a step is one training step of the layer instead: the
forward keeping what the backward needs, then the whole backward (combine^T,
GELU and down-projection backward, up-projection backward, expert weight
gradients, gate backward, gate weight gradients, dispatch^T).
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

METRIC = "MoE fwd tokens/s on 1 GPU + expert GEMM % bf16 MFMA peak, HBM % peak"
PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The clocks ramp up over the first few launches after idle; 20 steps
    # (about 60 ms of work) reach the sustained state.
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="large-experts-e8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step (forward + backward) instead of the forward")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the steps, as a "
                         "known-size reference for memory-traffic counters")
    return ap.parse_args(argv)


# the sources each GEMM kernel family is built from (hashed into its summaries)
GEMM_SOURCES = {
    "gemm_mfma": ["mixture_experts_layer_49_amd/csrc/gemm_mfma.hip",
                  "mixture_experts_layer_49_amd/csrc/ffn_common.h",
                  "mixture_experts_layer_49_amd/csrc/moe_internal.h"],
    "gemm_frag": ["mixture_experts_layer_49_amd/csrc/gemm_frag.hip",
                  "mixture_experts_layer_49_amd/csrc/gemm_frag.h",
                  "mixture_experts_layer_49_amd/csrc/gemm_mfma.hip",   # the split fix-up kernel
                  "mixture_experts_layer_49_amd/csrc/ffn_common.h",
                  "mixture_experts_layer_49_amd/csrc/moe_internal.h"],
}


def measured_traffic(which: str, workload: str, family: str = "gemm_mfma"):
    """HBM bytes per launch of one GEMM kind (up, down, dh, dx, dw2, dw1) from
    the committed rocprofv3 summary (profiles/<family>_<which>_<workload>.md;
    for gemm_mfma the GEMM kernel plus its split fix-up kernel when tiles
    split, the two kernels the launch's HIP events time), or None when there
    is none or the kernel source changed after the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "%s_%s_%s.md" % (family, which, workload))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256"):
            key, val = line.split(":", 1)
            fields[key] = val.strip()
    h = hashlib.sha256()
    for f in GEMM_SOURCES[family]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def cpu_baseline(inp, cfg):
    """The CPU oracle, as it stands, on the full batch of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    t0 = time.perf_counter()
    O.forward(inp, cfg.dtype, cfg.k, cfg.cf, cfg.alpha)
    dt = time.perf_counter() - t0
    return {"value": cfg.T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "full batch: %d tokens, every step (gate, softmax, top-k, dispatch, "
                      "FFN on all kept rows, combine, aux) in float64 numpy; %.1f s wall"
                      % (cfg.T, dt), "seconds": dt}


def cpu_baseline_backward(inp, cfg, n_tokens):
    """The CPU oracle's forward + backward on the first n_tokens tokens of the
    same workload (the whole batch would take minutes)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from mixture_experts_layer_49_amd import inputs as I
    from oracle import moe_oracle as O

    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    sub = dict(inp)
    sub["x"] = inp["x"][:n_tokens]
    dy = I.upstream_grad(n_tokens, cfg.d, 77).astype(np.float64)
    t0 = time.perf_counter()
    fwd = O.forward(sub, cfg.dtype, cfg.k, cfg.cf, cfg.alpha)
    O.backward(sub, fwd, dy, cfg.dtype, cfg.k, alpha=cfg.alpha)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "first %d of the %d tokens (capacity from the sample's own T), forward + "
                      "backward in float64 numpy; %.1f s wall" % (n_tokens, cfg.T, dt),
            "seconds": dt}


# bench step name -> GEMM kind (the profile summaries are named after kinds)
KIND_OF = {"down_bwd": "dh", "up_bwd": "dx", "dw2": "dw2", "dw1": "dw1"}


def copy_probe(args, torch, device):
    """One plain device copy of --copy-probe-mib MiB: a known-size reference for
    the memory-traffic counters of a profiled run."""
    if args.copy_probe_mib <= 0:
        return
    n = args.copy_probe_mib << 20
    src_probe = torch.ones(n // 4, dtype=torch.float32, device=device)
    dst_probe = torch.empty_like(src_probe)
    torch.cuda.synchronize()
    dst_probe.copy_(src_probe)
    torch.cuda.synchronize()
    del src_probe, dst_probe


def bench_backward(args, cfg, inp, ops, torch, np):
    """One training step per timed step; prints the JSON line."""
    from mixture_experts_layer_49_amd import inputs as I

    def dev(a, bf16):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16).view(torch.bfloat16) if bf16 else t).to("cuda:0")

    bf = cfg.dtype == "bf16"
    if not cfg.routed:
        print("--backward runs routed workloads", file=sys.stderr)
        return 2
    x, w1, w2 = dev(inp["x"], bf), dev(inp["w1"], bf), dev(inp["w2"], bf)
    wg = dev(inp["w_gate"], bf)
    bias = dev(inp["bias"], False) if inp["bias"] is not None else None
    dy = dev(I.upstream_grad(cfg.T, cfg.d, 77), False)
    C = ops.moe_capacity(cfg.T, cfg.E, cfg.cf)
    b = ops.MoEBuffers(cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, C, x.dtype, x.device, True,
                       save_for_backward=True)
    g = ops.MoEGrads(cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, b.rows_max, x.dtype, x.device, True)
    stream = torch.cuda.current_stream()
    T, d, dff, E, k = cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k
    R_max = b.rows_max

    names = ["router", "dispatch_plan", "permute", "up_gelu_z", "down", "combine", "aux",
             "combine_bwd", "down_bwd", "up_bwd", "dw2", "dw1", "gate_bwd", "gate_wgrad",
             "dispatch_bwd"]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        ops.moe_router_topk_ex(x, wg, bias, k, 0, 1.0, None, True, True, b.topk_idx, b.topk_w,
                               b.probs, b.lse)
        rec(1)
        ops.moe_dispatch_plan(b.topk_idx, E, C, b.counts, b.offsets, b.dest, b.src, b.ws_dispatch)
        rec(2)
        ops.moe_permute(x, b.src, b.offsets, R_max, b.x_perm)
        rec(3)
        ops.moe_expert_up_gelu_z(b.x_perm, b.offsets, w1, R_max, b.h, b.z, b.ws_ffn)
        rec(4)
        ops.moe_expert_down(b.h, b.offsets, w2, R_max, b.y_perm, b.ws_ffn)
        rec(5)
        ops.moe_combine(b.y_perm, b.dest, b.topk_w, d, torch.float32, b.y)
        rec(6)
        ops.moe_aux_loss(b.probs, b.counts, k, cfg.alpha, b.loss, b.ws_aux)
        rec(7)
        ops.moe_combine_backward(dy, b.y_perm, b.dest, b.topk_w, x.dtype, R_max, g.d_out_perm,
                                 g.d_topk_w)
        rec(8)
        ops.moe_expert_down_backward(g.d_out_perm, b.offsets, w2, b.z, R_max, g.dz, b.ws_ffn)
        rec(9)
        ops.moe_expert_up_backward(g.dz, b.offsets, w1, R_max, g.dx_perm, b.ws_ffn)
        rec(10)
        ops.moe_expert_weight_grads(None, b.h, g.d_out_perm, None, b.offsets, E, R_max, d, dff,
                                    x.dtype, None, g.dw2, want_dw1=False)
        rec(11)
        ops.moe_expert_weight_grads(b.x_perm, None, None, g.dz, b.offsets, E, R_max, d, dff,
                                    x.dtype, g.dw1, None, want_dw2=False)
        rec(12)
        ops.moe_gate_backward(g.d_topk_w, b.topk_idx, b.topk_w, b.probs, b.counts, k, cfg.alpha,
                              1.0, 0, 1.0, None, 0.0, g.d_logits)
        rec(13)
        ops.moe_gate_weight_grads(g.d_logits, x, E, g.dw_gate, g.d_bias, True, g.ws_gate)
        rec(14)
        ops.moe_dispatch_backward(g.dx_perm, b.dest, d, x.dtype, g.d_logits, wg, g.dx)
        rec(15)

    copy_probe(args, torch, x.device)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(len(names))] for e in evs]).mean(0)
    us = dict(zip(names, (per * 1e3).tolist()))
    R = int(b.offsets.cpu().numpy()[-1])
    s2 = 2 if bf else 4
    nch = ops.moe_gate_weight_grads_workspace_bytes(T, d, E) // (4 * E * (d + 1))
    gemm_flops = 2.0 * R * d * dff
    hbm = {
        "combine_bwd": T * d * 4 + R * d * 4 + R * d * s2 + T * k * 16,
        "gate_bwd": T * k * 12 + T * E * 8 + T * 4,
        "gate_wgrad": T * E * 4 + T * d * s2 + 2 * nch * E * d * 4 + E * d * 4,
        "dispatch_bwd": R * d * 4 + T * d * 4 + T * E * 4 + T * k * 4,
    }
    breakdown = {}
    for n in names:
        v = {"us": us[n]}
        if n in ("down_bwd", "up_bwd", "dw2", "dw1"):
            v["TFLOP/s"] = gemm_flops / (us[n] * 1e-6) / 1e12
            v["mfma_frac"] = v["TFLOP/s"] / PEAK_MFMA_TFLOPS
        if n in hbm:
            v["bytes"] = hbm[n]
            v["GB/s"] = hbm[n] / (us[n] * 1e-6) / 1e9
            v["hbm_frac"] = v["GB/s"] / PEAK_HBM_GBS
        breakdown[n] = v
    bwd_names = names[7:]
    bwd_us = sum(us[n] for n in bwd_names)
    dom = max(("down_bwd", "up_bwd", "dw2", "dw1"), key=lambda n: us[n])
    out = {
        "metric": "MoE training step (fwd+bwd) tokens/s on 1 GPU + backward GEMM % bf16 MFMA peak",
        "value": T * args.steps / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded; inputs and upstream gradient resident in HBM before timing)",
        "config": {"workload": cfg.name, "T": T, "d": d, "d_ff": dff, "E": E, "k": k,
                   "capacity_factor": cfg.cf, "capacity": C, "kept_rows": R,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "grouped_gemm_mfma<%s>" % KIND_OF[dom], "bound": "mfma",
                     "achieved": breakdown[dom]["TFLOP/s"], "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": breakdown[dom]["mfma_frac"],
                     "traffic": measured_traffic(KIND_OF[dom], cfg.name),
                     "flops_per_launch": gemm_flops, "launch_us": us[dom]},
        "backward_ms": bwd_us * 1e-3,
        "backward_gemm_mfma_frac": 4 * gemm_flops / (sum(us[n] for n in ("down_bwd", "up_bwd", "dw2", "dw1")) * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS,
        "breakdown": breakdown,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (forward + backward) on the host ...")
        out["cpu_baseline"] = cpu_baseline_backward(inp, cfg, 256)
    print(json.dumps(out))
    return 0


def main(argv=None) -> int:
    args = parse(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mixture_experts_layer_49_amd import inputs as I
    from mixture_experts_layer_49_amd import ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    cfg = I.config(args.workload)
    t0 = time.perf_counter()
    inp = I.make_inputs(cfg)
    log("inputs generated in %.1f s" % (time.perf_counter() - t0))
    if args.backward:
        return bench_backward(args, cfg, inp, ops, torch, np)

    def dev(a, bf16):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16).view(torch.bfloat16) if bf16 else t).to("cuda:0")

    bf = cfg.dtype == "bf16"
    x, w1, w2 = dev(inp["x"], bf), dev(inp["w1"], bf), dev(inp["w2"], bf)
    wg = dev(inp["w_gate"], bf) if cfg.routed else None
    bias = dev(inp["bias"], False) if cfg.routed and inp["bias"] is not None else None
    given_idx = dev(inp["topk_idx"], False) if not cfg.routed else None
    given_w = dev(inp["topk_w"], False) if not cfg.routed else None
    C = ops.moe_capacity(cfg.T, cfg.E, cfg.cf)
    b = ops.MoEBuffers(cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, C, x.dtype, x.device, cfg.routed)
    # inference weight format: W2 in fp16, converted once (exact; the kernels
    # would otherwise convert each W2 value in registers on every step)
    w2h = ops.moe_weights_bf16_to_f16(w2) if bf else None
    # fragment-ordered path: h stays in fragment order for the down-projection
    hfrag = (torch.empty((ops.moe_frag_rows(b.rows_max, cfg.E), cfg.d_ff), dtype=torch.float16,
                         device=x.device) if b.frag and cfg.d_ff % 256 == 0 else None)
    stream = torch.cuda.current_stream()

    names = ["router", "dispatch_plan", "permute", "up_gelu", "down", "combine", "aux"]
    # one set of boundary events per timed step, all on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        if cfg.routed:
            ops.moe_router_topk(x, wg, bias, cfg.k, 0, True, b.topk_idx, b.topk_w, b.probs)
            idx, w = b.topk_idx, b.topk_w
        else:
            idx, w = given_idx, given_w
        rec(1)
        ops.moe_dispatch_plan(idx, cfg.E, C, b.counts, b.offsets, b.dest, b.src, b.ws_dispatch)
        rec(2)
        if hfrag is not None:
            ops.moe_permute_frag(x, b.src, b.offsets, b.rows_max, b.x_frag)
            rec(3)
            ops.moe_expert_up_gelu_frag(b.x_frag, b.offsets, w1, b.rows_max, hfrag, True)
            rec(4)
            ops.moe_expert_down_frag(hfrag, b.offsets, w2h, b.rows_max, b.y_perm, b.ws_ffn)
            rec(5)
            ops.moe_combine(b.y_perm, b.dest, w, cfg.d, torch.float32, b.y)
            rec(6)
            if cfg.routed:
                ops.moe_aux_loss(b.probs, b.counts, cfg.k, cfg.alpha, b.loss, b.ws_aux)
            rec(7)
            return
        if b.frag:
            ops.moe_permute_frag(x, b.src, b.offsets, b.rows_max, b.x_frag)
            rec(3)
            ops.moe_expert_up_gelu_frag(b.x_frag, b.offsets, w1, b.rows_max, b.h)
        else:
            ops.moe_permute(x, b.src, b.offsets, b.rows_max, b.x_perm)
            rec(3)
            ops.moe_expert_up_gelu(b.x_perm, b.offsets, w1, b.rows_max, b.h, b.ws_ffn)
        rec(4)
        if w2h is not None:
            ops.moe_expert_down_f16w(b.h, b.offsets, w2h, b.rows_max, b.y_perm, b.ws_ffn)
        else:
            ops.moe_expert_down(b.h, b.offsets, w2, b.rows_max, b.y_perm, b.ws_ffn)
        rec(5)
        ops.moe_combine(b.y_perm, b.dest, w, cfg.d, torch.float32, b.y)
        rec(6)
        if cfg.routed:
            ops.moe_aux_loss(b.probs, b.counts, cfg.k, cfg.alpha, b.loss, b.ws_aux)
        rec(7)

    copy_probe(args, torch, x.device)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(len(names))] for e in evs]).mean(0)

    counts = b.counts.cpu().numpy()
    R = int(b.offsets.cpu().numpy()[-1])
    T, d, dff, E, k = cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k
    s = 2 if bf else 4
    flops_up = 2.0 * R * d * dff
    flops_down = 2.0 * R * dff * d
    bytes_router = T * d * s + E * d * s + T * k * 8 + T * E * 4 if cfg.routed else 0
    bytes_plan = T * k * 4 * 2 + R * 4 + 2 * E * 4
    bytes_permute = 2 * R * d * s + R * 4
    bytes_combine = R * d * 4 + T * d * 4 + T * k * 8
    bytes_aux = T * E * 4 if cfg.routed else 0
    us = dict(zip(names, (per * 1e3).tolist()))
    breakdown = {
        "router": {"us": us["router"], "GB/s": bytes_router / (per[0] * 1e-3) / 1e9 if per[0] else None},
        # the plan is integer work of a few hundred KB: latency, reported in us only
        "dispatch_plan": {"us": us["dispatch_plan"], "bytes": bytes_plan},
        "permute": {"us": us["permute"], "GB/s": bytes_permute / (per[2] * 1e-3) / 1e9},
        "up_gelu": {"us": us["up_gelu"], "TFLOP/s": flops_up / (per[3] * 1e-3) / 1e12},
        "down": {"us": us["down"], "TFLOP/s": flops_down / (per[4] * 1e-3) / 1e12},
        "combine": {"us": us["combine"], "GB/s": bytes_combine / (per[5] * 1e-3) / 1e9},
        "aux": {"us": us["aux"]},
    }
    for key, v in breakdown.items():
        if "GB/s" in v and v["GB/s"] is not None:
            v["hbm_frac"] = v["GB/s"] / PEAK_HBM_GBS
        if "TFLOP/s" in v:
            v["mfma_frac"] = v["TFLOP/s"] / PEAK_MFMA_TFLOPS
    dom = "up_gelu" if per[3] >= per[4] else "down"
    dom_frag = b.frag and (dom == "up_gelu" or hfrag is not None)
    dom_which = ("up" if dom == "up_gelu" else
                 "down" if hfrag is not None or w2h is None else "down_f16w")
    dom_kernel = ("frag_gemm_kernel<%s>" % ("up_frag" if hfrag is not None else "up_rows")
                  if dom_frag and dom == "up_gelu" else
                  "frag_gemm_kernel<down>" if dom_frag else "grouped_gemm_mfma<%s>" % dom_which)
    achieved = breakdown[dom]["TFLOP/s"]
    ffn_tflops = (flops_up + flops_down) / ((per[3] + per[4]) * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": T * args.steps / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded; inputs resident in HBM before timing)",
        "config": {"workload": cfg.name, "T": T, "d": d, "d_ff": dff, "E": E, "k": k,
                   "capacity_factor": cfg.cf, "capacity": C, "kept_rows": R,
                   "max_over_mean_load": float(counts.max() / counts.mean()),
                   "activation_layout": ("fragment-ordered x and h" if hfrag is not None else
                                         "fragment-ordered x" if b.frag else "row-major"),
                   "w2_storage": "fp16 (converted once from the bf16 weights, exact)" if bf else "f32",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": dom_kernel, "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_TFLOPS,
                     "traffic": measured_traffic(dom_which, cfg.name,
                                                 "gemm_frag" if dom_frag else "gemm_mfma"),
                     "flops_per_launch": flops_up if dom == "up_gelu" else flops_down,
                     "launch_us": us[dom]},
        "ffn_mfma_frac": ffn_tflops / PEAK_MFMA_TFLOPS,
        "breakdown": breakdown,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(inp, cfg)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
