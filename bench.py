"""Benchmark: one MoE layer forward per step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--backward]

A step is the whole forward -- gate + softmax + top-k, dispatch (index build +
permute), grouped expert FFN (up-projection + GELU, down-projection), weighted
combine, aux loss -- over one batch of synthetic tokens already resident in
HBM. Default workload: large-experts-e8 (T=8192 tokens, d=4096,
d_ff=16384, E=8, top-2, capacity factor 1.25, bf16); the receiver share
ep8-receiver-share (8192 received rows, 8 local experts of the same size,
Zipf(1.2) loads) is timed after it with the same steps and reported under
"also".

Before the warm-up steps an untimed ramp runs until the clocks have settled
(its length is in the line). Prints ONE JSON line: tokens/s, ms per step,
the roofline of the dominant kernel (timed live with HIP events on the
launch stream, in a second pass of the same steps so that the events do not
add to the whole-job time), the graphics clock under the dominant GEMM (from its
profile) and right after the GEMMs (a live probe), the matrix-core ceiling
under the power cap (an MFMA-only loop with no memory traffic), a per-call
breakdown, the HBM-bound calls again with cold caches
next to a plain-read and a copy reference of the same bytes, and the CPU
oracle timed on this host as a baseline.

With --backward a step is one training step of the layer instead: the
forward keeping what the backward needs, then the whole backward (combine^T,
GELU and down-projection backward, up-projection backward, expert weight
gradients, gate backward, gate weight gradients, dispatch^T).
"""
from __future__ import annotations

import argparse
import gc
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
    ap.add_argument("--also", default="ep8-receiver-share",
                    help="comma-separated workloads also timed (same steps and warm-up) and "
                         "reported under 'also'; 'none' for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step (forward + backward) instead of the forward")
    ap.add_argument("--dense-reference", action="store_true",
                    help="time the vendor library's dense bf16 GEMM (torch.matmul -> hipBLASLt) on the "
                         "workload's expert-GEMM shape (all kept rows as one M) instead of the layer: a "
                         "reference for the clock and matrix-core busy fraction, not the metric")
    ap.add_argument("--path", default="auto", choices=["auto", "frag", "gather", "rows"],
                    help="activation layout of a bf16 forward: what the layer picks (auto), the "
                         "fragment-ordered copy (frag), row-major with the permute folded into the "
                         "up-projection (gather) or row-major with x_perm stored (rows)")
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


def profile_fields(which: str, workload: str, family: str = "gemm_mfma") -> dict:
    """Fields of the committed rocprofv3 summary of one GEMM kind (up, down,
    dh, dx, dw2, dw1) on one workload (profiles/<family>_<which>_<workload>.md),
    or {} when there is none or the kernel sources changed after it was made."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "%s_%s_%s.md" % (family, which, workload))
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "`")):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    h = hashlib.sha256()
    for f in GEMM_SOURCES[family]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return fields if fields.get("source_sha256") == h.hexdigest() else {}


def measured_traffic(which: str, workload: str, family: str = "gemm_mfma"):
    """HBM bytes per launch of one GEMM kind from its committed summary (for
    gemm_mfma the GEMM kernel plus its split fix-up kernel when tiles split,
    the two kernels the launch's HIP events time), or None."""
    v = profile_fields(which, workload, family).get("traffic_bytes_per_launch")
    return float(v) if v else None


def profiled_sclk(which: str, workload: str, family: str = "gemm_mfma"):
    """The graphics clock under one GEMM launch from its committed summary:
    GRBM_GUI_ACTIVE cycles per XCD / the launch's duration, or None."""
    v = profile_fields(which, workload, family).get("sclk_mhz_under_kernel")
    return float(v) if v else None


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


def timed_steps(step, steps, torch, stream):
    """Milliseconds for `steps` back-to-back steps, bracketed by a device
    synchronisation and two events on the launch stream; nothing else is
    recorded inside, so the figure is the whole-job time. Python's garbage
    collector is held off meanwhile: a collection pause on the launching
    thread would leave the GPU idle inside the timed region (the callers
    collect before their warm-up steps, so no long host pause sits between
    those and the timed steps either: an idle GPU lowers its clock)."""
    import gc

    gc.disable()
    try:
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        h0 = time.perf_counter()
        for _ in range(steps):
            step()
        host = time.perf_counter() - h0
        stop.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    timed_steps.host_us_per_step = host * 1e6 / max(steps, 1)
    return start.elapsed_time(stop)


def kernel_breakdown(step, evs, n, torch, stream, np):
    """Mean milliseconds of each of the n calls of a step, from boundary events
    recorded between the calls in a second pass of the same steps (each event
    record costs a few microseconds of stream time, which is why the whole-job
    time is taken without them)."""
    torch.cuda.synchronize()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    return np.array([[e[i].elapsed_time(e[i + 1]) for i in range(n)] for e in evs]).mean(0)


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
    gc.collect()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    total_ms = timed_steps(step, args.steps, torch, stream)
    per = kernel_breakdown(step, evs, len(names), torch, stream, np)
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
        "breakdown_pass": {"how": "events between the calls, in a second pass of the same steps",
                           "ms_per_step": float(per.sum())},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (forward + backward) on the host ...")
        out["cpu_baseline"] = cpu_baseline_backward(inp, cfg, 256)
    print(json.dumps(out))
    return 0


def clock_ramp(step, torch, stream, min_ms=400.0, max_ms=4000.0, window=5):
    """Untimed steps until the clocks have settled: windows of `window` steps
    until at least min_ms of work ran and three windows in a row agree to 1%
    (at most max_ms). Returns what ran."""
    times, total, n = [], 0.0, 0
    while True:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(window):
            step()
        b.record(stream)
        b.synchronize()
        t = a.elapsed_time(b)
        times.append(t / window)
        total += t
        n += window
        settled = (len(times) >= 3 and abs(times[-1] - times[-2]) <= 0.01 * times[-1]
                   and abs(times[-2] - times[-3]) <= 0.01 * times[-2])
        if (total >= min_ms and settled) or total >= max_ms:
            return {"steps": n, "ms": total, "settled": settled,
                    "ms_per_step_first_last": [times[0], times[-1]]}


def measure_clock(step, kernels, torch, stream, device, n=10, ticks=1000):
    """The graphics clock right after each expert GEMM: after the timed steps,
    n more steps (untimed) with a clock probe (libmoe_bench.so: shader-clock
    counter against the 100 MHz counter over `ticks` real-time ticks, one
    wave) launched right after the up- and after the down-projection. The
    clock recovers within microseconds once the matrix cores go idle, so this
    reads higher than the clock under the GEMM itself (GRBM_GUI_ACTIVE in the
    profiles)."""
    import ctypes

    L = bench_lib()
    buf = torch.zeros(4 * n, dtype=torch.int64, device=device)
    strm = ctypes.c_void_p(stream.cuda_stream)

    def probe(slot):
        ptr = ctypes.c_void_p(buf.data_ptr() + 16 * slot)
        if L.probe_clock(ptr, ticks, strm) != 0:
            raise RuntimeError("probe_clock failed")

    for i in range(n):
        for j, kern in enumerate(kernels):
            kern()
            if j == 3:
                probe(2 * i)
            elif j == 4:
                probe(2 * i + 1)
    torch.cuda.synchronize()
    v = buf.cpu().numpy().reshape(2 * n, 2).astype(float)
    mhz = sorted(100.0 * v[:, 0] / v[:, 1])
    return {"sclk_mhz": mhz[len(mhz) // 2], "sclk_mhz_min": mhz[0], "sclk_mhz_max": mhz[-1],
            "probes": len(mhz),
            "source": "shader-clock counter / 100 MHz counter over 10 us, one wave launched right "
                      "after each expert GEMM of %d untimed steps (median); the clock recovers "
                      "once the matrix cores idle" % n}


def cold_us(fn, flush, torch, stream, reps=10):
    """Median time of fn() with the caches flushed before each call (a plain
    read of 1 GiB leaves the L2s and the 256 MiB infinity cache holding other,
    clean lines: nothing has to be written back when the call's data comes
    in)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for r in range(reps):
        flush(r)
        evs[r][0].record(stream)
        fn()
        evs[r][1].record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return t[len(t) // 2]


def measure_mfma_ceiling(torch, stream, device, form="32x32x16", iters=20000, reps=5):
    """The matrix-core ceiling under the power cap: libmoe_bench.so's MFMA-only
    loop (form "32x32x16": v_mfma_f32_32x32x16_bf16, 16 accumulators;
    "16x16x32": v_mfma_f32_16x16x32_bf16, 64 accumulators, twice the
    iterations; operands in registers, one workgroup of four waves per CU, no
    memory traffic), a few warm launches then `reps` timed ones; its TFLOP/s,
    the fraction of the nominal peak and the clock it held (shader-clock
    against 100 MHz ticks over workgroup 0's loop)."""
    import ctypes

    L = bench_lib()
    grid = torch.cuda.get_device_properties(device).multi_processor_count
    out = torch.empty(grid * 256, dtype=torch.float32, device=device)
    clk = torch.zeros(2, dtype=torch.int64, device=device)
    strm = ctypes.c_void_p(stream.cuda_stream)
    small = form == "16x16x32"
    fn = L.probe_mfma_loop16 if small else L.probe_mfma_loop
    n_it = 2 * iters if small else iters

    def launch():
        if fn(ctypes.c_void_p(out.data_ptr()), n_it, ctypes.c_void_p(clk.data_ptr()), grid, strm) != 0:
            raise RuntimeError("probe_mfma_loop failed")

    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flop = float(grid) * 4 * n_it * (64 * 16384.0 if small else 16 * 32768.0)
    c = clk.cpu().numpy().astype(float)
    tf = flop / (ms * 1e-3) / 1e12
    return {"TFLOP/s": tf, "frac": tf / PEAK_MFMA_TFLOPS, "sclk_mhz": 100.0 * c[0] / c[1],
            "what": "v_mfma_f32_%s_bf16 on register operands, %d accumulators, no memory traffic, one "
                    "workgroup of 4 waves per CU (%d), %.2f ms per launch"
                    % (form, 64 if small else 16, grid, ms)}


def bench_lib():
    """libmoe_bench.so: the streaming-read reference kernel, the clock probe
    and the MFMA-only loop."""
    import ctypes

    path = os.path.join(ROOT, "mixture_experts_layer_49_amd", "libmoe_bench.so")
    if not os.path.exists(path):
        raise RuntimeError("libmoe_bench.so is not built: run `python -m mixture_experts_layer_49_amd.build`")
    L = ctypes.CDLL(path)
    L.probe_stream_read.restype = ctypes.c_int
    L.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    for fn in (L.probe_mfma_loop, L.probe_mfma_loop16):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return L


def forward_workload(args, name, ops, torch, np, I, want_cpu):
    """Times the layer forward on one workload; returns the result object."""
    import ctypes

    cfg = I.config(name)
    t0 = time.perf_counter()
    inp = I.make_inputs(cfg)
    log("%s: inputs generated in %.1f s" % (name, time.perf_counter() - t0))

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
    frag, gather = {"auto": (None, None), "frag": (True, False), "gather": (False, True),
                    "rows": (False, False)}[args.path if bf else "auto"]
    b = ops.MoEBuffers(cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, C, x.dtype, x.device, cfg.routed,
                       w2_f16=bf, frag=frag, gather=gather)
    # inference weight format: W2 in fp16, converted once (the kernels would
    # otherwise round each W2 value to fp16 in registers on every step, the
    # same way); the report counts values that lost bits or overflowed
    w2_report = None
    if bf:
        rep = torch.zeros(2, dtype=torch.int64, device=x.device)
        w2h = ops.moe_weights_bf16_to_f16(w2, report=rep)
        w2_report = [int(v) for v in rep.cpu()]
        del w2
    else:
        w2h = None
    hfrag = b.h_frag
    stream = torch.cuda.current_stream()

    names = ["router", "dispatch_plan", "permute", "up_gelu", "down", "combine"]
    if b.gather:
        names.remove("permute")   # no launch of its own: the up-projection reads x through src

    # routed bf16 layers with few enough (tile, expert) cells: the router counts
    # its token tiles' choices and sums their softmax columns, and the plan (with
    # the aux loss) is built from those in one launch
    tiles = cfg.routed and b.tiles

    def k_router():
        if tiles:
            ops.moe_router_topk_tiles(x, wg, bias, cfg.k, 0, True, True, b.topk_idx, b.topk_w, b.probs,
                                      b.tile_counts, b.tile_colsum)
        elif cfg.routed:
            ops.moe_router_topk(x, wg, bias, cfg.k, 0, True, b.topk_idx, b.topk_w, b.probs)

    idx, w = (b.topk_idx, b.topk_w) if cfg.routed else (given_idx, given_w)

    def k_plan():
        # routed layers: the plan with the aux loss folded in (moe_dispatch_plan_tiles
        # or moe_dispatch_plan_aux)
        if tiles:
            ops.moe_dispatch_plan_tiles(idx, b.tile_counts, b.tile_colsum, cfg.E, C, cfg.alpha, b.counts,
                                        b.offsets, b.dest, b.src, b.loss)
        elif cfg.routed:
            ops.moe_dispatch_plan_aux(idx, b.probs, cfg.E, C, cfg.alpha, b.counts, b.offsets, b.dest, b.src,
                                      b.loss, b.ws_plan_aux)
        else:
            ops.moe_dispatch_plan(idx, cfg.E, C, b.counts, b.offsets, b.dest, b.src, b.ws_dispatch)

    def k_permute():
        # (with b.gather the up-projection reads x through src: no launch here)
        if b.frag:
            ops.moe_permute_frag(x, b.src, b.offsets, b.rows_max, b.x_frag)
        elif not b.gather:
            ops.moe_permute(x, b.src, b.offsets, b.rows_max, b.x_perm)

    def k_up():
        if hfrag is not None:
            ops.moe_expert_up_gelu_frag(b.x_frag, b.offsets, w1, b.rows_max, hfrag, True)
        elif b.frag:
            ops.moe_expert_up_gelu_frag(b.x_frag, b.offsets, w1, b.rows_max, b.h)
        elif b.gather:
            ops.moe_expert_up_gelu_gather(x, b.src, b.offsets, w1, b.rows_max, b.h, b.ws_ffn)
        else:
            ops.moe_expert_up_gelu(b.x_perm, b.offsets, w1, b.rows_max, b.h, b.ws_ffn)

    def k_down():
        if hfrag is not None:
            ops.moe_expert_down_frag(hfrag, b.offsets, w2h, b.rows_max, b.y_perm, b.ws_ffn)
        elif w2h is not None:
            ops.moe_expert_down_f16w(b.h, b.offsets, w2h, b.rows_max, b.y_perm, b.ws_ffn)
        else:
            ops.moe_expert_down(b.h, b.offsets, w2, b.rows_max, b.y_perm, b.ws_ffn)

    def k_combine():
        ops.moe_combine(b.y_perm, b.dest, w, cfg.d, torch.float32, b.y)

    kernels = [k_router, k_plan, k_permute, k_up, k_down, k_combine]
    if b.gather:
        kernels.remove(k_permute)

    def step(ev=None):
        for i, kern in enumerate(kernels):
            if ev is not None:
                ev[i].record(stream)
            kern()
        if ev is not None:
            ev[len(kernels)].record(stream)

    copy_probe(args, torch, x.device)
    # one set of boundary events per step of the second pass, all on the
    # launch stream (made before the warm-up, so that nothing but the
    # synchronisation separates the warm-up from the timed steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    gc.collect()
    ramp = clock_ramp(step, torch, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    total_ms = timed_steps(step, args.steps, torch, stream)
    after = measure_clock(step, kernels, torch, stream, x.device)
    # both MFMA forms: the fragment-ordered GEMM multiplies with 16x16x32, the
    # row-major one with 32x32x16
    ceilings = {f: measure_mfma_ceiling(torch, stream, x.device, f) for f in ("16x16x32", "32x32x16")}
    ms_per_step = total_ms / args.steps
    per = kernel_breakdown(step, evs, len(names), torch, stream, np)
    us = dict(zip(names, (per * 1e3).tolist()))
    us.setdefault("permute", 0.0)

    counts = b.counts.cpu().numpy()
    R = int(b.offsets.cpu().numpy()[-1])
    T, d, dff, E, k = cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k
    s = 2 if bf else 4
    flops_up = 2.0 * R * d * dff
    flops_down = 2.0 * R * dff * d
    hbm = {"router": T * d * s + E * d * s + T * k * 8 + T * E * 4 if cfg.routed else 0,
           "permute": 0 if b.gather else 2 * R * d * s + R * 4,
           "combine": R * d * 4 + T * d * 4 + T * k * 8}
    breakdown = {
        "router": {"us": us["router"]},
        # the plan is integer work of a few hundred KB: latency, reported in us
        # only; on routed layers it also forms the aux loss
        "dispatch_plan": {"us": us["dispatch_plan"], "bytes": T * k * 4 * 2 + R * 4 + 2 * E * 4,
                          "includes_aux_loss": bool(cfg.routed),
                          "from_router_tiles": bool(tiles)},
        "permute": ({"us": us["permute"], "folded_into": "up_gelu (x read through src)"} if b.gather
                    else {"us": us["permute"]}),
        "up_gelu": {"us": us["up_gelu"], "TFLOP/s": flops_up / (us["up_gelu"] * 1e-6) / 1e12},
        "down": {"us": us["down"], "TFLOP/s": flops_down / (us["down"] * 1e-6) / 1e12},
        "combine": {"us": us["combine"]},
    }
    for key, nb in hbm.items():
        if nb and us[key] > 0:
            breakdown[key].update(bytes=nb, **{"GB/s": nb / (us[key] * 1e-6) / 1e9})
            breakdown[key]["hbm_frac"] = breakdown[key]["GB/s"] / PEAK_HBM_GBS
    for key in ("up_gelu", "down"):
        breakdown[key]["mfma_frac"] = breakdown[key]["TFLOP/s"] / PEAK_MFMA_TFLOPS

    # the same HBM-bound kernels with cold caches, and the plain-read and
    # copy references for the same bytes
    L = bench_lib()
    grid = 4096
    sink = torch.empty(grid, dtype=torch.int32, device=x.device)
    sptr, strm = ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream)

    def stream_read(ptr, nbytes):
        if L.probe_stream_read(ctypes.c_void_p(ptr), nbytes, sptr, grid, strm) != 0:
            raise RuntimeError("probe_stream_read failed")

    flush_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=x.device)
    torch.cuda.synchronize()
    flush = lambda r: stream_read(flush_buf.data_ptr(), flush_buf.numel())
    cold = {}
    for key, fn in (("router", k_router), ("permute", k_permute), ("combine", k_combine)):
        if not hbm[key]:
            continue
        t = cold_us(fn, flush, torch, stream)
        cold[key] = {"us": t, "bytes": hbm[key], "GB/s": hbm[key] / (t * 1e-6) / 1e9,
                     "hbm_frac": hbm[key] / (t * 1e-6) / 1e9 / PEAK_HBM_GBS,
                     "in_pipeline_us": us[key]}
    xb = x.numel() * x.element_size()
    t = cold_us(lambda: stream_read(x.data_ptr(), xb), flush, torch, stream)
    cold["read_floor"] = {"us": t, "bytes": xb, "GB/s": xb / (t * 1e-6) / 1e9,
                          "hbm_frac": xb / (t * 1e-6) / 1e9 / PEAK_HBM_GBS,
                          "what": "plain streaming read of x (16-byte loads, 8 in flight per thread, "
                                  "%d workgroups) after the same flush" % grid}
    if "router" in cold:
        cold["router"]["over_read_floor"] = cold["router"]["us"] / t
    half = R * d * s
    if half:
        ca = torch.empty(half, dtype=torch.uint8, device=x.device)
        cb = torch.empty_like(ca)
        t = cold_us(lambda: cb.copy_(ca), flush, torch, stream)
        cold["copy_floor"] = {"us": t, "bytes": 2 * half, "GB/s": 2 * half / (t * 1e-6) / 1e9,
                              "hbm_frac": 2 * half / (t * 1e-6) / 1e9 / PEAK_HBM_GBS,
                              "what": "torch copy_ of the permute's bytes (R d s read + written) "
                                      "after the same flush"}
        if "permute" in cold:
            cold["permute"]["over_copy_floor"] = cold["permute"]["us"] / t
        del ca, cb
    del flush_buf

    dom = "up_gelu" if us["up_gelu"] >= us["down"] else "down"
    dom_frag = b.frag and (dom == "up_gelu" or hfrag is not None)
    dom_which = (("up_gather" if b.gather else "up") if dom == "up_gelu" else
                 "down" if hfrag is not None or w2h is None else "down_f16w")
    dom_kernel = ("frag_gemm_kernel<%s>" % ("up_frag" if hfrag is not None else "up_rows")
                  if dom_frag and dom == "up_gelu" else
                  "frag_gemm_kernel<down>" if dom_frag else "grouped_gemm_mfma<%s>" % dom_which)
    achieved = breakdown[dom]["TFLOP/s"]
    ceiling = dict(ceilings["16x16x32" if dom_frag else "32x32x16"])
    ceiling["other_form"] = ceilings["32x32x16" if dom_frag else "16x16x32"]
    ffn_tflops = (flops_up + flops_down) / ((us["up_gelu"] + us["down"]) * 1e-6) / 1e12
    fam = "gemm_frag" if dom_frag else "gemm_mfma"
    under = profiled_sclk(dom_which, cfg.name, fam)
    clock = {"under_dominant_gemm_mhz": under,
             "under_source": ("rocprofv3 GRBM_GUI_ACTIVE per XCD / duration, profiles/%s_%s_%s.md "
                              "(same kernel sources)" % (fam, dom_which, cfg.name) if under else
                              "profiles/%s_%s_%s.md gives no clock: launches under 100 us are too "
                              "short for the counter" % (fam, dom_which, cfg.name)
                              if profile_fields(dom_which, cfg.name, fam) else
                              "no profile summary of the current kernel sources"),
             "after_gemm_probe": after}
    out = {
        "value": T * args.steps / (total_ms * 1e-3),
        "unit": "tokens/s" if cfg.routed else "rows/s",
        "ms_per_step": ms_per_step,
        # host time to enqueue one step (the binding's argument marshalling and
        # the launches); at or above ms_per_step the step would be launch-bound
        "host_enqueue_us_per_step": timed_steps.host_us_per_step,
        "config": {"workload": cfg.name, "T": T, "d": d, "d_ff": dff, "E": E, "k": k,
                   "capacity_factor": cfg.cf, "capacity": C, "kept_rows": R,
                   "max_over_mean_load": float(counts.max() / counts.mean()),
                   "activation_layout": ("fragment-ordered x and h" if hfrag is not None else
                                         "fragment-ordered x" if b.frag else
                                         "row-major, the permute folded into the up-projection "
                                         "(x read through src)" if b.gather else "row-major"),
                   "w2_storage": ("fp16, converted once from the bf16 weights (round to nearest "
                                  "even; %d values lost low bits, %d overflowed)" % tuple(w2_report)
                                  if bf else "f32"),
                   "parallelism": "single GPU"},
        "roofline": {"kernel": dom_kernel, "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_TFLOPS,
                     "traffic": measured_traffic(dom_which, cfg.name,
                                                 "gemm_frag" if dom_frag else "gemm_mfma"),
                     "flops_per_launch": flops_up if dom == "up_gelu" else flops_down,
                     "launch_us": us[dom]},
        "ffn_mfma_frac": ffn_tflops / PEAK_MFMA_TFLOPS,
        "clock": clock,
        "mfma_ceiling": ceiling,
        "ramp": ramp,
        "breakdown": breakdown,
        "breakdown_pass": {"how": "events between the calls, in a second pass of the same steps",
                           "ms_per_step": float(per.sum())},
        "hbm_cold": cold,
    }
    # the dominant GEMM against what the matrix cores reach on this chip with
    # no memory traffic at all (the power cap holds the clock below 2.4 GHz)
    out["roofline"]["frac_of_mfma_ceiling"] = achieved / ceiling["TFLOP/s"]
    if under:
        # the same fraction against the MFMA peak at the clock the kernel ran at
        out["roofline"]["sclk_mhz"] = under
        out["roofline"]["frac_at_sclk"] = achieved / (PEAK_MFMA_TFLOPS * under / 2400.0)
    if want_cpu:
        log("timing the CPU oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(inp, cfg)
    del b, x, w1, w2h, inp
    torch.cuda.empty_cache()
    return out


def dense_reference(args, I, torch) -> int:
    """torch.matmul (hipBLASLt) on one dense bf16 GEMM of the expert GEMM's
    size: M = the workload's kept rows (T k, capped by E C), N = d_ff, K = d,
    with the same clock ramp and step counts; one JSON line."""
    cfg = I.config(args.workload)
    C = round(cfg.T / cfg.E * cfg.cf)
    M = min(cfg.T * cfg.k, cfg.E * C) if cfg.routed else cfg.T
    g = torch.Generator(device="cuda:0").manual_seed(0)
    A = torch.randn(M, cfg.d, device="cuda:0", generator=g).to(torch.bfloat16)
    B = torch.randn(cfg.d_ff, cfg.d, device="cuda:0", generator=g).to(torch.bfloat16)
    Cm = torch.empty(M, cfg.d_ff, device="cuda:0", dtype=torch.bfloat16)
    stream = torch.cuda.current_stream()
    step = lambda: torch.matmul(A, B.t(), out=Cm)
    ramp = clock_ramp(step, torch, stream)
    for _ in range(args.warmup):
        step()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / args.steps * 1e3
    fl = 2.0 * M * cfg.d * cfg.d_ff
    print(json.dumps({"metric": "dense bf16 GEMM reference (torch.matmul, vendor library), not the layer",
                      "value": fl / (us * 1e-6) / 1e12, "unit": "TFLOP/s", "frac": fl / (us * 1e-6) / 1e12 /
                      PEAK_MFMA_TFLOPS, "us": us, "shape": {"M": M, "N": cfg.d_ff, "K": cfg.d},
                      "steps": args.steps, "warmup": args.warmup, "ramp": ramp, "dtype": "bf16"}))
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
    if args.dense_reference:
        return dense_reference(args, I, torch)
    if args.backward:
        cfg = I.config(args.workload)
        t0 = time.perf_counter()
        inp = I.make_inputs(cfg)
        log("inputs generated in %.1f s" % (time.perf_counter() - t0))
        return bench_backward(args, cfg, inp, ops, torch, np)

    res = forward_workload(args, args.workload, ops, torch, np, I, not args.no_cpu_baseline)
    out = {"metric": METRIC, "value": res.pop("value"), "unit": res.pop("unit"), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if I.config(args.workload).dtype == "bf16" else "f32",
           "data": "synthetic (seeded; inputs resident in HBM before timing)"}
    out.update(res)
    also = [n for n in args.also.split(",") if n and n != "none" and n != args.workload]
    for name in also:
        # the second target workload, same steps and warm-up, under its own key
        out.setdefault("also", {})[name] = forward_workload(args, name, ops, torch, np, I, False)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
