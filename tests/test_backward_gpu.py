"""GPU parity of the layer backward: the HIP path (through the C ABI) against
the CPU oracle's backward on the same seeded inputs and the GPU's own routing
(indices, weights, probabilities, dispatch plan and log-sum-exp are taken from
the GPU forward, so a near-tie cannot cascade).

Small workloads compare every gradient element by element. f32 layers: within
1e-5 of (|ref| + rms). bf16 layers: the outputs the expert chain produces
(z, d_out_perm, dz, dx_perm, dx, dW1, dW2) within 7 standard deviations of
the error their 16-bit storage roundings imply, element by element (the
model and its derivation: bwd_tolerance.py); the gate's outputs (dw, d_logits,
dWg, db), which see only f32 arithmetic on the forward's outputs, within
2e-2 max-abs / rms as the forward.
The full-size bench workload compares every kept row and every token, the
whole weight gradients of two experts, and the gate weight gradient as the
product it is.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_49_amd import inputs as I
from mixture_experts_layer_49_amd import ops
from oracle import moe_oracle as O
from bwd_tolerance import expert_sigmas_torch, layer_sigmas, within
from parity_helpers import cached_inputs, close, dev, host, say

pytestmark = pytest.mark.gpu

CASES = [
    I.small("bwd-small-bf16"),
    I.small("bwd-small-f32", dtype="f32", T=200, d=36, d_ff=52, E=5, k=2, seed=7),
    I.small("bwd-ragged-bf16", T=517, d=200, d_ff=328, E=7, k=3, cf=1.0, seed=8),
    I.small("bwd-max-experts", T=300, d=64, d_ff=64, E=256, k=8, cf=2.0, seed=9),
    I.small("bwd-one-expert-nodrop", T=100, d=64, d_ff=96, E=1, k=1, cf=0.0, seed=10),
    I.small("bwd-all-dropped", T=64, d=64, d_ff=64, E=4, k=2, cf=0.01, seed=12),
    I.small("bwd-zipf-bias", T=600, d=256, d_ff=256, E=16, k=2, cf=1.0, gate_bias="zipf", seed=13),
    I.small("bwd-receiver", T=700, d=128, d_ff=256, E=8, k=1, cf=1.25, routed=False, seed=14),
    I.small("bwd-single-token", T=1, d=64, d_ff=64, E=4, k=2, cf=1.25, seed=15),
    I.small("bwd-multi-tile", T=1200, d=512, d_ff=576, E=3, k=2, cf=1.25, seed=16),
    I.small("bwd-split-k2-ragged", T=300, d=1024, d_ff=1032, E=2, k=2, cf=1.25, seed=17),
    I.small("bwd-long-rows", T=2000, d=256, d_ff=512, E=2, k=1, cf=1.25, seed=19),
    # wide gates (the gate weight gradients on the f32 matrix cores, dispatch^T
    # with several 16-expert gate chunks): ragged tokens and columns, bf16 and
    # f32 gates
    I.small("bwd-wide-gate", T=517, d=200, d_ff=128, E=40, k=2, cf=1.25, seed=21),
    I.small("bwd-wide-gate-f32", dtype="f32", T=333, d=36, d_ff=52, E=24, k=3, cf=1.25, seed=22),
]
# routing knobs: (flags, temperature, noise scale, z_coeff)
VARIANTS = {"plain": (0, 1.0, 0.0, 0.0), "renorm-temp-noise-zloss": (ops.MOE_RENORM, 1.6, 0.3, 0.05)}


def run_gpu(inp, cfg, variant="plain", aux_grad=0.7):
    flags, tau, noise_scale, zc = VARIANTS[variant]
    x = dev(inp["x"], cfg.dtype)
    w1, w2 = dev(inp["w1"], cfg.dtype), dev(inp["w2"], cfg.dtype)
    wg = dev(inp["w_gate"], cfg.dtype) if cfg.routed else None
    bias = dev(inp["bias"], "f32") if cfg.routed and inp["bias"] is not None else None
    given_idx = dev(inp["topk_idx"], "f32") if not cfg.routed else None
    given_w = dev(inp["topk_w"], "f32") if not cfg.routed else None
    noise = (I.routing_noise(cfg.T, cfg.E, noise_scale, 900 + cfg.seed)
             if noise_scale and cfg.routed else None)
    C = ops.moe_capacity(cfg.T, cfg.E, cfg.cf)
    b = ops.moe_forward(x, w1, w2, cfg.k, C, w_gate=wg, bias=bias, topk_idx=given_idx,
                        topk_w=given_w, alpha=cfg.alpha, flags=flags, save_for_backward=True,
                        temperature=tau, noise=None if noise is None else dev(noise, "f32"))
    dy_np = I.upstream_grad(cfg.T, cfg.d, 500 + cfg.seed)
    dy = dev(dy_np, "f32")
    g = ops.moe_backward(x, w1, w2, cfg.k, b, dy, w_gate=wg, alpha=cfg.alpha, aux_grad=aux_grad,
                         flags=flags, temperature=tau, z_coeff=zc)
    torch.cuda.synchronize()
    R = int(host(b.offsets)[-1])
    fwd = {"topk_idx": host(b.topk_idx).astype(np.int64) if cfg.routed else inp["topk_idx"].astype(np.int64),
           "topk_w": host(b.topk_w) if cfg.routed else inp["topk_w"],
           "counts": host(b.counts), "offsets": host(b.offsets).astype(np.int64),
           "dest": host(b.dest).astype(np.int64), "src": host(b.src[:R]).astype(np.int64)}
    if cfg.routed:
        fwd["probs"] = host(b.probs)
        fwd["lse"] = host(b.lse[:cfg.T])
    gpu = {"z_perm": host(b.z[:R]), "d_out_perm": host(g.d_out_perm[:R]), "dw": host(g.d_topk_w),
           "dz_perm": host(g.dz[:R]), "dx_perm": host(g.dx_perm[:R]), "dw1": host(g.dw1),
           "dw2": host(g.dw2), "dx": host(g.dx)}
    if cfg.routed:
        gpu.update(dl=host(g.d_logits), dwg=host(g.dw_gate), db=host(g.d_bias))
    knobs = dict(renorm=bool(flags & 1), temperature=tau, z_coeff=zc)
    return gpu, fwd, dy_np, knobs, (b, g)


MODELLED = ("z_perm", "d_out_perm", "dz_perm", "dx_perm", "dx", "dw1", "dw2")


def compare(gpu, ref, cfg, names, sig=None, inp=None):
    for n in names:
        if ref[n].size == 0:
            continue
        what = "%s %s" % (cfg.name, n)
        if cfg.dtype == "bf16" and n in MODELLED:
            extra = 0.0
            if n == "dx" and "dl" in ref:
                # the gate's share d_logits Wg, with d_logits held to 2e-2 of its rms
                wg = O.decode(inp["w_gate"], cfg.dtype)
                extra = 2e-2 * float(np.sqrt(np.mean(ref["dl"] ** 2))) * np.abs(wg).sum(axis=0)
            within(gpu[n], ref[n], sig[n], what, extra)
        else:
            close(gpu[n], ref[n], cfg.dtype, what)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_backward_small(cfg):
    say("  backward %s" % (cfg,))
    inp = I.make_inputs(cfg)
    gpu, fwd, dy, knobs, _ = run_gpu(inp, cfg)
    ref = O.backward(inp, fwd, dy, cfg.dtype, cfg.k, alpha=cfg.alpha, aux_scale=0.7, **knobs)
    sig = layer_sigmas(inp, fwd, ref) if cfg.dtype == "bf16" else None
    compare(gpu, ref, cfg, ["z_perm", "d_out_perm", "dw", "dz_perm", "dx_perm", "dw1", "dw2", "dx"],
            sig, inp)
    if cfg.routed:
        compare(gpu, ref, cfg, ["dl", "dwg", "db"])
    # an expert with no rows gets an all-zero weight gradient
    empty = np.nonzero(np.diff(fwd["offsets"]) == 0)[0]
    assert not gpu["dw1"][empty].any() and not gpu["dw2"][empty].any()


@pytest.mark.parametrize("cfg", [c for c in CASES if c.routed and c.name in
                                 ("bwd-small-bf16", "bwd-small-f32", "bwd-ragged-bf16",
                                  "bwd-max-experts", "bwd-zipf-bias")], ids=lambda c: c.name)
def test_backward_routing_variants(cfg):
    inp = I.make_inputs(cfg)
    gpu, fwd, dy, knobs, _ = run_gpu(inp, cfg, "renorm-temp-noise-zloss")
    ref = O.backward(inp, fwd, dy, cfg.dtype, cfg.k, alpha=cfg.alpha, aux_scale=0.7, **knobs)
    sig = layer_sigmas(inp, fwd, ref) if cfg.dtype == "bf16" else None
    compare(gpu, ref, cfg, ["dw", "dl", "dwg", "db", "dx", "dw1", "dw2"], sig, inp)


def test_backward_is_deterministic():
    cfg = CASES[2]
    inp = I.make_inputs(cfg)
    a, _, _, _, _ = run_gpu(inp, cfg)
    b, _, _, _, _ = run_gpu(inp, cfg)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


@pytest.mark.timeout(900)
def test_backward_full_size():
    """large-experts-e8 at its real size against the oracle: every kept row's
    z, dz and dx_perm, every token's combine-weight gradient, d_logits and
    dx, and the whole weight gradients dW1, dW2 of the first and the last
    expert; the gate weight gradient as the product d_logits^T x."""
    cfg = I.config("large-experts-e8")
    inp = cached_inputs(cfg)
    gpu, fwd, dy, knobs, _ = run_gpu(inp, cfg)
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    R = int(fwd["offsets"][-1])
    x = O.decode(inp["x"], cfg.dtype)
    # every kept row's output gradient: w * dy
    d_out_all, _ = O.combine_backward(dy, np.zeros((R, d)), fwd["dest"], fwd["topk_w"], R)
    within(gpu["d_out_perm"], d_out_all, 2.0 ** -8 / np.sqrt(3) * np.abs(d_out_all), "d_out_perm")
    y_perm = np.zeros((R, d))
    dx_perm = np.zeros((R, d))
    s_dx_perm = np.zeros((R, d))
    whole = (0, E - 1)      # experts whose weight gradients are checked whole
    for e in range(E):
        a, b = int(fwd["offsets"][e]), int(fwd["offsets"][e + 1])
        if a == b:
            continue
        w1e, w2e = O.decode(inp["w1"][e], cfg.dtype), O.decode(inp["w2"][e], cfg.dtype)
        xr = x[fwd["src"][a:b]]
        g = O.expert_backward(xr, d_out_all[a:b], w1e, w2e, weight_grads=e in whole)
        y_perm[a:b] = g["y"]
        sg = expert_sigmas_torch(xr, d_out_all[a:b], w1e, w2e, weight_grads=e in whole)
        within(gpu["z_perm"][a:b], g["z"], sg["z"], "z, expert %d (%d rows)" % (e, b - a))
        within(gpu["dz_perm"][a:b], g["dz"], sg["dz"], "dz, expert %d" % e)
        within(gpu["dx_perm"][a:b], g["dx_perm"], sg["dx_perm"], "dx_perm, expert %d" % e)
        dx_perm[a:b], s_dx_perm[a:b] = g["dx_perm"], sg["dx_perm"]
        if e in whole:
            within(gpu["dw1"][e], g["dw1"], sg["dw1"], "dW1[%d], every hidden unit" % e)
            within(gpu["dw2"][e], g["dw2"], sg["dw2"], "dW2[%d], every hidden unit" % e)
        del w1e, w2e, g, sg
    # combine backward and the gate backward on every token
    _, dw = O.combine_backward(dy, y_perm, fwd["dest"], fwd["topk_w"], R)
    close(gpu["dw"], dw, cfg.dtype, "dw, every token")
    dl = O.gate_backward(dw, fwd["topk_idx"], fwd["topk_w"], fwd["probs"], fwd["counts"], k,
                         cfg.alpha, 0.7)
    close(gpu["dl"], dl, cfg.dtype, "d_logits, every token")
    wg = O.decode(inp["w_gate"], cfg.dtype)
    ref_dx = dl @ wg
    var = np.zeros((T, d))
    np.add.at(ref_dx, fwd["src"], dx_perm)
    np.add.at(var, fwd["src"], s_dx_perm ** 2)
    extra = 2e-2 * float(np.sqrt(np.mean(dl ** 2))) * np.abs(wg).sum(axis=0)
    within(gpu["dx"], ref_dx, np.sqrt(var), "dx, every token", extra)
    # gate weight gradient: the product of the GPU's own d_logits with x
    dlg = gpu["dl"].astype(np.float64)
    close(gpu["dwg"], dlg.T @ x, "f32", "dWg = d_logits^T x")
    close(gpu["db"], dlg.sum(axis=0), "f32", "db = sum_t d_logits")


@pytest.mark.parametrize("T,d,E,dt", [(20000, 256, 8, "bf16"), (9000, 72, 20, "f32"), (3, 64, 5, "bf16"),
                                      (4100, 520, 70, "bf16"), (16384, 2048, 64, "bf16")])
def test_gate_weight_grads_any_batch(T, d, E, dt):
    """dWg = d_logits^T x and db = column sums, for batches whose token chunks
    are longer than one staging block (T > 8192), an expert count that is not a
    multiple of 8, a batch of three tokens, and wide gates (the f32-MFMA path:
    20 experts with f32 x; 70, which spills into a second 64-expert block,
    with ragged tokens and columns; the 64-expert workload's shape); against
    float64."""
    rng = np.random.default_rng(T + d + E)
    dl = rng.standard_normal((T, E)).astype(np.float32)
    x_np = rng.standard_normal((T, d)).astype(np.float32)
    if dt == "bf16":
        x_bits = (torch.from_numpy(x_np).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16))
        x = dev(x_bits, "bf16")
        x64 = O.decode(x_bits, "bf16")
    else:
        x, x64 = dev(x_np, "f32"), x_np.astype(np.float64)
    dwg, db = ops.moe_gate_weight_grads(dev(dl, "f32"), x, E)
    torch.cuda.synchronize()
    close(host(dwg), dl.astype(np.float64).T @ x64, "f32", "dWg T=%d" % T)
    close(host(db), dl.astype(np.float64).sum(axis=0), "f32", "db T=%d" % T)
