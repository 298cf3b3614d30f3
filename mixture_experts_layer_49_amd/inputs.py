"""Seeded synthetic inputs for the MoE layer forward.

This module is shared by the GPU path and by the CPU oracle, so it holds no
step of the method itself: it only draws numbers. Every array is produced on
the host as numpy; bf16 tensors are returned as their raw uint16 bit
patterns, rounded from fp32 draws by torch's round-to-nearest-even cast.

Workload shapes follow what the pages describe:
  * 8192 tokens = max_length 4096 x per-device batch 2 (ms-swift MoE
    acceleration page, section 2.3 launch command);
  * 4096 -> 16384 -> 4096 experts with weights w1 / w2 (ETP expert-parallel
    page, the ETP section's up/down projection example);
  * 16 experts (ms-swift page, model list), 64 experts split 8 per GPU
    (SP/EP page, EP section; EP tutorial, section 4.1 DeepSpeed config);
  * capacity factor 1.0 - 1.25 (EP tutorial, section 2.2);
  * hot experts (SP/EP page, EP section, "hot-spot experts").

Draw order per config (numpy PCG64, seed = config index unless given):
x, gate weight, W1 expert by expert, W2 expert by expert, then extras.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class MoEConfig:
    """One MoE-layer workload.

    T      tokens entering the layer (rows received, for a receiver share)
    d      model width;  d_ff  expert hidden width
    E      experts;      k     experts per token
    cf     capacity factor (<= 0 means no dropping)
    dtype  "f32" or "bf16" for activations and weights
    alpha  aux-loss weight
    gate_bias  "none" | "zipf": per-expert logit bias log Zipf(s) (hot expert 0)
    routed     False for a receiver share: no gate, labels and weights are given
    recv_zipf_s  Zipf exponent of the per-expert received-row counts
    etp, etp_rank  expert tensor parallelism: this GPU holds slice etp_rank of
               etp equal slices of the hidden width -- rows of W1, columns of
               W2 -- of a layer whose hidden width is d_ff * etp (the weights
               are drawn for that layer, then sliced); its y is a partial sum
    """

    name: str
    T: int
    d: int
    d_ff: int
    E: int
    k: int
    cf: float
    dtype: str
    alpha: float = 0.01
    gate_bias: str = "none"
    zipf_s: float = 1.0
    routed: bool = True
    recv_zipf_s: float = 1.2
    seed: int = 0
    etp: int = 1
    etp_rank: int = 0


CONFIGS = [
    MoEConfig("tiny-fp32", 512, 64, 256, 8, 2, 1.25, F32, seed=0),
    MoEConfig("e16-zipf-bias", 4096, 1024, 4096, 16, 2, 1.0, BF16,
              gate_bias="zipf", zipf_s=1.0, seed=1),
    MoEConfig("fine-grained-e64", 16384, 2048, 1024, 64, 2, 1.25, BF16,
              alpha=0.01, seed=2),
    MoEConfig("large-experts-e8", 8192, 4096, 16384, 8, 2, 1.25, BF16, seed=3),
    MoEConfig("ep8-receiver-share", 8192, 4096, 16384, 8, 1, 1.25, BF16,
              routed=False, recv_zipf_s=1.2, seed=4),
]


# Workloads beyond the five above. The ETP share: one GPU's quarter of the
# large-experts layer's 4096 -> 16384 -> 4096 experts at ETP 4, W1 split by
# output columns and W2 by input columns (ETP expert-parallel page, ETP
# section); same tokens, gate and routing as large-experts-e8.
EXTRA_CONFIGS = [
    MoEConfig("etp4-share-e8", 8192, 4096, 4096, 8, 2, 1.25, BF16, seed=3, etp=4, etp_rank=0),
]


def config(i_or_name) -> MoEConfig:
    if isinstance(i_or_name, int):
        return CONFIGS[i_or_name]
    for c in CONFIGS + EXTRA_CONFIGS:
        if c.name == i_or_name:
            return c
    raise KeyError(i_or_name)


def small(name="small", **kw) -> MoEConfig:
    """A custom workload for quick parity cases."""
    base = dict(name=name, T=300, d=192, d_ff=320, E=6, k=2, cf=1.25,
                dtype=BF16, seed=123)
    base.update(kw)
    return MoEConfig(**base)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, via torch's cast) -> uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a if dtype == F32 else to_bf16_bits(a)


def routing_noise(T: int, E: int, scale: float, seed: int) -> np.ndarray:
    """A caller-drawn routing perturbation [T, E] f32: N(0, scale^2), its own
    PCG64 stream (seed), independent of the layer inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(size=(T, E), dtype=np.float32) * np.float32(scale)).astype(np.float32)


def zipf_counts(n: int, E: int, s: float) -> np.ndarray:
    """Per-expert counts of n rows following Zipf(s) over experts 0..E-1,
    rounded to integers by largest remainder (ties: lower expert first)."""
    w = np.array([(e + 1) ** -s for e in range(E)], dtype=np.float64)
    q = n * w / w.sum()
    c = np.floor(q).astype(np.int64)
    rem = n - int(c.sum())
    order = np.argsort(-(q - c), kind="stable")
    c[order[:rem]] += 1
    return c


def zipf_log_bias(E: int, s: float) -> np.ndarray:
    """Per-expert gate-logit bias b_e = log of the Zipf(s) pmf at rank e+1."""
    h = sum((e + 1) ** -s for e in range(E))
    return np.array([-s * math.log(e + 1) - math.log(h) for e in range(E)],
                    dtype=np.float32)


def make_inputs(cfg: MoEConfig, seed: int | None = None) -> dict:
    """Draw every input of one layer forward for `cfg`.

    Returned keys (numpy, host):
      x      [T, d]          f32, or uint16 bf16 bits
      w_gate [E, d]          (routed only)
      bias   [E] f32 or None (routed only)
      w1     [E, d_ff, d]    expert up-projection, K (= d) contiguous
      w2     [E, d, d_ff]    expert down-projection, K (= d_ff) contiguous
      topk_idx [T, 1] int32, topk_w [T, 1] f32   (receiver share only)
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    T, d, E = cfg.T, cfg.d, cfg.E
    dff = cfg.d_ff * cfg.etp   # drawn for the whole layer; an ETP share is sliced below
    out = {"cfg": cfg}
    out["x"] = _normal(rng, (T, d), 1.0, cfg.dtype)
    if cfg.routed:
        out["w_gate"] = _normal(rng, (E, d), 1.0 / math.sqrt(d), cfg.dtype)
    w1 = np.empty((E, dff, d), dtype=np.float32 if cfg.dtype == F32 else np.uint16)
    w2 = np.empty((E, d, dff), dtype=w1.dtype)
    for e in range(E):
        w1[e] = _normal(rng, (dff, d), 1.0 / math.sqrt(d), cfg.dtype)
    for e in range(E):
        w2[e] = _normal(rng, (d, dff), 1.0 / math.sqrt(dff), cfg.dtype)
    if cfg.etp > 1:
        lo, hi = cfg.etp_rank * cfg.d_ff, (cfg.etp_rank + 1) * cfg.d_ff
        w1 = np.ascontiguousarray(w1[:, lo:hi, :])
        w2 = np.ascontiguousarray(w2[:, :, lo:hi])
    out["w1"], out["w2"] = w1, w2
    if cfg.routed:
        out["bias"] = zipf_log_bias(E, cfg.zipf_s) if cfg.gate_bias == "zipf" else None
    else:
        counts = zipf_counts(T, E, cfg.recv_zipf_s)
        labels = np.repeat(np.arange(E, dtype=np.int32), counts)
        labels = labels[rng.permutation(T)]
        out["topk_idx"] = np.ascontiguousarray(labels.reshape(T, 1), dtype=np.int32)
        out["topk_w"] = rng.uniform(0.0, 1.0, size=(T, 1)).astype(np.float32)
    return out


def upstream_grad(T: int, d: int, seed: int) -> np.ndarray:
    """Seeded gradient of the loss with respect to the layer output, [T, d]
    f32, standard normal (what a next layer would hand back)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((T, d), dtype=np.float32)
