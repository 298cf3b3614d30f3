"""Shared pieces of the GPU parity tests: moving seeded inputs to the device,
the tolerances, and the routing-gap rule."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

from mixture_experts_layer_49_amd import inputs as I
from oracle import moe_oracle as O

# Tolerances (fixed by the workload definitions): float32 outputs agree to
# 1e-5 relative, bf16 outputs (fp32 accumulate) to 2e-2 max-abs / output RMS.
F32_RTOL = 1e-5
BF16_MAX_OVER_RMS = 2e-2
GAP = 1e-4            # tokens whose top-k logit gap is below this may route differently


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype: str):
    """numpy input (f32 values or bf16 bits) -> torch tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to("cuda:0")


def host(t) -> np.ndarray:
    """Device tensor -> numpy. Slice to the written rows before calling: rows
    past them hold whatever the allocation held, signalling-NaN patterns
    included, and converting those raises floating-point warnings."""
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def close_f32(got, ref, what="output"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bound = F32_RTOL * (np.abs(ref) + rms)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), "%s: %d elements beyond 1e-5*(|ref|+rms); worst %.3e" % (
        what, int(bad.sum()), float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-300))))


def close_bf16(got, ref, what="output"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got)))
    say("  %s: max|err|/rms = %.3e (bound %.0e)" % (what, err, BF16_MAX_OVER_RMS))
    assert err <= BF16_MAX_OVER_RMS, "%s: max|err|/rms = %.3e" % (what, err)
    return err


def close(got, ref, dtype, what="output"):
    return close_f32(got, ref, what) if dtype == "f32" else close_bf16(got, ref, what)


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the smallest gap between consecutive sorted logits among the
    first k+1 (covers both the chosen set and the slot order)."""
    s = -np.sort(-logits, axis=1)
    kk = min(k + 1, logits.shape[1])
    if kk < 2:
        return np.full(logits.shape[0], np.inf)
    return np.min(s[:, :kk - 1] - s[:, 1:kk], axis=1)


@functools.lru_cache(maxsize=2)
def cached_inputs(cfg: I.MoEConfig):
    say("  generating inputs for %s" % (cfg,))
    return I.make_inputs(cfg)


def unfrag(x_frag, offsets, d: int):
    """Row-major x_perm rows [offsets[E], d] read back from the fragment-ordered
    copy, and the padding rows of every segment, from the layout's definition:
    segment e starts at padded row pad[e] = sum of roundup(kept, 32) before it,
    and element (padded row r, column c) sits at
    ((r // 32) (d // 16) + c // 16) 512 + ((r % 32) + 32 ((c // 8) % 2)) 8 + c % 8."""
    off = [int(v) for v in offsets]
    kept = [b - a for a, b in zip(off[:-1], off[1:])]
    pad_total = sum((n + 31) // 32 * 32 for n in kept)
    flat = x_frag.reshape(-1)[: pad_total * d]
    # (block, 16-column group, column half, row in block, column in half)
    rows = flat.reshape(pad_total // 32, d // 16, 2, 32, 8).permute(0, 3, 1, 2, 4).reshape(pad_total, d)
    parts, pads, p = [], [], 0
    for n in kept:
        parts.append(rows[p:p + n])
        pads.append(rows[p + n:p + (n + 31) // 32 * 32])
        p += (n + 31) // 32 * 32
    cat = lambda ts: torch.cat(ts) if ts else rows[:0]
    return cat(parts), cat(pads), pad_total
