"""GPU: a bounded randomised sweep of the fragment-ordered GEMM (16x16x32
MFMAs) against the row-major one (32x32x16), the oracle-checked reference of
the layer parity tests. 16 seeded cases draw the expert count, the segment
lengths (empty, a few rows, ragged, several 256-row tiles), d and d_ff, so
that workgroups run from a single unit to many and tiles from 4 to 64
stages; each case is printed before it runs and the sweep stops at its first
failure. Per case (test_frag_gpu.run_case): the permuted rows bit for bit,
padding rows zero and nothing past them written; h (row-major and fragment
order, the same values bit for bit) against the row-major GEMM's to one
fp16 step; y_perm from fragment-ordered h against the row-major
down-projection to float32 summation order; then the down-projection with
the workspace (short last rounds split along K) against the same without it,
and deterministic."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_49_amd import ops
from parity_helpers import say
from test_frag_gpu import f32_close, run_case

pytestmark = pytest.mark.gpu


def draw_case(i):
    rng = np.random.default_rng(9100 + i)
    E = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64]))
    kind = rng.random(E)
    counts = np.where(kind < 0.15, 0,
                      np.where(kind < 0.35, rng.integers(1, 40, E),
                               np.where(kind < 0.8, rng.integers(40, 700, E), rng.integers(700, 1600, E))))
    d = int(256 * rng.choice([1, 2, 3, 4, 8, 16]))
    d_ff = int(256 * rng.choice([1, 2, 3, 5, 8, 16]))
    # keep a case to about 200 MB of weights and 20 M activation values
    while E * d * d_ff > 100_000_000:   # halve, staying a multiple of 256
        if d >= d_ff and d % 512 == 0:
            d //= 2
        elif d_ff % 512 == 0:
            d_ff //= 2
        else:
            break
    while int(counts.sum()) * max(d, d_ff) > 20_000_000 and counts.max() > 1:
        counts = counts // 2
    return [int(c) for c in counts], d, d_ff


def split_check(counts, d, d_ff, seed):
    g = torch.Generator().manual_seed(seed)
    E, R = len(counts), int(sum(counts))
    rows_max = R + 3
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda:0")
    x = torch.randn(max(R, 1), d, generator=g).to(torch.bfloat16).to("cuda:0")
    w1 = (torch.randn(E, d_ff, d, generator=g) / d ** 0.5).to(torch.bfloat16).to("cuda:0")
    src = torch.arange(max(R, 1), dtype=torch.int32, device="cuda:0")
    xf = ops.moe_permute_frag(x, src, off, rows_max)
    hf = ops.moe_expert_up_gelu_frag(xf, off, w1, rows_max, frag_out=True)
    w2h = (torch.randn(E, d, d_ff, generator=g) / d_ff ** 0.5).to(torch.float16).to("cuda:0")
    ws = torch.empty(ops.moe_ffn_workspace_bytes(torch.bfloat16), dtype=torch.uint8, device="cuda:0")
    yu = ops.moe_expert_down_frag(hf, off, w2h, rows_max)
    ys = ops.moe_expert_down_frag(hf, off, w2h, rows_max, workspace=ws)
    ys2 = ops.moe_expert_down_frag(hf, off, w2h, rows_max, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(ys[:R], ys2[:R]), "split down-projection not deterministic"
    f32_close(ys[:R], yu[:R], "y_perm split vs unsplit", tol=1e-4)


@pytest.mark.timeout(600)
def test_frag_gemm_random_sweep():
    for i in range(16):
        counts, d, d_ff = draw_case(i)
        say("sweep case %d: E=%d R=%d d=%d d_ff=%d counts[:8]=%s" % (i, len(counts), sum(counts), d, d_ff,
                                                                     counts[:8]))
        run_case(counts, d, d_ff, seed=100 + i)
        if sum(counts) > 0:
            split_check(counts, d, d_ff, seed=200 + i)
