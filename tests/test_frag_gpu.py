"""GPU: the fragment-ordered permute and up-projection against the row-major
ones, on the same segments. The permuted rows are bit-exact (read back through
the layout's definition, padding rows zero), h is bit-identical to
moe_expert_up_gelu without a workspace (the same MFMA operands in the same
order), and rows past the segments are left alone. The row-major up-projection
is itself checked against the oracle by the layer parity tests."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_49_amd import ops
from parity_helpers import say, unfrag

pytestmark = pytest.mark.gpu

SENT_H = 0x7E55     # an fp16 NaN pattern no result has
SENT_X = 0x5A5A


def run_case(counts, d, d_ff, slack=17, seed=0):
    g = torch.Generator().manual_seed(seed)
    E = len(counts)
    R = int(sum(counts))
    rows_max = R + slack
    T = max(R // 2, 1)
    say("  case E=%d R=%d d=%d d_ff=%d rows_max=%d" % (E, R, d, d_ff, rows_max))
    x = (torch.randn(T, d, generator=g)).to(torch.bfloat16).to("cuda:0")
    w1 = (torch.randn(E, d_ff, d, generator=g) / d ** 0.5).to(torch.bfloat16).to("cuda:0")
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda:0")
    src = torch.randint(0, T, (max(rows_max, 1),), generator=g, dtype=torch.int32).to("cuda:0")

    x_perm = ops.moe_permute(x, src, off, rows_max)
    h_ref = torch.empty(max(rows_max, 1), d_ff, dtype=torch.float16, device="cuda:0")
    ops.moe_expert_up_gelu(x_perm, off, w1, rows_max, h=h_ref)

    nf = ops.moe_frag_rows(rows_max, E)
    x_frag = torch.full((nf, d), SENT_X, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    ops.moe_permute_frag(x, src, off, rows_max, x_frag)
    h = torch.full((max(rows_max, 1), d_ff), SENT_H, dtype=torch.int16, device="cuda:0").view(torch.float16)
    ops.moe_expert_up_gelu_frag(x_frag, off, w1, rows_max, h=h)
    torch.cuda.synchronize()

    rows, pads, pad_total = unfrag(x_frag.cpu(), counts_to_offsets(counts), d)
    assert pad_total <= nf
    assert torch.equal(rows, x.cpu()[src.cpu()[:R].long()]), "permuted rows differ"
    assert (pads.view(torch.int16) == 0).all(), "padding rows are not zero"
    assert (x_frag.view(torch.int16)[pad_total:].cpu() == SENT_X).all(), "rows past the padded segments written"
    same = torch.equal(h[:R].view(torch.int16), h_ref[:R].view(torch.int16))
    if not same:
        diff = (h[:R].float() - h_ref[:R].float()).abs()
        bad = torch.nonzero(diff > 0)
        say("  %d values differ, first at %s" % (bad.shape[0], bad[:4].tolist()))
    assert same, "h differs from the row-major up-projection"
    assert (h[R:].view(torch.int16) == SENT_H).all(), "rows past offsets[E] written"
    return R


def counts_to_offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def test_frag_ragged_segments():
    """Segments of 37, 0, 300, 1 and 64 rows (none a multiple of 32 but the
    last), a d_ff tail (776 = 3 x 256 + 8)."""
    run_case([37, 0, 300, 1, 64], d=512, d_ff=776)


def test_frag_several_tiles_per_workgroup_short_k():
    """d = 256: four 64-deep stages per tile, so every stage of a tile but the
    first prefetches the next tile; about 600 tiles, several per workgroup."""
    rng = np.random.default_rng(3)
    counts = rng.integers(600, 1100, size=6).tolist()
    run_case(counts, d=256, d_ff=6144, seed=1)


def test_frag_many_sparse_experts():
    """256 experts, most of them empty, the rest 1 to 70 rows."""
    rng = np.random.default_rng(5)
    counts = np.where(rng.random(256) < 0.2, rng.integers(1, 71, size=256), 0).tolist()
    run_case(counts, d=512, d_ff=264, seed=2)


def test_frag_no_rows():
    run_case([0, 0, 0, 0], d=256, d_ff=256, slack=64, seed=3)
    # rows_max == 0 is a no-op
    x = torch.zeros(1, 256, dtype=torch.bfloat16, device="cuda:0")
    off = torch.zeros(5, dtype=torch.int32, device="cuda:0")
    w1 = torch.zeros(4, 256, 256, dtype=torch.bfloat16, device="cuda:0")
    xf = ops.moe_permute_frag(x, off, off, 0)
    ops.moe_expert_up_gelu_frag(xf, off, w1, 0)
    torch.cuda.synchronize()


def test_frag_large_experts_shape():
    """The large-experts shape (d 4096, d_ff 16384, eight experts of about
    1280 rows), with ragged segment lengths."""
    counts = [1283, 1250, 1301, 1222, 1279, 1340, 1197, 1368]
    run_case(counts, d=4096, d_ff=16384, seed=4)
