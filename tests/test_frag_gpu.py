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
    if d_ff % 256 == 0:
        # h in fragment order: the same values, padding rows zero, nothing past the padded segments;
        # then the down-projection from it against the row-major one on the same h (no workspace)
        hf = torch.full((ops.moe_frag_rows(rows_max, E), d_ff), SENT_H, dtype=torch.int16,
                        device="cuda:0").view(torch.float16)
        ops.moe_expert_up_gelu_frag(x_frag, off, w1, rows_max, h=hf, frag_out=True)
        w2h = (torch.randn(E, d, d_ff, generator=g) / d_ff ** 0.5).to(torch.float16).to("cuda:0")
        y_ref = ops.moe_expert_down_f16w(h_ref, off, w2h, rows_max)
        y = torch.full((max(rows_max, 1), d), float("nan"), device="cuda:0")
        ops.moe_expert_down_frag(hf, off, w2h, rows_max, y_perm=y)
        torch.cuda.synchronize()
        hrows, hpads, hpt = unfrag(hf.cpu(), counts_to_offsets(counts), d_ff)
        assert torch.equal(hrows.view(torch.int16), h_ref[:R].cpu().view(torch.int16)), "fragment-ordered h differs"
        assert (hpads.view(torch.int16) == 0).all(), "padding rows of h are not zero"
        assert (hf.view(torch.int16)[hpt:].cpu() == SENT_H).all(), "rows past the padded segments of h written"
        assert torch.equal(y[:R].view(torch.int32), y_ref[:R].view(torch.int32)), \
            "down-projection from fragment-ordered h differs: max|diff| %.3g" % (y[:R] - y_ref[:R]).abs().max().item()
        assert torch.isnan(y[R:]).all(), "rows past offsets[E] of y_perm written"
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


# ---------------------------------------------------------------- fp16 W2 --
def test_weights_bf16_to_f16_every_value():
    """All 65536 bf16 bit patterns (plus a ragged tail of 5): the conversion
    against torch's bf16 -> fp16 (round to nearest even); NaNs stay NaN."""
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    w = torch.cat([bits, bits[1000:1005]]).view(torch.bfloat16)
    got = ops.moe_weights_bf16_to_f16(w.to("cuda:0"))
    torch.cuda.synchronize()
    got = got.cpu()
    want = w.to(torch.float16)
    nan = torch.isnan(want)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(got[~nan].view(torch.int16), want[~nan].view(torch.int16))


@pytest.mark.parametrize("counts,d,d_ff", [([37, 0, 300, 1, 64], 512, 776),
                                           ([150, 290], 1024, 8200),
                                           ([1283, 1250, 1301, 1222, 1279, 1340, 1197, 1368], 4096, 16384)])
def test_down_f16w_equals_in_register_conversion(counts, d, d_ff):
    """The down-projection on the fp16 copy of W2 against the one converting
    bf16 W2 in registers: bit-identical, with and without split tiles."""
    g = torch.Generator().manual_seed(7)
    E, R = len(counts), int(sum(counts))
    rows_max = R + 9
    say("  case E=%d R=%d d=%d d_ff=%d" % (E, R, d, d_ff))
    h = torch.randn(rows_max, d_ff, generator=g).to(torch.float16).to("cuda:0")
    w2 = (torch.randn(E, d, d_ff, generator=g) / d_ff ** 0.5).to(torch.bfloat16).to("cuda:0")
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda:0")
    w2h = ops.moe_weights_bf16_to_f16(w2)
    ws = torch.empty(ops.moe_ffn_workspace_bytes(torch.bfloat16), dtype=torch.uint8, device="cuda:0")
    for workspace in (None, ws):
        a = ops.moe_expert_down(h, off, w2, rows_max, workspace=workspace)
        b = ops.moe_expert_down_f16w(h, off, w2h, rows_max, workspace=workspace)
        torch.cuda.synchronize()
        assert torch.equal(a[:R].view(torch.int32), b[:R].view(torch.int32)), \
            "workspace %s: max|diff| %.3g" % (workspace is not None, (a[:R] - b[:R]).abs().max().item())


@pytest.mark.parametrize("frag", [False, True])
def test_forward_with_f16_w2_is_bit_identical(frag):
    """The layer forward given moe_weights_bf16_to_f16(W2) against the same
    forward converting W2 in registers: the same y, bit for bit."""
    from mixture_experts_layer_49_amd import inputs as I
    from parity_helpers import dev
    cfg = I.small("f16w", T=600, d=256, d_ff=512, E=4, k=2, cf=1.25, seed=71)
    inp = I.make_inputs(cfg)
    x, w1, w2, wg = (dev(inp[n], "bf16") for n in ("x", "w1", "w2", "w_gate"))
    C = ops.moe_capacity(cfg.T, cfg.E, cfg.cf)
    ys = []
    for w2h in (None, ops.moe_weights_bf16_to_f16(w2)):
        b = ops.MoEBuffers(cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, C, x.dtype, x.device, frag=frag)
        ops.moe_forward(x, w1, w2, cfg.k, C, w_gate=wg, bufs=b, w2_f16=w2h)
        torch.cuda.synchronize()
        ys.append(b.y.clone())
    assert torch.equal(ys[0].view(torch.int32), ys[1].view(torch.int32))


@pytest.mark.parametrize("counts,d,d_ff", [([1283, 1250, 1301, 1222, 1279, 1340, 1197, 1368], 4096, 16384),
                                           ([700, 720, 690, 745, 701, 680, 730, 747], 4096, 16384),
                                           ([150, 290, 77], 512, 8192)])
def test_down_frag_split_tiles(counts, d, d_ff):
    """The fragment-ordered down-projection with the workspace (a short last
    round split along K, pieces added up by the fix-up kernel) against the
    same without it: equal up to float32 summation order, the same on every
    call. The first shape leaves half a round of tiles (2-way split), the
    second (the receiver share's) and third other splits."""
    g = torch.Generator().manual_seed(11)
    E, R = len(counts), int(sum(counts))
    rows_max = R + 5
    say("  case E=%d R=%d d=%d d_ff=%d" % (E, R, d, d_ff))
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda:0")
    # h in fragment order, written by the up-projection (its padding rows zero)
    x = torch.randn(R, d, generator=g).to(torch.bfloat16).to("cuda:0")
    w1 = (torch.randn(E, d_ff, d, generator=g) / d ** 0.5).to(torch.bfloat16).to("cuda:0")
    src = torch.arange(R, dtype=torch.int32, device="cuda:0")
    xf = ops.moe_permute_frag(x, src, off, rows_max)
    hf = ops.moe_expert_up_gelu_frag(xf, off, w1, rows_max, frag_out=True)
    del w1, x
    w2h = (torch.randn(E, d, d_ff, generator=g) / d_ff ** 0.5).to(torch.float16).to("cuda:0")
    ws = torch.empty(ops.moe_ffn_workspace_bytes(torch.bfloat16), dtype=torch.uint8, device="cuda:0")
    ws.fill_(0x7F)
    yu = ops.moe_expert_down_frag(hf, off, w2h, rows_max)
    ys = ops.moe_expert_down_frag(hf, off, w2h, rows_max, workspace=ws)
    ys2 = ops.moe_expert_down_frag(hf, off, w2h, rows_max, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(ys[:R], ys2[:R])
    a, b = ys[:R].double(), yu[:R].double()
    err = ((a - b).abs().max() / b.pow(2).mean().sqrt()).item()
    moved = (a != b).float().mean().item()
    say("  split vs unsplit: max|diff|/rms %.2e, %.2f%% of values differ" % (err, 100 * moved))
    # float32 sums of 16384 products in another order: the difference grows
    # like sqrt(K) * 2^-24 times the terms' size (measured up to 1.2e-5 of the
    # output RMS); the row-major GEMM's split test allows 1e-3
    assert err <= 1e-4, err
