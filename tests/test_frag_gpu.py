"""GPU: the fragment-ordered permute and up-projection against the row-major
ones, on the same segments. The permuted rows are bit-exact (read back through
the layout's definition, padding rows zero), and rows past the segments are
left alone. The fragment-ordered GEMM multiplies with 16 x 16 x 32 MFMAs and
the row-major one with 32 x 32 x 16 MFMAs: the same products, added in float32
in another order, so h agrees with moe_expert_up_gelu's to one fp16 rounding
step (plus the absolute change of a reordered float32 sum near zero) and y_perm
to float32 summation order. The row-major GEMM is itself checked against the
oracle by the layer parity tests, and so is the fragment-ordered path at every
workload's full size."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_49_amd import ops
from parity_helpers import say, unfrag

pytestmark = pytest.mark.gpu

SENT_H = 0x7E55     # an fp16 NaN pattern no result has
SENT_X = 0x5A5A


def fp16_close(got, ref, what):
    """got and ref (fp16, same shape) agree to one fp16 rounding step of ref
    plus 2^-17: the float32 sums of d products behind them differ only in the
    order of their additions, which moves the pre-activation by about
    sqrt(d) 2^-24 of the partial sums' size and gelu by at most 1.13 times
    that; after the fp16 rounding, values next to a rounding boundary move by
    one step, and near zero (fp16 subnormals, step 2^-24) by that absolute
    change. Few values may move at all."""
    a, b = got.double().cpu(), ref.double().cpu()
    assert torch.isfinite(a).all() == torch.isfinite(b).all()
    step = torch.where(b.abs() < 2.0 ** -14, torch.full_like(b, 2.0 ** -24),
                       torch.exp2(torch.floor(torch.log2(b.abs().clamp_min(2.0 ** -14)))) * 2.0 ** -10)
    diff = (a - b).abs()
    bad = diff > step * 1.0001 + 2.0 ** -17
    moved = (diff > 0).double().mean().item() if diff.numel() else 0.0
    say("  %s: %.4f%% of values differ, max|diff| %.3g, %d beyond the bound"
        % (what, 100 * moved, diff.max().item() if diff.numel() else 0.0, int(bad.sum())))
    assert not bad.any(), "%s differs by more than one fp16 step" % what
    assert moved < 0.02, "%s: %.4f of the values differ" % (what, moved)


def f32_close(got, ref, what, tol=1e-4):
    """float32 results of the same products summed in another order: max|diff|
    within tol of the reference's RMS."""
    a, b = got.double().cpu(), ref.double().cpu()
    rms = b.pow(2).mean().sqrt().item() if b.numel() else 0.0
    err = ((a - b).abs().max().item() / rms) if rms > 0 else (a - b).abs().max().item() if a.numel() else 0.0
    say("  %s: max|diff|/rms %.2e" % (what, err))
    assert err <= tol, "%s: max|diff|/rms %.3e" % (what, err)


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
    fp16_close(h[:R], h_ref[:R], "h (row-major) vs the row-major GEMM's")
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
        assert torch.equal(hrows.view(torch.int16), h[:R].cpu().view(torch.int16)), \
            "fragment-ordered h differs from the same kernel's row-major h"
        assert (hpads.view(torch.int16) == 0).all(), "padding rows of h are not zero"
        assert (hf.view(torch.int16)[hpt:].cpu() == SENT_H).all(), "rows past the padded segments of h written"
        # the down-projection from fragment-ordered h against the row-major one
        # on the row-major kernel's h: both the h values (one fp16 step apart
        # in a few places) and the summation order differ
        f32_close(y[:R], y_ref[:R], "y_perm from fragment-ordered h", tol=1e-3)
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


def _f16_flags(w_bf16: torch.Tensor):
    """Host reference of the conversion report: (inexact, overflow) counts of
    bf16 -> fp16 round to nearest even, from torch's CPU casts."""
    f = w_bf16.float()
    h = w_bf16.to(torch.float16).float()
    fin = torch.isfinite(f)
    over = fin & torch.isinf(h)
    inexact = fin & ~torch.isinf(h) & (h != f)
    return int(inexact.sum()), int(over.sum())


def test_weights_bf16_to_f16_report_every_value():
    """The report on all 65536 bf16 bit patterns (and a ragged tail): its two
    counts equal the host's, and the flagged values lie in the documented
    ranges (exact for 0 and 2^-17 <= |w| <= 65280, +-inf from 65536 up)."""
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    w = torch.cat([bits, bits[1000:1005]]).view(torch.bfloat16)
    rep = torch.full((2,), -1, dtype=torch.int64, device="cuda:0")
    ops.moe_weights_bf16_to_f16(w.to("cuda:0"), report=rep)
    torch.cuda.synchronize()
    got = tuple(int(v) for v in rep.cpu())
    want = _f16_flags(w)
    say("  report %s, host %s" % (got, want))
    assert got == want
    # where the flags fall: bits are lost only below 2^-17 (and there only
    # where a value has bits below fp16's subnormal step 2^-24: every nonzero
    # value under 2^-25 rounds away), inf only from 65536 up
    f = w.float().abs()
    h = w.to(torch.float16).float()
    fin = torch.isfinite(f)
    lost = fin & ~torch.isinf(h) & (h != w.float())
    assert not (lost & (f >= 2.0 ** -17)).any()
    assert lost[fin & (f > 0) & (f < 2.0 ** -25)].all()
    assert torch.equal(fin & torch.isinf(h), fin & (f >= 65536.0))


def test_weights_bf16_to_f16_report_small_and_large_w2():
    """W2 holding values of 2^-20 (with low bits that fp16 cannot hold) and
    7e4 (beyond fp16): the report counts them, the converted values are the
    round-to-nearest-even ones (2^-20 and +-inf), and a down-projection on
    that W2 gives non-finite output exactly in the columns of the
    overflowing weights of the rows that use them."""
    g = torch.Generator().manual_seed(5)
    E, d, d_ff = 2, 256, 512
    w2 = (torch.randn(E, d, d_ff, generator=g) / d_ff ** 0.5).to(torch.bfloat16)
    tiny = torch.tensor((1.0 + 2.0 ** -7) * 2.0 ** -20).to(torch.bfloat16)   # bits below 2^-24
    w2[0, 3, 5] = tiny
    w2[1, 200, 77] = -tiny
    w2[1, 9, 300] = 7e4
    w2[0, 100, 0] = -7e4
    rep = torch.zeros(2, dtype=torch.int64, device="cuda:0")
    w2h = ops.moe_weights_bf16_to_f16(w2.to("cuda:0"), report=rep)
    torch.cuda.synchronize()
    inexact, over = _f16_flags(w2)
    assert tuple(int(v) for v in rep.cpu()) == (inexact, over) and over == 2 and inexact >= 2
    hh = w2h.cpu()
    assert float(hh[0, 3, 5]) == 2.0 ** -20 and float(hh[1, 200, 77]) == -(2.0 ** -20)
    assert torch.isinf(hh[1, 9, 300]) and hh[1, 9, 300] > 0
    assert torch.isinf(hh[0, 100, 0]) and hh[0, 100, 0] < 0
    # down-projection on that W2: rows of expert 1 are non-finite in column 9,
    # rows of expert 0 in column 100, every other value finite
    rows = [40, 33]
    off = torch.tensor([0, rows[0], rows[0] + rows[1]], dtype=torch.int32, device="cuda:0")
    h = (torch.rand(sum(rows), d_ff, generator=g) + 0.5).to(torch.float16).to("cuda:0")
    y = ops.moe_expert_down_f16w(h, off, w2h, sum(rows))
    torch.cuda.synchronize()
    bad = ~torch.isfinite(y[:sum(rows)].cpu())
    want = torch.zeros_like(bad)
    want[:rows[0], 100] = True
    want[rows[0]:, 9] = True
    assert torch.equal(bad, want)


def test_hidden_overflow_gives_nonfinite_rows():
    """h is fp16: a row whose pre-activation reaches 65520 or more stores
    +-inf there, as documented, and only that token's output is non-finite."""
    from mixture_experts_layer_49_amd import inputs as I
    from parity_helpers import dev
    cfg = I.small("h-overflow", T=64, d=256, d_ff=256, E=2, k=1, cf=0.0, seed=77)
    inp = I.make_inputs(cfg)
    x = dev(inp["x"], "bf16")
    w1 = dev(inp["w1"], "bf16")
    # token 7: x = 2e4 * sign(W1[e, 0, :]), the same row in both experts, so
    # that z[., 0] = 2e4 * sum |W1[e, 0, :]| (about 2.6e5) is far above 65520
    w1[1, 0] = w1[0, 0]
    x[7] = (2e4 * torch.where(w1[0, 0].float() >= 0, 1.0, -1.0)).to(torch.bfloat16)
    w2 = dev(inp["w2"], "bf16")
    idx = torch.randint(0, 2, (cfg.T, 1), dtype=torch.int32, device="cuda:0")
    wt = torch.ones(cfg.T, 1, device="cuda:0")
    for frag in (False, True):
        b = ops.MoEBuffers(cfg.T, cfg.d, cfg.d_ff, cfg.E, 1, -1, x.dtype, x.device, routed=False,
                           frag=frag)
        ops.moe_forward(x, w1, w2, 1, -1, topk_idx=idx, topk_w=wt, bufs=b)
        torch.cuda.synchronize()
        fin = torch.isfinite(b.y.cpu()).all(dim=1)
        assert not fin[7] and fin[torch.arange(cfg.T) != 7].all()


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


@pytest.mark.parametrize("frag,hfrag", [(False, False), (True, False), (True, True)])
def test_forward_with_f16_w2(frag, hfrag):
    """The layer forward given moe_weights_bf16_to_f16(W2) against the same
    forward converting W2 in registers: with h row-major (both forwards run
    the same kernels) the same y, bit for bit; with h kept in fragment order
    (the down-projection then runs the fragment-ordered GEMM, whose float32
    sums are added in another order) y to float32 summation order."""
    from mixture_experts_layer_49_amd import inputs as I
    from parity_helpers import dev
    cfg = I.small("f16w", T=600, d=256, d_ff=512, E=4, k=2, cf=1.25, seed=71)
    inp = I.make_inputs(cfg)
    x, w1, w2, wg = (dev(inp[n], "bf16") for n in ("x", "w1", "w2", "w_gate"))
    C = ops.moe_capacity(cfg.T, cfg.E, cfg.cf)
    ys = []
    for w2h in (None, ops.moe_weights_bf16_to_f16(w2)):
        b = ops.MoEBuffers(cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, C, x.dtype, x.device, frag=frag,
                           w2_f16=hfrag and w2h is not None)
        ops.moe_forward(x, w1, w2, cfg.k, C, w_gate=wg, bufs=b, w2_f16=w2h)
        assert (b.h_frag is not None) == (hfrag and w2h is not None)
        torch.cuda.synchronize()
        ys.append(b.y.clone())
    if hfrag:
        f32_close(ys[1], ys[0], "y with h in fragment order", tol=1e-4)
    else:
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
