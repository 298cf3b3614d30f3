"""CPU: the host side of the fragment-ordered path -- which layers take it,
the buffer sizes, and the test helper that reads the layout back, pinned to
the layout's definition element by element (written out here with plain
loops, independent of the helper's reshapes)."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_49_amd import ops
from parity_helpers import unfrag


def frag_index(r, c, d):
    """Element (padded row r, column c) of a fragment-ordered [rows, d] buffer."""
    return ((r // 32) * (d // 16) + c // 16) * 512 + ((r % 32) + 32 * ((c // 8) % 2)) * 8 + c % 8


@pytest.mark.parametrize("counts,d", [([5, 0, 40], 32), ([33], 48), ([0, 0], 16), ([64, 1], 16)])
def test_unfrag_reads_the_documented_layout(counts, d):
    rng = np.random.default_rng(0)
    off = np.concatenate([[0], np.cumsum(counts)])
    pads = [(n + 31) // 32 * 32 for n in counts]
    total = sum(pads)
    rows = rng.integers(-1000, 1000, size=(int(off[-1]), d)).astype(np.int16)
    buf = np.full(max(total, 32) * d, 7, dtype=np.int16)   # padding rows hold 7 here
    p = 0
    for e, n in enumerate(counts):
        for i in range(n):
            for c in range(d):
                buf[frag_index(p + i, c, d)] = rows[off[e] + i, c]
        p += pads[e]
    got, pad_rows, pt = unfrag(torch.from_numpy(buf).reshape(-1, d), off, d)
    assert pt == total
    assert np.array_equal(got.numpy(), rows)
    assert (pad_rows.numpy() == 7).all() and pad_rows.shape[0] == total - off[-1]


def test_fragment_path_choice_and_sizes():
    bf = torch.bfloat16
    assert ops.frag_eligible(bf, 4096) and ops.frag_eligible(bf, 8192)
    assert not ops.frag_eligible(bf, 2048) and not ops.frag_eligible(bf, 1024)
    assert not ops.frag_eligible(bf, 4096 + 8)
    assert not ops.frag_eligible(torch.float32, 4096)
    # MoEBuffers on the host (sizes only): the fragment copy replaces x_perm
    b = ops.MoEBuffers(64, 4096, 256, 4, 2, 40, bf, "cpu")
    assert b.frag and b.x_perm is None
    assert b.x_frag.shape == (ops.moe_frag_rows(b.rows_max, 4), 4096)
    assert not ops.MoEBuffers(64, 4096, 256, 4, 2, 40, bf, "cpu", save_for_backward=True).frag
    assert not ops.MoEBuffers(64, 1024, 256, 4, 2, 40, bf, "cpu").frag
    # the row-major bf16 forward without a backward folds the permute into the
    # up-projection (no x_perm); a backward or f32 keeps x_perm
    g = ops.MoEBuffers(64, 1024, 256, 4, 2, 40, bf, "cpu")
    assert g.gather and g.x_perm is None and not b.gather
    assert not ops.MoEBuffers(64, 1024, 256, 4, 2, 40, bf, "cpu", save_for_backward=True).gather
    assert not ops.MoEBuffers(64, 1024, 256, 4, 2, 40, torch.float32, "cpu").gather
    assert ops.MoEBuffers(64, 1024, 256, 4, 2, 40, bf, "cpu", gather=False).x_perm is not None
    with pytest.raises(ValueError):
        ops.MoEBuffers(64, 1024, 256, 4, 2, 40, torch.float32, "cpu", gather=True)
    with pytest.raises(ValueError):
        ops.MoEBuffers(64, 2048, 256, 4, 2, 40, bf, "cpu", frag=True, gather=True)
    with pytest.raises(ValueError):
        ops.MoEBuffers(64, 2048, 256, 4, 2, 40, torch.float32, "cpu", frag=True)
    with pytest.raises(ValueError):
        ops.MoEBuffers(64, 2048, 256, 4, 2, 40, bf, "cpu", frag=True, save_for_backward=True)
