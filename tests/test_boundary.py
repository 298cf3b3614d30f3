"""The C-ABI library on the CPU: it loads, exports every declared entry point,
computes its host-side sizes correctly and rejects bad arguments before any
HIP call (no kernel is launched here)."""
import ctypes
import json
import os
import re

import pytest

from mixture_experts_layer_49_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = ops.lib()
    names = declared_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(L, n), n
    assert sorted(ops.EXPORTS) == names


def test_capacity_matches_hand_cases():
    with open(os.path.join(ROOT, "tests", "golden", "capacity_hand.json")) as f:
        for c in json.load(f)["cases"]:
            assert ops.moe_capacity(c["n"], c["E"], c["cf"]) == c["C"], c
    assert ops.moe_capacity(-1, 4, 1.0) == -2
    assert ops.moe_capacity(10, 0, 1.0) == -2


def test_rows_max():
    assert ops.moe_rows_max(8192, 2, 8, 1280) == 10240
    assert ops.moe_rows_max(4096, 2, 16, 256) == 4096
    assert ops.moe_rows_max(100, 2, 4, 1000) == 200
    assert ops.moe_rows_max(100, 2, 4, -1) == 200
    assert ops.moe_rows_max(0, 2, 4, 10) == 0


def test_workspace_sizes():
    assert ops.moe_dispatch_workspace_bytes(0, 2, 8) == 0
    assert ops.moe_dispatch_workspace_bytes(512, 2, 8) == 2 * 2 * 8 * 4
    assert ops.moe_dispatch_workspace_bytes(16384, 2, 64) == 2 * 64 * 64 * 4
    assert ops.moe_aux_loss_workspace_bytes(16384, 64) > 0


FAKE = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never dereferenced: calls fail first


def _rc(fn, *args):
    return getattr(ops.lib(), fn)(*args)


def test_router_argument_errors():
    L = ops.lib()
    good = [FAKE, FAKE, None, 16, 64, 8, 2, 1, 0, FAKE, FAKE, None, None]
    def call(**kw):
        a = list(good)
        pos = {"x": 0, "wg": 1, "T": 3, "d": 4, "E": 5, "k": 6, "dt": 7, "flags": 8, "idx": 9, "w": 10}
        for k, v in kw.items():
            a[pos[k]] = v
        return L.moe_router_topk(*a)
    assert call(x=None) == -1
    assert call(idx=None) == -1
    assert call(T=-1) == -1
    assert call(d=0) == -1
    assert call(E=0) == -3
    assert call(E=257) == -3
    assert call(k=0) == -3
    assert call(k=9, E=16) == -3
    assert call(k=3, E=2) == -3
    assert call(dt=7) == -2
    assert call(flags=4) == -1
    assert call(d=60) == -6                       # bf16 rows must be a multiple of 8
    assert call(x=ctypes.c_void_p((1 << 20) + 2)) == -6
    assert b"x" in L.moe_last_error()
    assert call(T=0) == 0                         # empty batch: no-op, nothing launched


def test_dispatch_argument_errors():
    L = ops.lib()
    need = L.moe_dispatch_workspace_bytes(100, 2, 8)
    base = [FAKE, 100, 2, 8, 25, FAKE, 64, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None]
    def call(i, v):
        a = list(base)
        a[i] = v
        return L.moe_dispatch(*a)
    assert call(13, None) == -4                  # no workspace
    assert call(14, need - 1) == -4              # too small
    assert call(0, None) == -1
    assert call(8, None) == -1
    assert call(3, 300) == -3
    assert call(7, 5) == -2
    assert call(6, 12) == -6
    assert call(13, ctypes.c_void_p((1 << 20) + 2)) == -6
    # T == 0 skips every per-token pointer check but still needs counts/offsets
    a = list(base); a[1] = 0; a[8] = None
    assert L.moe_dispatch(*a) == -1


def test_router_ex_and_z_loss_argument_errors():
    L = ops.lib()
    base = [FAKE, FAKE, None, None, 100, 64, 8, 2, 1, 0, 1.0, FAKE, FAKE, None, None, None]

    def call(i, v):
        a = list(base); a[i] = v
        return L.moe_router_topk_ex(*a)
    assert call(10, 0.0) == -1                    # temperature must be > 0
    assert call(10, -2.0) == -1
    assert call(10, float("nan")) == -1
    assert call(10, float("inf")) == -1
    assert call(9, 0x4) == -1                     # unknown flag
    assert call(7, 9) == -3                       # k > E
    assert call(5, 60) == -6                      # bf16 d % 8
    assert call(0, None) == -1
    # moe_z_loss(lse, T, coeff, loss, ws, ws_bytes, stream)
    need = L.moe_z_loss_workspace_bytes(100)
    assert need > 0
    assert L.moe_z_loss(FAKE, -1, 1.0, FAKE, FAKE, need, None) == -1
    assert L.moe_z_loss(FAKE, 100, 1.0, None, FAKE, need, None) == -1
    assert L.moe_z_loss(None, 100, 1.0, FAKE, FAKE, need, None) == -1
    assert L.moe_z_loss(FAKE, 100, 1.0, FAKE, FAKE, need - 1, None) == -4
    assert L.moe_z_loss(FAKE, 100, 1.0, FAKE, ctypes.c_void_p((1 << 20) + 4), need, None) == -6


def test_plan_and_permute_argument_errors():
    L = ops.lib()
    need = L.moe_dispatch_workspace_bytes(100, 2, 8)
    ok = [FAKE, 100, 2, 8, 30, FAKE, FAKE, FAKE, FAKE, FAKE, need, None]

    def plan(i, v):
        a = list(ok); a[i] = v
        return L.moe_dispatch_plan(*a)
    assert plan(3, 0) == -3                      # E = 0
    assert plan(2, 9) == -3                      # k > E
    assert plan(1, -1) == -1                     # T < 0
    assert plan(5, None) == -1                   # counts
    assert plan(0, None) == -1                   # topk_idx with T > 0
    assert plan(10, need - 1) == -4              # workspace too small
    assert plan(9, ctypes.c_void_p((1 << 20) + 2)) == -6
    a = list(ok); a[1] = 0; a[0] = None; a[7] = None; a[8] = None; a[9] = None; a[10] = 0; a[5] = None
    assert L.moe_dispatch_plan(*a) == -1         # T == 0 still needs counts and offsets
    # moe_dispatch_plan_aux(topk_idx, probs, T, k, E, capacity, alpha, counts, offsets, dest, src,
    #                       loss, ws, ws_bytes, stream)
    need_aux = L.moe_dispatch_plan_aux_workspace_bytes(100, 2, 8)
    assert need_aux == need + 1 * 8 * 8            # the plan's ints, then a double per (chunk, expert)
    okx = [FAKE, FAKE, 100, 2, 8, 30, ctypes.c_float(0.01), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need_aux, None]

    def plan_aux(i, v):
        a = list(okx); a[i] = v
        return L.moe_dispatch_plan_aux(*a)
    assert plan_aux(4, 0) == -3                  # E = 0
    assert plan_aux(1, None) == -1               # probs with T > 0
    assert plan_aux(11, None) == -1              # loss
    assert plan_aux(13, need_aux - 1) == -4      # workspace too small
    assert plan_aux(12, ctypes.c_void_p((1 << 20) + 4)) == -6   # workspace alignment
    assert plan_aux(1, ctypes.c_void_p((1 << 20) + 4)) == -6    # probs alignment
    # moe_dispatch_plan_noalloc(topk_idx, T, k, E, capacity, counts, offsets, dest, src, stream):
    # the same checks without a workspace; a plan beyond the static scratch is
    # refused before anything is enqueued
    assert L.moe_dispatch_plan_noalloc_scratch_bytes() == 1 << 20
    assert L.moe_dispatch_plan_noalloc(FAKE, 100, 2, 0, 30, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert L.moe_dispatch_plan_noalloc(FAKE, 100, 9, 8, 30, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert L.moe_dispatch_plan_noalloc(FAKE, -1, 2, 8, 30, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert L.moe_dispatch_plan_noalloc(None, 100, 2, 8, 30, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert L.moe_dispatch_plan_noalloc(FAKE, 100, 2, 8, 30, FAKE, FAKE, None, FAKE, None) == -1
    assert L.moe_dispatch_plan_noalloc(FAKE, 131073, 2, 256, 30, FAKE, FAKE, FAKE, FAKE, None) == -4
    assert L.moe_dispatch_workspace_bytes(131072, 2, 256) == 1 << 20   # the largest that fits
    # moe_permute(x, d, dtype, src, offsets, E, rows_max, x_perm, stream)
    assert L.moe_permute(FAKE, 64, 1, FAKE, FAKE, 8, 10, FAKE, None) != -1
    assert L.moe_permute(FAKE, 60, 1, FAKE, FAKE, 8, 10, FAKE, None) == -6
    assert L.moe_permute(FAKE, 64, 7, FAKE, FAKE, 8, 10, FAKE, None) == -2
    assert L.moe_permute(None, 64, 1, FAKE, FAKE, 8, 10, FAKE, None) == -1
    assert L.moe_permute(FAKE, 64, 1, FAKE, FAKE, 0, 10, FAKE, None) == -3
    assert L.moe_permute(None, 64, 1, None, None, 8, 0, None, None) == 0
    assert L.moe_permute(FAKE, 64, 1, FAKE, FAKE, 8, 10, ctypes.c_void_p((1 << 20) + 4), None) == -6


def test_ffn_combine_aux_argument_errors():
    L = ops.lib()
    assert L.moe_grouped_ffn(FAKE, FAKE, 0, 10, 64, 128, FAKE, FAKE, 1, FAKE, FAKE, None, 0, None) == -3
    assert L.moe_grouped_ffn(FAKE, FAKE, 8, 10, 60, 128, FAKE, FAKE, 1, FAKE, FAKE, None, 0, None) == -6
    assert L.moe_grouped_ffn(FAKE, FAKE, 8, 10, 64, 128, FAKE, FAKE, 3, FAKE, FAKE, None, 0, None) == -2
    assert L.moe_grouped_ffn(None, FAKE, 8, 10, 64, 128, FAKE, FAKE, 1, FAKE, FAKE, None, 0, None) == -1
    assert L.moe_grouped_ffn(FAKE, FAKE, 8, -1, 64, 128, FAKE, FAKE, 1, FAKE, FAKE, None, 0, None) == -1
    assert L.moe_grouped_ffn(None, None, 8, 0, 64, 128, None, None, 1, None, None, None, 0, None) == 0
    assert L.moe_expert_up_gelu(FAKE, FAKE, 8, 10, 64, 130, FAKE, 1, FAKE, None, 0, None) == -6
    assert L.moe_expert_down(FAKE, None, 8, 10, 64, 128, FAKE, 1, FAKE, None, 0, None) == -1
    # the FFN workspace is optional, but a given one must be large enough and 16-B aligned
    need = L.moe_ffn_workspace_bytes(1)
    assert L.moe_expert_down(FAKE, FAKE, 8, 10, 64, 128, FAKE, 1, FAKE, FAKE, need - 1, None) == -4
    assert L.moe_expert_up_gelu(FAKE, FAKE, 8, 10, 64, 128, FAKE, 1, FAKE, FAKE, need - 1, None) == -4
    assert L.moe_grouped_ffn(FAKE, FAKE, 8, 10, 64, 128, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, None) == -4
    # moe_expert_up_gelu_gather(x, T, src, offsets, E, rows_max, d, d_ff, w1, h, ws, ws_bytes, stream)
    G = L.moe_expert_up_gelu_gather
    assert G(FAKE, 100, FAKE, FAKE, 8, 10, 64, 130, FAKE, FAKE, None, 0, None) == -6      # d_ff % 8
    assert G(FAKE, 100, FAKE, FAKE, 8, 10, 60, 128, FAKE, FAKE, None, 0, None) == -6      # d % 8
    assert G(FAKE, -1, FAKE, FAKE, 8, 10, 64, 128, FAKE, FAKE, None, 0, None) == -1       # T < 0
    assert G(FAKE, 100, None, FAKE, 8, 10, 64, 128, FAKE, FAKE, None, 0, None) == -1      # src
    assert G(FAKE, 1 << 24, FAKE, FAKE, 8, 10, 64, 128, FAKE, FAKE, None, 0, None) == -3  # x of 2^31 bytes
    assert G(FAKE, 100, FAKE, FAKE, 300, 10, 64, 128, FAKE, FAKE, None, 0, None) == -3    # E
    assert G(FAKE, 100, FAKE, FAKE, 8, 10, 64, 128, FAKE, FAKE, FAKE, need - 1, None) == -4
    assert G(None, 0, None, None, 8, 0, 64, 128, None, None, None, 0, None) == 0
    assert L.moe_expert_down(FAKE, FAKE, 8, 10, 64, 128, FAKE, 1, FAKE,
                             ctypes.c_void_p((1 << 20) + 8), need, None) == -6
    assert L.moe_combine(FAKE, FAKE, FAKE, 10, 9, 64, FAKE, 0, None) == -1
    assert L.moe_combine(FAKE, FAKE, FAKE, 10, 2, 62, FAKE, 0, None) == -6
    assert L.moe_combine(FAKE, None, FAKE, 10, 2, 64, FAKE, 0, None) == -1
    assert L.moe_combine(None, None, None, 0, 2, 64, None, 0, None) == 0
    assert L.moe_aux_loss(FAKE, FAKE, 10, 8, 2, 0.01, FAKE, None, 0, None) == -4
    assert L.moe_aux_loss(FAKE, FAKE, 10, 8, 2, 0.01, None, FAKE, 1 << 20, None) == -1
    assert L.moe_aux_loss(FAKE, FAKE, 10, 8, 9, 0.01, FAKE, FAKE, 1 << 20, None) == -3


def test_fragment_path_argument_errors_and_sizes():
    L = ops.lib()
    # padded rows: every segment rounds up to 32, so rows_max + 31 E, rounded up to 32, bounds them
    assert L.moe_frag_rows(0, 1) == 32
    assert L.moe_frag_rows(10240, 8) == 10496
    assert L.moe_frag_rows(1, 256) == (1 + 31 * 256 + 31) // 32 * 32
    assert L.moe_frag_rows(-1, 8) == -1 and L.moe_frag_rows(10, 0) == -1 and L.moe_frag_rows(10, 257) == -1
    # moe_permute_frag(x, d, src, offsets, E, rows_max, x_frag, stream)
    assert L.moe_permute_frag(FAKE, 264, FAKE, FAKE, 8, 10, FAKE, None) == -6      # d % 16
    assert L.moe_permute_frag(FAKE, 60, FAKE, FAKE, 8, 10, FAKE, None) == -6       # d % 8
    assert L.moe_permute_frag(None, 256, FAKE, FAKE, 8, 10, FAKE, None) == -1
    assert L.moe_permute_frag(FAKE, 256, FAKE, None, 8, 10, FAKE, None) == -1
    assert L.moe_permute_frag(FAKE, 256, FAKE, FAKE, 0, 10, FAKE, None) == -3
    assert L.moe_permute_frag(FAKE, 256, FAKE, FAKE, 8, -1, FAKE, None) == -1
    assert L.moe_permute_frag(FAKE, 256, FAKE, FAKE, 8, 10, ctypes.c_void_p((1 << 20) + 4), None) == -6
    assert L.moe_permute_frag(None, 256, None, None, 8, 0, None, None) == 0
    # moe_expert_up_gelu_frag(x_frag, offsets, E, rows_max, d, d_ff, w1, h, h_order, stream)
    assert L.moe_expert_up_gelu_frag(FAKE, FAKE, 8, 10, 256, 128, FAKE, FAKE, 2, None) == -1   # h_order
    assert L.moe_expert_up_gelu_frag(FAKE, FAKE, 8, 10, 256, 264, FAKE, FAKE, 1, None) == -6   # frag h: d_ff % 256
    # moe_expert_down_frag(h_frag, offsets, E, rows_max, d, d_ff, w2_f16, y_perm, ws, ws_bytes, stream)
    need = L.moe_ffn_workspace_bytes(1)
    assert L.moe_expert_down_frag(FAKE, FAKE, 8, 10, 256, 264, FAKE, FAKE, None, 0, None) == -6
    assert L.moe_expert_down_frag(FAKE, None, 8, 10, 256, 256, FAKE, FAKE, None, 0, None) == -1
    assert L.moe_expert_down_frag(FAKE, FAKE, 8, 10, 256, 256, FAKE, FAKE, FAKE, need - 1, None) == -4
    assert L.moe_expert_down_frag(FAKE, FAKE, 0, 10, 256, 256, FAKE, FAKE, None, 0, None) == -3
    assert L.moe_expert_down_frag(None, None, 8, 0, 256, 256, None, None, None, 0, None) == 0
    assert L.moe_expert_up_gelu_frag(FAKE, FAKE, 8, 10, 264, 128, FAKE, FAKE, 0, None) == -6   # d % 256
    assert L.moe_expert_up_gelu_frag(FAKE, FAKE, 8, 10, 256, 130, FAKE, FAKE, 0, None) == -6   # d_ff % 8
    assert L.moe_expert_up_gelu_frag(FAKE, FAKE, 300, 10, 256, 128, FAKE, FAKE, 0, None) == -3
    assert L.moe_expert_up_gelu_frag(FAKE, None, 8, 10, 256, 128, FAKE, FAKE, 0, None) == -1
    assert L.moe_expert_up_gelu_frag(FAKE, FAKE, 8, 10, 256, 128, FAKE, None, 0, None) == -1
    assert L.moe_expert_up_gelu_frag(FAKE, FAKE, 8, 10, 1 << 21, 128, FAKE, FAKE, 0, None) == -3
    assert L.moe_expert_up_gelu_frag(None, None, 8, 0, 256, 128, None, None, 0, None) == 0


def test_f16_weight_argument_errors():
    L = ops.lib()
    # moe_weights_bf16_to_f16(w, n, w_f16, report, stream)
    assert L.moe_weights_bf16_to_f16(FAKE, -1, FAKE, None, None) == -1
    assert L.moe_weights_bf16_to_f16(None, 0, None, None, None) == 0
    assert L.moe_weights_bf16_to_f16(None, 8, FAKE, None, None) == -1
    assert L.moe_weights_bf16_to_f16(FAKE, 8, ctypes.c_void_p((1 << 20) + 2), None, None) == -6
    assert L.moe_weights_bf16_to_f16(FAKE, 8, FAKE, ctypes.c_void_p((1 << 20) + 4), None) == -6
    # moe_expert_down_f16w(h, offsets, E, rows_max, d, d_ff, w2_f16, y_perm, ws, ws_bytes, stream)
    need = L.moe_ffn_workspace_bytes(1)
    assert L.moe_expert_down_f16w(FAKE, FAKE, 0, 10, 64, 128, FAKE, FAKE, None, 0, None) == -3
    assert L.moe_expert_down_f16w(FAKE, FAKE, 8, 10, 60, 128, FAKE, FAKE, None, 0, None) == -6
    assert L.moe_expert_down_f16w(FAKE, None, 8, 10, 64, 128, FAKE, FAKE, None, 0, None) == -1
    assert L.moe_expert_down_f16w(FAKE, FAKE, 8, 10, 64, 128, FAKE, FAKE, FAKE, need - 1, None) == -4
    assert L.moe_expert_down_f16w(None, None, 8, 0, 64, 128, None, None, None, 0, None) == 0


def test_ffn_workspace_bytes():
    L = ops.lib()
    assert L.moe_ffn_workspace_bytes(0) == 0           # f32 kernels never split a tile
    n = L.moe_ffn_workspace_bytes(1)
    # two 256 x 256 f32 partial tiles per workgroup (a multiple of 8 workgroups)
    assert n > 0 and n % (2 * 8 * 256 * 256 * 4) == 0, n


def test_binding_raises_typed_errors():
    with pytest.raises(ops.MoEError) as e:
        ops._check(-3)
    assert e.value.status == -3


def test_backward_argument_errors():
    L = ops.lib()
    # moe_combine_backward(dy, y_perm, dest, topk_w, T, k, d, dtype, d_out, d_topk_w, stream)
    cb = [FAKE, FAKE, FAKE, FAKE, 100, 2, 64, 1, FAKE, FAKE, None]

    def comb(i, v):
        a = list(cb); a[i] = v
        return L.moe_combine_backward(*a)
    assert comb(0, None) == -1
    assert comb(9, None) == -1
    assert comb(6, 60) == -6                      # bf16 rows: multiple of 8
    assert comb(7, 3) == -2
    assert comb(5, 9) == -1
    assert comb(4, 0) == 0                        # empty batch: nothing launched
    # moe_expert_down_backward(d_out, offsets, E, rows_max, d, d_ff, w2, z, dtype, dz, ws, wsb, s)
    db = [FAKE, FAKE, 8, 1000, 64, 128, FAKE, FAKE, 1, FAKE, None, 0, None]

    def down(i, v):
        a = list(db); a[i] = v
        return L.moe_expert_down_backward(*a)
    assert down(7, None) == -1                    # the forward's pre-activation is required
    assert down(2, 0) == -3
    a = list(db); a[4] = 1 << 16; a[5] = 1 << 14; a[3] = 8
    assert L.moe_expert_down_backward(*a) == -3   # d * d_ff >= 2^30
    assert down(3, 0) == 0                        # no rows: nothing launched
    assert down(10, FAKE) == -4                   # workspace given but too small
    # moe_expert_up_backward(dz, offsets, E, rows_max, d, d_ff, w1, dtype, dx_perm, ws, wsb, s)
    ub = [FAKE, FAKE, 8, 1000, 64, 128, FAKE, 1, FAKE, None, 0, None]
    a = list(ub); a[8] = None
    assert L.moe_expert_up_backward(*a) == -1
    a = list(ub); a[3] = 1 << 20; a[5] = 1 << 12
    assert L.moe_expert_up_backward(*a) == -3     # rows_max * d_ff >= 2^30
    # moe_expert_weight_grads(x_perm, h, d_out, dz, offsets, E, rows_max, d, d_ff, dtype, dw1, dw2, s)
    wb = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1000, 64, 128, 1, FAKE, FAKE, None]

    def wgr(i, v):
        a = list(wb); a[i] = v
        return L.moe_expert_weight_grads(*a)
    assert wgr(3, None) == -1                     # dW1 needs dz
    assert wgr(1, None) == -1                     # dW2 needs h
    assert wgr(4, None) == -1
    assert wgr(8, 100) == -6
    assert wgr(11, ctypes.c_void_p((1 << 20) + 4)) == -6
    # moe_gate_backward(dw, idx, w, probs, counts, lse, T, E, k, flags, tau, alpha, aux, zc, dl, s)
    gb = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 100, 8, 2, 0, 1.0, 0.01, 1.0, 0.0, FAKE, None]

    def gate(i, v):
        a = list(gb); a[i] = v
        return L.moe_gate_backward(*a)
    assert gate(10, 0.0) == -1                    # temperature
    assert gate(10, float("nan")) == -1
    assert gate(12, float("inf")) == -1           # aux_grad must be finite
    assert gate(13, 0.5) == -1                    # z-loss gradient needs lse
    assert gate(7, 0) == -3
    assert gate(8, 9) == -3
    assert gate(14, None) == -1
    a = list(gb); a[2] = None; a[9] = 1           # renormalised weights need topk_w
    assert L.moe_gate_backward(*a) == -1
    assert gate(6, 0) == 0
    # moe_gate_weight_grads(dl, x, T, d, E, dtype, dwg, db, ws, wsb, s)
    need = L.moe_gate_weight_grads_workspace_bytes(8192, 4096, 8)
    assert need >= 8 * 4096 * 4
    assert L.moe_gate_weight_grads_workspace_bytes(100, 64, 8) < need
    gw = [FAKE, FAKE, 8192, 4096, 8, 1, FAKE, FAKE, FAKE, need, None]

    def gwg(i, v):
        a = list(gw); a[i] = v
        return L.moe_gate_weight_grads(*a)
    assert gwg(9, need - 4) == -4
    assert gwg(8, None) == -4
    assert gwg(6, None) == -1
    assert gwg(3, 4092) == -6
    assert gwg(4, 300) == -3
    # moe_dispatch_backward(dx_perm, dest, dl, w_gate, T, k, d, E, dtype, dx, s)
    dbk = [FAKE, FAKE, FAKE, FAKE, 100, 2, 64, 8, 1, FAKE, None]

    def disp(i, v):
        a = list(dbk); a[i] = v
        return L.moe_dispatch_backward(*a)
    assert disp(2, None) == -1                    # d_logits and w_gate go together
    assert disp(3, None) == -1
    assert disp(9, None) == -1
    assert disp(6, 12) == -6
    assert disp(7, 0) == -3
    assert disp(4, 0) == 0


def test_bench_probe_library_exports_and_argument_checks():
    """libmoe_bench.so (the benchmark's measurement kernels) loads, exports its
    four probes, and rejects bad arguments before any launch."""
    path = os.path.join(os.path.dirname(ops.LIB_PATH), "libmoe_bench.so")
    if not os.path.exists(path):
        pytest.skip("libmoe_bench.so not built")
    L = ctypes.CDLL(path)
    for name in ("probe_stream_read", "probe_clock", "probe_mfma_loop", "probe_mfma_loop16"):
        assert hasattr(L, name), name
    L.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.probe_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.probe_mfma_loop16.argtypes = L.probe_mfma_loop.argtypes
    assert L.probe_stream_read(None, 16, None, 1, None) == -1
    assert L.probe_stream_read(ctypes.c_void_p(16), 15, ctypes.c_void_p(16), 1, None) == -1   # not a multiple of 16
    assert L.probe_stream_read(ctypes.c_void_p(8), 16, ctypes.c_void_p(16), 1, None) == -1    # misaligned
    assert L.probe_clock(None, 10, None) == -1
    assert L.probe_clock(ctypes.c_void_p(16), 0, None) == -1
    assert L.probe_mfma_loop(None, 1, ctypes.c_void_p(16), 1, None) == -1
    assert L.probe_mfma_loop(ctypes.c_void_p(16), 0, ctypes.c_void_p(16), 1, None) == -1
    assert L.probe_mfma_loop(ctypes.c_void_p(16), 1, ctypes.c_void_p(16), 0, None) == -1
    for fn in (L.probe_mfma_loop, L.probe_mfma_loop16):
        assert fn(None, 1, ctypes.c_void_p(16), 1, None) == -1
        assert fn(ctypes.c_void_p(16), 0, ctypes.c_void_p(16), 1, None) == -1
        assert fn(ctypes.c_void_p(16), 1, ctypes.c_void_p(16), 0, None) == -1


def test_router_tiles_and_plan_tiles_argument_errors():
    L = ops.lib()
    assert L.moe_router_tiles(0, 8) == 0 and L.moe_router_tiles(8192, 0) == 0 and L.moe_router_tiles(1, 257) == 0
    assert L.moe_router_tiles(8192, 8) == 512 and L.moe_router_tiles(16384, 64) == 256
    assert L.moe_router_tiles(17, 16) == 2 and L.moe_router_tiles(100, 100) == 7
    p = ctypes.c_void_p(4096)
    # f32: the tile outputs come from the bf16 router only
    assert L.moe_router_topk_tiles(p, p, None, 16, 64, 8, 2, 0, 0, p, p, None, p, None, None) == -2
    assert L.moe_router_topk_tiles(p, p, None, 16, 64, 8, 9, 1, 0, p, p, None, p, None, None) == -3   # k > E
    assert L.moe_router_topk_tiles(p, p, None, 16, 64, 8, 2, 1, 0, p, p, None, None, None, None) == -1   # no counts
    assert L.moe_router_topk_tiles(p, p, None, 16, 64, 8, 2, 1, 0, p, p, None, p, ctypes.c_void_p(4100),
                                   None) == -6   # colsum alignment
    assert L.moe_router_topk_tiles(p, p, None, 0, 64, 8, 2, 1, 0, None, None, None, None, None, None) == 0
    # plan from tiles: colsum and loss go together; too many cells; alignment
    assert L.moe_dispatch_plan_tiles(p, p, p, 16, 2, 8, 4, 0.01, p, p, p, p, None, None) == -1
    assert L.moe_dispatch_plan_tiles(p, p, None, 16, 2, 8, 4, 0.0, p, p, p, p, p, None) == -1
    assert L.moe_dispatch_plan_tiles(p, p, None, 40000, 2, 8, 4, 0.0, p, p, p, p, None, None) == -3
    assert L.moe_dispatch_plan_tiles(p, ctypes.c_void_p(4100), None, 16, 2, 8, 4, 0.0, p, p, p, p, None,
                                     None) == -6
    assert L.moe_dispatch_plan_tiles(p, None, None, 16, 2, 8, 4, 0.0, p, p, p, p, None, None) == -1
