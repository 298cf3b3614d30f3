"""Python binding of libmoe.so: argument marshalling only.

Every function has the name of the C entry point it wraps (include/moe.h),
takes torch tensors that already live on the GPU, allocates missing outputs
with torch (device memory is torch's job here), launches on the current torch
stream and raises MoEError on a non-OK status. No step of the layer runs in
Python: if libmoe.so is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB names another build of the same library (the host-sanitizer build
# libmoe_san.so, for instance); the default is the in-tree libmoe.so.
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_PKG, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_RENORM = 0x1
MOE_MAX_E, MOE_MAX_K = 256, 8
STATUS = {0: "MOE_OK", -1: "MOE_ERR_ARG", -2: "MOE_ERR_DTYPE", -3: "MOE_ERR_SHAPE",
          -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_HIP", -6: "MOE_ERR_ALIGN"}

EXPORTS = ["moe_capacity", "moe_rows_max", "moe_router_topk", "moe_router_topk_ex", "moe_dispatch_workspace_bytes",
           "moe_dispatch", "moe_dispatch_plan", "moe_dispatch_plan_aux",
           "moe_dispatch_plan_aux_workspace_bytes", "moe_dispatch_plan_noalloc",
           "moe_dispatch_plan_noalloc_scratch_bytes", "moe_router_tiles", "moe_router_topk_tiles",
           "moe_dispatch_plan_tiles", "moe_permute", "moe_grouped_ffn", "moe_expert_up_gelu",
           "moe_expert_up_gelu_gather", "moe_expert_down",
           "moe_ffn_workspace_bytes", "moe_frag_rows", "moe_permute_frag", "moe_expert_up_gelu_frag",
           "moe_weights_bf16_to_f16", "moe_expert_down_f16w", "moe_expert_down_frag", "moe_combine", "moe_aux_loss_workspace_bytes", "moe_aux_loss", "moe_z_loss_workspace_bytes",
           "moe_z_loss", "moe_expert_up_gelu_z", "moe_combine_backward", "moe_expert_down_backward",
           "moe_expert_up_backward", "moe_expert_weight_grads", "moe_gate_backward",
           "moe_gate_weight_grads_workspace_bytes", "moe_gate_weight_grads", "moe_dispatch_backward",
           "moe_last_error"]


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, msg))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoe.so is not built (%s); run `python -m "
                           "mixture_experts_layer_49_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U32, F32, F64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_uint32, ctypes.c_float, ctypes.c_double,
                                      ctypes.c_size_t)
    sig = {
        "moe_capacity": (I64, [I64, I32, F64]),
        "moe_rows_max": (I64, [I64, I32, I32, I64]),
        "moe_router_topk": (ctypes.c_int, [P, P, P, I64, I64, I32, I32, I32, U32, P, P, P, P]),
        "moe_router_topk_ex": (ctypes.c_int, [P, P, P, P, I64, I64, I32, I32, I32, U32, F32, P, P, P,
                                              P, P]),
        "moe_z_loss_workspace_bytes": (SZ, [I64]),
        "moe_z_loss": (ctypes.c_int, [P, I64, F32, P, P, SZ, P]),
        "moe_dispatch_workspace_bytes": (SZ, [I64, I32, I32]),
        "moe_dispatch": (ctypes.c_int, [P, I64, I32, I32, I64, P, I64, I32, P, P, P, P, P, P, SZ, P]),
        "moe_dispatch_plan": (ctypes.c_int, [P, I64, I32, I32, I64, P, P, P, P, P, SZ, P]),
        "moe_dispatch_plan_noalloc": (ctypes.c_int, [P, I64, I32, I32, I64, P, P, P, P, P]),
        "moe_dispatch_plan_aux_workspace_bytes": (SZ, [I64, I32, I32]),
        "moe_dispatch_plan_aux": (ctypes.c_int, [P, P, I64, I32, I32, I64, F32, P, P, P, P, P, P, SZ, P]),
        "moe_dispatch_plan_noalloc_scratch_bytes": (SZ, []),
        "moe_router_tiles": (I64, [I64, I32]),
        "moe_router_topk_tiles": (ctypes.c_int, [P, P, P, I64, I64, I32, I32, I32, U32, P, P, P, P, P, P]),
        "moe_dispatch_plan_tiles": (ctypes.c_int, [P, P, P, I64, I32, I32, I64, F32, P, P, P, P, P, P]),
        "moe_permute": (ctypes.c_int, [P, I64, I32, P, P, I32, I64, P, P]),
        "moe_grouped_ffn": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, P, I32, P, P, P, SZ, P]),
        "moe_expert_up_gelu": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, I32, P, P, SZ, P]),
        "moe_expert_up_gelu_gather": (ctypes.c_int, [P, I64, P, P, I32, I64, I64, I64, P, P, P, SZ, P]),
        "moe_expert_down": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, I32, P, P, SZ, P]),
        "moe_ffn_workspace_bytes": (SZ, [I32]),
        "moe_frag_rows": (I64, [I64, I32]),
        "moe_weights_bf16_to_f16": (ctypes.c_int, [P, I64, P, P, P]),
        "moe_expert_down_f16w": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, P, P, SZ, P]),
        "moe_permute_frag": (ctypes.c_int, [P, I64, P, P, I32, I64, P, P]),
        "moe_expert_up_gelu_frag": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, P, I32, P]),
        "moe_expert_down_frag": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, P, P, SZ, P]),
        "moe_combine": (ctypes.c_int, [P, P, P, I64, I32, I64, P, I32, P]),
        "moe_aux_loss_workspace_bytes": (SZ, [I64, I32]),
        "moe_aux_loss": (ctypes.c_int, [P, P, I64, I32, I32, F32, P, P, SZ, P]),
        "moe_expert_up_gelu_z": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, I32, P, P, P, SZ, P]),
        "moe_combine_backward": (ctypes.c_int, [P, P, P, P, I64, I32, I64, I32, P, P, P]),
        "moe_expert_down_backward": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, P, I32, P, P, SZ, P]),
        "moe_expert_up_backward": (ctypes.c_int, [P, P, I32, I64, I64, I64, P, I32, P, P, SZ, P]),
        "moe_expert_weight_grads": (ctypes.c_int, [P, P, P, P, P, I32, I64, I64, I64, I32, P, P, P]),
        "moe_gate_backward": (ctypes.c_int, [P, P, P, P, P, P, I64, I32, I32, U32, F32, F32, F32, F32,
                                             P, P]),
        "moe_gate_weight_grads_workspace_bytes": (SZ, [I64, I64, I32]),
        "moe_gate_weight_grads": (ctypes.c_int, [P, P, I64, I64, I32, I32, P, P, P, SZ, P]),
        "moe_dispatch_backward": (ctypes.c_int, [P, P, P, P, I64, I32, I64, I32, I32, P, P]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise MoEError(rc, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MOE_F32
    if dt == torch.bfloat16:
        return MOE_BF16
    raise MoEError(-2, "unsupported dtype %s" % dt)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def hidden_dtype(dt: torch.dtype) -> torch.dtype:
    """Storage of the FFN hidden activation h: f32 for f32 layers, fp16 for
    bf16 layers (see moe_grouped_ffn in include/moe.h)."""
    return torch.float32 if dt == torch.float32 else torch.float16


def grad_dtype(dt: torch.dtype) -> torch.dtype:
    """Storage of the backward's per-row gradients (d_out_perm, dz): bf16 for
    bf16 layers, f32 for f32 layers (see the backward section of include/moe.h)."""
    return dt


# ------------------------------------------------------------------ calls --
def moe_capacity(n_tokens: int, n_experts: int, capacity_factor: float) -> int:
    return int(lib().moe_capacity(n_tokens, n_experts, capacity_factor))


def moe_rows_max(T: int, k: int, E: int, capacity: int) -> int:
    return int(lib().moe_rows_max(T, k, E, capacity))


def moe_router_topk(x, w_gate, bias, k: int, flags: int = 0, want_probs: bool = True,
                    topk_idx=None, topk_w=None, probs=None, stream=None):
    T, d = x.shape
    E = w_gate.shape[0]
    topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    if want_probs and probs is None:
        probs = _empty((T, E), torch.float32, x)
    _check(lib().moe_router_topk(_ptr(x), _ptr(w_gate), _ptr(bias), T, d, E, k,
                                 dtype_code(x.dtype), flags, _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(probs), _stream(stream)))
    return topk_idx, topk_w, probs


def moe_router_topk_ex(x, w_gate, bias, k: int, flags: int = 0, temperature: float = 1.0,
                       noise=None, want_probs: bool = True, want_lse: bool = True,
                       topk_idx=None, topk_w=None, probs=None, lse=None, stream=None):
    """Router with temperature, a caller-drawn perturbation `noise` [T, E] f32
    and the per-token log-sum-exp `lse` [T] of the scores (see include/moe.h)."""
    T, d = x.shape
    E = w_gate.shape[0]
    topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    if want_probs and probs is None:
        probs = _empty((T, E), torch.float32, x)
    if want_lse and lse is None:
        lse = _empty((max(T, 1),), torch.float32, x)
    _check(lib().moe_router_topk_ex(_ptr(x), _ptr(w_gate), _ptr(bias), _ptr(noise), T, d, E, k,
                                    dtype_code(x.dtype), flags, float(temperature),
                                    _ptr(topk_idx), _ptr(topk_w), _ptr(probs), _ptr(lse),
                                    _stream(stream)))
    return topk_idx, topk_w, probs, lse


def moe_z_loss_workspace_bytes(T: int) -> int:
    return int(lib().moe_z_loss_workspace_bytes(T))


def moe_z_loss(lse, T: int, coeff: float, loss=None, workspace=None, stream=None):
    """coeff * mean over tokens of lse^2."""
    loss = _empty((1,), torch.float32, lse) if loss is None else loss
    if workspace is None:
        workspace = _empty((max(moe_z_loss_workspace_bytes(T), 8),), torch.uint8, lse)
    _check(lib().moe_z_loss(_ptr(lse), T, float(coeff), _ptr(loss), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)))
    return loss


def moe_dispatch_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().moe_dispatch_workspace_bytes(T, k, E))


def moe_dispatch(topk_idx, E: int, capacity: int, x, counts=None, offsets=None, dest=None,
                 src=None, x_perm=None, workspace=None, stream=None):
    T, k = topk_idx.shape
    d = x.shape[1]
    rows = moe_rows_max(T, k, E, capacity)
    counts = _empty((E,), torch.int32, x) if counts is None else counts
    offsets = _empty((E + 1,), torch.int32, x) if offsets is None else offsets
    dest = _empty((T, k), torch.int32, x) if dest is None else dest
    src = _empty((max(rows, 1),), torch.int32, x) if src is None else src
    x_perm = _empty((max(rows, 1), d), x.dtype, x) if x_perm is None else x_perm
    if workspace is None:
        workspace = _empty((max(moe_dispatch_workspace_bytes(T, k, E), 4),), torch.uint8, x)
    _check(lib().moe_dispatch(_ptr(topk_idx), T, k, E, capacity, _ptr(x), d, dtype_code(x.dtype),
                              _ptr(counts), _ptr(offsets), _ptr(dest), _ptr(src), _ptr(x_perm),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)))
    return counts, offsets, dest, src, x_perm


def moe_dispatch_plan(topk_idx, E: int, capacity: int, counts=None, offsets=None, dest=None,
                      src=None, workspace=None, stream=None):
    T, k = topk_idx.shape
    rows = moe_rows_max(T, k, E, capacity)
    counts = _empty((E,), torch.int32, topk_idx) if counts is None else counts
    offsets = _empty((E + 1,), torch.int32, topk_idx) if offsets is None else offsets
    dest = _empty((T, k), torch.int32, topk_idx) if dest is None else dest
    src = _empty((max(rows, 1),), torch.int32, topk_idx) if src is None else src
    if workspace is None:
        workspace = _empty((max(moe_dispatch_workspace_bytes(T, k, E), 4),), torch.uint8, topk_idx)
    _check(lib().moe_dispatch_plan(_ptr(topk_idx), T, k, E, capacity, _ptr(counts), _ptr(offsets),
                                   _ptr(dest), _ptr(src), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return counts, offsets, dest, src


def moe_dispatch_plan_aux_workspace_bytes(T: int, k: int, E: int) -> int:
    return lib().moe_dispatch_plan_aux_workspace_bytes(T, k, E)


def moe_dispatch_plan_aux(topk_idx, probs, E: int, capacity: int, alpha: float, counts=None,
                          offsets=None, dest=None, src=None, loss=None, workspace=None, stream=None):
    """moe_dispatch_plan and moe_aux_loss in one pass; returns counts,
    offsets, dest, src, loss."""
    T, k = topk_idx.shape
    rows = moe_rows_max(T, k, E, capacity)
    counts = _empty((E,), torch.int32, topk_idx) if counts is None else counts
    offsets = _empty((E + 1,), torch.int32, topk_idx) if offsets is None else offsets
    dest = _empty((T, k), torch.int32, topk_idx) if dest is None else dest
    src = _empty((max(rows, 1),), torch.int32, topk_idx) if src is None else src
    loss = _empty((1,), torch.float32, topk_idx) if loss is None else loss
    if workspace is None:
        workspace = _empty((max(moe_dispatch_plan_aux_workspace_bytes(T, k, E), 8),), torch.uint8, topk_idx)
    _check(lib().moe_dispatch_plan_aux(_ptr(topk_idx), _ptr(probs), T, k, E, capacity, alpha,
                                       _ptr(counts), _ptr(offsets), _ptr(dest), _ptr(src), _ptr(loss),
                                       _ptr(workspace), _ws_size(workspace), _stream(stream)))
    return counts, offsets, dest, src, loss


def moe_router_tiles(T: int, E: int) -> int:
    return lib().moe_router_tiles(T, E)


def moe_router_topk_tiles(x, w_gate, bias, k: int, flags: int = 0, want_probs: bool = True,
                          want_colsum: bool = True, topk_idx=None, topk_w=None, probs=None,
                          tile_counts=None, tile_colsum=None, stream=None):
    """The bf16 router that also counts each token tile's choices per expert
    (and sums its softmax columns in double); returns topk_idx, topk_w, probs,
    tile_counts, tile_colsum."""
    T, d = x.shape
    E = w_gate.shape[0]
    n = max(moe_router_tiles(T, E), 1)
    topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    if want_probs and probs is None:
        probs = _empty((T, E), torch.float32, x)
    tile_counts = _empty((n, E), torch.int32, x) if tile_counts is None else tile_counts
    if want_colsum and tile_colsum is None:
        tile_colsum = _empty((n, E), torch.float64, x)
    _check(lib().moe_router_topk_tiles(_ptr(x), _ptr(w_gate), _ptr(bias), T, d, E, k, dtype_code(x.dtype), flags,
                                       _ptr(topk_idx), _ptr(topk_w), _ptr(probs), _ptr(tile_counts),
                                       _ptr(tile_colsum), _stream(stream)))
    return topk_idx, topk_w, probs, tile_counts, tile_colsum


def moe_dispatch_plan_tiles(topk_idx, tile_counts, tile_colsum, E: int, capacity: int, alpha: float = 0.0,
                            counts=None, offsets=None, dest=None, src=None, loss=None, stream=None):
    """moe_dispatch_plan (and, with tile_colsum, the aux loss) from the
    router's per-tile counts; returns counts, offsets, dest, src, loss."""
    T, k = topk_idx.shape
    rows = moe_rows_max(T, k, E, capacity)
    counts = _empty((E,), torch.int32, topk_idx) if counts is None else counts
    offsets = _empty((E + 1,), torch.int32, topk_idx) if offsets is None else offsets
    dest = _empty((T, k), torch.int32, topk_idx) if dest is None else dest
    src = _empty((max(rows, 1),), torch.int32, topk_idx) if src is None else src
    if tile_colsum is not None and loss is None:
        loss = _empty((1,), torch.float32, topk_idx)
    _check(lib().moe_dispatch_plan_tiles(_ptr(topk_idx), _ptr(tile_counts), _ptr(tile_colsum), T, k, E, capacity,
                                         alpha, _ptr(counts), _ptr(offsets), _ptr(dest), _ptr(src),
                                         _ptr(loss if tile_colsum is not None else None), _stream(stream)))
    return counts, offsets, dest, src, (loss if tile_colsum is not None else None)


def tiles_eligible(dtype, T: int, E: int) -> bool:
    """Whether the router can hand the dispatch plan its per-tile counts:
    bf16 and at most 16384 (tile, expert) count cells."""
    return dtype == torch.bfloat16 and moe_router_tiles(T, E) * E <= 16384


def moe_dispatch_plan_noalloc(topk_idx, E: int, capacity: int, counts, offsets, dest, src,
                              stream=None):
    """moe_dispatch_plan on the library's own scratch: every output buffer is
    the caller's and nothing is allocated here or in the library."""
    T, k = topk_idx.shape
    _check(lib().moe_dispatch_plan_noalloc(_ptr(topk_idx), T, k, E, capacity, _ptr(counts),
                                           _ptr(offsets), _ptr(dest), _ptr(src), _stream(stream)))
    return counts, offsets, dest, src


def moe_dispatch_plan_noalloc_scratch_bytes() -> int:
    return lib().moe_dispatch_plan_noalloc_scratch_bytes()


def moe_permute(x, src, offsets, rows_max: int, x_perm=None, stream=None):
    d = x.shape[1]
    E = offsets.numel() - 1
    x_perm = _empty((max(rows_max, 1), d), x.dtype, x) if x_perm is None else x_perm
    _check(lib().moe_permute(_ptr(x), d, dtype_code(x.dtype), _ptr(src), _ptr(offsets), E, rows_max,
                             _ptr(x_perm), _stream(stream)))
    return x_perm


def moe_ffn_workspace_bytes(dtype) -> int:
    return int(lib().moe_ffn_workspace_bytes(dtype_code(dtype)))


def _ws_size(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def moe_expert_up_gelu(x_perm, offsets, w1, rows_max: int, h=None, workspace=None, stream=None):
    """workspace: a device buffer of moe_ffn_workspace_bytes(dtype) bytes, or
    None (then no output tile is split along K)."""
    E, d_ff, d = w1.shape
    h = _empty((max(rows_max, 1), d_ff), hidden_dtype(w1.dtype), x_perm) if h is None else h
    _check(lib().moe_expert_up_gelu(_ptr(x_perm), _ptr(offsets), E, rows_max, d, d_ff, _ptr(w1),
                                    dtype_code(w1.dtype), _ptr(h), _ptr(workspace),
                                    _ws_size(workspace), _stream(stream)))
    return h


def moe_expert_up_gelu_gather(x, src, offsets, w1, rows_max: int, h=None, workspace=None, stream=None):
    """moe_permute then moe_expert_up_gelu in one kernel (bf16): the
    up-projection reads row r as x[src[r]]."""
    T, d = x.shape
    E, d_ff, _ = w1.shape
    h = _empty((max(rows_max, 1), d_ff), hidden_dtype(w1.dtype), x) if h is None else h
    _check(lib().moe_expert_up_gelu_gather(_ptr(x), T, _ptr(src), _ptr(offsets), E, rows_max, d, d_ff,
                                           _ptr(w1), _ptr(h), _ptr(workspace), _ws_size(workspace),
                                           _stream(stream)))
    return h


def moe_expert_down(h, offsets, w2, rows_max: int, y_perm=None, workspace=None, stream=None):
    E, d, d_ff = w2.shape
    y_perm = _empty((max(rows_max, 1), d), torch.float32, h) if y_perm is None else y_perm
    _check(lib().moe_expert_down(_ptr(h), _ptr(offsets), E, rows_max, d, d_ff, _ptr(w2),
                                 dtype_code(w2.dtype), _ptr(y_perm), _ptr(workspace),
                                 _ws_size(workspace), _stream(stream)))
    return y_perm


def moe_frag_rows(rows_max: int, E: int) -> int:
    """Rows to allocate for the fragment-ordered copy of x_perm."""
    return int(lib().moe_frag_rows(rows_max, E))


def frag_eligible(dtype, d: int) -> bool:
    """Whether moe_forward takes the fragment-ordered path for this layer:
    bf16, d a multiple of 256 and at least 4096. Measured on the workloads,
    whole forward with fp16 W2, against the row-major path that folds the
    permute into the up-projection: -9% at d = 4096 (8 experts, also the
    receiver share and the ETP share; more since the fragment GEMM moved to
    16x16x32 MFMAs), +2% at d = 2048 (64 experts: the fragment-order permute
    pass costs more than the GEMMs gain), -1.7% at d = 1024 (16 experts,
    within the spread between boxes; left on the row-major path)."""
    return dtype == torch.bfloat16 and d % 256 == 0 and d >= 4096


def moe_permute_frag(x, src, offsets, rows_max: int, x_frag=None, stream=None):
    """x_perm rows in matrix-core fragment order, expert segments padded to
    multiples of 32 rows (bf16)."""
    d = x.shape[1]
    E = offsets.numel() - 1
    if x_frag is None:
        x_frag = _empty((max(moe_frag_rows(rows_max, E), 1), d), x.dtype, x)
    _check(lib().moe_permute_frag(_ptr(x), d, _ptr(src), _ptr(offsets), E, rows_max, _ptr(x_frag),
                                  _stream(stream)))
    return x_frag


MOE_ORDER_ROWS, MOE_ORDER_FRAG = 0, 1


def moe_expert_up_gelu_frag(x_frag, offsets, w1, rows_max: int, h=None, frag_out: bool = False,
                            stream=None):
    """moe_expert_up_gelu (without a workspace) from the fragment-ordered copy;
    h row-major [rows_max, d_ff], or with frag_out in fragment order
    [moe_frag_rows(rows_max, E), d_ff] (what moe_expert_down_frag reads)."""
    E, d_ff, d = w1.shape
    if h is None:
        rows = moe_frag_rows(rows_max, E) if frag_out else rows_max
        h = _empty((max(rows, 1), d_ff), hidden_dtype(w1.dtype), x_frag)
    _check(lib().moe_expert_up_gelu_frag(_ptr(x_frag), _ptr(offsets), E, rows_max, d, d_ff, _ptr(w1),
                                         _ptr(h), MOE_ORDER_FRAG if frag_out else MOE_ORDER_ROWS,
                                         _stream(stream)))
    return h


def moe_expert_down_frag(h_frag, offsets, w2_f16, rows_max: int, y_perm=None, workspace=None,
                         stream=None):
    """Down-projection from fragment-ordered h on W2 in fp16."""
    E, d, d_ff = w2_f16.shape
    y_perm = _empty((max(rows_max, 1), d), torch.float32, h_frag) if y_perm is None else y_perm
    _check(lib().moe_expert_down_frag(_ptr(h_frag), _ptr(offsets), E, rows_max, d, d_ff, _ptr(w2_f16),
                                      _ptr(y_perm), _ptr(workspace), _ws_size(workspace),
                                      _stream(stream)))
    return y_perm


def moe_weights_bf16_to_f16(w, out=None, report=None, stream=None):
    """fp16 copy of a bf16 weight (round to nearest even), for the
    down-projection's fp16 products. `report`: an int64 device tensor of two
    elements to receive the counts of values that lost bits and of values
    that became +-inf."""
    out = torch.empty(w.shape, dtype=torch.float16, device=w.device) if out is None else out
    if report is not None and (report.dtype != torch.int64 or report.numel() < 2):
        raise MoEError(-1, "report must be an int64 tensor of two elements")
    _check(lib().moe_weights_bf16_to_f16(_ptr(w), w.numel(), _ptr(out), _ptr(report),
                                         _stream(stream)))
    return out


def moe_expert_down_f16w(h, offsets, w2_f16, rows_max: int, y_perm=None, workspace=None, stream=None):
    """moe_expert_down of a bf16 layer with W2 given as moe_weights_bf16_to_f16(W2)."""
    E, d, d_ff = w2_f16.shape
    y_perm = _empty((max(rows_max, 1), d), torch.float32, h) if y_perm is None else y_perm
    _check(lib().moe_expert_down_f16w(_ptr(h), _ptr(offsets), E, rows_max, d, d_ff, _ptr(w2_f16),
                                      _ptr(y_perm), _ptr(workspace), _ws_size(workspace), _stream(stream)))
    return y_perm


def moe_grouped_ffn(x_perm, offsets, w1, w2, rows_max: int, h=None, y_perm=None, workspace=None,
                    stream=None):
    E, d_ff, d = w1.shape
    h = _empty((max(rows_max, 1), d_ff), hidden_dtype(w1.dtype), x_perm) if h is None else h
    y_perm = _empty((max(rows_max, 1), d), torch.float32, x_perm) if y_perm is None else y_perm
    _check(lib().moe_grouped_ffn(_ptr(x_perm), _ptr(offsets), E, rows_max, d, d_ff, _ptr(w1),
                                 _ptr(w2), dtype_code(x_perm.dtype), _ptr(h), _ptr(y_perm),
                                 _ptr(workspace), _ws_size(workspace), _stream(stream)))
    return h, y_perm


def moe_combine(y_perm, dest, topk_w, d: int, out_dtype=torch.float32, y=None, stream=None):
    T, k = dest.shape
    y = _empty((T, d), out_dtype, dest) if y is None else y
    _check(lib().moe_combine(_ptr(y_perm), _ptr(dest), _ptr(topk_w), T, k, d, _ptr(y),
                             dtype_code(y.dtype), _stream(stream)))
    return y


def moe_aux_loss_workspace_bytes(T: int, E: int) -> int:
    return int(lib().moe_aux_loss_workspace_bytes(T, E))


def moe_aux_loss(probs, counts, k: int, alpha: float, loss=None, workspace=None, stream=None):
    T, E = probs.shape
    loss = _empty((1,), torch.float32, probs) if loss is None else loss
    if workspace is None:
        workspace = _empty((max(moe_aux_loss_workspace_bytes(T, E), 8),), torch.uint8, probs)
    _check(lib().moe_aux_loss(_ptr(probs), _ptr(counts), T, E, k, alpha, _ptr(loss),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)))
    return loss


# --------------------------------------------------------------- backward --
def moe_expert_up_gelu_z(x_perm, offsets, w1, rows_max: int, h=None, z=None, workspace=None,
                         stream=None):
    """Up-projection + GELU that also keeps the pre-activation z."""
    E, d_ff, d = w1.shape
    hd = hidden_dtype(x_perm.dtype)
    h = _empty((max(rows_max, 1), d_ff), hd, x_perm) if h is None else h
    z = _empty((max(rows_max, 1), d_ff), hd, x_perm) if z is None else z
    _check(lib().moe_expert_up_gelu_z(_ptr(x_perm), _ptr(offsets), E, rows_max, d, d_ff, _ptr(w1),
                                      dtype_code(x_perm.dtype), _ptr(h), _ptr(z), _ptr(workspace),
                                      _ws_size(workspace), _stream(stream)))
    return h, z


def moe_combine_backward(dy, y_perm, dest, topk_w, dtype, rows_max: int, d_out_perm=None,
                         d_topk_w=None, stream=None):
    """d_out_perm [rows, d] in the gradient storage of `dtype`, d_topk_w [T, k] f32."""
    T, k = dest.shape
    d = dy.shape[1]
    d_out_perm = (_empty((max(rows_max, 1), d), grad_dtype(dtype), dy) if d_out_perm is None
                  else d_out_perm)
    d_topk_w = _empty((T, k), torch.float32, dy) if d_topk_w is None else d_topk_w
    _check(lib().moe_combine_backward(_ptr(dy), _ptr(y_perm), _ptr(dest), _ptr(topk_w), T, k, d,
                                      dtype_code(dtype), _ptr(d_out_perm), _ptr(d_topk_w),
                                      _stream(stream)))
    return d_out_perm, d_topk_w


def moe_expert_down_backward(d_out_perm, offsets, w2, z, rows_max: int, dz=None, workspace=None,
                             stream=None):
    E, d, d_ff = w2.shape
    dz = _empty((max(rows_max, 1), d_ff), d_out_perm.dtype, d_out_perm) if dz is None else dz
    _check(lib().moe_expert_down_backward(_ptr(d_out_perm), _ptr(offsets), E, rows_max, d, d_ff,
                                          _ptr(w2), _ptr(z), dtype_code(w2.dtype), _ptr(dz),
                                          _ptr(workspace), _ws_size(workspace), _stream(stream)))
    return dz


def moe_expert_up_backward(dz, offsets, w1, rows_max: int, dx_perm=None, workspace=None,
                           stream=None):
    E, d_ff, d = w1.shape
    dx_perm = _empty((max(rows_max, 1), d), torch.float32, dz) if dx_perm is None else dx_perm
    _check(lib().moe_expert_up_backward(_ptr(dz), _ptr(offsets), E, rows_max, d, d_ff, _ptr(w1),
                                        dtype_code(w1.dtype), _ptr(dx_perm), _ptr(workspace),
                                        _ws_size(workspace), _stream(stream)))
    return dx_perm


def moe_expert_weight_grads(x_perm, h, d_out_perm, dz, offsets, E: int, rows_max: int, d: int,
                            d_ff: int, dtype, dw1=None, dw2=None, want_dw1=True, want_dw2=True,
                            stream=None):
    like = x_perm if x_perm is not None else d_out_perm
    if want_dw1 and dw1 is None:
        dw1 = _empty((E, d_ff, d), torch.float32, like)
    if want_dw2 and dw2 is None:
        dw2 = _empty((E, d, d_ff), torch.float32, like)
    _check(lib().moe_expert_weight_grads(_ptr(x_perm), _ptr(h), _ptr(d_out_perm), _ptr(dz),
                                         _ptr(offsets), E, rows_max, d, d_ff, dtype_code(dtype),
                                         _ptr(dw1 if want_dw1 else None),
                                         _ptr(dw2 if want_dw2 else None), _stream(stream)))
    return dw1, dw2


def moe_gate_backward(d_topk_w, topk_idx, topk_w, probs, counts, k: int, alpha: float,
                      aux_grad: float = 1.0, flags: int = 0, temperature: float = 1.0,
                      lse=None, z_coeff: float = 0.0, d_logits=None, stream=None):
    T, E = probs.shape
    d_logits = _empty((T, E), torch.float32, probs) if d_logits is None else d_logits
    _check(lib().moe_gate_backward(_ptr(d_topk_w), _ptr(topk_idx), _ptr(topk_w), _ptr(probs),
                                   _ptr(counts), _ptr(lse), T, E, k, flags, float(temperature),
                                   float(alpha), float(aux_grad), float(z_coeff), _ptr(d_logits),
                                   _stream(stream)))
    return d_logits


def moe_gate_weight_grads_workspace_bytes(T: int, d: int, E: int) -> int:
    return int(lib().moe_gate_weight_grads_workspace_bytes(T, d, E))


def moe_gate_weight_grads(d_logits, x, E: int, d_w_gate=None, d_bias=None, want_bias=True,
                          workspace=None, stream=None):
    T, d = x.shape
    d_w_gate = _empty((E, d), torch.float32, x) if d_w_gate is None else d_w_gate
    if want_bias and d_bias is None:
        d_bias = _empty((E,), torch.float32, x)
    if workspace is None:
        workspace = _empty((max(moe_gate_weight_grads_workspace_bytes(T, d, E), 16),), torch.uint8, x)
    _check(lib().moe_gate_weight_grads(_ptr(d_logits), _ptr(x), T, d, E, dtype_code(x.dtype),
                                       _ptr(d_w_gate), _ptr(d_bias if want_bias else None),
                                       _ptr(workspace), _ws_size(workspace), _stream(stream)))
    return d_w_gate, d_bias


def moe_dispatch_backward(dx_perm, dest, d, dtype, d_logits=None, w_gate=None, dx=None,
                          stream=None):
    T, k = dest.shape
    E = w_gate.shape[0] if w_gate is not None else 1
    dx = _empty((T, d), torch.float32, dest) if dx is None else dx
    _check(lib().moe_dispatch_backward(_ptr(dx_perm), _ptr(dest), _ptr(d_logits), _ptr(w_gate), T,
                                       k, d, E, dtype_code(dtype), _ptr(dx), _stream(stream)))
    return dx


# ------------------------------------------------------------ whole layer --
class MoEBuffers:
    """Every intermediate of one layer forward, allocated once for a shape so
    repeated forwards allocate nothing."""

    def __init__(self, T, d, d_ff, E, k, capacity, dtype, device, routed=True, want_probs=True,
                 save_for_backward=False, frag=None, w2_f16=False, gather=None):
        z = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)
        self.T, self.d, self.d_ff, self.E, self.k, self.capacity = T, d, d_ff, E, k, capacity
        self.rows_max = moe_rows_max(T, k, E, capacity)
        R = max(self.rows_max, 1)
        self.topk_idx = z((T, k), torch.int32)
        self.topk_w = z((T, k), torch.float32)
        self.probs = z((T, E), torch.float32) if (routed and want_probs) else None
        self.counts = z((E,), torch.int32)
        self.offsets = z((E + 1,), torch.int32)
        self.dest = z((T, k), torch.int32)
        self.src = z((R,), torch.int32)
        # bf16 forward without a backward: the permuted rows in fragment order
        # (x_frag) instead of row-major (x_perm); frag=None picks it when eligible
        if frag is None:
            frag = frag_eligible(dtype, d) and not save_for_backward
        if frag and (save_for_backward or dtype != torch.bfloat16 or d % 256 != 0):
            raise ValueError("the fragment-ordered path needs bf16, d % 256 == 0 and no backward")
        self.frag = bool(frag)
        # the row-major bf16 forward without a backward reads x through src in
        # the up-projection (moe_expert_up_gelu_gather): x_perm is not stored
        if gather is None:
            gather = not self.frag and dtype == torch.bfloat16 and not save_for_backward
        if gather and (self.frag or save_for_backward or dtype != torch.bfloat16):
            raise ValueError("the gathered up-projection needs the row-major bf16 path and no backward")
        self.gather = bool(gather)
        self.x_perm = None if (self.frag or self.gather) else z((R, d), dtype)
        self.x_frag = z((max(moe_frag_rows(self.rows_max, E), 1), d), dtype) if self.frag else None
        # forwards that will pass W2 in fp16 (w2_f16) on the fragment-ordered
        # path keep h in fragment order too when d_ff % 256 == 0: only that
        # buffer is allocated, the row-major h is not
        self.h_frag = (z((max(moe_frag_rows(self.rows_max, E), 1), d_ff), torch.float16)
                       if self.frag and w2_f16 and d_ff % 256 == 0 else None)
        self.h = z((R, d_ff), hidden_dtype(dtype)) if self.h_frag is None else None
        # the pre-activation, kept for the backward
        self.z = z((R, d_ff), hidden_dtype(dtype)) if save_for_backward else None
        self.lse = z((max(T, 1),), torch.float32) if (routed and save_for_backward) else None
        self.y_perm = z((R, d), torch.float32)
        self.y = z((T, d), torch.float32)
        self.loss = z((1,), torch.float32)
        self.ws_dispatch = z((max(moe_dispatch_workspace_bytes(T, k, E), 4),), torch.uint8)
        # the plan with the aux loss folded in (routed layers with probabilities)
        self.ws_plan_aux = (z((max(moe_dispatch_plan_aux_workspace_bytes(T, k, E), 8),), torch.uint8)
                            if self.probs is not None else None)
        self.ws_aux = z((max(moe_aux_loss_workspace_bytes(T, E), 8),), torch.uint8)
        # the router's per-tile counts (and column sums) for the plan that
        # needs no histogram pass (bf16, few enough tile x expert cells)
        nt = max(moe_router_tiles(T, E), 1)
        self.tiles = routed and tiles_eligible(dtype, T, E)
        self.tile_counts = z((nt, E), torch.int32) if self.tiles else None
        self.tile_colsum = z((nt, E), torch.float64) if (self.tiles and self.probs is not None) else None
        self.used_idx, self.used_w = self.topk_idx, self.topk_w
        nb = moe_ffn_workspace_bytes(dtype)
        self.ws_ffn = z((nb,), torch.uint8) if nb > 0 else None


def moe_forward(x, w1, w2, k: int, capacity: int, w_gate=None, bias=None, topk_idx=None,
                topk_w=None, alpha: float = 0.01, flags: int = 0, bufs: MoEBuffers = None,
                stream=None, save_for_backward: bool = False, temperature: float = 1.0,
                noise=None, w2_f16=None) -> MoEBuffers:
    """router -> dispatch -> grouped FFN -> combine -> aux loss, all on one
    stream. With `w_gate` None, `topk_idx`/`topk_w` are taken as given (a
    receiver's share: the rows it got and their weights). With
    `save_for_backward` the up-projection also keeps the pre-activation and
    the router its log-sum-exp (what moe_backward needs). Without a backward,
    bf16 layers that frag_eligible() accepts run the permute and the
    up-projection on the fragment-ordered copy (bufs.frag; 16x16x32 MFMAs:
    h equal to the row-major up-projection's without a workspace up to
    float32 summation order, bit for bit on every shape tested), and the other
    bf16 layers fold the permute into the up-projection (bufs.gather: the
    same h bit for bit, x_perm not stored). `w2_f16`, for
    bf16 layers: moe_weights_bf16_to_f16(w2), prepared once; the
    down-projection then reads it instead of converting W2 in registers
    (y_perm bit for bit the same on the row-major kernel), and on the fragment-ordered path with
    d_ff % 256 == 0 and buffers made with w2_f16=True, h stays in fragment
    order (bufs.h_frag) for a down-projection that loads it straight into
    registers (bufs.h is then not allocated). Nothing here allocates when
    `bufs` is given."""
    T, d = x.shape
    E, d_ff, _ = w1.shape
    routed = w_gate is not None
    if bufs is None:
        bufs = MoEBuffers(T, d, d_ff, E, k, capacity, x.dtype, x.device, routed,
                          save_for_backward=save_for_backward, w2_f16=w2_f16 is not None)
    # the plain bf16 router can count its tiles' choices for the plan
    tiles = (routed and bufs.tiles and temperature == 1.0 and noise is None and bufs.lse is None)
    if routed:
        if temperature != 1.0 or noise is not None or bufs.lse is not None:
            moe_router_topk_ex(x, w_gate, bias, k, flags, temperature, noise,
                               bufs.probs is not None, bufs.lse is not None, bufs.topk_idx,
                               bufs.topk_w, bufs.probs, bufs.lse, stream)
        elif tiles:
            moe_router_topk_tiles(x, w_gate, bias, k, flags, bufs.probs is not None, bufs.tile_colsum is not None,
                                  bufs.topk_idx, bufs.topk_w, bufs.probs, bufs.tile_counts, bufs.tile_colsum,
                                  stream)
        else:
            moe_router_topk(x, w_gate, bias, k, flags, bufs.probs is not None, bufs.topk_idx,
                            bufs.topk_w, bufs.probs, stream)
        idx, w = bufs.topk_idx, bufs.topk_w
    else:
        idx, w = topk_idx, topk_w
    bufs.used_idx, bufs.used_w = idx, w   # the routing the layer ran with (given or computed)
    if w2_f16 is not None and x.dtype != torch.bfloat16:
        raise ValueError("w2_f16 is for bf16 layers")

    def down():
        if w2_f16 is not None:
            moe_expert_down_f16w(bufs.h, bufs.offsets, w2_f16, bufs.rows_max, bufs.y_perm,
                                 bufs.ws_ffn, stream)
        else:
            moe_expert_down(bufs.h, bufs.offsets, w2, bufs.rows_max, bufs.y_perm, bufs.ws_ffn,
                            stream)

    # the dispatch plan, with the aux loss folded in where the router's
    # probabilities are kept
    aux_done = routed and bufs.probs is not None and (bufs.ws_plan_aux is not None or tiles)
    if tiles:
        moe_dispatch_plan_tiles(idx, bufs.tile_counts, bufs.tile_colsum, E, capacity, alpha, bufs.counts,
                                bufs.offsets, bufs.dest, bufs.src, bufs.loss if bufs.tile_colsum is not None
                                else None, stream)
    elif aux_done:
        moe_dispatch_plan_aux(idx, bufs.probs, E, capacity, alpha, bufs.counts, bufs.offsets, bufs.dest,
                              bufs.src, bufs.loss, bufs.ws_plan_aux, stream)
    else:
        moe_dispatch_plan(idx, E, capacity, bufs.counts, bufs.offsets, bufs.dest, bufs.src,
                          bufs.ws_dispatch, stream)
    if bufs.frag:
        moe_permute_frag(x, bufs.src, bufs.offsets, bufs.rows_max, bufs.x_frag, stream)
        if w2_f16 is not None and bufs.h_frag is not None:
            # h stays in fragment order between the two projections
            moe_expert_up_gelu_frag(bufs.x_frag, bufs.offsets, w1, bufs.rows_max, bufs.h_frag, True,
                                    stream)
            moe_expert_down_frag(bufs.h_frag, bufs.offsets, w2_f16, bufs.rows_max, bufs.y_perm,
                                 bufs.ws_ffn, stream)
        else:
            if bufs.h is None:
                raise MoEError(-1, "these buffers keep h in fragment order: pass w2_f16")
            moe_expert_up_gelu_frag(bufs.x_frag, bufs.offsets, w1, bufs.rows_max, bufs.h, False, stream)
            down()
    elif bufs.gather:
        # the permute happens inside the up-projection's loads
        moe_expert_up_gelu_gather(x, bufs.src, bufs.offsets, w1, bufs.rows_max, bufs.h, bufs.ws_ffn, stream)
        down()
    else:
        moe_permute(x, bufs.src, bufs.offsets, bufs.rows_max, bufs.x_perm, stream)
        if bufs.z is not None:
            moe_expert_up_gelu_z(bufs.x_perm, bufs.offsets, w1, bufs.rows_max, bufs.h, bufs.z,
                                 bufs.ws_ffn, stream)
            down()
        elif w2_f16 is not None:
            moe_expert_up_gelu(bufs.x_perm, bufs.offsets, w1, bufs.rows_max, bufs.h, bufs.ws_ffn,
                               stream)
            down()
        else:
            moe_grouped_ffn(bufs.x_perm, bufs.offsets, w1, w2, bufs.rows_max, bufs.h, bufs.y_perm,
                            bufs.ws_ffn, stream)
    moe_combine(bufs.y_perm, bufs.dest, w, d, torch.float32, bufs.y, stream)
    if routed and bufs.probs is not None and not aux_done:
        moe_aux_loss(bufs.probs, bufs.counts, k, alpha, bufs.loss, bufs.ws_aux, stream)
    return bufs


class MoEGrads:
    """Every intermediate and result of one layer backward, allocated once."""

    def __init__(self, T, d, d_ff, E, k, rows_max, dtype, device, routed=True):
        z = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)
        R = max(rows_max, 1)
        self.d_out_perm = z((R, d), grad_dtype(dtype))
        self.d_topk_w = z((T, k), torch.float32)
        self.dz = z((R, d_ff), grad_dtype(dtype))
        self.dx_perm = z((R, d), torch.float32)
        self.dw1 = z((E, d_ff, d), torch.float32)
        self.dw2 = z((E, d, d_ff), torch.float32)
        self.dx = z((T, d), torch.float32)
        self.d_logits = z((T, E), torch.float32) if routed else None
        self.dw_gate = z((E, d), torch.float32) if routed else None
        self.d_bias = z((E,), torch.float32) if routed else None
        self.ws_gate = (z((max(moe_gate_weight_grads_workspace_bytes(T, d, E), 16),), torch.uint8)
                        if routed else None)


def moe_backward(x, w1, w2, k: int, bufs: MoEBuffers, dy, w_gate=None, alpha: float = 0.01,
                 aux_grad: float = 1.0, flags: int = 0, temperature: float = 1.0,
                 z_coeff: float = 0.0, grads: MoEGrads = None, stream=None) -> MoEGrads:
    """Gradients of <dy, y> + aux_grad * L_aux + z_coeff * mean(lse^2) for a
    forward run with save_for_backward: combine^T, down-projection and GELU
    backward, up-projection backward, expert weight gradients, gate backward,
    gate weight gradients, dispatch^T; all on one stream."""
    T, d = x.shape
    E, d_ff, _ = w1.shape
    routed = w_gate is not None
    if bufs.z is None:
        raise MoEError(-1, "the forward did not keep the pre-activation (save_for_backward)")
    if grads is None:
        grads = MoEGrads(T, d, d_ff, E, k, bufs.rows_max, x.dtype, x.device, routed)
    R = bufs.rows_max
    moe_combine_backward(dy, bufs.y_perm, bufs.dest, bufs.used_w, x.dtype, R, grads.d_out_perm,
                         grads.d_topk_w, stream)
    moe_expert_down_backward(grads.d_out_perm, bufs.offsets, w2, bufs.z, R, grads.dz, bufs.ws_ffn,
                             stream)
    moe_expert_up_backward(grads.dz, bufs.offsets, w1, R, grads.dx_perm, bufs.ws_ffn, stream)
    moe_expert_weight_grads(bufs.x_perm, bufs.h, grads.d_out_perm, grads.dz, bufs.offsets, E, R, d,
                            d_ff, x.dtype, grads.dw1, grads.dw2, stream=stream)
    if routed:
        moe_gate_backward(grads.d_topk_w, bufs.topk_idx, bufs.topk_w, bufs.probs, bufs.counts, k,
                          alpha, aux_grad, flags, temperature, bufs.lse, z_coeff, grads.d_logits,
                          stream)
        moe_gate_weight_grads(grads.d_logits, x, E, grads.dw_gate, grads.d_bias, True,
                              grads.ws_gate, stream)
    moe_dispatch_backward(grads.dx_perm, bufs.dest, d, x.dtype, grads.d_logits if routed else None,
                          w_gate, grads.dx, stream)
    return grads
