"""Per-element error model of the bf16 layer backward, for its parity tests.

Every value the bf16 path stores in 16 bits carries one round-to-nearest
error, uniform within half an ulp: standard deviation u |v| / sqrt(3) with
u = 2^-8 for bf16 (d_out_perm, dz, h on its way into dW2) and u = 2^-11 for
fp16 (z, h). The products accumulate in f32 (relative error near 2^-24 per
term, negligible next to these). Independent roundings add in quadrature
through each sum, so an output element's error has a standard deviation that
this module carries through the same chain the oracle computes:

  dh   = d_out W2              s_dh = sqrt(s_dout^2 W2^2)
  dz   = dh gelu'(z)           s_dz = sqrt((gelu'(z) s_dh)^2 + (dh s_z)^2 + (u_b dz / sqrt3)^2)
                               (|gelu''| <= 1 bounds the effect of z's rounding)
  dx_perm = dz W1              s = sqrt(s_dz^2 W1^2)
  dW1  = dz^T x_perm           s = sqrt((s_dz^2)^T x^2)
  dW2  = d_out^T h             s = sqrt((s_dout^2)^T h^2 + (d_out^2)^T s_h^2)
  dx   = sum of dx_perm rows   s = sqrt(sum of s_dx_perm^2)

The tests accept |gpu - exact| <= 7 s + 1e-5 (|exact| + rms): a sum of many
independent roundings is close to Gaussian, and 7 standard deviations are
not reached by chance over the sizes tested, while a wrong index or operand
gives errors of the order of the values themselves."""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O

U_BF16 = 2.0 ** -8
U_FP16 = 2.0 ** -11
K_SIGMA = 7.0
_S3 = np.sqrt(3.0)


def expert_sigmas(x_rows, d_out_rows, w1_e, w2_e, fcols=None, weight_grads=True) -> dict:
    """Error standard deviations of one expert block, in the shapes that
    O.expert_backward returns for the same arguments."""
    w1s = w1_e if fcols is None else w1_e[fcols]
    w2s = w2_e if fcols is None else w2_e[:, fcols]
    z = x_rows @ w1s.T
    h = O.gelu_tanh(z)
    g = O.gelu_tanh_grad(z)
    dh = d_out_rows @ w2s
    dz = dh * g
    s_dout = U_BF16 / _S3 * np.abs(d_out_rows)
    s_z = U_FP16 / _S3 * np.abs(z)
    s_dh = np.sqrt(s_dout ** 2 @ w2s ** 2)
    s_dz = np.sqrt((g * s_dh) ** 2 + (dh * s_z) ** 2 + (U_BF16 / _S3 * dz) ** 2)
    s_h = np.sqrt((U_FP16 / _S3 * h) ** 2 + (U_BF16 / _S3 * h) ** 2 + (g * s_z) ** 2)
    out = {"z": s_z, "dz": s_dz}
    if weight_grads:
        out["dw1"] = np.sqrt(s_dz.T ** 2 @ x_rows ** 2)
        out["dw2"] = np.sqrt(s_dout.T ** 2 @ h ** 2 + d_out_rows.T ** 2 @ s_h ** 2)
    if fcols is None:
        out["dx_perm"] = np.sqrt(s_dz ** 2 @ w1_e ** 2)
    return out


def expert_sigmas_torch(x_rows, d_out_rows, w1_e, w2_e, weight_grads=True) -> dict:
    """expert_sigmas without `fcols`, the same chain in float32 torch CPU ops
    (multi-threaded: the full-size case has 21 M hidden values per expert).
    GELU and its derivative are the tanh form's formulas written out here;
    they only scale the error model."""
    import torch

    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    x, d_out, w1, w2 = f(x_rows), f(d_out_rows), f(w1_e), f(w2_e)
    c = float(np.sqrt(2.0 / np.pi))
    z = x @ w1.T
    th = torch.tanh(c * (z + 0.044715 * z * z * z))
    h = 0.5 * z * (1.0 + th)
    g = 0.5 * (1.0 + th) + 0.5 * z * (1.0 - th * th) * c * (1.0 + 3.0 * 0.044715 * z * z)
    dh = d_out @ w2
    dz = dh * g
    ub, uf = U_BF16 / _S3, U_FP16 / _S3
    s_dout = ub * d_out.abs()
    s_z = uf * z.abs()
    s_dh = torch.sqrt(s_dout.square() @ w2.square())
    s_dz = torch.sqrt((g * s_dh).square() + (dh * s_z).square() + (ub * dz).square())
    out = {"z": s_z, "dz": s_dz, "dx_perm": torch.sqrt(s_dz.square() @ w1.square())}
    if weight_grads:
        s_h = torch.sqrt((uf * h).square() + (ub * h).square() + (g * s_z).square())
        out["dw1"] = torch.sqrt(s_dz.T.square() @ x.square())
        out["dw2"] = torch.sqrt(s_dout.T.square() @ h.square() + d_out.T.square() @ s_h.square())
    return {k: v.double().numpy() for k, v in out.items()}


def layer_sigmas(inp, fwd, ref, dtype="bf16") -> dict:
    """Standard deviations for every modelled output of a whole (small) layer,
    keyed like O.backward's result."""
    x = O.decode(inp["x"], dtype)
    w1, w2 = O.decode(inp["w1"], dtype), O.decode(inp["w2"], dtype)
    off, src, dest = fwd["offsets"], fwd["src"], fwd["dest"]
    d_out = ref["d_out_perm"]
    s = {"d_out_perm": U_BF16 / _S3 * np.abs(d_out), "z_perm": np.zeros_like(ref["z_perm"]),
         "dz_perm": np.zeros_like(ref["dz_perm"]), "dx_perm": np.zeros_like(ref["dx_perm"]),
         "dw1": np.zeros_like(ref["dw1"]), "dw2": np.zeros_like(ref["dw2"])}
    for e in range(w1.shape[0]):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        g = expert_sigmas(x[src[a:b]], d_out[a:b], w1[e], w2[e])
        s["z_perm"][a:b], s["dz_perm"][a:b], s["dx_perm"][a:b] = g["z"], g["dz"], g["dx_perm"]
        s["dw1"][e], s["dw2"][e] = g["dw1"], g["dw2"]
    var = np.zeros_like(ref["dx"])
    for j in range(dest.shape[1]):
        keep = dest[:, j] >= 0
        var[keep] += s["dx_perm"][dest[keep, j]] ** 2
    s["dx"] = np.sqrt(var)
    return s


def within(got, ref, sigma, what, extra=0.0):
    """|got - ref| <= 7 sigma + extra + 1e-5 (|ref| + rms); prints the worst ratio."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bound = K_SIGMA * np.asarray(sigma) + extra + 1e-5 * (np.abs(ref) + rms)
    ratio = np.abs(got - ref) / np.maximum(bound, 1e-300)
    worst = float(np.max(ratio))
    print("  %s: worst |err| / (7 sigma + ...) = %.3f" % (what, worst), flush=True)
    assert worst <= 1.0, "%s: %d elements beyond the rounding-error bound (worst %.3f)" % (
        what, int((ratio > 1).sum()), worst)
    return worst
