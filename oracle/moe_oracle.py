"""CPU oracle of the MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this module. The product path (the HIP library and its Python
binding) never does, and this module imports nothing from it.

Plain numpy in float64, written step by step from the pages:
  * gate: a lightweight linear layer scoring every token against every expert
    (EP tutorial "专家并行：混合专家模型的分布式训练方案", section 1.1);
  * the gate's output is a per-token expert-assignment probability
    (fine-grained EP deployment guide "细粒度专家并行部署实践与优化指南",
    section 5 step 3); softmax is the reading taken for "probability";
  * top-K expert selection, only chosen experts compute (EP tutorial 1.1,
    2.1 step 1; deployment guide section 7 example, topk of gate_probs, k=2);
  * capacity = round((total tokens / experts) x capacity factor), tokens over
    capacity dropped (EP tutorial, section 2.2);
  * dispatch plan, tokens grouped contiguously per expert (EP tutorial 2.1
    step 2 and 5.3);
  * per-expert FFN: up-projection w1, activation, down-projection w2
    (ETP expert-parallel page "ETP专家并行加速MoE模型", the ETP section:
    4096 -> 16384 -> 4096, w1 split by columns, w2 by rows); GELU-tanh is the
    activation this workload names, written from its textbook definition;
  * combine: results returned to their original token positions (EP tutorial
    2.1 step 5), weighted by the gate probabilities;
  * L_aux = alpha * num_experts * sum_i f_i * P_i (EP tutorial, section 5.1).

Readings where the pages are silent (each also listed in the design notes):
  * probabilities are a softmax over all E logits, taken before top-k;
  * experts are ranked on their logits (float64 here), larger first, ties to
    the lower expert index; the combine weight of a chosen expert is its
    softmax probability (not renormalised unless `renorm`);
  * the capacity formula's "total tokens" is n = T (the tokens entering the
    layer); round() is round-half-even; cf <= 0 disables dropping;
  * dropping keeps, per expert, the first C assignments in token order;
    a dropped assignment contributes 0 and surviving weights are not
    renormalised;
  * f_i counts router assignments before dropping, divided by T*k;
    P_i is the mean over all T tokens of the full softmax.
  * routing knobs against hot experts: the SP/EP page (EP section) adjusts
    the routing temperature and adds a random perturbation, the ETP page
    names a routing z-loss; none gives a formula. Read as: scores
    s = (l + noise) / temperature replace the logits in softmax and top-k
    (the caller draws the noise), and the z-loss is the mean over tokens of
    (log sum_e exp(s[t, e]))^2, the usual router z-loss.
  * backward (the pages train the layer and give the aux loss for its
    gradient, no formulas): the routing choice and the counts in f_i are
    constants; the caller's noise is an input.
"""
from __future__ import annotations

import numpy as np


def decode(a, dtype: str) -> np.ndarray:
    """Input tensor -> float64. bf16 is the upper half of a binary32 word."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def capacity(n_tokens: int, n_experts: int, cf: float) -> int:
    """Expert capacity = round((total tokens / experts) x capacity factor)
    (EP tutorial, section 2.2). Python's round() is round-half-even.
    cf <= 0 means no dropping and returns -1."""
    if cf <= 0:
        return -1
    return int(round((n_tokens / n_experts) * cf))


def gate_logits(x64: np.ndarray, wg64: np.ndarray, bias=None) -> np.ndarray:
    """l[t, e] = sum_c x[t, c] * Wg[e, c] + b[e] (EP tutorial 1.1: the gate is
    a linear layer over the token representation)."""
    l = x64 @ wg64.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def softmax(logits: np.ndarray) -> np.ndarray:
    """Row-wise softmax, max-subtracted."""
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def topk(logits: np.ndarray, probs: np.ndarray, k: int, renorm: bool = False):
    """Top-k experts per token (EP tutorial 1.1 and 2.1 step 1).

    Key: logit descending, then expert index ascending. Slot j holds the j-th
    best expert. Weight = the expert's softmax probability.
    Returns (idx [T,k] int64, w [T,k] float64)."""
    T, E = logits.shape
    eidx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((eidx, -logits), axis=-1)   # primary key is the last one
    idx = order[:, :k].astype(np.int64)
    w = np.take_along_axis(probs, idx, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w


def dispatch(topk_idx: np.ndarray, n_experts: int, cap: int):
    """Capacity-limited dispatch plan (EP tutorial 2.1 step 2, 2.2, 5.3).

    Assignments are visited in token order (t, then slot j); each expert hands
    out positions 0, 1, 2, ... in that order and keeps the assignment iff its
    position is below the capacity. Kept rows are laid out expert by expert.

    Returns counts[E] (assignments before dropping), offsets[E+1] (exclusive
    scan of kept rows), dest[T,k] (row in the grouped layout, or -1 when
    dropped) and src[R] (token of each grouped row)."""
    T, k = topk_idx.shape
    fill = np.zeros(n_experts, dtype=np.int64)
    pos = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(topk_idx[t, j])
            pos[t, j] = fill[e]
            fill[e] += 1
    counts = fill
    kept = counts.copy() if cap < 0 else np.minimum(counts, cap)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    keep = np.ones((T, k), dtype=bool) if cap < 0 else pos < cap
    dest = np.where(keep, offsets[topk_idx] + pos, -1)
    src = np.empty(int(offsets[-1]), dtype=np.int64)
    tok = np.broadcast_to(np.arange(T)[:, None], (T, k))
    src[dest[keep]] = tok[keep]
    return counts, offsets, dest, src


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def expert_ffn(x_rows: np.ndarray, w1_e: np.ndarray, w2_e: np.ndarray) -> np.ndarray:
    """One expert's FFN on a block of rows: gelu(X W1^T) W2^T, where W1 is
    [d_ff, d] and W2 is [d, d_ff] (ETP page: up-projection w1, down w2)."""
    return gelu_tanh(x_rows @ w1_e.T) @ w2_e.T


def combine(y_perm: np.ndarray, dest: np.ndarray, topk_w: np.ndarray, T: int) -> np.ndarray:
    """y[t] = sum over kept slots j of w[t,j] * y_perm[dest[t,j]]; a token with
    no kept slot gets 0 (EP tutorial 2.1 step 5 and 2.2)."""
    d = y_perm.shape[1] if y_perm.ndim == 2 else 0
    y = np.zeros((T, d), dtype=np.float64)
    for j in range(dest.shape[1]):
        keep = dest[:, j] >= 0
        y[keep] += topk_w[keep, j][:, None] * y_perm[dest[keep, j]]
    return y


def aux_loss(probs: np.ndarray, counts: np.ndarray, k: int, alpha: float) -> float:
    """L_aux = alpha * E * sum_i f_i * P_i (EP tutorial, section 5.1), with
    f_i = counts_i / (T k) and P_i the mean gate probability of expert i."""
    T, E = probs.shape
    if T == 0:
        return 0.0
    f = counts / float(T * k)
    P = probs.mean(axis=0)
    return float(alpha * E * np.sum(f * P))


def balance_scores(logits: np.ndarray, temperature: float = 1.0, noise=None) -> np.ndarray:
    """Routing scores with the pages' balancing knobs (SP/EP page, EP section:
    routing temperature and a random perturbation):
    s = (l + noise) / temperature; temperature 1 and no noise give l."""
    s = logits if noise is None else logits + np.asarray(noise, dtype=np.float64)
    return s / float(temperature)


def log_sum_exp(scores: np.ndarray) -> np.ndarray:
    """log sum_e exp(s[t, e]) per token, max-subtracted."""
    m = scores.max(axis=1)
    return m + np.log(np.exp(scores - m[:, None]).sum(axis=1))


def z_loss_terms(scores: np.ndarray) -> np.ndarray:
    """Per-token term of the router z-loss (ETP page: routing z-loss spreads
    the gate's attention): (log sum_e exp(s[t, e]))^2."""
    return log_sum_exp(scores) ** 2


def z_loss(scores: np.ndarray, coeff: float) -> float:
    """Router z-loss = coeff * mean over tokens of z_loss_terms."""
    if scores.shape[0] == 0:
        return 0.0
    return float(coeff * z_loss_terms(scores).mean())


def route(x, w_gate, bias, dtype: str, k: int, renorm: bool = False, temperature: float = 1.0,
          noise=None):
    """Gate -> (balancing knobs) -> softmax -> top-k on the given input bits.
    `logits` in the result are the scores that softmax and top-k see."""
    l = gate_logits(decode(x, dtype), decode(w_gate, dtype), bias)
    s = balance_scores(l, temperature, noise)
    p = softmax(s)
    idx, w = topk(s, p, k, renorm)
    lse = log_sum_exp(s)
    return {"logits": s, "probs": p, "topk_idx": idx, "topk_w": w, "lse": lse, "zsq": lse ** 2}


def forward(inp: dict, dtype: str, k: int, cf: float, alpha: float = 0.01,
            renorm: bool = False, sample_tokens=None, temperature: float = 1.0,
            noise=None) -> dict:
    """The whole layer: route (unless `inp` carries topk_idx/topk_w), dispatch,
    expert FFN, combine, aux loss.

    With `sample_tokens` (an index array) the FFN and combine are evaluated
    for those tokens only: `y` then has one row per sampled token, and only
    the grouped rows listed in `y_perm_rows` of `y_perm` are filled."""
    x = inp["x"]
    T = x.shape[0]
    E = inp["w1"].shape[0]
    out = {}
    if inp.get("w_gate") is not None:
        out.update(route(x, inp["w_gate"], inp.get("bias"), dtype, k, renorm, temperature, noise))
    else:
        out["topk_idx"] = np.asarray(inp["topk_idx"], dtype=np.int64)
        out["topk_w"] = np.asarray(inp["topk_w"], dtype=np.float64)
        k = out["topk_idx"].shape[1]
    C = capacity(T, E, cf)
    counts, offsets, dest, src = dispatch(out["topk_idx"], E, C)
    out.update(capacity=C, counts=counts, offsets=offsets, dest=dest, src=src)
    if "probs" in out:
        out["aux"] = aux_loss(out["probs"], counts, k, alpha)

    toks = np.arange(T) if sample_tokens is None else np.asarray(sample_tokens)
    need = dest[toks]
    rows = np.unique(need[need >= 0])                       # grouped rows needed
    d = inp["w2"].shape[1]
    y_perm = np.zeros((int(offsets[-1]), d))
    for e in range(E):
        sel = rows[(rows >= offsets[e]) & (rows < offsets[e + 1])]
        if sel.size:
            y_perm[sel] = expert_ffn(decode(x[src[sel]], dtype),
                                     decode(inp["w1"][e], dtype),
                                     decode(inp["w2"][e], dtype))
    out["y_perm"] = y_perm
    out["y_perm_rows"] = rows
    out["y"] = combine(y_perm, need, out["topk_w"][toks], toks.size)
    return out


# ----------------------------------------------------------------- backward --
# The layer's backward (EP tutorial section 5.1: the aux loss exists for its
# gradient; the pages' reverse path runs combine, expert FFN, dispatch and the
# gate in reverse). Readings: the routing choice (top-k indices, capacity
# drops) and the counts in f_i are constants; gradients flow through the
# chosen experts' weights, the FFN, the softmax and the gate; the noise is
# an input, so only 1/temperature scales the gate gradient.

def gelu_tanh_grad(z: np.ndarray) -> np.ndarray:
    """d/dz of gelu_tanh: 0.5 (1 + tanh u) + 0.5 z (1 - tanh^2 u) u',
    u = sqrt(2/pi)(z + 0.044715 z^3), u' = sqrt(2/pi)(1 + 3 * 0.044715 z^2)."""
    c = np.sqrt(2.0 / np.pi)
    u = c * (z + 0.044715 * z ** 3)
    th = np.tanh(u)
    return 0.5 * (1.0 + th) + 0.5 * z * (1.0 - th * th) * c * (1.0 + 3.0 * 0.044715 * z * z)


def combine_backward(dy: np.ndarray, y_perm: np.ndarray, dest: np.ndarray, topk_w: np.ndarray,
                     R: int):
    """Transpose of the weighted combine y[t] = sum_j w[t,j] o[dest[t,j]]:
    d_out[dest[t,j]] = w[t,j] dy[t] and dw[t,j] = dy[t] . o[dest[t,j]];
    a dropped slot gets dw = 0."""
    T, k = dest.shape
    d = dy.shape[1]
    d_out = np.zeros((R, d))
    dw = np.zeros((T, k))
    for j in range(k):
        keep = dest[:, j] >= 0
        r = dest[keep, j]
        d_out[r] = topk_w[keep, j][:, None] * dy[keep]
        dw[keep, j] = np.sum(dy[keep] * y_perm[r], axis=1)
    return d_out, dw


def gate_backward(dw: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, probs: np.ndarray,
                  counts: np.ndarray, k: int, alpha: float, aux_grad: float, renorm: bool = False,
                  temperature: float = 1.0, lse=None, z_coeff: float = 0.0,
                  n_tokens=None) -> np.ndarray:
    """Gradient of the gate's linear output (the logits before the routing
    knobs) from: the combine weights' gradient dw, aux_grad times the aux
    loss (EP tutorial 5.1), and z_coeff times the mean over tokens of lse^2.

    p = softmax(s), s = (l + noise) / temperature. Chosen weight w_j = p_j,
    or p_j / S with S = sum over the chosen p when renormalised, whose
    gradient with respect to a chosen p_m is (dw_m - sum_j dw_j w_j) / S.
    dL_aux/dp[t, i] = alpha E f_i / T with f_i = counts_i / (T k).
    Softmax: ds = p (dp - sum_e p dp); z-loss: ds += z_coeff 2 lse p / T;
    dl = ds / temperature. The rows may be a sample of the layer's tokens:
    `n_tokens` is then the layer's T."""
    E = probs.shape[1]
    T = probs.shape[0] if n_tokens is None else int(n_tokens)
    p = np.asarray(probs, dtype=np.float64)
    w = np.asarray(topk_w, dtype=np.float64)
    g = np.asarray(dw, dtype=np.float64).copy()
    if renorm:
        S = np.take_along_axis(p, topk_idx, axis=1).sum(axis=1, keepdims=True)
        g = (g - np.sum(g * w, axis=1, keepdims=True)) / S
    n = probs.shape[0]
    dp = np.zeros((n, E))
    for j in range(topk_idx.shape[1]):
        np.add.at(dp, (np.arange(n), topk_idx[:, j]), g[:, j])
    if T > 0:
        f = np.asarray(counts, dtype=np.float64) / float(T * k)
        dp += aux_grad * alpha * E * f[None, :] / T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    if z_coeff != 0.0 and T > 0:
        ds += z_coeff * 2.0 * np.asarray(lse, dtype=np.float64)[:, None] * p / T
    return ds / float(temperature)


def expert_backward(x_rows: np.ndarray, d_out_rows: np.ndarray, w1_e: np.ndarray,
                    w2_e: np.ndarray, fcols=None, weight_grads: bool = True) -> dict:
    """One expert's FFN backward on a block of its rows (optionally only the
    hidden units `fcols`): z = X W1^T, h = gelu(z), dz = (D W2) * gelu'(z),
    dW1 = dz^T X, dW2 = D^T h (left out when not `weight_grads`) and, over all
    hidden units, dx_perm = dz W1 and the rows' forward output y = h W2^T
    (what the combine weights' gradient needs)."""
    w1s = w1_e if fcols is None else w1_e[fcols]
    w2s = w2_e if fcols is None else w2_e[:, fcols]
    z = x_rows @ w1s.T
    h = gelu_tanh(z)
    dz = (d_out_rows @ w2s) * gelu_tanh_grad(z)
    out = {"z": z, "h": h, "dz": dz}
    if weight_grads:
        out["dw1"], out["dw2"] = dz.T @ x_rows, d_out_rows.T @ h
    if fcols is None:
        out["dx_perm"] = dz @ w1_e
        out["y"] = h @ w2_e.T
    return out


def backward(inp: dict, fwd: dict, dy: np.ndarray, dtype: str, k: int, alpha: float = 0.01,
             aux_scale: float = 1.0, renorm: bool = False, temperature: float = 1.0,
             z_coeff: float = 0.0) -> dict:
    """Gradients of L = sum(dy * y) + aux_scale * L_aux + z_coeff * mean(lse^2)
    with respect to x, the gate weight and bias, W1 and W2, given the
    forward's routing and dispatch (`fwd`: topk_idx, topk_w, probs, counts,
    offsets, dest, src, y_perm, lse).

    Expert part, for each kept row r (token t = src[r]):
      d_out_r, dw from combine_backward;  z_r = W1 x_t;  h_r = gelu(z_r);
      dz_r = (W2^T d_out_r) * gelu'(z_r);  dW2 += d_out_r h_r^T;
      dW1 += dz_r x_t^T;  dx_perm_r = W1^T dz_r;  dx_t += dx_perm_r.
    Gate: dl from gate_backward; dWg = dl^T x; db = sum_t dl_t; dx += dl Wg.
    Also returns the per-row intermediates (z_perm, h_perm, d_out_perm,
    dz_perm, dx_perm)."""
    x = decode(inp["x"], dtype)
    w1 = decode(inp["w1"], dtype)
    w2 = decode(inp["w2"], dtype)
    T, d = x.shape
    E, dff = w1.shape[0], w1.shape[1]
    dy = np.asarray(dy, dtype=np.float64)
    dest, src, offsets = fwd["dest"], fwd["src"], fwd["offsets"]
    tw = np.asarray(fwd["topk_w"], dtype=np.float64)
    R = int(offsets[-1])
    xp = x[src]
    y_perm = np.zeros((R, d))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        y_perm[a:b] = gelu_tanh(xp[a:b] @ w1[e].T) @ w2[e].T
    d_out, dw = combine_backward(dy, y_perm, dest, tw, R)
    z = np.zeros((R, dff))
    h = np.zeros((R, dff))
    dz = np.zeros((R, dff))
    dx_perm = np.zeros((R, d))
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        g = expert_backward(xp[a:b], d_out[a:b], w1[e], w2[e])
        z[a:b], h[a:b], dz[a:b], dx_perm[a:b] = g["z"], g["h"], g["dz"], g["dx_perm"]
        dw1[e], dw2[e] = g["dw1"], g["dw2"]
    dx = np.zeros((T, d))
    np.add.at(dx, src, dx_perm)
    out = {"dx_experts": dx.copy(), "dw1": dw1, "dw2": dw2, "dw": dw, "z_perm": z, "h_perm": h,
           "d_out_perm": d_out, "dz_perm": dz, "dx_perm": dx_perm}
    if inp.get("w_gate") is not None:
        wg = decode(inp["w_gate"], dtype)
        dl = gate_backward(dw, fwd["topk_idx"], tw, fwd["probs"], fwd["counts"], k, alpha,
                           aux_scale, renorm, temperature, fwd.get("lse"), z_coeff)
        out.update(dl=dl, dwg=dl.T @ x, db=dl.sum(axis=0))
        dx += dl @ wg
    out["dx"] = dx
    return out
