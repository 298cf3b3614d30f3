"""CPU: randomised property tests of the oracle (hypothesis): random token
counts, expert counts, k, capacity factors and logits with injected ties,
each case checked against what the method fixes independently of the
oracle's own code -- brute-force subset ranking for top-k, a per-expert
queue simulation for the dispatch, exact rational arithmetic for the
capacity, and invariances of the aux loss and of the layer."""
import fractions
import itertools

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import moe_oracle as O

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def routing(draw, max_T=120, max_E=12):
    """A routing problem: T tokens, E experts, k distinct experts per token
    from integer-valued logits (many exact ties), and a capacity."""
    T = draw(st.integers(0, max_T))
    E = draw(st.integers(1, max_E))
    k = draw(st.integers(1, min(4, E)))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    levels = draw(st.integers(1, 4))          # few distinct values: ties everywhere
    rng = np.random.default_rng(seed)
    logits = rng.integers(-levels, levels + 1, size=(T, E)).astype(np.float64)
    cf = draw(st.sampled_from([0.0, -1.0, 0.25, 0.5, 1.0, 1.25, 2.0, 3.0]))
    return logits, k, cf


def brute_topk(row, k):
    """The unique k-subset whose members all outrank every non-member under
    (value descending, index ascending), listed best first."""
    E = len(row)
    better = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
    for S in itertools.combinations(range(E), k):
        if all(better(a, b) for a in S for b in range(E) if b not in S):
            return sorted(S, key=lambda a: sum(better(b, a) for b in S))
    raise AssertionError("no dominating subset")


@SETTINGS
@given(routing(max_T=25, max_E=7))
def test_topk_equals_brute_force_with_ties(case):
    logits, k, _ = case
    idx, w = O.topk(logits, O.softmax(logits) if logits.size else logits, k)
    for t in range(logits.shape[0]):
        assert list(idx[t]) == brute_topk(logits[t], k)


@SETTINGS
@given(st.integers(0, 10 ** 6), st.integers(1, 256),
       st.fractions(min_value=fractions.Fraction(1, 64), max_value=fractions.Fraction(4), max_denominator=64))
def test_capacity_is_round_half_even_of_the_exact_quotient(n, E, cf):
    """C = round(n / E * cf) with ties to even, from exact rationals (cf is a
    dyadic-friendly fraction; floats of the same value give the same C)."""
    exact = fractions.Fraction(n, E) * cf
    fl, fr = exact.numerator // exact.denominator, exact - exact.numerator // exact.denominator
    want = fl + (1 if fr > fractions.Fraction(1, 2) or (fr == fractions.Fraction(1, 2) and fl % 2 == 1) else 0)
    got = O.capacity(n, E, float(cf))
    # a float quotient within a few ulps of a .5 tie may round either way
    if abs(float(fr) - 0.5) > 1e-9:
        assert got == want, (n, E, cf, got, want)


@SETTINGS
@given(routing())
def test_dispatch_equals_queue_simulation(case):
    logits, k, cf = case
    T, E = logits.shape
    idx, _ = O.topk(logits, O.softmax(logits) if T else logits, k)
    C = O.capacity(T, E, cf)
    counts, offsets, dest, src = O.dispatch(idx, E, C)
    # independent: each expert keeps a queue; assignments arrive in token order
    queues = [[] for _ in range(E)]
    drops = set()
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if C < 0 or len(queues[e]) < C:
                queues[e].append((t, j))
            else:
                drops.add((t, j))
    assert counts.sum() == T * k
    assert offsets[0] == 0 and list(np.diff(offsets)) == [len(q) for q in queues]
    for e in range(E):
        assert C < 0 or len(queues[e]) <= C
        for pos, (t, j) in enumerate(queues[e]):
            assert dest[t, j] == offsets[e] + pos and src[offsets[e] + pos] == t
    for (t, j) in drops:
        assert dest[t, j] == -1
    assert ((dest >= 0).sum(axis=1) <= k).all()          # at most k experts per token


@SETTINGS
@given(routing(), st.floats(1e-4, 1.0))
def test_aux_loss_invariances(case, alpha):
    logits, k, _ = case
    T, E = logits.shape
    if T == 0:
        assert O.aux_loss(np.zeros((0, E)), np.zeros(E), k, alpha) == 0.0
        return
    p = O.softmax(logits)
    idx, _ = O.topk(logits, p, k)
    counts = np.bincount(idx.ravel(), minlength=E)
    L = O.aux_loss(p, counts, k, alpha)
    assert L >= 0
    # linear in alpha, invariant under relabelling the experts
    assert np.isclose(O.aux_loss(p, counts, k, 2 * alpha), 2 * L, rtol=1e-12)
    perm = np.random.default_rng(E + T).permutation(E)
    assert np.isclose(O.aux_loss(p[:, perm], counts[perm], k, alpha), L, rtol=1e-12)
    # bounded by alpha E (all mass and all assignments on one expert)
    assert L <= alpha * E * (1 + 1e-12)


@SETTINGS
@given(st.integers(1, 40), st.integers(1, 6), st.integers(1, 3), st.integers(0, 2 ** 31 - 1))
def test_layer_without_dropping_is_the_dense_masked_sum(T, E, k, seed):
    """cf <= 0: every assignment kept; y = sum over each token's top-k of
    p * FFN_e(x), evaluated densely, for any shape."""
    k = min(k, E)
    rng = np.random.default_rng(seed)
    d, dff = 6, 9
    inp = {"x": rng.standard_normal((T, d)), "w_gate": rng.standard_normal((E, d)),
           "w1": rng.standard_normal((E, dff, d)) * 0.5, "w2": rng.standard_normal((E, d, dff)) * 0.5}
    out = O.forward(inp, "f32", k=k, cf=0.0)
    logits = inp["x"] @ inp["w_gate"].T
    p = O.softmax(logits)
    y = np.zeros((T, d))
    for t in range(T):
        for e in brute_topk(logits[t], k):
            h = inp["x"][t] @ inp["w1"][e].T
            h = 0.5 * h * (1 + np.tanh(np.sqrt(2 / np.pi) * (h + 0.044715 * h ** 3)))
            y[t] += p[t, e] * (h @ inp["w2"][e].T)
    np.testing.assert_allclose(out["y"], y, rtol=1e-10, atol=1e-12)
