"""Pins of the oracle's optional routing features: a selection-only expert
bias, per-expert capacity with token dropping, and the router's
load-balancing statistics.  Closed forms, hand-worked cases, the pages'
printed numbers and invariants; no GPU."""
import numpy as np
import pytest

import oracle
import synth

RNG = np.random.default_rng(99)


def _f64(a):
    return synth.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _silu(z):
    return z / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------- bias

def test_bias_space_worked_example():
    """One token, logits (2, 1, 0), softmax scores (.665, .245, .090), bias
    (0, .5, 0), k = 1.  On logits the keys are (2, 1.5, 0): expert 0.  On
    scores they are (.665, .745, .090): expert 1.  Either way the gate is the
    unbiased score (renormalised over one expert: 1; raw: s)."""
    lg = np.array([[2.0, 1.0, 0.0]])
    b = np.array([0.0, 0.5, 0.0])
    s = np.exp(lg[0]) / np.exp(lg[0]).sum()
    r = oracle.route(lg, 1, bias=b, bias_on_scores=0, renormalize=0)
    assert r["ids"].tolist() == [[0]]
    np.testing.assert_allclose(r["gates"][0, 0], s[0], rtol=1e-15)
    np.testing.assert_allclose(r["gap_logit"][0], 0.5, rtol=1e-15)
    r = oracle.route(lg, 1, bias=b, bias_on_scores=1, renormalize=0)
    assert r["ids"].tolist() == [[1]]
    np.testing.assert_allclose(r["gates"][0, 0], s[1], rtol=1e-15)
    np.testing.assert_allclose(r["gap_logit"][0], (s[1] + 0.5) - s[0], rtol=1e-14)
    r = oracle.route(lg, 1, bias=b, bias_on_scores=1, renormalize=1)
    assert r["gates"][0, 0] == 1.0


@pytest.mark.parametrize("score_fn", [oracle.SOFTMAX, oracle.SIGMOID])
def test_score_bias_zero_and_forcing(score_fn):
    """A zero bias on the scores selects like no bias (scores are increasing
    in the logits); a huge bias on expert e puts e first for every token,
    with the unbiased gates renormalised over the chosen set."""
    lg = RNG.normal(size=(80, 32))
    r0 = oracle.route(lg, 6, score_fn)
    rz = oracle.route(lg, 6, score_fn, bias=np.zeros(32), bias_on_scores=1)
    assert np.array_equal(r0["ids"], rz["ids"])
    b = np.zeros(32)
    b[17] = 1e3
    rb = oracle.route(lg, 6, score_fn, bias=b, bias_on_scores=1)
    assert (rb["ids"][:, 0] == 17).all()
    s = np.exp(lg - lg.max(1, keepdims=True))
    s = s / s.sum(1, keepdims=True) if score_fn == oracle.SOFTMAX else 1 / (1 + np.exp(-lg))
    sel = np.take_along_axis(s, rb["ids"].astype(np.int64), 1)
    np.testing.assert_allclose(rb["gates"], sel / sel.sum(1, keepdims=True), rtol=1e-13)
    # the other five are the top five of the rest, by score
    for t in range(80):
        rest = [e for e in np.argsort(-s[t], kind="stable") if e != 17][:5]
        assert rb["ids"][t, 1:].tolist() == rest


def test_score_bias_by_enumeration():
    """Brute force: the chosen set maximises the sum of score + bias over all
    C(8, 3) subsets."""
    import itertools
    lg = RNG.normal(size=(30, 8))
    b = RNG.normal(scale=0.2, size=8)
    r = oracle.route(lg, 3, oracle.SIGMOID, bias=b, bias_on_scores=1)
    s = 1 / (1 + np.exp(-lg))
    for t in range(30):
        best = max(itertools.combinations(range(8), 3), key=lambda c: sum(s[t, e] + b[e] for e in c))
        assert set(r["ids"][t].tolist()) == set(best)


# --------------------------------------------------------------------------- capacity

def test_capacity_page_example():
    """4,096 tokens, 64 experts, top-8, factor 1.0: 512 slots per expert; an
    expert picked 600 times drops 88 ('from the router to the all-to-all',
    Capacity and token dropping).  The dropped ones are its last 88 pairs in
    token order."""
    T, E, k = 4096, 64, 8
    C = oracle.capacity(T, k, E, 1.0)
    assert C == 512
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        others = RNG.permutation(np.arange(1, E))[:k - 1]
        ids[t] = np.concatenate([[0], others]) if t < 600 else RNG.permutation(np.arange(1, E))[:k]
    d = oracle.dispatch(ids, E, cap=C)
    p0 = np.nonzero(ids.ravel() == 0)[0]
    assert p0.size == 600
    assert d["counts"][0] == 512
    assert (d["pair_pos"][p0[:512]] >= 0).all() and (d["pair_pos"][p0[512:]] == -1).all()
    assert int((d["pair_pos"] == -1).sum()) == 88 + sum(max(0, int(c) - 512) for c in
                                                         np.bincount(ids.ravel(), minlength=E)[1:])
    assert oracle.capacity(T, k, E, 1.25) == 640 and oracle.capacity(10, 2, 3, 1.0) == 7
    # the overflow the statistics report is that expert's 88 plus the others'
    st = oracle.router_stats(np.full((T, E), 1.0 / E), ids, alpha=1.0, cap=C)
    assert st["overflow"] == 88 + sum(max(0, int(c) - 512) for c in np.bincount(ids.ravel(), minlength=E)[1:])


def test_capacity_rounding():
    """ceil(T k / E * factor) with the factor read as the decimal it is
    written as: exact products stay exact (640 * 1.1
    is 704, though 640 * 1.1 in binary doubles is 704.0000000000001), and a
    fractional slot count rounds up."""
    assert oracle.capacity(80, 8, 1, 1.1) == 704
    assert oracle.capacity(333, 2, 8, 1.0) == 84            # 83.25
    assert oracle.capacity(4096, 2, 8, 1.25) == 1280
    assert oracle.capacity(4096, 8, 64, 1.1) == 564         # 563.2
    assert oracle.capacity(100, 3, 7, 2.0) == 86            # 85.71...
    assert oracle.capacity(0, 8, 64, 1.25) == 0


def test_stats_overflow_counts_dropped_pairs():
    """Capacity overflow ('T2.6 -- What Mixture of Experts Changes', In
    practice): the pairs the capacity drops, the same count the dispatch
    leaves out (pair_pos -1); none without a capacity or with a capacity at
    or above every count."""
    T, E, k = 300, 16, 4
    ids = np.stack([np.concatenate([[e % 3], RNG.permutation(np.arange(3, E))[:k - 1]])
                    for e in range(T)]).astype(np.int32)
    s = np.full((T, E), 1.0 / E)
    n = np.bincount(ids.ravel(), minlength=E)
    for cap in (1, 40, 75, int(n.max())):
        st = oracle.router_stats(s, ids, alpha=1.0, cap=cap)
        assert st["overflow"] == int((oracle.dispatch(ids, E, cap=cap)["pair_pos"] < 0).sum())
    assert oracle.router_stats(s, ids)["overflow"] == 0
    assert oracle.router_stats(s, ids, cap=int(n.max()))["overflow"] == 0


@pytest.mark.parametrize("T,E,k,cap", [(200, 8, 2, 30), (333, 64, 8, 20), (50, 16, 4, 1)])
def test_capacity_keeps_each_experts_first_pairs(T, E, k, cap):
    ids = np.stack([RNG.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    flat = ids.ravel()
    d = oracle.dispatch(ids, E, cap=cap)
    full = oracle.dispatch(ids, E)
    n = np.bincount(flat, minlength=E)
    np.testing.assert_array_equal(d["counts"], np.minimum(n, cap))
    np.testing.assert_array_equal(d["offsets"], np.concatenate([[0], np.cumsum(d["counts"])]))
    kept = d["offsets"][E]
    for e in range(E):
        mine = np.nonzero(flat == e)[0][:cap]          # first pairs in token order
        np.testing.assert_array_equal(d["sorted_pairs"][d["offsets"][e]:d["offsets"][e + 1]], mine)
    assert (d["sorted_pairs"][kept:] == -1).all()
    live = d["pair_pos"] >= 0
    np.testing.assert_array_equal(d["sorted_pairs"][d["pair_pos"][live]], np.nonzero(live)[0])
    # a capacity at or above every count drops nothing
    big = oracle.dispatch(ids, E, cap=int(n.max()))
    for key in ("counts", "offsets", "sorted_pairs", "pair_pos"):
        np.testing.assert_array_equal(big[key], full[key])


def test_dropped_pairs_contribute_nothing():
    """y with dropped pairs = y without them: sum over kept j of g_j f_j(x);
    a token whose every pair is dropped gets only the shared expert."""
    sh = synth.LayerShape("t", T=12, d=16, E=4, k=2, d_ff=24, num_shared=1, d_ff_shared=8,
                          dtype=synth.F32)
    inp = synth.make_inputs(sh, 4)
    toks = np.arange(12)
    full = oracle.forward_tokens(inp, 2, toks)
    keep = np.ones((12, 2), dtype=np.int32)
    keep[3, 1] = 0
    keep[7] = 0
    part = oracle.forward_tokens(inp, 2, toks, keep=keep)
    x = _f64(inp["x"])
    wg, wu, wd = (_f64(inp[n]) for n in ("w_gate", "w_up", "w_down"))
    e = full["ids"][3, 1]
    f3 = (_silu(wg[e] @ x[3]) * (wu[e] @ x[3])) @ wd[e].T
    np.testing.assert_allclose(part["y"][3], full["y"][3] - full["gates"][3, 1] * f3, rtol=1e-11, atol=1e-13)
    fs = (_silu(_f64(inp["ws_gate"]) @ x[7]) * (_f64(inp["ws_up"]) @ x[7])) @ _f64(inp["ws_down"]).T
    np.testing.assert_allclose(part["y"][7], fs, rtol=1e-11, atol=1e-13)
    others = [t for t in toks if t not in (3, 7)]
    np.testing.assert_array_equal(part["y"][others], full["y"][others])


# --------------------------------------------------------------------------- router statistics

def test_stats_uniform_top1_gives_alpha():
    """Uniform routing, k = 1: f_e = P_e = 1/E, so L_aux = alpha whatever E is
    ('from the router to the all-to-all', Load balancing; '8.6 Mixture of
    Experts', sec. 3.1)."""
    for E in (4, 8, 64):
        T = 3 * E
        lg = np.zeros((T, E))                          # equal logits: uniform probabilities
        ids = (np.arange(T) % E).reshape(T, 1)
        s = oracle.route(lg, 1)["scores"]
        st = oracle.router_stats(s, ids, alpha=0.01)
        np.testing.assert_allclose(st["l_aux"], 0.01, rtol=1e-13)
        np.testing.assert_allclose(st["f"], 1 / E, rtol=1e-15)
        assert st["max_over_mean"] == 1.0


def test_stats_worked_example_and_k_factor():
    """Two tokens, two experts, k = 1: token 0 -> expert 0 with p = (.8, .2),
    token 1 -> expert 0 with p = (.6, .4).  f = (1, 0), P = (.7, .3),
    L_aux = alpha * 2 * .7; max/mean = 2.  With k = E every f_e is 1 and
    L_aux = alpha * E * sum P = alpha * E (the k factor: sum f = k)."""
    s = np.array([[0.8, 0.2], [0.6, 0.4]])
    st = oracle.router_stats(s, np.array([[0], [0]]), alpha=0.5)
    np.testing.assert_allclose(st["f"], [1.0, 0.0])
    np.testing.assert_allclose(st["P"], [0.7, 0.3])
    np.testing.assert_allclose(st["l_aux"], 0.5 * 2 * 0.7)
    assert st["max_over_mean"] == 2.0
    lg = RNG.normal(size=(40, 6))
    r = oracle.route(lg, 6)
    st = oracle.router_stats(r["scores"], r["ids"], alpha=1.0)
    np.testing.assert_allclose(st["f"].sum(), 6.0)
    np.testing.assert_allclose(st["l_aux"], 6.0, rtol=1e-12)


def test_stats_sigmoid_probabilities_are_normalised():
    lg = RNG.normal(size=(50, 16))
    r = oracle.route(lg, 4, oracle.SIGMOID)
    st = oracle.router_stats(r["scores"], r["ids"], oracle.SIGMOID)
    np.testing.assert_allclose(st["P"].sum(), 1.0, rtol=1e-13)
    np.testing.assert_allclose(st["f"].sum(), 4.0, rtol=1e-15)
    sg = 1 / (1 + np.exp(-lg))
    np.testing.assert_allclose(st["P"], (sg / sg.sum(1, keepdims=True)).mean(0), rtol=1e-12)
