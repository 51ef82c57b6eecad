"""Pins of the oracle's backward pass: central finite differences of the
oracle's own forward (fp64 inputs, routing held fixed) in random directions
of every input and weight tensor, and closed forms.  No GPU."""
import numpy as np
import pytest

import oracle
import synth

RNG = np.random.default_rng(2024)


def _inputs(T, d, E, k, f, S=0, f_s=0, seed=0):
    sh = synth.LayerShape("t", T=T, d=d, E=E, k=k, d_ff=f, num_shared=S, d_ff_shared=f_s, dtype=synth.F32)
    inp = synth.make_inputs(sh, seed)
    return {n: (None if a is None else a.astype(np.float64)) for n, a in inp.items()}


def _loss(inp, ids, dy, score_fn, renorm):
    T = inp["x"].shape[0]
    y = oracle.forward_tokens(inp, ids.shape[1], np.arange(T), score_fn, renorm, forced_ids=ids)["y"]
    return float(np.sum(dy * y))


GRAD_OF = {"x": "dx", "w_router": "dw_router", "w_gate": "dw_gate", "w_up": "dw_up", "w_down": "dw_down",
           "ws_gate": "ds_gate", "ws_up": "ds_up", "ws_down": "ds_down"}


@pytest.mark.parametrize("score_fn,renorm,S", [(oracle.SOFTMAX, 1, 0), (oracle.SOFTMAX, 0, 1),
                                               (oracle.SIGMOID, 1, 1), (oracle.SIGMOID, 0, 0)])
def test_gradients_match_finite_differences(score_fn, renorm, S):
    T, d, E, k, f = 5, 8, 6, 2, 12
    inp = _inputs(T, d, E, k, f, S, 4 if S else 0, seed=3)
    for n in ("x", "w_router"):
        inp[n] = inp[n] * 2.0            # livelier gates
    lg = oracle.logits(inp["x"], inp["w_router"])
    ids = oracle.route(lg, k, score_fn, renorm)["ids"]
    dy = RNG.normal(size=(T, d))
    g = oracle.backward(inp, ids, dy, score_fn, renorm)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if inp.get(name) is None:
            continue
        v = RNG.normal(size=inp[name].shape)
        plus, minus = dict(inp), dict(inp)
        plus[name] = inp[name] + eps * v
        minus[name] = inp[name] - eps * v
        fd = (_loss(plus, ids, dy, score_fn, renorm) - _loss(minus, ids, dy, score_fn, renorm)) / (2 * eps)
        an = float(np.sum(g[gname] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}: finite difference {fd} vs gradient {an}"


def test_single_renormalised_choice_gives_no_router_gradient():
    """k = 1 with renormalisation: the gate is 1 whatever the logits, so the
    router gets no gradient and dx has only the expert path."""
    inp = _inputs(7, 8, 4, 1, 12, seed=5)
    lg = oracle.logits(inp["x"], inp["w_router"])
    ids = oracle.route(lg, 1)["ids"]
    dy = RNG.normal(size=(7, 8))
    g = oracle.backward(inp, ids, dy, oracle.SOFTMAX, 1)
    np.testing.assert_allclose(g["dw_router"], 0.0, atol=1e-14)   # the Jacobian terms cancel
    # the expert path alone: dx = W_gate^T da + W_up^T du for the chosen expert
    x, wg, wu, wd = (inp[n] for n in ("x", "w_gate", "w_up", "w_down"))
    for t in range(7):
        e = ids[t, 0]
        a, u = wg[e] @ x[t], wu[e] @ x[t]
        sig = 1 / (1 + np.exp(-a))
        dh = wd[e].T @ dy[t]
        da = dh * u * (sig + a * sig * (1 - sig))
        du = dh * a * sig
        np.testing.assert_allclose(g["dx"][t], wg[e].T @ da + wu[e].T @ du, rtol=1e-12, atol=1e-14)


def test_weight_gradients_are_outer_product_sums():
    """dW_down of an expert is the sum over its pairs of (g dy) h^T: with all
    tokens sent to one expert and k = 1, renorm = 0 (Switch), it equals
    (g * dy)^T H computed with plain matmuls."""
    inp = _inputs(9, 8, 3, 1, 10, seed=8)
    inp["w_router"] = inp["w_router"] * 0.0
    inp["w_router"][1] = 1.0              # expert 1 wins only where sum(x) > 0 ...
    inp["w_router"][:, 0] += np.array([0.0, 50.0, 0.0])   # ... so force it through x[:, 0]
    x = inp["x"]
    x[:, 0] = 1.0
    lg = oracle.logits(x, inp["w_router"])
    ids = oracle.route(lg, 1, oracle.SOFTMAX, 0)["ids"]
    assert (ids == 1).all()
    dy = RNG.normal(size=(9, 8))
    g = oracle.backward(inp, ids, dy, oracle.SOFTMAX, 0)
    s = np.exp(lg - lg.max(1, keepdims=True))
    s /= s.sum(1, keepdims=True)
    gate = s[:, 1]
    a, u = x @ inp["w_gate"][1].T, x @ inp["w_up"][1].T
    H = a / (1 + np.exp(-a)) * u
    np.testing.assert_allclose(g["dw_down"][1], (gate[:, None] * dy).T @ H, rtol=1e-12, atol=1e-14)
    assert np.all(g["dw_down"][0] == 0.0) and np.all(g["dw_down"][2] == 0.0)


@pytest.mark.parametrize("score_fn,renorm", [(oracle.SOFTMAX, 1), (oracle.SIGMOID, 1), (oracle.SOFTMAX, 0)])
def test_weight_samples_equal_full_backward(score_fn, renorm):
    """The element-wise weight gradients (for checking full-size layers on a
    sample) equal the entries of the whole backward, which the finite
    differences above pin; routed and shared, every kind."""
    T, d, E, k, f, f_s = 9, 8, 5, 2, 12, 6
    inp = _inputs(T, d, E, k, f, 1, f_s, seed=7)
    inp["x"] = inp["x"] * 2.0
    ids = oracle.route(oracle.logits(inp["x"], inp["w_router"]), k, score_fn, renorm)["ids"]
    dy = RNG.normal(size=(T, d))
    g = oracle.backward(inp, ids, dy, score_fn, renorm)
    samples = []
    for e in range(E):
        samples += [("dw_gate", e, int(RNG.integers(f)), int(RNG.integers(d))),
                    ("dw_up", e, int(RNG.integers(f)), int(RNG.integers(d))),
                    ("dw_down", e, int(RNG.integers(d)), int(RNG.integers(f)))]
    samples += [("ds_gate", 0, 1, 2), ("ds_up", 0, 5, 7), ("ds_down", 0, 3, 4), ("ds_down", 0, 7, 0)]
    got = oracle.backward_weight_samples(inp, ids, dy, samples, score_fn, renorm)
    for (name, e, i, j), v in zip(samples, got):
        want = g[name][i, j] if name.startswith("ds_") else g[name][e, i, j]
        assert abs(v - want) <= 1e-12 * max(1.0, abs(want)), (name, e, i, j, v, want)


def test_dx_only_equals_full_backward():
    """weights=False (dx only, for full-size samples) gives the same dx."""
    inp = _inputs(6, 8, 5, 2, 12, 1, 6, seed=9)
    ids = oracle.route(oracle.logits(inp["x"], inp["w_router"]), 2, oracle.SIGMOID, 1)["ids"]
    dy = RNG.normal(size=(6, 8))
    full = oracle.backward(inp, ids, dy, oracle.SIGMOID, 1)
    only = oracle.backward(inp, ids, dy, oracle.SIGMOID, 1, weights=False)
    assert set(only) == {"dx"}
    np.testing.assert_array_equal(only["dx"], full["dx"])


def _loss_keep(inp, ids, dy, score_fn, renorm, keep):
    T = inp["x"].shape[0]
    y = oracle.forward_tokens(inp, ids.shape[1], np.arange(T), score_fn, renorm, forced_ids=ids, keep=keep)["y"]
    return float(np.sum(dy * y))


@pytest.mark.parametrize("score_fn,renorm,S", [(oracle.SOFTMAX, 1, 1), (oracle.SIGMOID, 1, 0), (oracle.SOFTMAX, 0, 0)])
def test_capacity_drops_match_finite_differences(score_fn, renorm, S):
    """Pairs an expert capacity dropped add nothing to y: the backward with
    the same keep mask matches central finite differences of the forward
    with that mask, for every input and weight tensor."""
    T, d, E, k, f = 8, 8, 4, 2, 12
    inp = _inputs(T, d, E, k, f, S, 4 if S else 0, seed=11)
    for n in ("x", "w_router"):
        inp[n] = inp[n] * 2.0
    ids = oracle.route(oracle.logits(inp["x"], inp["w_router"]), k, score_fn, renorm)["ids"]
    keep = (oracle.dispatch(ids, E, 3)["pair_pos"] >= 0).reshape(T, k)
    assert 0 < keep.sum() < T * k            # some pairs dropped, some kept
    dy = RNG.normal(size=(T, d))
    g = oracle.backward(inp, ids, dy, score_fn, renorm, keep=keep)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if inp.get(name) is None:
            continue
        v = RNG.normal(size=inp[name].shape)
        plus, minus = dict(inp), dict(inp)
        plus[name] = inp[name] + eps * v
        minus[name] = inp[name] - eps * v
        fd = (_loss_keep(plus, ids, dy, score_fn, renorm, keep) -
              _loss_keep(minus, ids, dy, score_fn, renorm, keep)) / (2 * eps)
        an = float(np.sum(g[gname] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}: finite difference {fd} vs gradient {an}"


def test_keep_all_equals_plain_backward():
    inp = _inputs(6, 8, 5, 2, 12, 1, 6, seed=12)
    ids = oracle.route(oracle.logits(inp["x"], inp["w_router"]), 2)["ids"]
    dy = RNG.normal(size=(6, 8))
    a = oracle.backward(inp, ids, dy)
    b = oracle.backward(inp, ids, dy, keep=np.ones((6, 2), bool))
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])


def _l_aux(lg, ids, score_fn, alpha):
    scores = oracle.route(lg, ids.shape[1], score_fn, 1, forced_ids=ids)["scores"]
    return oracle.router_stats(scores, ids, score_fn, alpha)["l_aux"]


@pytest.mark.parametrize("score_fn", [oracle.SOFTMAX, oracle.SIGMOID])
def test_aux_loss_gradient_matches_finite_differences(score_fn):
    """dL_aux/dl (the written-out probability Jacobian) against central finite
    differences of router_stats' L_aux in random logit directions, the
    assignment (hence f) held fixed."""
    T, E, k = 7, 6, 2
    lg = RNG.normal(size=(T, E)) * 1.5
    ids = oracle.route(lg, k, score_fn)["ids"]
    g = oracle.aux_loss_logit_grad(lg, ids, score_fn, 0.3)
    eps = 1e-6
    for _ in range(4):
        v = RNG.normal(size=lg.shape)
        fd = (_l_aux(lg + eps * v, ids, score_fn, 0.3) - _l_aux(lg - eps * v, ids, score_fn, 0.3)) / (2 * eps)
        an = float(np.sum(g * v))
        assert abs(fd - an) <= 1e-8 * max(1.0, abs(an)), (fd, an)


def test_aux_loss_gradient_vanishes_for_balanced_assignment():
    """With every expert picked equally often (f_e the same for all e), L_aux
    = alpha E f sum_e P_e = alpha E f, a constant: the probabilities of each
    token sum to 1 whatever the logits, so the gradient is zero."""
    T, E, k = 4, 8, 2
    lg = RNG.normal(size=(T, E)) * 2.0
    ids = np.array([[0, 1], [2, 3], [4, 5], [6, 7]])     # f_e = 1/4 for every e
    for score_fn in (oracle.SOFTMAX, oracle.SIGMOID):
        g = oracle.aux_loss_logit_grad(lg, ids, score_fn, 1.0)
        assert np.abs(g).max() < 1e-15


@pytest.mark.parametrize("score_fn,S", [(oracle.SOFTMAX, 1), (oracle.SIGMOID, 0)])
def test_backward_with_aux_loss_matches_finite_differences(score_fn, S):
    """L = sum(dy * y) + L_aux: the backward with aux_alpha against finite
    differences of the forward plus router_stats' L_aux, in x and W_r (the
    expert weights do not enter L_aux)."""
    T, d, E, k, f = 6, 8, 5, 2, 12
    inp = _inputs(T, d, E, k, f, S, 4 if S else 0, seed=13)
    for n in ("x", "w_router"):
        inp[n] = inp[n] * 2.0
    ids = oracle.route(oracle.logits(inp["x"], inp["w_router"]), k, score_fn, 1)["ids"]
    dy = RNG.normal(size=(T, d))
    alpha = 0.7
    g = oracle.backward(inp, ids, dy, score_fn, 1, aux_alpha=alpha)

    def loss(p):
        return _loss(p, ids, dy, score_fn, 1) + _l_aux(oracle.logits(p["x"], p["w_router"]), ids, score_fn, alpha)

    eps = 1e-6
    for name, gname in (("x", "dx"), ("w_router", "dw_router")):
        v = RNG.normal(size=inp[name].shape)
        plus, minus = dict(inp), dict(inp)
        plus[name] = inp[name] + eps * v
        minus[name] = inp[name] - eps * v
        fd = (loss(plus) - loss(minus)) / (2 * eps)
        an = float(np.sum(g[gname] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}: finite difference {fd} vs gradient {an}"
