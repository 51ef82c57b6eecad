"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a closed
form worked by hand, a special case that reduces to a different computation
(a dense softmax ensemble, a library routine, brute force over all expert
subsets), an invariant the pages state, or a count the pages print
(``tests/golden``).  The cases are chosen so that a plausible slip anywhere in
the oracle (SiLU on the wrong projection, a transposed operand, a dropped
shared-expert term, a wrong gate normaliser, a wrong tie order, an unstable
dispatch) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _f32_inputs(T, d, E, k, f, S=0, f_s=0, seed=0):
    sh = synth.LayerShape("t", T=T, d=d, E=E, k=k, d_ff=f, num_shared=S, d_ff_shared=f_s,
                          dtype=synth.F32)
    return sh, synth.make_inputs(sh, seed)


def _f64(a):
    return synth.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _dense_expert(x, wg, wu, wd):
    """f(x) = W_down (silu(W_gate x) * W_up x) for rows of x, by plain matmuls."""
    return (_silu(x @ wg.T) * (x @ wu.T)) @ wd.T


# --------------------------------------------------------------------------- closed forms

def test_closed_form_one_token_switch():
    """Hand-worked layer: E=2, d=2, d_ff=1, top-1.

    x = (1, 0), W_r = [[1,0],[0,0]] -> logits (1, 0): expert 0 wins with
    p0 = e/(e+1) = 0.7310585786300049.  Expert 0: W_gate x = 2, W_up x = 3,
    h = silu(2)*3 = 6/(1+e^-2) = 5.284782467867294 (SiLU on the up
    projection instead would give 5.7154447609345995), W_down = (1, -2)^T,
    so f_0(x) = (5.2848, -10.5696).  Switch form (no renorm):
    y = p0 f_0(x) = (3.8634855593278337, -7.726971118655667); with renorm
    over the single chosen expert y = f_0(x).
    """
    x = np.array([[1.0, 0.0]], dtype=np.float32)
    wr = np.array([[1.0, 0.0], [0.0, 0.0]], dtype=np.float32)
    wg = np.array([[[2.0, 5.0]], [[9.0, 9.0]]], dtype=np.float32)      # [E, d_ff=1, d]
    wu = np.array([[[3.0, 7.0]], [[9.0, 9.0]]], dtype=np.float32)
    wd = np.array([[[1.0], [-2.0]], [[9.0], [9.0]]], dtype=np.float32)  # [E, d, d_ff=1]
    inp = dict(x=x, w_router=wr, w_gate=wg, w_up=wu, w_down=wd)
    r = oracle.forward_tokens(inp, 1, [0], renormalize=0)
    assert r["ids"].tolist() == [[0]]
    np.testing.assert_allclose(r["gates"], [[0.7310585786300049]], rtol=1e-15)
    np.testing.assert_allclose(r["y"], [[3.8634855593278337, -7.726971118655667]], rtol=1e-14)
    r = oracle.forward_tokens(inp, 1, [0], renormalize=1)
    np.testing.assert_allclose(r["y"], [[5.284782467867294, -10.569564935734588]], rtol=1e-14)
    # same through the expert-loop form
    lg = oracle.logits(x, wr)
    rr = oracle.route(lg, 1, renormalize=0)
    y = oracle.forward_expert_loop(inp, rr["ids"], rr["gates"])
    np.testing.assert_allclose(y, [[3.8634855593278337, -7.726971118655667]], rtol=1e-14)


def test_closed_form_softmax_scores():
    """logits (0, ln2, ln3, ln4): softmax = (1,2,3,4)/10.  Top-2 = experts
    3, 2; renormalised gates 4/7, 3/7; raw gates 0.4, 0.3."""
    lg = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    r = oracle.route(lg, 2, oracle.SOFTMAX, 1)
    assert r["ids"].tolist() == [[3, 2]]
    np.testing.assert_allclose(r["gates"], [[4 / 7, 3 / 7]], rtol=1e-15)
    np.testing.assert_allclose(r["scores"], [[0.1, 0.2, 0.3, 0.4]], rtol=1e-15)
    np.testing.assert_allclose(r["gap_score"], [0.1], rtol=1e-13)
    np.testing.assert_allclose(r["gap_logit"], [math.log(1.5)], rtol=1e-13)
    r = oracle.route(lg, 2, oracle.SOFTMAX, 0)
    np.testing.assert_allclose(r["gates"], [[0.4, 0.3]], rtol=1e-15)


def test_closed_form_sigmoid_scores():
    """logits (0, ln3, -ln3, 2 ln3): sigmoid = (1/2, 3/4, 1/4, 9/10).  Top-2 =
    experts 3, 1; normalised among the selected: 0.9/1.65, 0.75/1.65."""
    l3 = math.log(3.0)
    lg = np.array([[0.0, l3, -l3, 2 * l3]])
    r = oracle.route(lg, 2, oracle.SIGMOID, 1)
    assert r["ids"].tolist() == [[3, 1]]
    np.testing.assert_allclose(r["scores"], [[0.5, 0.75, 0.25, 0.9]], rtol=1e-15)
    np.testing.assert_allclose(r["gates"], [[0.9 / 1.65, 0.75 / 1.65]], rtol=1e-15)
    r = oracle.route(lg, 2, oracle.SIGMOID, 0)
    np.testing.assert_allclose(r["gates"], [[0.9, 0.75]], rtol=1e-15)


def test_page_top2_example():
    g = json.load(open(os.path.join(GOLD, "top2_example.json")))
    lg = np.full((1, g["E"]), -10.0)
    lg[0, 7] = 0.0
    lg[0, 3] = math.log(g["gates"][0] / g["gates"][1])
    r = oracle.route(lg, g["k"], oracle.SOFTMAX, 1)
    assert r["ids"][0].tolist() == g["ids"]
    np.testing.assert_allclose(r["gates"][0], g["gates"], rtol=1e-14)


# --------------------------------------------------------------------------- routing invariants

@pytest.mark.parametrize("score_fn", [oracle.SOFTMAX, oracle.SIGMOID])
@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (16, 5), (64, 8), (256, 8), (7, 7)])
def test_renorm_gates_sum_to_one(score_fn, E, k):
    lg = RNG.normal(size=(200, E)) * 3
    r = oracle.route(lg, k, score_fn, 1)
    np.testing.assert_allclose(r["gates"].sum(1), 1.0, atol=1e-15 * k)
    assert (r["gates"] > 0).all()
    assert all(len(set(row)) == k for row in r["ids"].tolist())


@pytest.mark.parametrize("E,k", [(6, 1), (6, 2), (8, 3), (9, 4)])
def test_topk_is_best_subset_by_enumeration(E, k):
    """The chosen set maximises the sum of logits over all C(E,k) subsets
    (distinct logits), and the ids come in descending logit order."""
    lg = RNG.normal(size=(300, E))
    r = oracle.route(lg, k, oracle.SOFTMAX, 1)
    subsets = list(itertools.combinations(range(E), k))
    for t in range(lg.shape[0]):
        best = max(subsets, key=lambda s: sum(lg[t, list(s)]))
        assert set(r["ids"][t].tolist()) == set(best)
        assert np.all(np.diff(lg[t, r["ids"][t]]) < 0)


def test_two_gate_forms_agree():
    """Softmax over all E, keep the top-k and renormalise ('Mixture-of-Experts
    Internals', sec. 2.1) equals a softmax over the chosen logits alone
    ('8.6 Mixture of Experts', sec. 2)."""
    lg = RNG.normal(size=(500, 64)) * 4
    r = oracle.route(lg, 8, oracle.SOFTMAX, 1)
    sel = np.take_along_axis(lg, r["ids"].astype(np.int64), 1)
    ex = np.exp(sel - sel.max(1, keepdims=True))
    np.testing.assert_allclose(r["gates"], ex / ex.sum(1, keepdims=True), rtol=1e-13)


def test_ties_go_to_lower_index():
    lg = np.zeros((3, 8))
    r = oracle.route(lg, 3, oracle.SOFTMAX, 1)
    assert r["ids"].tolist() == [[0, 1, 2]] * 3
    np.testing.assert_allclose(r["gates"], 1 / 3, rtol=1e-15)
    lg = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    assert oracle.route(lg, 2)["ids"].tolist() == [[1, 2]]
    assert oracle.route(lg, 4)["ids"].tolist() == [[1, 2, 4, 3]]
    assert oracle.route(lg, 1)["ids"].tolist() == [[1]]
    lg = np.array([[-0.0, 0.0, 0.0]])   # -0 and +0 are equal logits
    assert oracle.route(lg, 2)["ids"].tolist() == [[0, 1]]


def test_selection_bias_changes_choice_not_gates():
    """Selection on h + b, gates from the unbiased scores ('Mixture-of-Experts
    Internals', sec. 3.3): b = 0 changes nothing; a huge b_e puts e in every
    token's set while its gate stays its unbiased renormalised score."""
    lg = RNG.normal(size=(100, 16))
    r0 = oracle.route(lg, 4)
    rb = oracle.route(lg, 4, bias=np.zeros(16))
    assert (r0["ids"] == rb["ids"]).all() and np.array_equal(r0["gates"], rb["gates"])
    b = np.zeros(16)
    b[5] = 1e6
    rb = oracle.route(lg, 4, bias=b)
    assert (rb["ids"][:, 0] == 5).all()
    s = np.exp(lg - lg.max(1, keepdims=True))
    sel = np.take_along_axis(s, rb["ids"].astype(np.int64), 1)
    np.testing.assert_allclose(rb["gates"], sel / sel.sum(1, keepdims=True), rtol=1e-13)


# --------------------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (333, 64, 8), (50, 256, 8), (1, 4, 4)])
def test_dispatch_is_stable_grouping(T, E, k):
    ids = np.stack([RNG.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch(ids, E)
    flat = ids.ravel()
    # counts: one per pair; they sum to T*k ("8.6 Mixture of Experts", sec. 3.1: sum_e f_e = k)
    assert d["counts"].sum() == T * k
    np.testing.assert_array_equal(d["counts"], np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(d["offsets"], np.concatenate([[0], np.cumsum(d["counts"])]))
    # the grouping is the library's stable sort of pairs by expert id
    np.testing.assert_array_equal(d["sorted_pairs"], np.argsort(flat, kind="stable"))
    # pair_pos is the inverse permutation
    np.testing.assert_array_equal(d["sorted_pairs"][d["pair_pos"]], np.arange(T * k))


def test_union_read_matches_page():
    """Batch of 32 tokens, each picking 8 of 64 experts uniformly: the share of
    experts the batch touches is 1 - (56/64)^32 (page prints about 98.6%)."""
    g = json.load(open(os.path.join(GOLD, "page_counts.json")))["union_read_fraction"]
    assert abs((1 - (56 / 64) ** 32) - g["value"]) < g["tolerance"]
    rng = np.random.default_rng(7)
    trials, touched = 3000, 0
    for _ in range(trials):
        ids = np.stack([rng.permutation(64)[:8] for _ in range(32)]).astype(np.int32)
        touched += int((oracle.dispatch(ids, 64)["counts"] > 0).sum())
    assert abs(touched / (trials * 64) - g["value"]) < 0.002


# --------------------------------------------------------------------------- single expert, row ranges

@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
def test_expert_rows_is_the_dense_expert(dtype):
    """expert_rows(e, rows) is expert e's SwiGLU on the listed token rows
    ('8.6 Mixture of Experts', sec. 2; 'What Actually Happens...', Step 4):
    h = silu(W_gate,e x) * (W_up,e x) and o = W_down,e h, equal to plain
    matmuls on the widened inputs, for experts past the first, rows out of
    order and repeated, d != d_ff; the o of a call without h is the same."""
    sh = synth.LayerShape("t", T=23, d=48, E=5, k=2, d_ff=40, dtype=dtype)
    inp = synth.make_inputs(sh, 21)
    x = _f64(inp["x"])
    rows = np.array([7, 0, 22, 7, 13, 13, 1], dtype=np.int32)
    for e in (1, 4):
        wg, wu, wd = (_f64(inp[n][e]) for n in ("w_gate", "w_up", "w_down"))
        h_want = _silu(x[rows] @ wg.T) * (x[rows] @ wu.T)
        h, o = oracle.expert_rows(e, inp["x"], rows, inp["w_gate"], inp["w_up"], inp["w_down"], want_h=True)
        assert h.shape == (rows.size, 40) and o.shape == (rows.size, 48)
        np.testing.assert_allclose(h, h_want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(o, h_want @ wd.T, rtol=1e-12, atol=1e-14)
        h0, o0 = oracle.expert_rows(e, inp["x"], rows, inp["w_gate"], inp["w_up"], inp["w_down"])
        assert h0 is None
        np.testing.assert_array_equal(o0, o)


def test_expert_rows_matches_top1_layer():
    """Top-1 with renormalisation: each token's y is its one expert's output
    (the Switch form, 'from the router to the all-to-all', The router), so
    expert_rows on the tokens that chose e equals forward_tokens' y there."""
    sh, inp = _f32_inputs(T=31, d=32, E=4, k=1, f=48, seed=17)
    r = oracle.forward_tokens(inp, 1, np.arange(31))
    for e in range(4):
        toks = np.nonzero(r["ids"][:, 0] == e)[0].astype(np.int32)
        if toks.size == 0:
            continue
        _, o = oracle.expert_rows(e, inp["x"], toks, inp["w_gate"], inp["w_up"], inp["w_down"])
        np.testing.assert_allclose(o, r["y"][toks], rtol=1e-12, atol=1e-13)


def test_logits_of_a_row_range():
    """logits(rows=slice(a, b)) is rows a..b-1 of x W_r^T (plain matmul)."""
    sh, inp = _f32_inputs(T=29, d=24, E=7, k=2, f=16, seed=19)
    want = _f64(inp["x"]) @ _f64(inp["w_router"]).T
    np.testing.assert_allclose(oracle.logits(inp["x"], inp["w_router"], rows=slice(5, 17)), want[5:17],
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(oracle.logits(inp["x"], inp["w_router"], rows=slice(20, None)), want[20:],
                               rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- whole layer

def test_dense_softmax_ensemble_when_k_equals_E():
    """k = E with softmax: y = sum_e softmax(h)_e f_e(x), computed densely with
    no selection or grouping (renorm on or off gives the same)."""
    sh, inp = _f32_inputs(T=40, d=32, E=6, k=6, f=48)
    x = _f64(inp["x"])
    lg = x @ _f64(inp["w_router"]).T
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = sum(p[:, e:e + 1] * _dense_expert(x, _f64(inp["w_gate"][e]), _f64(inp["w_up"][e]),
                                             _f64(inp["w_down"][e])) for e in range(6))
    for renorm in (0, 1):
        r = oracle.forward(inp, 6, renormalize=renorm)
        np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)
        r = oracle.forward_tokens(inp, 6, np.arange(40), renormalize=renorm)
        np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


def test_switch_top1():
    """k=1 without renorm: y = p_i f_i(x), p_i the full-softmax probability of
    the argmax; with renorm y = f_i(x)."""
    sh, inp = _f32_inputs(T=50, d=32, E=8, k=1, f=64, seed=3)
    x = _f64(inp["x"])
    lg = x @ _f64(inp["w_router"]).T
    i = lg.argmax(1)
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    fx = np.stack([_dense_expert(x[t:t + 1], _f64(inp["w_gate"][i[t]]), _f64(inp["w_up"][i[t]]),
                                 _f64(inp["w_down"][i[t]]))[0] for t in range(50)])
    r0 = oracle.forward(inp, 1, renormalize=0)
    np.testing.assert_array_equal(r0["ids"][:, 0], i)
    np.testing.assert_allclose(r0["y"], p[np.arange(50), i][:, None] * fx, rtol=1e-12, atol=1e-13)
    r1 = oracle.forward(inp, 1, renormalize=1)
    np.testing.assert_allclose(r1["y"], fx, rtol=1e-12, atol=1e-13)


def test_identical_experts_give_the_single_expert():
    """All experts equal + renorm: the output is a convex combination of equal
    vectors, so y = f(x) whatever the routing."""
    sh, inp = _f32_inputs(T=30, d=32, E=8, k=3, f=40, seed=5)
    for n in ("w_gate", "w_up", "w_down"):
        inp[n] = np.ascontiguousarray(np.repeat(inp[n][:1], 8, axis=0))
    x = _f64(inp["x"])
    want = _dense_expert(x, _f64(inp["w_gate"][0]), _f64(inp["w_up"][0]), _f64(inp["w_down"][0]))
    r = oracle.forward(inp, 3)
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


def test_zero_tokens():
    """x = 0: every logit is 0, so ids are 0..k-1 with gates 1/k, and
    silu(0)*0 = 0 makes y = 0."""
    sh, inp = _f32_inputs(T=5, d=16, E=8, k=3, f=32)
    inp["x"] = np.zeros_like(inp["x"])
    r = oracle.forward(inp, 3)
    assert r["ids"].tolist() == [[0, 1, 2]] * 5
    np.testing.assert_allclose(r["gates"], 1 / 3, rtol=1e-15)
    assert np.all(r["y"] == 0.0)


def test_shared_expert_is_additive():
    """y(with shared) - y(without) = f_shared(x), ungated
    ('8.6 Mixture of Experts', sec. 4.1)."""
    sh, inp = _f32_inputs(T=20, d=32, E=8, k=2, f=48, S=1, f_s=64, seed=9)
    r1 = oracle.forward(inp, 2)
    noshared = dict(inp, ws_gate=None, ws_up=None, ws_down=None)
    r0 = oracle.forward(noshared, 2)
    x = _f64(inp["x"])
    fs = _dense_expert(x, _f64(inp["ws_gate"]), _f64(inp["ws_up"]), _f64(inp["ws_down"]))
    np.testing.assert_allclose(r1["y"] - r0["y"], fs, rtol=1e-11, atol=1e-12)
    t1 = oracle.forward_tokens(inp, 2, np.arange(20))
    np.testing.assert_allclose(t1["y"], r1["y"], rtol=1e-12, atol=1e-13)


def test_relabelling_experts_permutes_ids_only():
    sh, inp = _f32_inputs(T=60, d=32, E=8, k=2, f=48, seed=11)
    perm = RNG.permutation(8)          # new expert j is old expert perm[j]
    inv = np.argsort(perm)
    inp2 = dict(inp)
    for n in ("w_router", "w_gate", "w_up", "w_down"):
        inp2[n] = np.ascontiguousarray(inp[n][perm])
    r1, r2 = oracle.forward(inp, 2), oracle.forward(inp2, 2)
    np.testing.assert_array_equal(inv[r1["ids"]], r2["ids"])
    np.testing.assert_allclose(r1["y"], r2["y"], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("name", ["tiny"])
def test_torch_module_crosscheck(name):
    """The layer written as the page's PyTorch module (nn.Linear router and
    experts, softmax, topk, renorm, per-expert masked loop) in float64 on the
    CPU agrees with the oracle."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    sh = synth.SHAPES[name]
    inp = synth.make_inputs(sh, 0)
    x = torch.from_numpy(_f64(inp["x"]))
    wr = torch.from_numpy(_f64(inp["w_router"]))
    with torch.no_grad():
        probs = F.softmax(F.linear(x, wr), dim=-1)
        tp, ti = torch.topk(probs, sh.k, dim=-1)
        tp = tp / tp.sum(-1, keepdim=True)
        y = torch.zeros_like(x)
        for e in range(sh.E):
            mask = (ti == e)
            rows = mask.any(1)
            if not rows.any():
                continue
            xe = x[rows]
            g = torch.from_numpy(_f64(inp["w_gate"][e]))
            u = torch.from_numpy(_f64(inp["w_up"][e]))
            dn = torch.from_numpy(_f64(inp["w_down"][e]))
            out = F.linear(F.silu(F.linear(xe, g)) * F.linear(xe, u), dn)
            w = (tp * mask)[rows].sum(1, keepdim=True)
            y[rows] += w * out
    r = oracle.forward(inp, sh.k)
    assert (r["gap_logit"] > 1e-9).all()      # no ties: torch's tie order is unspecified
    np.testing.assert_array_equal(np.sort(r["ids"], 1), np.sort(ti.numpy(), 1))
    np.testing.assert_allclose(r["y"], y.numpy(), rtol=1e-12, atol=1e-13)


def test_two_layer_forms_agree_bf16():
    """Expert-loop form == per-token form on bf16 inputs with k=8 and a
    shared expert (sum orders differ, so within fp64 rounding)."""
    sh = synth.LayerShape("t", T=48, d=64, E=32, k=8, d_ff=64, num_shared=1, d_ff_shared=64,
                          score_fn=synth.SIGMOID)
    inp = synth.make_inputs(sh, 2)
    r = oracle.forward(inp, 8, score_fn=oracle.SIGMOID)
    t = oracle.forward_tokens(inp, 8, np.arange(48), score_fn=oracle.SIGMOID)
    assert (r["ids"] == t["ids"]).all()
    np.testing.assert_allclose(t["y"], r["y"], rtol=1e-12, atol=1e-13)


def test_forced_ids_reproduce_and_override():
    sh, inp = _f32_inputs(T=16, d=32, E=8, k=2, f=32, seed=4)
    r = oracle.forward_tokens(inp, 2, np.arange(16))
    f = oracle.forward_tokens(inp, 2, np.arange(16), forced_ids=r["ids"])
    np.testing.assert_array_equal(f["y"], r["y"])
    swapped = r["ids"][:, ::-1].copy()
    g = oracle.forward_tokens(inp, 2, np.arange(16), forced_ids=swapped)
    np.testing.assert_allclose(g["gates"], r["gates"][:, ::-1], rtol=1e-15)
    np.testing.assert_allclose(g["y"], r["y"], rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- shapes

def test_layer_shapes_match_page_counts():
    g = json.load(open(os.path.join(GOLD, "page_counts.json")))
    S = synth.SHAPES
    assert 3 * S["hunyuan_a13b"].d * S["hunyuan_a13b"].d_ff == g["hunyuan_a13b_expert_weights"]["value"]
    assert S["hunyuan_a13b"].E * S["hunyuan_a13b"].d == g["hunyuan_a13b_router_weights"]["value"]
    assert 3 * S["deepseek_v3"].d * S["deepseek_v3"].d_ff == g["deepseek_v3_expert_weights"]["value"]
    assert S["mixtral_prefill"].E * S["mixtral_prefill"].d == g["mixtral_router_weights"]["value"]
    assert S["deepseek_v3"].k * S["deepseek_v3"].d == g["deepseek_v3_token_fanout"]["value"]
    c = g["combinations"]["values"]
    assert math.comb(8, 2) == c["C(8,2)"] and math.comb(32, 8) == c["C(32,8)"]
    assert math.comb(16, 2) == c["C(16,2)"] and math.comb(64, 8) == c["C(64,8)"]
    # ~22.5 GB of routed bf16 weights in the DeepSeek-V3-shaped layer
    assert abs(256 * g["deepseek_v3_expert_weights"]["value"] * 2 / 1e9 - 22.55) < 0.01
