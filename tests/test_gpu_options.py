"""GPU parity of the optional routing features against the CPU oracle:
selection-only expert bias (on logits or on scores), per-expert capacity with
dropped pairs, and router load statistics.  Same rules as the plain layer:
ids in order except at near-ties of the selection key, bit-exact dispatch,
gates within 1e-5, y within tau * max|y| with the oracle given the GPU's ids
(and its dropped pairs)."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import LOGIT_TIE, NEAR_TIE, TAU, DeviceLayer, assert_close, check_ids, to_dev, to_host, torch

pytestmark = pytest.mark.gpu
S = synth.LayerShape


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch().cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    import mixture_experts_sparse_moe_amd as moe
    moe.lib()


def moe_mod():
    import mixture_experts_sparse_moe_amd as moe
    return moe


def selection_keys(lg, scores, b, on_scores, score_fn):
    """The oracle's selection key [T,E] for a selection bias b, and the key in
    score space: key = score + b (already a score), or key = logit + b,
    whose score image is the score function of the biased logits (softmax
    over the experts, or the sigmoid)."""
    if on_scores:
        key = scores + b
        return key, key
    key = lg + b
    if score_fn == synth.SIGMOID:
        return key, 1.0 / (1.0 + np.exp(-key))
    e = np.exp(key - key.max(1, keepdims=True))
    return key, e / e.sum(1, keepdims=True)


def check_ids_keyspace(gids, ref, key, key_score, on_scores):
    """Ids in order against the oracle's biased selection, by the near-tie
    rule of the plain path (check_ids): every differing slot sits at a
    near-tie of the selection key (score space 1e-6; a logit key also within
    the fp32 logit band).  Returns exempt tokens."""
    return check_ids(gids, ref["ids"], key, key_score, NEAR_TIE if on_scores else LOGIT_TIE, NEAR_TIE)


def run_route_ex(L, opts):
    t = torch()
    sh = L.sh
    ids = t.empty(sh.T, sh.k, dtype=t.int32, device="cuda")
    wts = t.empty(sh.T, sh.k, dtype=t.float32, device="cuda")
    gap = t.empty(sh.T, 2, dtype=t.float32, device="cuda")
    moe_mod().moe_route_ex(L.cfg, opts, L.d["x"], L.d["w_router"], ids, wts, gap, ws=L.ws)
    return ids, wts, gap


def run_forward_ex(L, opts):
    t = torch()
    sh = L.sh
    y = L.empty_act(sh.T, sh.d)
    ids = t.empty(sh.T, sh.k, dtype=t.int32, device="cuda")
    wts = t.empty(sh.T, sh.k, dtype=t.float32, device="cuda")
    counts = t.empty(sh.E, dtype=t.int32, device="cuda")
    gap = t.empty(sh.T, 2, dtype=t.float32, device="cuda")
    dv = L.d
    moe_mod().moe_forward_ex(L.cfg, opts, dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                             dv["ws_gate"], dv["ws_up"], dv["ws_down"], y, ids, wts, counts, L.ws, topk_gap=gap)
    return dict(y=y, ids=ids, weights=wts, counts=counts, gap=gap)


BIAS_CASES = {
    # name: (shape, bias_on_scores, bias scale)
    "logit_softmax_e64": (S("c", T=300, d=256, E=64, k=6, d_ff=128), 0, 1.0),
    "score_sigmoid_e256_shared": (S("c", T=260, d=256, E=256, k=8, d_ff=64, num_shared=1, d_ff_shared=128,
                                    score_fn=synth.SIGMOID), 1, 0.05),
    "score_softmax_e16_raw": (S("c", T=200, d=128, E=16, k=2, d_ff=128, renormalize=0), 1, 0.05),
    "score_sigmoid_decode": (S("c", T=24, d=1024, E=64, k=6, d_ff=128, score_fn=synth.SIGMOID), 1, 0.05),
    "fp32_logit_e8": (S("c", T=64, d=64, E=8, k=2, d_ff=128, dtype=synth.F32), 0, 1.0),
}


@pytest.mark.parametrize("name", sorted(BIAS_CASES))
def test_selection_bias(name):
    sh, on_scores, scale = BIAS_CASES[name]
    say(f"[case] bias {name} {sh}")
    inp = synth.make_inputs(sh, 11)
    rng = np.random.default_rng(5)
    b = (rng.normal(size=sh.E) * scale).astype(np.float32)
    L = DeviceLayer(sh, inp)
    moe = moe_mod()
    bd = to_dev(b)
    opts = moe.MoeOptions.of(expert_bias=bd, bias_on_scores=on_scores)
    ids, wts, gap = run_route_ex(L, opts)
    fw = run_forward_ex(L, opts)
    torch().cuda.synchronize()
    lg = oracle.logits(inp["x"], inp["w_router"])
    ref = oracle.route(lg, sh.k, sh.score_fn, sh.renormalize, bias=b.astype(np.float64),
                       bias_on_scores=on_scores)
    plain = oracle.route(lg, sh.k, sh.score_fn, sh.renormalize)
    changed = int((ref["ids"] != plain["ids"]).any(1).sum())
    key, key_score = selection_keys(lg, plain["scores"], b.astype(np.float64), on_scores, sh.score_fn)
    gids = to_host(ids)
    ex = check_ids_keyspace(gids, ref, key, key_score, on_scores)
    fids = to_host(fw["ids"])
    fex = check_ids_keyspace(fids, ref, key, key_score, on_scores)
    rf = oracle.route(lg, sh.k, sh.score_fn, sh.renormalize, forced_ids=gids)
    np.testing.assert_allclose(to_host(wts), rf["gates"], atol=1e-5, rtol=0)
    # margins: the selection key's (score-space keys to fp32 score accuracy,
    # logit keys as the plain logits), and the unbiased score margin of the
    # same two experts
    for g, skip in ((to_host(gap), ex), (to_host(fw["gap"]), fex)):
        ok = np.setdiff1d(np.arange(sh.T), skip)
        np.testing.assert_allclose(g[ok, 0], ref["gap_logit"][ok], atol=2e-6 if on_scores else 1e-3,
                                   rtol=1e-3 if on_scores else 1e-4, err_msg="key margin")
        np.testing.assert_allclose(g[ok, 1], ref["gap_score"][ok], atol=2e-6, rtol=1e-3, err_msg="score margin")
    rff = oracle.route(lg, sh.k, sh.score_fn, sh.renormalize, forced_ids=fids)
    np.testing.assert_allclose(to_host(fw["weights"]), rff["gates"], atol=1e-5, rtol=0)
    toks = np.arange(sh.T) if sh.T <= 64 else np.unique(np.concatenate([[0, sh.T - 1],
                                                                          rng.integers(0, sh.T, 30)]))
    r = oracle.forward_tokens(inp, sh.k, toks, sh.score_fn, sh.renormalize, forced_ids=fids[toks])
    widen = synth.bf16_to_f64 if sh.dtype == synth.BF16 else (lambda a: a.astype(np.float64))
    rel = assert_close(widen(to_host(fw["y"]))[toks], r["y"], TAU[sh.dtype], "y of moe_forward_ex")
    say(f"[ok] bias moved {changed}/{sh.T} tokens' choices, near-ties {ex.tolist()}, rel {rel:.2e}")
    assert changed > 0 or sh.T < 32


def test_huge_bias_forces_an_expert():
    sh = S("c", T=150, d=128, E=32, k=4, d_ff=64, score_fn=synth.SIGMOID)
    inp = synth.make_inputs(sh, 2)
    L = DeviceLayer(sh, inp)
    moe = moe_mod()
    for on_scores in (0, 1):
        b = np.zeros(sh.E, dtype=np.float32)
        b[9] = 1e4
        opts = moe.MoeOptions.of(expert_bias=to_dev(b), bias_on_scores=on_scores)
        ids, wts, _ = run_route_ex(L, opts)
        torch().cuda.synchronize()
        gids = to_host(ids)
        assert (gids[:, 0] == 9).all()
        lg = oracle.logits(inp["x"], inp["w_router"])
        rf = oracle.route(lg, sh.k, sh.score_fn, 1, forced_ids=gids)
        np.testing.assert_allclose(to_host(wts), rf["gates"], atol=1e-5, rtol=0)


CAP_CASES = {
    # skewed loads so that capacity drops pairs; one decode-sized case (fused
    # router + dispatch), one with several dispatch chunks
    "zipf_e64_k8": (S("c", T=520, d=256, E=64, k=8, d_ff=256, zipf_s=1.1), 1.0),
    "x4router_e8_k2": (S("c", T=600, d=256, E=8, k=2, d_ff=384, router_scale=4.0), 0.9),
    "decode_e16_k4": (S("c", T=20, d=1024, E=16, k=4, d_ff=128), 0.8),
    "chunks_e32_k4": (S("c", T=1300, d=128, E=32, k=4, d_ff=64, zipf_s=1.1), 1.1),
    "fp32_e8_k2": (S("c", T=64, d=64, E=8, k=2, d_ff=128, dtype=synth.F32), 0.75),
    # 640 or more rows per expert: the tile height chosen on the device from
    # the kept counts, and a combine for each down K split
    "fixed_tile_choice_e8_k2": (S("c", T=3264, d=256, E=8, k=2, d_ff=8192), 1.0),
}


@pytest.mark.parametrize("name", sorted(CAP_CASES))
def test_capacity_drops(name):
    sh, factor = CAP_CASES[name]
    say(f"[case] capacity {name} {sh} factor {factor}")
    inp = synth.make_inputs(sh, 3)
    L = DeviceLayer(sh, inp)
    moe = moe_mod()
    t = torch()
    cap = moe.capacity(sh.T, sh.k, sh.E, factor)
    assert cap == oracle.capacity(sh.T, sh.k, sh.E, factor)
    stats = t.full((2 * sh.E + 3,), -1.0, dtype=t.float32, device="cuda")
    opts = moe.MoeOptions.of(expert_capacity=cap, router_stats=stats)
    st = L.steps()                                   # plain routing: the ids to dispatch
    P = sh.T * sh.k
    counts = t.empty(sh.E, dtype=t.int32, device="cuda")
    offsets = t.empty(sh.E + 1, dtype=t.int32, device="cuda")
    sp = t.full((P,), -7, dtype=t.int32, device="cuda")
    pp = t.empty(P, dtype=t.int32, device="cuda")
    moe.moe_dispatch_ex(L.cfg, opts, st["ids"], counts, offsets, sp, pp, L.ws)
    fw = run_forward_ex(L, opts)
    t.cuda.synchronize()
    gids = to_host(st["ids"])
    d = oracle.dispatch(gids, sh.E, cap=cap)
    np.testing.assert_array_equal(to_host(counts), d["counts"])
    np.testing.assert_array_equal(to_host(offsets), d["offsets"])
    np.testing.assert_array_equal(to_host(pp), d["pair_pos"])
    kept = int(d["offsets"][sh.E])
    np.testing.assert_array_equal(to_host(sp)[:kept], d["sorted_pairs"][:kept])
    dropped = int((d["pair_pos"] < 0).sum())
    assert dropped > 0, "the case should drop pairs"
    # whole layer with the capacity: its own routing (the same ids unless at
    # a near-tie), its kept-pair counts, y with the dropped pairs left out
    fids = to_host(fw["ids"])
    fd = oracle.dispatch(fids, sh.E, cap=cap)
    np.testing.assert_array_equal(to_host(fw["counts"]), fd["counts"])
    # the statistics' overflow: the pairs this capacity drops from the call's routing
    lg = oracle.logits(inp["x"], inp["w_router"])
    sref = oracle.router_stats(oracle.route(lg, sh.k, sh.score_fn, sh.renormalize)["scores"], fids,
                               sh.score_fn, 0.0, cap=cap)
    g = to_host(stats)
    assert g[2 * sh.E + 2] == sref["overflow"] == int((fd["pair_pos"] < 0).sum())
    keep = (fd["pair_pos"] >= 0).reshape(sh.T, sh.k).astype(np.int32)
    rng = np.random.default_rng(1)
    toks = np.arange(sh.T) if sh.T <= 80 else np.unique(np.concatenate([[0, sh.T - 1],
                                                                          rng.integers(0, sh.T, 40)]))
    r = oracle.forward_tokens(inp, sh.k, toks, sh.score_fn, sh.renormalize, forced_ids=fids[toks],
                              keep=keep[toks])
    widen = synth.bf16_to_f64 if sh.dtype == synth.BF16 else (lambda a: a.astype(np.float64))
    rel = assert_close(widen(to_host(fw["y"]))[toks], r["y"], TAU[sh.dtype], "y with capacity")
    say(f"[ok] capacity {cap}: dropped {dropped}/{P} pairs, rel {rel:.2e}")


STATS_CASES = {
    "softmax_e8_k2": S("c", T=600, d=256, E=8, k=2, d_ff=128, router_scale=4.0),
    "sigmoid_e256_k8": S("c", T=300, d=256, E=256, k=8, d_ff=64, score_fn=synth.SIGMOID),
    "zipf_e64_k8": S("c", T=520, d=256, E=64, k=8, d_ff=64, zipf_s=1.1),
    "decode_e8_k2": S("c", T=32, d=1024, E=8, k=2, d_ff=128),
    "fp32_e8_k2": S("c", T=64, d=64, E=8, k=2, d_ff=128, dtype=synth.F32),
}


@pytest.mark.parametrize("name", sorted(STATS_CASES))
def test_router_stats(name):
    sh = STATS_CASES[name]
    say(f"[case] stats {name} {sh}")
    inp = synth.make_inputs(sh, 4)
    L = DeviceLayer(sh, inp)
    moe = moe_mod()
    t = torch()
    out = t.full((2 * sh.E + 3,), -1.0, dtype=t.float32, device="cuda")
    out2 = t.full((2 * sh.E + 3,), -1.0, dtype=t.float32, device="cuda")
    alpha = 0.01
    ids, _, _ = run_route_ex(L, moe.MoeOptions.of(router_stats=out, aux_alpha=alpha))
    fw = run_forward_ex(L, moe.MoeOptions.of(router_stats=out2, aux_alpha=alpha))
    t.cuda.synchronize()
    lg = oracle.logits(inp["x"], inp["w_router"])
    s = oracle.route(lg, sh.k, sh.score_fn, sh.renormalize)["scores"]
    for o, i in ((out, ids), (out2, fw["ids"])):
        g = to_host(o).astype(np.float64)
        ref = oracle.router_stats(s, to_host(i), sh.score_fn, alpha)
        E = sh.E
        np.testing.assert_allclose(g[:E], ref["f"], rtol=1e-6, atol=0)      # counts / T
        np.testing.assert_allclose(g[E:2 * E], ref["P"], atol=2e-6, rtol=1e-4)
        np.testing.assert_allclose(g[2 * E], ref["l_aux"], rtol=1e-4)
        np.testing.assert_allclose(g[2 * E + 1], ref["max_over_mean"], rtol=1e-6)
        assert g[2 * E + 2] == 0.0          # no capacity: no overflow
    say(f"[ok] L_aux {float(to_host(out)[2 * sh.E]):.5f} max/mean {float(to_host(out)[2 * sh.E + 1]):.3f}")


def test_options_leave_plain_results_unchanged():
    """All-zero options give bitwise the plain calls' results."""
    sh = S("c", T=333, d=192, E=8, k=2, d_ff=320)
    inp = synth.make_inputs(sh, 6)
    L = DeviceLayer(sh, inp)
    moe = moe_mod()
    a = L.forward()
    b = run_forward_ex(L, moe.MoeOptions.of())
    st = L.steps()
    ids, wts, gap = run_route_ex(L, moe.MoeOptions.of())
    torch().cuda.synchronize()
    for n in ("y", "ids", "weights", "counts"):
        np.testing.assert_array_equal(to_host(a[n]), to_host(b[n]), err_msg=n)
    np.testing.assert_array_equal(to_host(ids), to_host(st["ids"]))
    np.testing.assert_array_equal(to_host(wts), to_host(st["weights"]))
    np.testing.assert_array_equal(to_host(gap), to_host(st["gap"]))
