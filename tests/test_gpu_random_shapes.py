"""Seeded random layer shapes, beyond the hand-picked cases: both dtypes,
1 to 256 experts, k up to 16, widths in steps of 64 (ragged against every
tile), with or without a shared expert, softmax or sigmoid, renormalised or
raw gates, uniform or Zipf-skewed routing.  Every shape gets the full forward
check of test_gpu_parity (routing bit-exact, dispatch bit-exact, expert
outputs and y against the oracle); the shapes small enough for the oracle's
chain rule also get the backward check."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import TAU, DeviceLayer, assert_close, to_dev, to_host, torch
from test_gpu_backward import NAMES, run_backward
from test_gpu_parity import check_layer

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


def random_shapes(n=48, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = synth.F32 if i % 4 == 0 else synth.BF16
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 100, 256]))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.choice([1, 7, 32, 33, 100, 257, 600]))
        d = 64 * int(rng.integers(1, 9))
        d_ff = 64 * int(rng.integers(1, 9))
        shared = bool(rng.random() < 0.3)
        d_ff_s = 64 * int(rng.integers(1, 5)) if shared else 0
        score = synth.SIGMOID if rng.random() < 0.4 else synth.SOFTMAX
        renorm = 0 if rng.random() < 0.25 else 1
        # the skew shifts x along W_r^T (W_r W_r^T)^-1 b, which needs E <= d
        zipf = 1.1 if (rng.random() < 0.3 and 4 <= E <= d) else 0.0
        out.append(S(f"r{i:02d}", T=T, d=d, E=E, k=k, d_ff=d_ff, num_shared=int(shared), d_ff_shared=d_ff_s,
                     score_fn=score, renormalize=renorm, dtype=dtype, zipf_s=zipf))
    return out


SHAPES = {sh.name: sh for sh in random_shapes()}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_random_shape_forward(name):
    sh = SHAPES[name]
    check_layer(sh, synth.make_inputs(sh, 31))


def random_merged_shapes(n=6, seed=7):
    """bf16 layers whose shared expert moe_forward runs inside the routed
    GEMMs: as wide as the routed experts, about one M tile per expert (the
    tile queue), more than one dispatch chunk of pairs, d a multiple of 256."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([16, 32, 64, 100, 256]))
        k = int(rng.integers(1, min(E, 16) + 1))
        d = 256 * int(rng.integers(1, 4))
        d_ff = 128 * int(rng.integers(1, 5))
        T = int(rng.integers(200, 1500))
        P = T * k
        if not (P > 2048 and P < 640 * E and P > 32 * E):
            continue
        score = synth.SIGMOID if rng.random() < 0.5 else synth.SOFTMAX
        zipf = 1.1 if (rng.random() < 0.3 and E <= d) else 0.0
        out.append(S(f"m{len(out):02d}", T=T, d=d, E=E, k=k, d_ff=d_ff, num_shared=1, d_ff_shared=d_ff,
                     score_fn=score, zipf_s=zipf))
    return out


MERGED = {sh.name: sh for sh in random_merged_shapes()}


@pytest.mark.parametrize("name", sorted(MERGED))
def test_random_shape_forward_shared_merged(name):
    import mixture_experts_sparse_moe_amd as moe
    from gpu_harness import cfg_of
    sh = MERGED[name]
    assert moe.moe_forward_plan(cfg_of(sh))["shared_merged"], "the shape must take the merged path"
    check_layer(sh, synth.make_inputs(sh, 43))


def random_tall_shapes(n=6, seed=11):
    """bf16 layers whose routed GEMMs take 288-row tiles: 224 to 287 rows per
    expert on average, d a multiple of 256 and d_ff of 128 (the persistent
    kernels), with or without a shared expert (as wide as the routed ones,
    so inside their launches, or narrower), uniform or skewed routing."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([8, 16, 32, 64]))
        k = int(rng.integers(1, min(E, 16) + 1))
        d = 256 * int(rng.integers(1, 3))
        d_ff = 128 * int(rng.integers(1, 4))
        T = -(-E * int(rng.integers(224, 288)) // k)
        if not 224 * E <= T * k < 288 * E:
            continue
        shared = int(rng.integers(0, 3))           # none, same width, narrower
        d_ff_s = (d_ff, 128)[shared - 1] if shared else 0
        score = synth.SIGMOID if rng.random() < 0.5 else synth.SOFTMAX
        zipf = 1.1 if (rng.random() < 0.3 and E <= d) else 0.0
        out.append(S(f"t{len(out):02d}", T=T, d=d, E=E, k=k, d_ff=d_ff, num_shared=int(shared > 0),
                     d_ff_shared=d_ff_s, score_fn=score, zipf_s=zipf))
    return out


TALL = {sh.name: sh for sh in random_tall_shapes()}


@pytest.mark.parametrize("name", sorted(TALL))
def test_random_shape_forward_tall_tiles(name):
    import mixture_experts_sparse_moe_amd as moe
    from gpu_harness import cfg_of
    sh = TALL[name]
    assert moe.moe_forward_plan(cfg_of(sh))["tile_rows"] == 288, "the shape must take the 288-row tiles"
    check_layer(sh, synth.make_inputs(sh, 47))


# the oracle's chain rule costs about 12 d d_ff fp64 multiply-adds per pair
BACKWARD = sorted(n for n, sh in SHAPES.items() if sh.T * sh.k * sh.d * sh.d_ff <= 2.5e8)


@pytest.mark.parametrize("name", BACKWARD)
def test_random_shape_backward(name):
    sh = SHAPES[name]
    say(f"[case] backward {sh}")
    inp = synth.make_inputs(sh, 37)
    L = DeviceLayer(sh, inp)
    st = L.steps()
    dy_h = synth.normal(37, 99, sh.T * sh.d, 1.0, sh.dtype).reshape(sh.T, sh.d)
    dy_ref = synth.bf16_to_f64(dy_h) if sh.dtype == synth.BF16 else dy_h.astype(np.float64)
    out = run_backward(L, st["ids"], st["weights"], to_dev(dy_h))
    torch().cuda.synchronize()
    gids = to_host(st["ids"])
    ref = oracle.backward(inp, gids, dy_ref, sh.score_fn, sh.renormalize)
    tau = TAU[sh.dtype]
    worst = 0.0
    for gname, rname in NAMES:
        if gname not in out:
            continue
        want = ref[rname]
        got = to_host(out[gname]).astype(np.float64)
        if np.abs(want).max() < 1e-10:       # zero up to the oracle's rounding
            assert np.abs(got).max() <= 1e-6, f"{gname} should be zero"
            continue
        worst = max(worst, assert_close(got, want, tau, gname))
    say(f"[ok] worst max|err|/max|ref| = {worst:.2e}")


@pytest.mark.parametrize("name", BACKWARD)
def test_random_shape_capacity_and_aux_loss(name):
    """The same shapes trained with an expert capacity (factor 0.8, so pairs
    are dropped) and the load-balancing loss: moe_forward_ex's y against the
    oracle's forward without the dropped pairs, and moe_backward_ex's
    gradients against the oracle's backward with the same keep mask and
    alpha."""
    import mixture_experts_sparse_moe_amd as moe
    t = torch()
    sh = SHAPES[name]
    cap = moe.capacity(sh.T, sh.k, sh.E, 0.8)
    say(f"[case] capacity {cap} + aux loss {sh}")
    inp = synth.make_inputs(sh, 41)
    L = DeviceLayer(sh, inp)
    dv = L.d
    y = L.empty_act(sh.T, sh.d)
    ids = t.empty(sh.T, sh.k, dtype=t.int32, device="cuda")
    wts = t.empty(sh.T, sh.k, dtype=t.float32, device="cuda")
    moe.moe_forward_ex(L.cfg, moe.MoeOptions.of(expert_capacity=cap), dv["x"], dv["w_router"], dv["w_gate"],
                       dv["w_up"], dv["w_down"], dv["ws_gate"], dv["ws_up"], dv["ws_down"], y, ids, wts, None, L.ws)
    dy_h = synth.normal(41, 99, sh.T * sh.d, 1.0, sh.dtype).reshape(sh.T, sh.d)
    dy_ref = synth.bf16_to_f64(dy_h) if sh.dtype == synth.BF16 else dy_h.astype(np.float64)
    out = run_backward(L, ids, wts, to_dev(dy_h), moe.MoeOptions.of(expert_capacity=cap, aux_alpha=1.0))
    t.cuda.synchronize()
    gids = to_host(ids)
    keep = (oracle.dispatch(gids, sh.E, cap)["pair_pos"] >= 0).reshape(sh.T, sh.k)
    tau = TAU[sh.dtype]
    widen = synth.bf16_to_f64 if sh.dtype == synth.BF16 else (lambda a: a.astype(np.float64))
    r = oracle.forward_tokens(inp, sh.k, np.arange(sh.T), sh.score_fn, sh.renormalize, forced_ids=gids,
                              keep=keep.astype(np.int32))
    rel = assert_close(widen(to_host(y)), r["y"], tau, "y with capacity")
    ref = oracle.backward(inp, gids, dy_ref, sh.score_fn, sh.renormalize, keep=keep, aux_alpha=1.0)
    worst = 0.0
    for gname, rname in NAMES:
        if gname not in out:
            continue
        want = ref[rname]
        got = to_host(out[gname]).astype(np.float64)
        if np.abs(want).max() < 1e-10:
            assert np.abs(got).max() <= 1e-6, f"{gname} should be zero"
            continue
        worst = max(worst, assert_close(got, want, tau, gname))
    say(f"[ok] {int((~keep).sum())} of {sh.T * sh.k} pairs dropped; y {rel:.2e}, gradients {worst:.2e}")
