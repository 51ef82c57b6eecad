"""GPU parity of the backward pass (moe_backward) against the oracle's
chain-rule backward, for the GPU's own routing.  Every gradient must satisfy
max|err| <= tau * max|ref|: tau = 1e-4 for fp32 layers; 2e-2 for bf16 layers
(the recomputed a, u, h and the intermediate da, du, dO are rounded to bf16,
about five roundings of 2^-9 along any path)."""
import sys
import types

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import TAU, DeviceLayer, assert_close, to_dev, to_host, torch

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


CASES = {
    "fp32_e8_k2": S("b", T=64, d=64, E=8, k=2, d_ff=128, dtype=synth.F32),
    "fp32_e6_k3_sigmoid_raw_shared": S("b", T=40, d=64, E=6, k=3, d_ff=64, num_shared=1, d_ff_shared=64,
                                       score_fn=synth.SIGMOID, renormalize=0, dtype=synth.F32),
    "fp32_e6_k4_softmax_raw": S("b", T=50, d=64, E=6, k=4, d_ff=128, renormalize=0, dtype=synth.F32),
    "bf16_e8_k2": S("b", T=200, d=256, E=8, k=2, d_ff=384),
    "bf16_e32_k4_sigmoid_shared": S("b", T=150, d=128, E=32, k=4, d_ff=128, num_shared=1, d_ff_shared=192,
                                    score_fn=synth.SIGMOID),
    "bf16_e64_k8_zipf": S("b", T=300, d=256, E=64, k=8, d_ff=128, zipf_s=1.1),
    "bf16_decode_e8_k2": S("b", T=16, d=512, E=8, k=2, d_ff=256),
    "bf16_e4_k1": S("b", T=90, d=128, E=4, k=1, d_ff=128),
    # widths in multiples of 256: the GEMMs run on the forward's kernel over
    # transposed operands (per-expert K ranges padded to 128 for the weights)
    "bf16_w256_e8_k2": S("b", T=300, d=256, E=8, k=2, d_ff=512),
    "bf16_w256_e16_k4_sigmoid_shared": S("b", T=260, d=512, E=16, k=4, d_ff=256, num_shared=1, d_ff_shared=256,
                                         score_fn=synth.SIGMOID),
    "bf16_w256_e32_k2_zipf": S("b", T=100, d=256, E=32, k=2, d_ff=256, zipf_s=1.5),
    "bf16_w256_e4_k2_long_groups": S("b", T=1200, d=256, E=4, k=2, d_ff=256),
    # dx per pair with its K (2 d_ff = 3072) cut in two slices
    "bf16_w256_e8_k2_dx_split": S("b", T=200, d=256, E=8, k=2, d_ff=1536),
    # the limits: 256 experts, 16 per token (generic path); 256 groups of the
    # grouped-K weight gradients, many of them empty (persistent-kernel path)
    "bf16_e256_k16": S("b", T=100, d=128, E=256, k=16, d_ff=64),
    "bf16_w256_e256_k8_sigmoid": S("b", T=200, d=256, E=256, k=8, d_ff=256, score_fn=synth.SIGMOID),
    # 32 experts or more: dW_r as one product over 2 x 3072 token columns (dl
    # in bf16 high and low parts), its K cut in four fp32 slices
    "bf16_w256_e32_k2_router_slices": S("b", T=3000, d=256, E=32, k=2, d_ff=256),
}

NAMES = [("dx", "dx"), ("dw_router", "dw_router"), ("dw_gate", "dw_gate"), ("dw_up", "dw_up"),
         ("dw_down", "dw_down"), ("dws_gate", "ds_gate"), ("dws_up", "ds_up"), ("dws_down", "ds_down")]


def run_backward(L, ids, wts, dy_d, opts=None):
    import mixture_experts_sparse_moe_amd as moe
    t = torch()
    sh, dv = L.sh, L.d
    f32 = dict(dtype=t.float32, device="cuda")
    out = dict(dx=t.full((sh.T, sh.d), 7.0, **f32), dw_router=t.full((sh.E, sh.d), 7.0, **f32),
               dw_gate=t.full((sh.E, sh.d_ff, sh.d), 7.0, **f32), dw_up=t.full((sh.E, sh.d_ff, sh.d), 7.0, **f32),
               dw_down=t.full((sh.E, sh.d, sh.d_ff), 7.0, **f32))
    if sh.num_shared:
        fs = sh.d_ff_shared
        out.update(dws_gate=t.full((fs, sh.d), 7.0, **f32), dws_up=t.full((fs, sh.d), 7.0, **f32),
                   dws_down=t.full((sh.d, fs), 7.0, **f32))
    ws = moe.alloc_backward_workspace(L.cfg)
    args = (dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], dv["ws_gate"], dv["ws_up"],
            dv["ws_down"], dy_d, ids, wts, out["dx"], out["dw_router"], out["dw_gate"], out["dw_up"],
            out["dw_down"], out.get("dws_gate"), out.get("dws_up"), out.get("dws_down"))
    if opts is None:
        moe.moe_backward(L.cfg, *args, ws=ws)
    else:
        moe.moe_backward_ex(L.cfg, opts, *args, ws=ws)
    return out


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_matches_oracle(name):
    sh = CASES[name]
    say(f"[case] backward {name} {sh}")
    inp = synth.make_inputs(sh, 21)
    L = DeviceLayer(sh, inp)
    st = L.steps()
    # dy: seeded normals in the layer's dtype (tensor id 99: not used by the inputs)
    dy_h = synth.normal(21, 99, sh.T * sh.d, 1.0, sh.dtype).reshape(sh.T, sh.d)
    dy_ref = synth.bf16_to_f64(dy_h) if sh.dtype == synth.BF16 else dy_h.astype(np.float64)
    out = run_backward(L, st["ids"], st["weights"], to_dev(dy_h))
    out2 = run_backward(L, st["ids"], st["weights"], to_dev(dy_h))
    torch().cuda.synchronize()
    gids = to_host(st["ids"])
    ref = oracle.backward(inp, gids, dy_ref, sh.score_fn, sh.renormalize)
    tau = TAU[sh.dtype]
    worst = 0.0
    for gname, rname in NAMES:
        if gname not in out:
            continue
        got = to_host(out[gname]).astype(np.float64)
        np.testing.assert_array_equal(got, to_host(out2[gname]), err_msg=f"{gname} not deterministic")
        want = ref[rname]
        if np.abs(want).max() < 1e-10:       # zero up to the oracle's rounding (k = 1, renormalised)
            assert np.abs(got).max() <= 1e-6, f"{gname} should be zero"
            continue
        worst = max(worst, assert_close(got, want, tau, gname))
    # experts that no pair chose get exactly zero weight gradients
    unused = np.setdiff1d(np.arange(sh.E), gids.ravel())
    for gname in ("dw_gate", "dw_up", "dw_down"):
        assert not np.any(to_host(out[gname])[unused]), gname
    say(f"[ok] worst max|err|/max|ref| = {worst:.2e}, unused experts {unused.tolist()}")


@pytest.mark.parametrize("name", ["bf16_w256_e16_k4_sigmoid_shared", "bf16_e32_k4_sigmoid_shared", "fp32_e8_k2"])
def test_backward_empty_batch_zeroes_weight_grads(name):
    """T = 0: nothing routed, every weight gradient is written as exact zeros."""
    import dataclasses
    sh = dataclasses.replace(CASES[name], T=0)
    say(f"[case] backward empty batch {name}")
    inp = synth.make_inputs(sh, 21)
    L = DeviceLayer(sh, inp)
    t = torch()
    ids = t.empty((0, sh.k), dtype=t.int32, device="cuda")
    wts = t.empty((0, sh.k), dtype=t.float32, device="cuda")
    dy = t.empty((0, sh.d), dtype=t.bfloat16 if sh.dtype == synth.BF16 else t.float32, device="cuda")
    out = run_backward(L, ids, wts, dy)
    t.cuda.synchronize()
    for gname, _ in NAMES:
        if gname in out and gname != "dx":
            assert not np.any(to_host(out[gname])), gname


@pytest.mark.parametrize("name", ["mixtral_prefill", "deepseek_v3"])
def test_backward_full_size_sampled(name):
    """Full-size layers in the configuration the benchmark times: dx on
    sampled tokens (each depends on its own token only) and sampled elements
    of every expert weight gradient, each summed by the oracle over its
    expert's pairs; bound tau * (max |ref| over the tensor's samples).  The
    router weight gradient needs every token's expert outputs, so it is
    checked at the small shapes only."""
    import mixture_experts_sparse_moe_amd as moe
    t = torch()
    sh = synth.SHAPES[name]
    say(f"[gen] backward full size {name}")
    inp = synth.make_inputs(sh, 0)
    dv = {n: (None if a is None else to_dev(a)) for n, a in inp.items()}
    cfg = moe.MoeConfig.of(sh.T, sh.d, sh.E, sh.k, sh.d_ff, sh.num_shared, sh.d_ff_shared, sh.score_fn,
                           sh.renormalize)
    ids = t.empty(sh.T, sh.k, dtype=t.int32, device="cuda")
    wts = t.empty(sh.T, sh.k, dtype=t.float32, device="cuda")
    moe.moe_route(cfg, dv["x"], dv["w_router"], ids, wts)
    dy_h = synth.normal(0, 99, sh.T * sh.d, 1.0, sh.dtype).reshape(sh.T, sh.d)
    say(f"[gpu] backward {name}")
    out = run_backward(types.SimpleNamespace(sh=sh, d=dv, cfg=cfg), ids, wts, to_dev(dy_h))
    t.cuda.synchronize()
    gids = to_host(ids)
    dy_ref = synth.bf16_to_f64(dy_h)
    rng = np.random.default_rng(1)
    tau = TAU[sh.dtype]
    # dx on sampled tokens: the oracle's backward restricted to those tokens
    toks = np.unique(np.concatenate([[0, sh.T - 1], rng.integers(0, sh.T, 4)]))
    sub = dict(inp)
    sub["x"] = inp["x"][toks]
    say(f"[oracle] dx of tokens {toks.tolist()}")
    ref_dx = oracle.backward(sub, gids[toks], dy_ref[toks], sh.score_fn, sh.renormalize, weights=False)["dx"]
    got_dx = to_host(out["dx"][t.from_numpy(toks).cuda()]).astype(np.float64)
    assert_close(got_dx, ref_dx, tau, "dx (sampled tokens)")
    # weight gradients: 8 elements of each, experts and positions seeded
    kinds = [("dw_gate", sh.d_ff, sh.d), ("dw_up", sh.d_ff, sh.d), ("dw_down", sh.d, sh.d_ff)]
    if sh.num_shared:
        kinds += [("ds_gate", sh.d_ff_shared, sh.d), ("ds_up", sh.d_ff_shared, sh.d),
                  ("ds_down", sh.d, sh.d_ff_shared)]
    samples = [(n, int(rng.integers(sh.E)), int(rng.integers(a)), int(rng.integers(b)))
               for n, a, b in kinds for _ in range(8)]
    say(f"[oracle] {len(samples)} weight-gradient elements")
    ref = oracle.backward_weight_samples(inp, gids, dy_ref, samples, sh.score_fn, sh.renormalize)
    gpu_name = {"ds_gate": "dws_gate", "ds_up": "dws_up", "ds_down": "dws_down"}
    for n, _, _ in kinds:
        sel = [q for q, s in enumerate(samples) if s[0] == n]
        got = np.array([float(out[gpu_name.get(n, n)][s[2], s[3]] if n.startswith("ds_")
                              else out[n][s[1], s[2], s[3]]) for s in (samples[q] for q in sel)])
        want = ref[sel]
        scale = np.abs(want).max()
        err = np.abs(got - want).max()
        say(f"[{n}] max|err| {err:.3e}, max|ref| {scale:.3e}")
        assert err <= tau * scale, f"{n}: max|err| {err} > {tau} * {scale}"



CAPACITY = {
    # (shape, capacity factor or fixed capacity)
    "bf16_w256_e8_k2_zipf": (S("b", T=300, d=256, E=8, k=2, d_ff=512, zipf_s=1.2), 0.8),
    "bf16_w256_decode_e8_k2": (S("b", T=16, d=512, E=8, k=2, d_ff=256), 2),
    "bf16_e16_k4_sigmoid_shared": (S("b", T=150, d=128, E=16, k=4, d_ff=128, num_shared=1, d_ff_shared=128,
                                     score_fn=synth.SIGMOID), 1.0),
    "fp32_e8_k2": (S("b", T=64, d=64, E=8, k=2, d_ff=128, dtype=synth.F32), 0.75),
}


@pytest.mark.parametrize("name", sorted(CAPACITY))
def test_backward_with_capacity_matches_oracle(name):
    """moe_backward_ex with an expert capacity: the pairs each expert drops
    (past its first C in pair order) get no gradient; every gradient against
    the oracle's backward under the same keep mask (from the oracle's own
    dispatch of the GPU's ids)."""
    import mixture_experts_sparse_moe_amd as moe
    sh, cf = CAPACITY[name]
    cap = cf if isinstance(cf, int) else moe.capacity(sh.T, sh.k, sh.E, cf)
    say(f"[case] backward with capacity {cap}: {name} {sh}")
    inp = synth.make_inputs(sh, 23)
    L = DeviceLayer(sh, inp)
    st = L.steps()
    dy_h = synth.normal(23, 99, sh.T * sh.d, 1.0, sh.dtype).reshape(sh.T, sh.d)
    dy_ref = synth.bf16_to_f64(dy_h) if sh.dtype == synth.BF16 else dy_h.astype(np.float64)
    opts = moe.MoeOptions.of(expert_capacity=cap)
    out = run_backward(L, st["ids"], st["weights"], to_dev(dy_h), opts)
    out2 = run_backward(L, st["ids"], st["weights"], to_dev(dy_h), opts)
    torch().cuda.synchronize()
    gids = to_host(st["ids"])
    keep = (oracle.dispatch(gids, sh.E, cap)["pair_pos"] >= 0).reshape(sh.T, sh.k)
    dropped = int((~keep).sum())
    assert dropped > 0, "the case must drop pairs"
    ref = oracle.backward(inp, gids, dy_ref, sh.score_fn, sh.renormalize, keep=keep)
    tau = TAU[sh.dtype]
    worst = 0.0
    for gname, rname in NAMES:
        if gname not in out:
            continue
        got = to_host(out[gname]).astype(np.float64)
        np.testing.assert_array_equal(got, to_host(out2[gname]), err_msg=f"{gname} not deterministic")
        worst = max(worst, assert_close(got, ref[rname], tau, gname))
    say(f"[ok] {dropped} of {sh.T * sh.k} pairs dropped; worst max|err|/max|ref| = {worst:.2e}")


AUX = {
    "bf16_w256_e8_k2": (S("b", T=300, d=256, E=8, k=2, d_ff=512), 0),
    "bf16_e16_k4_sigmoid_shared_capacity": (S("b", T=150, d=128, E=16, k=4, d_ff=128, num_shared=1,
                                              d_ff_shared=128, score_fn=synth.SIGMOID), 40),
    "fp32_e8_k2_softmax_raw": (S("b", T=64, d=64, E=8, k=2, d_ff=128, renormalize=0, dtype=synth.F32), 0),
}


@pytest.mark.parametrize("name", sorted(AUX))
def test_backward_with_aux_loss_matches_oracle(name):
    """moe_backward_ex with aux_alpha: the gradient of the load-balancing loss
    (f fixed by the assignment, through the mean router probabilities) on top
    of the layer's.  Checked twice: the whole dx and dw_router against the
    oracle's backward with the same alpha, and the difference to the run
    without the loss (the aux term alone) against the oracle's aux term."""
    import mixture_experts_sparse_moe_amd as moe
    sh, cap = AUX[name]
    alpha = 2.0
    say(f"[case] backward with aux loss alpha {alpha}, capacity {cap}: {name} {sh}")
    inp = synth.make_inputs(sh, 29)
    L = DeviceLayer(sh, inp)
    st = L.steps()
    dy_h = synth.normal(29, 99, sh.T * sh.d, 1.0, sh.dtype).reshape(sh.T, sh.d)
    dy_ref = synth.bf16_to_f64(dy_h) if sh.dtype == synth.BF16 else dy_h.astype(np.float64)
    with_aux = run_backward(L, st["ids"], st["weights"], to_dev(dy_h),
                            moe.MoeOptions.of(expert_capacity=cap, aux_alpha=alpha))
    without = run_backward(L, st["ids"], st["weights"], to_dev(dy_h), moe.MoeOptions.of(expert_capacity=cap))
    torch().cuda.synchronize()
    gids = to_host(st["ids"])
    keep = None if not cap else (oracle.dispatch(gids, sh.E, cap)["pair_pos"] >= 0).reshape(sh.T, sh.k)
    ref = oracle.backward(inp, gids, dy_ref, sh.score_fn, sh.renormalize, keep=keep, aux_alpha=alpha)
    tau = TAU[sh.dtype]
    for gname in ("dx", "dw_router"):
        assert_close(to_host(with_aux[gname]).astype(np.float64), ref[gname], tau, gname)
    # the aux term alone
    dl = oracle.aux_loss_logit_grad(oracle.logits(inp["x"], inp["w_router"]), gids, sh.score_fn, alpha)
    xr = synth.bf16_to_f64(inp["x"]) if sh.dtype == synth.BF16 else inp["x"].astype(np.float64)
    wr = synth.bf16_to_f64(inp["w_router"]) if sh.dtype == synth.BF16 else inp["w_router"].astype(np.float64)
    for gname, want in (("dx", dl @ wr), ("dw_router", dl.T @ xr)):
        got = to_host(with_aux[gname]).astype(np.float64) - to_host(without[gname]).astype(np.float64)
        r = assert_close(got, want, tau, f"{gname} aux term")
        say(f"[{gname}] aux term max|ref| {np.abs(want).max():.3e}, rel err {r:.2e}")
    # the expert weight gradients do not see the loss
    for gname in ("dw_gate", "dw_up", "dw_down"):
        np.testing.assert_array_equal(to_host(with_aux[gname]), to_host(without[gname]), err_msg=gname)
