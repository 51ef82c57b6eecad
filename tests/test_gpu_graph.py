"""The layer under HIP graph capture: moe_forward and moe_backward enqueue only
kernels (no memsets, copies or host synchronisation), so a captured call can
be replayed.  Each case captures once, then replays several times; before each
replay it writes new input values into the captured buffers and overwrites
the outputs, runs the same call eagerly on those inputs into other buffers,
and requires the replay to match bit for bit."""
import sys

import numpy as np
import pytest

import synth
from gpu_harness import to_dev, torch

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


FORWARD = {
    # 32 tokens: K-split router whose last kernel also groups the pairs, 32-row GEMMs
    "decode_e8_k2": S("g", T=32, d=512, E=8, k=2, d_ff=512),
    # persistent 256 x 256 GEMMs with a K-split down projection, shared expert
    "prefill_e8_k2_shared": S("g", T=1024, d=512, E=8, k=2, d_ff=1024, num_shared=1, d_ff_shared=512),
    "prefill_e32_k4_sigmoid": S("g", T=512, d=256, E=32, k=4, d_ff=256, score_fn=synth.SIGMOID),
    # tile queue, shared expert as wide as the routed ones: it runs as one more
    # group of the routed GEMMs (the dispatch writes its rows on every replay)
    "prefill_e32_k4_shared_in_routed": S("g", T=1024, d=512, E=32, k=4, d_ff=512, num_shared=1,
                                         d_ff_shared=512, score_fn=synth.SIGMOID),
    # 640 or more rows per expert: both tile heights' GEMMs and both combines
    # are captured; the device picks one of each on every replay
    "prefill_e8_k2_tile_choice": S("g", T=3264, d=256, E=8, k=2, d_ff=8192),
}


def _cfg(sh):
    import mixture_experts_sparse_moe_amd as moe
    return moe.MoeConfig.of(sh.T, sh.d, sh.E, sh.k, sh.d_ff, sh.num_shared, sh.d_ff_shared, sh.score_fn,
                            sh.renormalize)


def _forward(moe, cfg, dv, out, ws):
    moe.moe_forward(cfg, dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], dv["ws_gate"],
                    dv["ws_up"], dv["ws_down"], out["y"], out["ids"], out["wts"], out["counts"], ws)


def _forward_bufs(t, sh):
    return dict(y=t.empty(sh.T, sh.d, dtype=t.bfloat16, device="cuda"),
                ids=t.empty(sh.T, sh.k, dtype=t.int32, device="cuda"),
                wts=t.empty(sh.T, sh.k, dtype=t.float32, device="cuda"),
                counts=t.empty(sh.E, dtype=t.int32, device="cuda"))


def _scribble(bufs):
    for b in bufs.values():
        if b is not None:
            b.fill_(7)


@pytest.mark.parametrize("name", sorted(FORWARD))
def test_forward_graph_replays_match_eager(name):
    import mixture_experts_sparse_moe_amd as moe
    t = torch()
    sh = FORWARD[name]
    say(f"[case] forward graph {name}")
    dv = {n: (None if a is None else to_dev(a)) for n, a in synth.make_inputs(sh, 0).items()}
    cfg = _cfg(sh)
    ws = moe.alloc_workspace(cfg)
    ws_eager = moe.alloc_workspace(cfg)
    cap = _forward_bufs(t, sh)
    ref = _forward_bufs(t, sh)
    side = t.cuda.Stream()
    with t.cuda.stream(side):            # warm-up off the default stream
        _forward(moe, cfg, dv, cap, ws)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        _forward(moe, cfg, dv, cap, ws)
    t.cuda.synchronize()
    for rep in range(4):
        x_new = synth.make_inputs(sh, 100 + rep)["x"]
        dv["x"].copy_(to_dev(x_new))
        _scribble(cap)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        _scribble(ref)
        _forward(moe, cfg, dv, ref, ws_eager)
        t.cuda.synchronize()
        for n in cap:
            assert t.equal(cap[n], ref[n]), f"replay {rep}: {n} differs from the eager call"
    say(f"[ok] {name}: 4 replays match")


def test_backward_graph_replays_match_eager():
    import mixture_experts_sparse_moe_amd as moe
    t = torch()
    sh = S("g", T=256, d=256, E=8, k=2, d_ff=512, num_shared=1, d_ff_shared=256)
    say("[case] backward graph")
    dv = {n: (None if a is None else to_dev(a)) for n, a in synth.make_inputs(sh, 0).items()}
    cfg = _cfg(sh)
    ids = t.empty(sh.T, sh.k, dtype=t.int32, device="cuda")
    wts = t.empty(sh.T, sh.k, dtype=t.float32, device="cuda")
    moe.moe_route(cfg, dv["x"], dv["w_router"], ids, wts)
    dy = to_dev(synth.normal(0, 99, sh.T * sh.d, 1.0, synth.BF16).reshape(sh.T, sh.d))
    f32 = dict(dtype=t.float32, device="cuda")

    def grads():
        return dict(dx=t.empty(sh.T, sh.d, **f32), dw_router=t.empty(sh.E, sh.d, **f32),
                    dw_gate=t.empty(sh.E, sh.d_ff, sh.d, **f32), dw_up=t.empty(sh.E, sh.d_ff, sh.d, **f32),
                    dw_down=t.empty(sh.E, sh.d, sh.d_ff, **f32), dws_gate=t.empty(sh.d_ff_shared, sh.d, **f32),
                    dws_up=t.empty(sh.d_ff_shared, sh.d, **f32), dws_down=t.empty(sh.d, sh.d_ff_shared, **f32))

    def run(out, ws):
        moe.moe_backward(cfg, dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], dv["ws_gate"],
                         dv["ws_up"], dv["ws_down"], dy, ids, wts, out["dx"], out["dw_router"], out["dw_gate"],
                         out["dw_up"], out["dw_down"], out["dws_gate"], out["dws_up"], out["dws_down"], ws=ws)

    ws, ws_eager = moe.alloc_backward_workspace(cfg), moe.alloc_backward_workspace(cfg)
    cap, ref = grads(), grads()
    side = t.cuda.Stream()
    with t.cuda.stream(side):
        run(cap, ws)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        run(cap, ws)
    t.cuda.synchronize()
    for rep in range(3):
        dy.copy_(to_dev(synth.normal(10 + rep, 99, sh.T * sh.d, 1.0, synth.BF16).reshape(sh.T, sh.d)))
        _scribble(cap)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        _scribble(ref)
        run(ref, ws_eager)
        t.cuda.synchronize()
        for n in cap:
            assert t.equal(cap[n], ref[n]), f"replay {rep}: {n} differs from the eager call"
        assert np.isfinite(cap["dx"].cpu().numpy()).all()
    say("[ok] backward: 3 replays match")
