"""moe_forward_noalloc, the forward for callers that cannot allocate (its
workspace is the library's fixed per-GPU device array), against moe_forward
with a workspace the caller allocated: four calls in a row on the same
array, each smaller than the one before (a layer whose shared expert runs
inside the routed GEMMs, on 288-row tiles, a prefill-sized layer whose GEMMs claim tiles
through counters kept in the array, a decode-sized layer on the 32-row
kernels with the router's fused dispatch, a five-token layer), every output
bitwise equal to moe_forward's (same kernels, same launches)."""
import sys

import numpy as np
import pytest

import synth
from gpu_harness import DeviceLayer, to_host, torch

pytestmark = pytest.mark.gpu
S = synth.LayerShape

CASES = [
    S("n0", T=1024, d=512, E=16, k=4, d_ff=512, num_shared=1, d_ff_shared=512, score_fn=synth.SIGMOID),
    S("n1", T=600, d=256, E=8, k=2, d_ff=384, router_scale=4.0),
    S("n2", T=48, d=1024, E=16, k=4, d_ff=512, num_shared=1, d_ff_shared=256, score_fn=synth.SIGMOID),
    S("n3", T=5, d=512, E=8, k=2, d_ff=256),
]


def _outputs(L, t):
    sh = L.sh
    return dict(y=L.empty_act(sh.T, sh.d), ids=t.empty(sh.T, sh.k, dtype=t.int32, device="cuda"),
                wts=t.empty(sh.T, sh.k, dtype=t.float32, device="cuda"),
                counts=t.empty(sh.E, dtype=t.int32, device="cuda"),
                gap=t.empty(sh.T, 2, dtype=t.float32, device="cuda"))


def test_noalloc_forward_equals_forward_with_workspace():
    import mixture_experts_sparse_moe_amd as moe
    t = torch()
    if not t.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    layers = [DeviceLayer(sh, synth.make_inputs(sh, 50 + i)) for i, sh in enumerate(CASES)]
    for L in layers:
        assert moe.moe_workspace_bytes(L.cfg) <= moe.NOALLOC_SCRATCH_BYTES
    assert moe.moe_forward_plan(layers[0].cfg)["shared_merged"]
    assert moe.moe_forward_plan(layers[0].cfg)["tile_rows"] == 288
    sizes = [moe.moe_workspace_bytes(L.cfg) for L in layers]
    assert sizes == sorted(sizes, reverse=True)
    got, want = [], []
    for L in layers:
        print(f"[case] noalloc {L.sh}", file=sys.stderr, flush=True)
        o = _outputs(L, t)
        dv = L.d
        moe.moe_forward_noalloc(L.cfg, dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                                dv["ws_gate"], dv["ws_up"], dv["ws_down"], o["y"], o["ids"], o["wts"],
                                o["counts"], o["gap"])
        got.append(o)
    t.cuda.synchronize()
    for L in layers:
        o = _outputs(L, t)
        dv = L.d
        moe.moe_forward(L.cfg, dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], dv["ws_gate"],
                        dv["ws_up"], dv["ws_down"], o["y"], o["ids"], o["wts"], o["counts"], L.ws,
                        topk_gap=o["gap"])
        want.append(o)
    t.cuda.synchronize()
    for L, g, w in zip(layers, got, want):
        for n in ("y", "ids", "wts", "counts", "gap"):
            np.testing.assert_array_equal(to_host(g[n]), to_host(w[n]), err_msg=f"{L.sh.name} {n}")
        assert np.abs(to_host(g["y"]).astype(np.int64)).sum() > 0
    # a second pass over the first layer: the array kept the last call's contents
    L = layers[0]
    o = _outputs(L, t)
    dv = L.d
    moe.moe_forward_noalloc(L.cfg, dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], dv["ws_gate"],
                            dv["ws_up"], dv["ws_down"], o["y"], o["ids"], o["wts"], o["counts"], o["gap"])
    t.cuda.synchronize()
    for n in ("y", "ids", "wts", "counts", "gap"):
        np.testing.assert_array_equal(to_host(o[n]), to_host(want[0][n]), err_msg=f"again {n}")
