"""moe_forward_staged: the same layer as moe_forward (y, ids, gates and counts
bitwise equal) with one event per stage; every stage's elapsed time is
non-negative, and the stages that moe_forward_plan says are empty are
(the shared expert inside the routed GEMMs; the dispatch inside the router's
last kernel for a batch of at most 32 tokens)."""
import sys

import pytest

import synth
from gpu_harness import cfg_of, to_dev, torch

pytestmark = pytest.mark.gpu
S = synth.LayerShape

EMPTY_MS = 0.02     # two back-to-back event records with nothing between them

CASES = {
    "shared_in_routed": S("s", T=1024, d=512, E=32, k=4, d_ff=512, num_shared=1, d_ff_shared=512,
                          score_fn=synth.SIGMOID),
    "shared_on_its_own": S("s", T=1024, d=512, E=8, k=2, d_ff=1024, num_shared=1, d_ff_shared=512),
    "decode": S("s", T=32, d=512, E=8, k=2, d_ff=512),
    # 640 or more rows per expert: the tile height is chosen on the device, so
    # both gate/up kernels run between events 1 and 2 (the first one's start,
    # the second one's end), and both combines of the two K splits
    "tile_choice": S("s", T=3264, d=256, E=8, k=2, d_ff=8192),
}


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch().cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    import mixture_experts_sparse_moe_amd as moe
    moe.lib()


@pytest.mark.parametrize("name", sorted(CASES))
def test_staged_matches_forward_and_marks_every_stage(name):
    import mixture_experts_sparse_moe_amd as moe
    t = torch()
    sh = CASES[name]
    cfg = cfg_of(sh)
    plan = moe.moe_forward_plan(cfg)
    say(f"[case] staged {name} {plan}")
    dv = {n: (None if a is None else to_dev(a)) for n, a in synth.make_inputs(sh, 5).items()}
    ws = moe.alloc_workspace(cfg)
    outs = []
    for staged in (False, True):
        y = t.empty(sh.T, sh.d, dtype=t.bfloat16, device="cuda")
        ids = t.empty(sh.T, sh.k, dtype=t.int32, device="cuda")
        wts = t.empty(sh.T, sh.k, dtype=t.float32, device="cuda")
        counts = t.empty(sh.E, dtype=t.int32, device="cuda")
        args = (cfg, dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], dv["ws_gate"], dv["ws_up"],
                dv["ws_down"], y)
        if staged:
            start = t.cuda.Event(enable_timing=True)
            evs = [t.cuda.Event(enable_timing=True) for _ in range(moe.MOE_NUM_STAGES)]
            moe.moe_forward_staged(*args, topk_ids=ids, topk_weights=wts, expert_counts=counts, ws=ws,
                                   start_event=start, stage_events=evs)
        else:
            moe.moe_forward(*args, ids, wts, counts, ws)
        t.cuda.synchronize()
        outs.append((y, ids, wts, counts))
    for a, b, what in zip(outs[0], outs[1], ("y", "ids", "weights", "counts")):
        assert t.equal(a, b), f"moe_forward_staged's {what} differs from moe_forward's"
    ms, prev = [], start
    for e in evs:
        ms.append(prev.elapsed_time(e))
        prev = e
    say("[stages ms] " + ", ".join(f"{n} {v:.4f}" for n, v in zip(moe.STAGE_NAMES, ms)))
    assert all(v >= 0.0 for v in ms)
    assert ms[2] > 0.0
    if sh.num_shared and plan["shared_merged"]:
        assert ms[4] + ms[5] < EMPTY_MS, "the shared expert ran outside the routed GEMMs"
    if sh.num_shared and not plan["shared_merged"]:
        assert ms[4] > 0.0 and ms[5] > 0.0
