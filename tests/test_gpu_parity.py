"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case uses seeded synthetic inputs (``synth``).  Rules:
  * routing ids bit-exact, in order, except at near-ties (score gap < 1e-6
    and logit gap < 1e-4 at the ranks involved), which are listed;
  * counts, offsets, grouped order and inverse order bit-exact;
  * gates within 1e-5 of the oracle's gates for the GPU's ids;
  * expert outputs and y within max|err| <= tau * max|ref|, tau = 2e-2 for
    bf16 and 1e-4 for fp32, the oracle evaluated with the GPU's ids.
  * the k-th/(k+1)-th margins (logit and score) of the step-by-step router
    and of moe_forward against the oracle's, tokens routed differently at a
    near-tie left out.
Small cases span several GEMM tiles in M, N and K with ragged tails; the
full-size layer shapes check all routing and dispatch outputs, and the
expert outputs and y on a stratified sample: the first and the last grouped
row of every M tile of every expert (both the 256-row tiles with a short last
one and the even split, so every tile of every schedule, the one-row tails
included) and their tokens.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import (TAU, DeviceLayer, assert_close, check_gaps, check_routing, oracle_routing, to_dev,
                         to_host, torch)

pytestmark = pytest.mark.gpu
S = synth.LayerShape

SMALL = {
    "tiny_fp32": synth.SHAPES["tiny"],
    "bf16_e8_k2_x4router": S("c", T=600, d=256, E=8, k=2, d_ff=384, router_scale=4.0),
    "bf16_e8_k2_n320": S("c", T=333, d=192, E=8, k=2, d_ff=320),
    "bf16_e64_k8_zipf": S("c", T=520, d=256, E=64, k=8, d_ff=256, zipf_s=1.1),
    "bf16_e256_k8_sigmoid_shared": S("c", T=300, d=256, E=256, k=8, d_ff=128, num_shared=1,
                                     d_ff_shared=192, score_fn=synth.SIGMOID),
    "bf16_e16_k1_switch": S("c", T=200, d=128, E=16, k=1, d_ff=128, renormalize=0),
    "bf16_e6_k4_softmax_raw": S("c", T=150, d=128, E=6, k=4, d_ff=192, renormalize=0),
    "bf16_e3_k2": S("c", T=97, d=64, E=3, k=2, d_ff=64),
    "bf16_e256_k16": S("c", T=100, d=128, E=256, k=16, d_ff=64),
    "fp32_e6_k6_dense": S("c", T=100, d=64, E=6, k=6, d_ff=128, dtype=synth.F32),
    # few tokens, wide rows: K-split router and the 32-row expert GEMMs
    "bf16_decode_e64_k6": S("c", T=40, d=1024, E=64, k=6, d_ff=192),
    "bf16_decode_e256_k8_shared": S("c", T=8, d=2048, E=256, k=8, d_ff=64, num_shared=1,
                                    d_ff_shared=128, score_fn=synth.SIGMOID),
    "bf16_decode_e100_k3": S("c", T=70, d=512, E=100, k=3, d_ff=320),
    "fp32_e32_k4_sigmoid_shared": S("c", T=130, d=128, E=32, k=4, d_ff=192, num_shared=1,
                                    d_ff_shared=128, score_fn=synth.SIGMOID, dtype=synth.F32),
    # a shared expert as wide as the routed ones, about one M tile per
    # expert: moe_forward runs it as one more group of the routed GEMMs
    "bf16_e64_k6_sigmoid_shared_same_width": S("c", T=700, d=512, E=64, k=6, d_ff=256, num_shared=1,
                                               d_ff_shared=256, score_fn=synth.SIGMOID),
    "bf16_e32_k4_zipf_shared_same_width": S("c", T=900, d=768, E=32, k=4, d_ff=384, num_shared=1,
                                            d_ff_shared=384, zipf_s=1.1),
    # 224 to 287 rows per expert on average: 288-row tiles on 12 waves (an
    # expert of 257..288 rows is one tile), with the shared expert inside the
    # routed GEMMs, on its own, and with skewed routing
    "bf16_e32_k8_sigmoid_shared_same_width_tall": S("c", T=1024, d=512, E=32, k=8, d_ff=256, num_shared=1,
                                                    d_ff_shared=256, score_fn=synth.SIGMOID),
    "bf16_e16_k4_shared_tall": S("c", T=1000, d=256, E=16, k=4, d_ff=384, num_shared=1, d_ff_shared=128),
    "bf16_e32_k8_zipf_tall": S("c", T=1024, d=256, E=32, k=8, d_ff=256, zipf_s=1.1),
    # 640 or more rows per expert: the tile height is chosen on the device
    # from the counts, and moe_forward splits the 256-row down GEMM in 4 K
    # ranges (the 288-row one never): experts of 761..867 rows take 288-row
    # tiles, experts of 633..733 rows 256-row ones (test_device_tile_choice)
    "bf16_e8_k2_fixed_choose288": S("c", T=3264, d=256, E=8, k=2, d_ff=8192),
    "bf16_e8_k2_fixed_choose256": S("c", T=2720, d=256, E=8, k=2, d_ff=8192),
}


def tile_choice_rows(counts, d_ff, slots=256):
    """The tile height the library chooses on the device for a layer of 640
    or more rows per expert (written out from its documented rule): 288 when
    the gate/up GEMM's 288-row tiles take fewer rounds of the persistent grid
    than 256-row ones, a 288-row round weighing 9/8."""
    tn = 2 * d_ff // 256
    r = {bm: -(-sum(-(-int(n) // bm) for n in counts) * tn // slots) for bm in (256, 288)}
    return 288 if 9 * r[288] < 8 * r[256] else 256


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    import mixture_experts_sparse_moe_amd as moe
    moe.lib()   # raises if the library is missing


def tile_edge_rows(offsets: np.ndarray, bms=(256, 288)) -> np.ndarray:
    """First and last grouped row of every M tile of every expert, for both
    tile heights bm of the persistent GEMMs and both ways they cut an
    expert's n rows into m = ceil(n / bm) tiles: full tiles of bm rows and a
    short last one, or m tiles of ceil(n / m) rows."""
    rows = []
    for e in range(offsets.size - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        n = b - a
        if n == 0:
            continue
        for bm in bms:
            m = -(-n // bm)
            for h in (bm, -(-n // m)):
                for r0 in range(a, b, h):
                    rows += [r0, min(r0 + h, b) - 1]
    return np.unique(np.array(rows, dtype=np.int64))


def check_layer(sh, inp, sample=None, check_expert_out=True, rows_sample=None):
    """Full set of checks for one layer; returns a small report.
    sample: tokens whose y is checked (all when None); check_expert_out: every
    expert row; rows_sample: instead, these grouped rows plus the tokens of
    rows_sample(offsets) (a function of the dispatch offsets)."""
    say(f"[case] {sh}")
    L = DeviceLayer(sh, inp)
    st = L.steps()
    fw = L.forward()
    torch().cuda.synchronize()
    ref = oracle_routing(inp, sh)
    gids = to_host(st["ids"])
    exempt = check_routing(gids, ref, sh.k)
    # the whole-layer call may sum the router logits and the down projection
    # over K ranges, which rounds differently from the step-by-step calls:
    # its routing is checked against the oracle by the same rules
    fids = to_host(fw["ids"])
    fexempt = check_routing(fids, ref, sh.k)
    # gates for the GPU's ids
    rf = oracle.route(ref["logits"], sh.k, sh.score_fn, sh.renormalize, forced_ids=gids)
    np.testing.assert_allclose(to_host(st["weights"]), rf["gates"], atol=1e-5, rtol=0)
    rff = oracle.route(ref["logits"], sh.k, sh.score_fn, sh.renormalize, forced_ids=fids)
    np.testing.assert_allclose(to_host(fw["weights"]), rff["gates"], atol=1e-5, rtol=0)
    # margins of the k-th choice, logit and score, from both router paths
    check_gaps(to_host(st["gap"]), ref, sh.k, sh.E, skip=exempt)
    check_gaps(to_host(fw["gap"]), ref, sh.k, sh.E, skip=fexempt)
    # dispatch, bit-exact
    d = oracle.dispatch(gids, sh.E)
    for n in ("counts", "offsets", "sorted_pairs", "pair_pos"):
        np.testing.assert_array_equal(to_host(st[n]), d[n], err_msg=n)
    np.testing.assert_array_equal(to_host(fw["counts"]), oracle.dispatch(fids, sh.E)["counts"])
    tau = TAU[sh.dtype]
    widen = synth.bf16_to_f64 if sh.dtype == synth.BF16 else (lambda a: a.astype(np.float64))
    # expert outputs, per expert in grouped order
    rows = None if rows_sample is None else rows_sample(d["offsets"])
    if rows is not None:
        out = widen(to_host(st["expert_out"]))
        grp = np.searchsorted(d["offsets"], rows, side="right") - 1
        for e in np.unique(grp):
            rr = rows[grp == e]
            _, o = oracle.expert_rows(int(e), inp["x"], d["sorted_pairs"][rr] // sh.k, inp["w_gate"],
                                      inp["w_up"], inp["w_down"])
            assert_close(out[rr], o, tau, f"expert_out of expert {e}, grouped rows {rr.tolist()[:6]}")
        say(f"[rows] {rows.size} grouped rows of {len(np.unique(grp))} experts checked")
        extra = np.unique(d["sorted_pairs"][rows] // sh.k)
        sample = extra if sample is None else np.union1d(np.asarray(sample), extra)
        if sh.num_shared:
            _, o = oracle.expert_rows(0, inp["x"], sample, inp["ws_gate"][None], inp["ws_up"][None],
                                      inp["ws_down"][None])
            assert_close(widen(to_host(st["shared_out"]))[sample], o, tau, "shared_out on the sampled tokens")
    elif check_expert_out:
        out = widen(to_host(st["expert_out"]))
        for e in range(sh.E):
            a, b = d["offsets"][e], d["offsets"][e + 1]
            if a == b:
                continue
            toks = d["sorted_pairs"][a:b] // sh.k
            _, o = oracle.expert_rows(e, inp["x"], toks, inp["w_gate"], inp["w_up"], inp["w_down"])
            assert_close(out[a:b], o, tau, f"expert_out of expert {e}")
        if sh.num_shared:
            _, o = oracle.expert_rows(0, inp["x"], np.arange(sh.T), inp["ws_gate"][None],
                                      inp["ws_up"][None], inp["ws_down"][None])
            assert_close(widen(to_host(st["shared_out"])), o, tau, "shared_out")
    # layer output
    toks = np.arange(sh.T) if sample is None else np.asarray(sample)
    r = oracle.forward_tokens(inp, sh.k, toks, sh.score_fn, sh.renormalize, forced_ids=gids[toks])
    y = widen(to_host(st["y"]))[toks]
    rel = assert_close(y, r["y"], tau, "y of the step-by-step calls")
    if not np.array_equal(fids[toks], gids[toks]):
        r = oracle.forward_tokens(inp, sh.k, toks, sh.score_fn, sh.renormalize, forced_ids=fids[toks])
    rel = max(rel, assert_close(widen(to_host(fw["y"]))[toks], r["y"], tau, "y of moe_forward"))
    say(f"[ok] max|err|/max|y| = {rel:.3e}, near-tie tokens {exempt.tolist()} / {fexempt.tolist()}, "
        f"counts max/mean {d['counts'].max() / max(d['counts'].mean(), 1e-9):.2f}")
    return dict(rel=rel, exempt=exempt, counts=d["counts"])


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_layer(name):
    sh = SMALL[name]
    check_layer(sh, synth.make_inputs(sh, 0))


FULL = ["mixtral_decode", "mixtral_prefill", "hunyuan_a13b", "deepseek_v3"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(name):
    """The full-size layer shapes: every routing and dispatch output; the
    expert outputs of the first and last grouped row of every (expert,
    256- or 288-row M tile) (decode: every row); y on those rows' tokens plus
    the first, the last and 22 seeded random tokens."""
    sh = synth.SHAPES[name]
    say(f"[gen] {name}")
    inp = synth.make_inputs(sh, 0)
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([[0, sh.T - 1], rng.integers(0, sh.T, 22)]))
    if sh.T <= 64:
        rep = check_layer(sh, inp, sample=sample, check_expert_out=True)
    else:
        rep = check_layer(sh, inp, sample=sample, check_expert_out=False, rows_sample=tile_edge_rows)
    say(f"[{name}] counts {rep['counts'].tolist()[:16]}{'...' if sh.E > 16 else ''}")


def test_zero_tokens_route_to_first_experts():
    """x = 0: all logits tie, so every token takes experts 0..k-1 with gates
    1/k (lowest-index tie-break), the first k experts get all T pairs, and
    y = 0."""
    sh = S("z", T=257, d=128, E=16, k=4, d_ff=128)
    inp = synth.make_inputs(sh, 1)
    inp["x"] = np.zeros_like(inp["x"])
    L = DeviceLayer(sh, inp)
    st = L.steps()
    torch().cuda.synchronize()
    assert to_host(st["ids"]).tolist() == [[0, 1, 2, 3]] * sh.T
    np.testing.assert_array_equal(to_host(st["weights"]), np.full((sh.T, 4), 0.25, np.float32))
    assert to_host(st["counts"]).tolist() == [sh.T] * 4 + [0] * 12
    assert not np.any(to_host(st["y"]).astype(np.uint16) & 0x7FFF)


def test_one_expert_top1():
    sh = S("one", T=70, d=128, E=1, k=1, d_ff=192)
    check_layer(sh, synth.make_inputs(sh, 2))


def test_single_token():
    sh = S("t1", T=1, d=256, E=64, k=8, d_ff=128, num_shared=1, d_ff_shared=64)
    check_layer(sh, synth.make_inputs(sh, 3))


def test_empty_batch():
    t = torch()
    sh = S("empty", T=0, d=128, E=8, k=2, d_ff=128)
    inp = synth.make_inputs(sh, 0)
    L = DeviceLayer(sh, inp)
    counts = t.full((8,), 7, dtype=t.int32, device="cuda")
    y = L.empty_act(0, sh.d)
    import mixture_experts_sparse_moe_amd as moe
    moe.moe_forward(L.cfg, L.d["x"], L.d["w_router"], L.d["w_gate"], L.d["w_up"], L.d["w_down"],
                    None, None, None, y, None, None, counts, L.ws)
    t.cuda.synchronize()
    assert to_host(counts).tolist() == [0] * 8


def test_deterministic_and_stream_independent():
    """Two runs, one on a side stream, are bitwise identical (no float atomics)."""
    t = torch()
    sh = SMALL["bf16_e64_k8_zipf"]
    L = DeviceLayer(sh, synth.make_inputs(sh, 5))
    a = L.forward()
    s = t.cuda.Stream()
    with t.cuda.stream(s):
        b = L.forward(stream=s)
    s.synchronize()
    t.cuda.synchronize()
    for n in ("y", "ids", "weights", "counts"):
        np.testing.assert_array_equal(to_host(a[n]), to_host(b[n]), err_msg=n)


def test_decode_paths_deterministic():
    """Few tokens (32-row expert GEMMs, K-split router): repeated whole-layer
    and expert-FFN calls give bitwise identical outputs.  Every expert block
    is checked against the oracle in test_small_layer; a race between a
    stage buffer's last reads and its refill showed up here as run-to-run
    differences in single row blocks."""
    t = torch()
    sh = SMALL["bf16_decode_e100_k3"]
    L = DeviceLayer(sh, synth.make_inputs(sh, 7))
    st = L.steps()
    ys = [to_host(L.forward()["y"]) for _ in range(6)]
    t.cuda.synchronize()
    for y in ys[1:]:
        np.testing.assert_array_equal(y, ys[0])
    import mixture_experts_sparse_moe_amd as moe
    outs = []
    for _ in range(6):
        out = L.empty_act(sh.T * sh.k, sh.d)
        moe.moe_expert_ffn(L.cfg, L.d["x"], st["sorted_pairs"], st["offsets"], L.d["w_gate"], L.d["w_up"],
                           L.d["w_down"], None, None, None, out, None, L.ws)
        outs.append(out)
    t.cuda.synchronize()
    for o in outs:
        np.testing.assert_array_equal(to_host(o), to_host(st["expert_out"]))


def test_nearly_empty_tiles_through_the_tile_queue():
    """Every other expert holds 257 rows (a full 256-row tile plus a one-row
    tile), the rest one row, at widths that give both routed GEMMs 960 tiles
    (3.75 rounds over 256 CUs), so the persistent kernels claim and steal
    tiles past their first three rounds.  moe_expert_ffn's rows against the
    oracle's expert FFN (both tile edges of every expert, and the one-row
    tiles), and three more calls bitwise equal to the first: which workgroup
    takes a tile changes between calls, the result may not."""
    import mixture_experts_sparse_moe_amd as moe
    t = torch()
    sh = S("q", T=1024, d=4096, E=40, k=8, d_ff=2048)
    inp = synth.make_inputs(sh, 11)
    L = DeviceLayer(sh, inp)
    counts = np.array([257 if e % 2 == 0 else 1 for e in range(sh.E)], dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    P = sh.T * sh.k
    pairs = np.random.default_rng(11).permutation(P).astype(np.int32)   # rows past offsets[E] unused
    say(f"[case] tile queue: {int(offsets[-1])} rows in {sh.E} experts, {sh}")
    sp, off = to_dev(pairs), to_dev(offsets)
    outs = []
    for _ in range(4):
        out = L.empty_act(P, sh.d)
        moe.moe_expert_ffn(L.cfg, L.d["x"], sp, off, L.d["w_gate"], L.d["w_up"], L.d["w_down"], None, None,
                           None, out, None, L.ws)
        outs.append(out)
    t.cuda.synchronize()
    n = int(offsets[-1])
    first = to_host(outs[0])[:n]
    for o in outs[1:]:
        np.testing.assert_array_equal(to_host(o)[:n], first)
    worst = 0.0
    for e in range(sh.E):
        local = [0, 255, 256] if counts[e] == 257 else [0]
        rows = offsets[e] + np.array(local)
        _, want = oracle.expert_rows(e, inp["x"], pairs[rows] // sh.k, inp["w_gate"], inp["w_up"], inp["w_down"])
        worst = max(worst, assert_close(synth.bf16_to_f64(first[rows]), want, TAU[sh.dtype], f"expert {e}"))
    say(f"[ok] worst max|err|/max|ref| = {worst:.2e}")


def test_tall_tiles_live_block_edges():
    """288-row tiles on 12 waves (a layer with 224 to 287 rows per expert on
    average): experts of 0..577 rows, at every edge of a wave's 32-row blocks
    (31/32/33), of a wave's 96 rows (95/96/97, 191/192/193), of the old and
    the new tile height (255..257, 287..289) and of two tiles (575..577), so
    waves run the three-, two- and zero-block K loops and the even split of
    the gate/up tiles and the full-plus-short split of the down tiles both
    occur.  Every row of moe_expert_ffn against the oracle's expert FFN, and
    two more calls bitwise equal to the first."""
    import mixture_experts_sparse_moe_amd as moe
    from gpu_harness import cfg_of
    t = torch()
    counts = np.array([0, 1, 31, 32, 33, 95, 96, 97, 191, 192, 193, 255, 256, 257, 287, 288, 289,
                       575, 576, 577, 300, 300, 300, 300], dtype=np.int32)
    sh = S("tall", T=691, d=512, E=counts.size, k=8, d_ff=256)
    assert moe.moe_forward_plan(cfg_of(sh))["tile_rows"] == 288
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    P = sh.T * sh.k
    assert offsets[-1] <= P
    inp = synth.make_inputs(sh, 13)
    L = DeviceLayer(sh, inp)
    pairs = np.random.default_rng(13).permutation(P).astype(np.int32)   # rows past offsets[E] unused
    say(f"[case] tall tiles: {int(offsets[-1])} rows in {sh.E} experts, {sh}")
    sp, off = to_dev(pairs), to_dev(offsets)
    outs = []
    for _ in range(3):
        out = L.empty_act(P, sh.d)
        moe.moe_expert_ffn(L.cfg, L.d["x"], sp, off, L.d["w_gate"], L.d["w_up"], L.d["w_down"], None, None,
                           None, out, None, L.ws)
        outs.append(out)
    t.cuda.synchronize()
    n = int(offsets[-1])
    first = to_host(outs[0])[:n]
    for o in outs[1:]:
        np.testing.assert_array_equal(to_host(o)[:n], first)
    worst = 0.0
    for e in range(sh.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        _, want = oracle.expert_rows(e, inp["x"], pairs[a:b] // sh.k, inp["w_gate"], inp["w_up"], inp["w_down"])
        worst = max(worst, assert_close(synth.bf16_to_f64(first[a:b]), want, TAU[sh.dtype],
                                        f"expert {e} ({b - a} rows)"))
    say(f"[ok] worst max|err|/max|ref| = {worst:.2e}")


def test_device_tile_choice():
    """The two fixed-schedule cases above take the tile height they are meant
    to cover (test_small_layer checks their outputs), and a layer whose experts
    sit at the edges of the 288-row kernel's row blocks and tiles (0, 1, 31..33,
    95..97, 287..289, 575..577 rows) among experts of 769..864 rows runs the
    288-row kernels on the fixed schedule: every row of moe_expert_ffn against
    the oracle's expert FFN, and two more calls bitwise equal to the first."""
    import mixture_experts_sparse_moe_amd as moe
    from gpu_harness import cfg_of
    t = torch()
    for name, want in (("bf16_e8_k2_fixed_choose288", 288), ("bf16_e8_k2_fixed_choose256", 256)):
        sh = SMALL[name]
        plan = moe.moe_forward_plan(cfg_of(sh))
        assert plan["tile_rows"] == 0 and plan["routed_splits"] == 4, plan
        inp = synth.make_inputs(sh, 0)
        counts = oracle_routing(inp, sh)
        counts = np.bincount(counts["ids"].ravel(), minlength=sh.E)
        assert tile_choice_rows(counts, sh.d_ff) == want, (name, counts.tolist())
        # Which kernels moe_forward ran, seen in its output: the step calls on
        # moe_forward's own routing never split the down GEMM (moe_expert_ffn
        # writes the finished product), so their y is bitwise moe_forward's
        # when it took the 288-row tiles (unsplit), and differs in the last
        # bits when it took the 256-row ones (four bf16 K slices).
        L = DeviceLayer(sh, inp)
        fw = L.forward()
        P = sh.T * sh.k
        counts_d = t.empty(sh.E, dtype=t.int32, device="cuda")
        offsets = t.empty(sh.E + 1, dtype=t.int32, device="cuda")
        sp = t.empty(P, dtype=t.int32, device="cuda")
        pp = t.empty(P, dtype=t.int32, device="cuda")
        moe.moe_dispatch(L.cfg, fw["ids"], counts_d, offsets, sp, pp, L.ws)
        out = L.empty_act(P, sh.d)
        moe.moe_expert_ffn(L.cfg, L.d["x"], sp, offsets, L.d["w_gate"], L.d["w_up"], L.d["w_down"], None, None,
                           None, out, None, L.ws)
        y = L.empty_act(sh.T, sh.d)
        moe.moe_combine(L.cfg, out, fw["weights"], pp, None, y)
        t.cuda.synchronize()
        same = np.array_equal(to_host(y), to_host(fw["y"]))
        assert same == (want == 288), f"{name}: moe_forward's y {'equals' if same else 'differs from'} the unsplit one"
    edges = [0, 1, 31, 32, 33, 95, 96, 97, 287, 288, 289, 575, 576, 577]
    counts = np.array(edges + [769 + 9 * i for i in range(11)], dtype=np.int32)
    sh = S("fixed288", T=2000, d=256, E=counts.size, k=8, d_ff=8192)
    assert sh.T * sh.k >= 640 * sh.E and int(counts.sum()) <= sh.T * sh.k
    assert moe.moe_forward_plan(cfg_of(sh))["tile_rows"] == 0
    assert tile_choice_rows(counts, sh.d_ff) == 288
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    P = sh.T * sh.k
    inp = synth.make_inputs(sh, 17)
    L = DeviceLayer(sh, inp)
    pairs = np.random.default_rng(17).permutation(P).astype(np.int32)   # rows past offsets[E] unused
    say(f"[case] fixed-schedule 288-row tiles: {int(offsets[-1])} rows in {sh.E} experts, {sh}")
    sp, off = to_dev(pairs), to_dev(offsets)
    outs = []
    for _ in range(3):
        out = L.empty_act(P, sh.d)
        moe.moe_expert_ffn(L.cfg, L.d["x"], sp, off, L.d["w_gate"], L.d["w_up"], L.d["w_down"], None, None,
                           None, out, None, L.ws)
        outs.append(out)
    t.cuda.synchronize()
    n = int(offsets[-1])
    first = to_host(outs[0])[:n]
    for o in outs[1:]:
        np.testing.assert_array_equal(to_host(o)[:n], first)
    worst = 0.0
    for e in range(sh.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        _, want = oracle.expert_rows(e, inp["x"], pairs[a:b] // sh.k, inp["w_gate"], inp["w_up"], inp["w_down"])
        worst = max(worst, assert_close(synth.bf16_to_f64(first[a:b]), want, TAU[sh.dtype],
                                        f"expert {e} ({b - a} rows)"))
    say(f"[ok] worst max|err|/max|ref| = {worst:.2e}")
