"""The C-ABI library on the host: it loads, exports every declared entry point,
and its validator rejects bad arguments with the documented status codes
before anything is enqueued (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

import mixture_experts_sparse_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="libmoe.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS), names
    L = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def declared_param_counts():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(moe_[a-z_]+)\s*\(([^;{]*?)\)\s*;", src):
        params = [p for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = len(params)
    return out


def test_binding_argument_counts_match_header():
    counts = declared_param_counts()
    L = moe.lib()
    for n in moe.EXPORTS:
        assert len(getattr(L, n).argtypes) == counts[n], n


def test_library_links_no_oracle_or_torch():
    """The product library depends on the HIP runtime only."""
    import subprocess
    out = subprocess.run(["ldd", moe.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out and "torch" not in out and "libsynth" not in out
    assert "amdhip64" in out


def cfg(**kw):
    base = dict(T=64, d=128, E=8, k=2, d_ff=256)
    base.update(kw)
    return moe.MoeConfig.of(base["T"], base["d"], base["E"], base["k"], base["d_ff"],
                            num_shared=kw.get("num_shared", 0), d_ff_shared=kw.get("d_ff_shared", 0),
                            score_fn=kw.get("score_fn", 0), renormalize=kw.get("renormalize", 1),
                            dtype=kw.get("dtype", moe.MOE_BF16))


FAKE = 0x10000   # an aligned, never-dereferenced address: validation fails first


def route(c, x=FAKE, w=FAKE, ids=FAKE, wts=FAKE, gap=None):
    return moe.lib().moe_route(ctypes.byref(c) if c is not None else None, x, w, ids, wts, gap, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), moe.MOE_ERR_SHAPE),
    (dict(d=0), moe.MOE_ERR_SHAPE),
    (dict(E=0), moe.MOE_ERR_SHAPE),
    (dict(k=0), moe.MOE_ERR_SHAPE),
    (dict(k=9), moe.MOE_ERR_SHAPE),                 # k > E
    (dict(d_ff=0), moe.MOE_ERR_SHAPE),
    (dict(num_shared=2, d_ff_shared=64), moe.MOE_ERR_SHAPE),
    (dict(num_shared=1, d_ff_shared=0), moe.MOE_ERR_SHAPE),
    (dict(E=257, k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=32, k=17), moe.MOE_ERR_UNSUPPORTED),
    (dict(d=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(num_shared=1, d_ff_shared=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(score_fn=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(renormalize=3), moe.MOE_ERR_UNSUPPORTED),
    (dict(dtype=5), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=2**28, k=8), moe.MOE_ERR_UNSUPPORTED),  # T*k >= 2^31
])
def test_config_validation(kw, status):
    c = cfg(**kw)
    assert route(c) == status
    assert moe.moe_workspace_bytes(c) == 0
    L = moe.lib()
    assert L.moe_forward(ctypes.byref(c), *([FAKE] * 13), FAKE, 1 << 40, None) == status
    assert moe.lib().moe_capacity(ctypes.byref(c), 1.0) == status
    assert L.moe_dispatch(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == status
    assert L.moe_combine(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None) == status


def test_null_and_alignment():
    c = cfg()
    L = moe.lib()
    assert L.moe_route(None, FAKE, FAKE, FAKE, FAKE, None, None) == moe.MOE_ERR_NULL
    assert route(c, x=None) == moe.MOE_ERR_NULL
    assert route(c, w=None) == moe.MOE_ERR_NULL
    assert route(c, ids=None) == moe.MOE_ERR_NULL
    assert route(c, x=FAKE + 2) == moe.MOE_ERR_ALIGN
    assert route(c, wts=FAKE + 8) == moe.MOE_ERR_ALIGN
    assert route(c, gap=FAKE + 4) == moe.MOE_ERR_ALIGN
    # shared expert weights are required only when num_shared == 1
    cs = cfg(num_shared=1, d_ff_shared=128)
    ffn = lambda c_, sg: L.moe_expert_ffn(ctypes.byref(c_), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, sg,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert ffn(cs, None) == moe.MOE_ERR_NULL


def test_workspace_checks():
    c = cfg()
    L = moe.lib()
    need = moe.moe_workspace_bytes(c)
    assert need > 0 and need % 256 == 0
    args = [FAKE] * 13
    assert L.moe_forward(ctypes.byref(c), *args, None, need, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_forward(ctypes.byref(c), *args, FAKE, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_forward_staged(ctypes.byref(c), *args, FAKE, need - 1, None, None, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_expert_ffn(ctypes.byref(c), *([FAKE] * 11), None, 0, None) == moe.MOE_ERR_WORKSPACE


def test_workspace_size_covers_intermediates():
    """The workspace holds at least the [T*k, d_ff] intermediate, the [T*k, d]
    expert outputs and the routing tables; the shared expert adds its own."""
    for dtype, eb in ((moe.MOE_BF16, 2), (moe.MOE_F32, 4)):
        c = cfg(T=1000, d=256, E=64, k=8, d_ff=512, dtype=dtype)
        P = 1000 * 8
        need = moe.moe_workspace_bytes(c)
        assert need >= P * 512 * eb + P * 256 * eb + 4 * P * 4
        cs = cfg(T=1000, d=256, E=64, k=8, d_ff=512, dtype=dtype, num_shared=1, d_ff_shared=384)
        assert moe.moe_workspace_bytes(cs) >= need + 1000 * 384 * eb + 1000 * 256 * eb


def test_empty_token_batch_is_a_noop():
    c = cfg(T=0)
    L = moe.lib()
    assert L.moe_route(ctypes.byref(c), None, FAKE, None, None, None, None) == moe.MOE_OK
    assert L.moe_combine(ctypes.byref(c), None, None, None, None, None, None) == moe.MOE_OK
    assert L.moe_expert_ffn(ctypes.byref(c), None, None, FAKE, FAKE, FAKE, FAKE, None, None, None,
                            None, None, None, 0, None) == moe.MOE_OK


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert moe.moe_status_str(s).startswith("MOE_")
    assert "unknown" in moe.moe_status_str(42)


def route_ex(c, opts, ws=None, ws_bytes=0):
    return moe.lib().moe_route_ex(ctypes.byref(c), ctypes.byref(opts) if opts is not None else None,
                                  FAKE, FAKE, FAKE, FAKE, None, ws, ws_bytes, None)


def test_options_are_validated_before_launch():
    c = cfg()
    O = moe.MoeOptions
    assert route_ex(c, O(None, 2, 0, None, 0.0)) == moe.MOE_ERR_UNSUPPORTED       # bias space 0/1
    assert route_ex(c, O(FAKE + 4, 0, 0, None, 0.0)) == moe.MOE_ERR_ALIGN        # bias alignment
    assert route_ex(c, O(None, 0, 0, FAKE + 8, 0.0)) == moe.MOE_ERR_ALIGN        # stats alignment
    assert route_ex(c, O(None, 0, 0, None, float("nan"))) == moe.MOE_ERR_SHAPE   # alpha
    # statistics need the workspace
    assert route_ex(c, O(None, 0, 0, FAKE, 0.01)) == moe.MOE_ERR_WORKSPACE
    assert route_ex(c, O(None, 0, 0, FAKE, 0.01), FAKE, 64) == moe.MOE_ERR_WORKSPACE
    # a bad config is still reported first
    assert route_ex(cfg(k=0), O(None, 0, 0, None, 0.0)) == moe.MOE_ERR_SHAPE


def test_capacity_matches_page():
    """moe_capacity: the page's 4,096 tokens, 64 experts, top-8, factor 1.0
    give 512 slots ('from the router to the all-to-all', Capacity and token
    dropping); factor 1.25 gives 640; a whole-number product stays whole
    although its doubles are not (640 * 8 / 8 * 1.1 = 704.0000000000001)."""
    assert moe.capacity(4096, 8, 64, 1.0) == 512
    assert moe.capacity(4096, 8, 64, 1.25) == 640
    assert moe.capacity(10, 2, 3, 1.0) == 7
    assert moe.capacity(640, 8, 8, 1.1) == 704
    assert moe.capacity(4096, 8, 64, 1.1) == 564
    assert moe.capacity(0, 8, 64, 1.25) == 0


def test_capacity_agrees_with_exact_rational():
    """The library's rounding against the oracle's exact rational ceiling over
    token counts, widths and decimal factors."""
    import oracle
    for T in (1, 7, 97, 333, 640, 1000, 4096, 8192, 65535):
        for E, k in ((8, 2), (64, 8), (256, 8), (6, 4), (3, 1), (100, 3)):
            for f in (0.5, 0.75, 0.8, 0.9, 1.0, 1.05, 1.1, 1.2, 1.25, 1.3, 1.5, 2.0, 3.7):
                assert moe.capacity(T, k, E, f) == oracle.capacity(T, k, E, f), (T, E, k, f)


def test_capacity_rejects_bad_factors():
    L = moe.lib()
    c = cfg()
    for f in (0.0, -1.0, float("nan"), float("inf")):
        assert L.moe_capacity(ctypes.byref(c), f) == moe.MOE_ERR_SHAPE
    assert L.moe_capacity(ctypes.byref(cfg(T=2**26, E=8, k=8)), 1e3) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_capacity(None, 1.0) == moe.MOE_ERR_NULL


def test_forward_entry_points_take_the_gap_after_the_counts():
    """moe_forward, moe_forward_staged and moe_forward_ex take a nullable
    float* topk_gap_out right after expert_counts_out (the near-ties of the
    call's own routing), and reject a misaligned one before any launch."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in ("moe_forward", "moe_forward_staged", "moe_forward_ex"):
        m = re.search(r"\b%s\s*\(([^;]*?)\)\s*;" % name, src)
        params = [p.strip() for p in m.group(1).split(",")]
        i = params.index("int32_t* expert_counts_out")
        assert params[i + 1] == "float* topk_gap_out", (name, params)
    c = cfg()
    L = moe.lib()
    need = moe.moe_workspace_bytes(c)
    args = [FAKE] * 12
    assert L.moe_forward(ctypes.byref(c), *args, FAKE + 4, FAKE, need, None) == moe.MOE_ERR_ALIGN
    assert L.moe_forward_staged(ctypes.byref(c), *args, FAKE + 4, FAKE, need, None, None, None) == \
        moe.MOE_ERR_ALIGN
    assert L.moe_forward_ex(ctypes.byref(c), None, *args, FAKE + 4, FAKE, need, None) == moe.MOE_ERR_ALIGN


def test_backward_options_are_validated_before_launch():
    """moe_backward_ex reads the capacity only; statistics are refused, bad
    options and a short workspace are reported before anything is enqueued."""
    c = cfg()
    O = moe.MoeOptions
    L = moe.lib()
    need = moe.moe_backward_workspace_bytes(c)
    assert need > 0 and need % 256 == 0

    def bwd(opts, ws=FAKE, ws_bytes=1 << 40):
        return L.moe_backward_ex(ctypes.byref(c), ctypes.byref(opts) if opts is not None else None,
                                 *([FAKE] * 16), None, None, None, ws, ws_bytes, None)

    assert bwd(O(None, 0, 0, FAKE, 0.01)) == moe.MOE_ERR_UNSUPPORTED       # no statistics in the backward
    assert bwd(O(None, 2, 0, None, 0.0)) == moe.MOE_ERR_UNSUPPORTED        # bias space 0/1
    assert bwd(O(FAKE + 4, 0, 0, None, 0.0)) == moe.MOE_ERR_ALIGN         # bias alignment
    assert bwd(O(None, 0, 64, None, 0.0), ws=FAKE, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert bwd(None, ws=None) == moe.MOE_ERR_WORKSPACE


def test_noalloc_rejects_layers_past_its_array():
    """moe_forward_noalloc refuses a layer whose workspace exceeds its fixed
    array (here the Mixtral-8x7B prefill layer) before touching the GPU; a
    bad config is still a config error."""
    L = moe.lib()
    big = moe.MoeConfig.of(4096, 4096, 8, 2, 14336)
    assert moe.moe_workspace_bytes(big) > moe.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(big), *([FAKE] * 13), None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_forward_noalloc(None, *([FAKE] * 13), None) == moe.MOE_ERR_NULL
    assert L.moe_forward_noalloc(ctypes.byref(cfg(k=9)), *([FAKE] * 13), None) == moe.MOE_ERR_SHAPE


def test_forward_plan():
    """moe_forward_plan (host only): DeepSeek-V3's shared expert, as wide as
    its routed experts, runs inside the routed GEMMs; a narrower one, an fp32
    layer, a capacity-free decode batch on 32-row tiles and a layer without a
    shared expert do not."""
    ds = moe.MoeConfig.of(8192, 7168, 256, 8, 2048, 1, 2048, moe.MOE_SCORE_SIGMOID)
    assert moe.moe_forward_plan(ds) == dict(tile_rows=288, routed_splits=1, shared_splits=1,
                                            shared_merged=True)
    narrow = moe.MoeConfig.of(8192, 7168, 256, 8, 2048, 1, 1024, moe.MOE_SCORE_SIGMOID)
    assert not moe.moe_forward_plan(narrow)["shared_merged"]
    f32 = moe.MoeConfig.of(512, 256, 8, 2, 256, 1, 256, dtype=moe.MOE_F32)
    assert not moe.moe_forward_plan(f32)["shared_merged"]
    dec = moe.MoeConfig.of(8, 2048, 256, 8, 256, 1, 256, moe.MOE_SCORE_SIGMOID)
    p = moe.moe_forward_plan(dec)
    assert p["tile_rows"] == 32 and not p["shared_merged"]
    mix = moe.MoeConfig.of(4096, 4096, 8, 2, 14336)
    p = moe.moe_forward_plan(mix)
    assert p["shared_splits"] == 0 and not p["shared_merged"] and p["routed_splits"] >= 1
    assert p["tile_rows"] == 0                            # chosen on the device per call
    odd = moe.MoeConfig.of(4096, 4096 + 128, 8, 2, 14336)   # d not a multiple of 256: no choice
    assert moe.moe_forward_plan(odd)["tile_rows"] == 256
    L = moe.lib()
    assert L.moe_forward_plan(ctypes.byref(ds), None) == moe.MOE_ERR_NULL
    out = (ctypes.c_int32 * 4)()
    assert L.moe_forward_plan(ctypes.byref(cfg(k=0)), out) == moe.MOE_ERR_SHAPE


def test_forward_plan_tile_rows_boundaries():
    """Rows per tile of the routed GEMMs (host only): 288 exactly when the
    experts hold 224 to 287 rows on average and the tile queue runs (bf16,
    over 32 and under 640 rows per expert); 0 (each call chooses 256 or 288
    on the device) for bf16 layers of 640 rows per expert or more whose
    widths fit both kernels; else 256 (32 for few rows)."""
    def rows(T, k, E, dtype=moe.MOE_BF16):
        c = moe.MoeConfig.of(T, 512, E, k, 512, 0, 0, moe.MOE_SCORE_SIGMOID, dtype=dtype)
        return moe.moe_forward_plan(c)["tile_rows"]

    assert rows(8192, 8, 256) == 288                      # 256 rows per expert
    assert rows(7168, 8, 256) == 288                      # 224: the lower end
    assert rows(7167, 8, 256) == 256                      # just under 224
    assert rows(9215, 8, 256) == 288                      # 287.97
    assert rows(9216, 8, 256) == 256                      # 288: the upper end is open
    assert rows(8192, 8, 256, moe.MOE_F32) == 256
    assert rows(1024, 2, 8) == 288                        # 256 per expert, 8 experts
    assert rows(900, 2, 8) == 288                         # 225 per expert
    assert rows(2048, 2, 8) == 256                        # 512 per expert (tile queue, two tiles)
    assert rows(4096, 2, 8) == 0                          # 1024 per expert (no tile queue): chosen on the device
    assert rows(4096, 2, 8, moe.MOE_F32) == 256
    assert rows(32, 8, 256) == 32                         # decode


def test_forward_plan_shared_placement_boundaries():
    """Where moe_forward_plan puts a same-width shared expert (host only):
    inside the routed GEMMs only with the tile queue (fewer than 640 pairs per
    expert), more than one dispatch chunk (over 2048 pairs), 256-row tiles
    (over 32 pairs per expert), d a multiple of 256 and d_ff of 128, bf16."""
    def plan(T, d, E, k, f, fs=None, dtype=moe.MOE_BF16):
        c = moe.MoeConfig.of(T, d, E, k, f, 1, f if fs is None else fs, moe.MOE_SCORE_SIGMOID, dtype=dtype)
        return moe.moe_forward_plan(c)["shared_merged"]

    assert plan(1024, 512, 32, 4, 512)                    # 4096 pairs, 128 per expert
    assert not plan(1024, 512, 32, 4, 512, fs=256)        # narrower shared expert
    assert not plan(1024, 512, 32, 4, 512, dtype=moe.MOE_F32)
    assert not plan(1024, 384, 32, 4, 512)                # d not a multiple of 256
    assert not plan(1024, 512, 32, 4, 448)                # d_ff not a multiple of 128
    assert not plan(512, 512, 32, 4, 512)                 # 2048 pairs: one dispatch chunk
    assert plan(513, 512, 32, 4, 512)                     # 2052 pairs: two chunks
    assert not plan(5120, 512, 8, 1, 512)                 # 640 pairs per expert: fixed schedule
    assert plan(5119, 512, 8, 1, 512)
    assert not plan(2100, 512, 256, 1, 512)               # 8 pairs per expert: 32-row kernels
