"""The device-side tile-height rule as the bench labels it and the GPU tests
expect it (host only).  The rule itself runs in the kernels
(tall_tiles_chosen); bench.device_tile_rows (and the parity tests'
tile_choice_rows) restate it from its documentation, and
test_device_tile_choice checks on the GPU, through moe_forward's output, that
the kernels take the height the restatement names.  Here: the bench's
restatement agrees with the rule written out once more by loops, and the
layer shapes whose routing the documentation quotes get the heights it names
(Mixtral prefill 288, Hunyuan-A13B 256)."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), ".."))

import bench  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402


def rows_by_rounds(counts, d_ff, slots=256):
    # written out once more, by loops: tiles per height, rounds, the 9/8 weight
    tn = 2 * d_ff // 256
    rounds = {}
    for bm in (256, 288):
        tiles = 0
        for n in counts:
            tiles += (int(n) + bm - 1) // bm
        rounds[bm] = (tiles * tn + slots - 1) // slots
    return 288 if 9 * rounds[288] < 8 * rounds[256] else 256


def test_restatements_agree_on_random_counts():
    rng = np.random.default_rng(0)
    for _ in range(300):
        E = int(rng.integers(1, 257))
        counts = rng.integers(0, 3000, E)
        d_ff = int(rng.choice([128, 512, 2048, 8192, 14336]))
        want = rows_by_rounds(counts, d_ff)
        assert bench.device_tile_rows(counts, d_ff) == want
    # equal rounds keep the 256-row tiles; 9/8 of the rounds decides
    assert bench.device_tile_rows([1024] * 8, 14336) == 256
    assert bench.device_tile_rows([1050] * 8, 14336) == 288     # 40 vs 32 tiles: 18 vs 14 rounds


def test_documented_layers():
    for name, want in (("mixtral_prefill", 288), ("hunyuan_a13b", 256)):
        sh = synth.SHAPES[name]
        x, w_router = synth.make_router_and_x(sh, 0)
        ids = oracle.route(oracle.logits(x, w_router), sh.k, sh.score_fn, sh.renormalize)["ids"]
        counts = np.bincount(ids.ravel(), minlength=sh.E)
        assert bench.device_tile_rows(counts, sh.d_ff) == want, (name, counts.min(), counts.max())
