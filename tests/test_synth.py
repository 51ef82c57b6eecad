"""The seeded input generator: known-answer Philox, slices, distributions."""
import numpy as np

import synth


def test_philox_known_answers():
    """Philox4x32-10 known-answer vectors (Salmon et al., SC'11 / Random123)."""
    assert synth.philox_block(0, 0, [0, 0, 0, 0]).tolist() == [
        0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]
    assert synth.philox_block(0xffffffff, 0xffffffff, [0xffffffff] * 4).tolist() == [
        0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]
    assert synth.philox_block(0xa4093822, 0x299f31d0,
                              [0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344]).tolist() == [
        0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]


def test_slices_are_consistent():
    full = synth.normal(5, 2, 10001, 0.5, synth.BF16)
    for first, n in [(0, 7), (1, 8), (4999, 1002), (10000, 1)]:
        part = synth.normal(5, 2, n, 0.5, synth.BF16, first=first)
        np.testing.assert_array_equal(part, full[first:first + n])
    rows = synth.normal_rows(5, 2, 3, 4, 9, 1000, 0.5, synth.BF16)
    np.testing.assert_array_equal(rows, np.stack([full[3 + r * 1000: 12 + r * 1000] for r in range(4)]))


def test_distribution_and_rounding():
    a = synth.normal(0, 1, 1 << 20, 2.0, synth.F32)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 2.0) < 0.01
    b = synth.normal(0, 1, 1 << 20, 2.0, synth.BF16)
    # bf16 is the round-to-nearest-even of the fp32 value
    u = a.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(b, rne)


def test_zipf_shift_sets_logit_offsets():
    sh = synth.SHAPES["hunyuan_a13b"].replace(T=16)
    x, wr = synth.make_router_and_x(sh, 0)
    m = synth.zipf_shift(sh, wr, 0)
    W = synth.bf16_to_f64(wr)
    ranks = synth.zipf_perm_ranks(sh, 0)
    p = np.arange(1, 65, dtype=float) ** -1.1
    p /= p.sum()
    np.testing.assert_allclose(W @ m, 0.6 * np.log(p[ranks - 1]), atol=1e-9)
    assert sorted(ranks.tolist()) == list(range(1, 65))
