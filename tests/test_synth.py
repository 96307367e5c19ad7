"""The seeded input generator G (host side)."""
import numpy as np

import synth


def test_splitmix64_published_sequence():
    """SplitMix64 from state 0: the first three outputs of Vigna's reference
    generator (state advanced by the golden gamma before each output)."""
    z = np.array([0, synth.GAMMA, (2 * synth.GAMMA) & synth.MASK64], dtype=np.uint64)
    got = [int(x) for x in synth.splitmix64(z)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert synth.splitmix64_int(0) == 0xE220A8397B1DCDAF


def test_values_unit_variance_and_bounded():
    v = synth.bf16_bits_to_f32(synth.bf16_at(3, synth.TAG_K, np.arange(2_000_000)))
    assert abs(float(v.mean())) < 2e-3
    assert abs(float(v.std()) - 1.0) < 2e-3
    assert float(np.abs(v).max()) <= 3.46


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert synth.f32_to_bf16_rne(f).tolist()[:3] == [0x3F80, 0x3F80, 0x3F82]


def test_layer0_shared_between_branches_and_aligned_needles():
    wl = synth.workloads()[1].replace(layers=3)
    for which in ("q", "k", "v"):
        a = synth.step_tensor(wl, which + "L", 5, 0)
        b = synth.step_tensor(wl, which + "F", 5, 0)
        assert np.array_equal(a, b)
        a = synth.step_tensor(wl, which + "L", 5, 1)
        b = synth.step_tensor(wl, which + "F", 5, 1)
        assert not np.array_equal(a, b)
    q = synth.step_tensor(wl, "qL", 8, 2)
    n = synth.aligned_needle(wl, 8)
    assert n == 1
    assert np.all(q == synth.needle_bits(wl.seed, n, 128)[None, None, :])
    rows = synth.cache_rows(wl, synth.TAG_K, 0, 0, 3, 495, 505)
    assert np.array_equal(rows[5], synth.needle_bits(wl.seed, 1, 128))


def test_block_tables_are_a_permutation():
    wl = synth.workloads()["5-4k"].replace(batch=4, t0=np.array([4096, 100, 17, 1]))
    tables, nb = synth.paged_block_tables(wl)
    used = tables[tables >= 0]
    assert sorted(used.tolist()) == list(range(nb))


def test_forced_rate_flags_exact_count():
    f = synth.forced_rate_flags(3, 128, 4, 0.125)
    assert f.sum() == 64 and f.shape == (128, 4)


def test_device_source_uses_the_same_scale_bits():
    """The device generator hard-codes float32(1/sqrt(21845)); it must be the
    host constant's bit pattern."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(synth.__file__), "csrc", "fill.hip")).read()
    m = re.search(r"__uint_as_float\(0x([0-9A-Fa-f]+)u\)", src)
    assert m and int(m.group(1), 16) == int(synth.VALUE_SCALE.view(np.uint32))
