"""The seeded generator shared by the oracle and the HIP path (CPU only)."""

import numpy as np

import synth
from synth import configs as C


def test_splitmix64_published_vector():
    # First five outputs of SplitMix64 seeded with 1234567, as published with
    # the reference implementation (Vigna, splitmix64.c test vector).
    out = [int(x) for x in synth.words(np.uint64(1234567), np.arange(5))]
    assert out == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_deterministic_and_indexable():
    a = synth.tensor(synth.BF16N, 3, 9, (4, 33))
    b = synth.tensor(synth.BF16N, 3, 9, (4, 33))
    assert np.array_equal(a, b)
    sub = synth.values(synth.BF16N, 3, 9, np.array([0, 5, 131]))
    assert np.array_equal(sub, a.reshape(-1)[[0, 5, 131]])
    assert not np.array_equal(a, synth.tensor(synth.BF16N, 3, 10, (4, 33)))
    assert not np.array_equal(a, synth.tensor(synth.BF16N, 4, 9, (4, 33)))


def test_value_ranges_and_moments():
    i8 = synth.tensor(synth.I8U4, 1, 1, (1 << 16,)).astype(np.int64)
    assert i8.min() == -8 and i8.max() == 7
    counts = np.bincount(i8 + 8, minlength=16)
    assert counts.min() > 3800 and counts.max() < 4400
    u4 = synth.as_float(synth.BF16U4, synth.tensor(synth.BF16U4, 1, 1, (1 << 12,)))
    assert np.array_equal(u4, np.round(u4)) and u4.min() == -8 and u4.max() == 7
    n = synth.as_float(synth.BF16N, synth.tensor(synth.BF16N, 1, 2, (1 << 18,)))
    assert abs(n.mean()) < 0.01 and abs(n.std() - 1.0) < 0.01 and np.abs(n).max() <= 6.0


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    assert list(back) == [1.0, 1.0, 1.0 + 4 * 2**-8, 1.0, -2.5]


def test_rows_matches_full():
    cfg = C.TINY
    full = C.make(cfg, cfg.k_spec(2))
    t = np.array([0, 17, 2047])
    got = C.rows(cfg, cfg.k_spec(2), (np.zeros_like(t), t))
    assert np.array_equal(got, full[0, t])
