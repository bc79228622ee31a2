"""Seeded input generators: determinism, shapes, encodings, distributions."""
import numpy as np
import pytest

import synth


def test_bf16_rounding_ties_to_even_and_bits_roundtrip():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, 3.0e38], dtype=np.float32)
    r = synth.round_to_bf16(x)
    assert r[1] == 1.0                      # tie -> even mantissa
    assert r[2] == 1.0 + 2 ** -6            # tie -> even (up)
    np.testing.assert_array_equal(synth.bits_to_f32(synth.bf16_bits(r)), r)
    with pytest.raises(ValueError):
        synth.bf16_bits(np.array([1.0 + 2 ** -10], dtype=np.float32))


def test_suite_shapes_and_determinism():
    a = synth.make_suite((8, 24, 40), 101, 3, 5, seed=7)
    b = synth.make_suite((8, 24, 40), 101, 3, 5, seed=7)
    assert a.n_tokens == 15
    assert [x.shape for x in a.h] == [(15, 8), (15, 24), (15, 40)]
    assert [x.shape for x in a.emb] == [(101, 8), (101, 16), (101, 16)]
    assert [x.shape for x in a.w] == [(101, 8), (101, 24), (101, 40)]
    for x, y in zip(a.h + a.emb + a.w, b.h + b.emb + b.w):
        np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(a.ids, b.ids)
    # next-token structure: labels are the ids shifted by one within a row
    np.testing.assert_array_equal(a.ids.reshape(3, 5)[:, 1:], a.labels.reshape(3, 5)[:, :-1])
    for x in a.h + a.emb + a.w:
        synth.bf16_bits(x)                  # raises unless bf16-exact


def test_distributions():
    s = synth.make_suite((256, 512), 4096, 4, 512, seed=1)
    assert abs(s.h[0].std() - 4.0) < 0.05
    assert abs(s.w[1].std() - 0.02) < 5e-4
    assert s.ids.min() >= 0 and s.ids.max() < 4096
    # Zipf(1.1): token 0 is the most frequent, about 1/H_{V,1.1} of the mass
    w = (np.arange(4096) + 1.0) ** -1.1
    p0 = 1.0 / w.sum()
    assert abs(np.mean(s.ids == 0) - p0) < 0.02
    u = synth.make_suite((8,), 64, 8, 256, seed=2, ids="uniform", dtype="f32")
    assert u.h[0].dtype == np.float32 and abs(np.mean(u.ids == 0) - 1 / 64) < 0.01


def test_named_workloads_metadata():
    assert len(synth.WORKLOADS) == 5
    t = synth.make_workload(0)
    assert t.widths == (64, 128, 256) and t.vocab == 512 and t.n_tokens == 128
    assert t.dtype == "f32" and t.alpha == 0.3
    assert synth.WORKLOADS[4][8] == (0, 2)
