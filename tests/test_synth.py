"""Seeded input generator: published SplitMix64 outputs, distribution sanity,
plant placement and bfloat16 rounding."""
import numpy as np
import pytest

import synth


def test_splitmix64_published_vector():
    # First outputs of SplitMix64 for seed 1234567, as published with the
    # generator's reference C code (Vigna, splitmix64.c) and its ports.
    got = [int(x) for x in synth.splitmix64(1234567, 5)]
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_stream_offsets_are_consistent():
    a = synth.splitmix64(42, 10)
    b = synth.splitmix64(42, 4, start=6)
    assert np.array_equal(a[6:], b)


def test_uniforms_in_half_open_unit_interval():
    u = synth.uniform53(7, 100000)
    assert u.min() > 0.0 and u.max() <= 1.0
    assert abs(u.mean() - 0.5) < 0.005


def test_normals_moments_and_determinism():
    z = synth.normal_f32(11, 200001)
    assert z.dtype == np.float32 and z.shape == (200001,)
    assert abs(float(z.mean())) < 0.01
    assert abs(float(z.var()) - 1.0) < 0.01
    assert np.array_equal(z, synth.normal_f32(11, 200001))
    assert not np.array_equal(z[:100], synth.normal_f32(12, 100))


def test_shapes_and_plants():
    q, k, v, pos = synth.case_planted_chunk(17, 31, 100, 3)
    assert q.shape == (17, 32, 64) and k.shape == (48, 8, 64) and v.shape == (48, 8, 64)
    assert len(set(pos)) == 3 and all(31 <= p < 48 for p in pos)
    for p in pos:
        assert np.all(q[p - 31, 0] == 4.0) and np.all(k[p, 0] == 4.0) and np.all(v[p, 0] == 4.0)
    # nothing else equals exactly 4.0 in head 0
    assert int((q[:, 0] == 4.0).all(axis=1).sum()) == 3


def test_last_key_case():
    q, k, v, pos = synth.case_last_key(8, 40, 400)
    assert pos == [47]
    assert np.all(k[47, 0] == 4.0) and np.all(q[7, 0] == 4.0)


def test_draw_distinct_rejects_impossible():
    with pytest.raises(ValueError):
        synth.draw_distinct(1, 0, 2, 3)


def test_bf16_round_to_nearest_even():
    # hand-made cases around ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5,
                  3.0e-39], np.float32)
    b = synth.to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                      # tie -> even (mantissa 0)
    assert back[2] == 1.0 + 4 * 2.0 ** -8      # tie -> even (round up)
    assert back[3] == 1.0 + 2.0 ** -7          # above the tie -> up
    assert back[4] == -2.5


def test_bf16_matches_torch_cast():
    torch = pytest.importorskip("torch")
    x = synth.normal_f32(5, 50000)
    ours = synth.to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
