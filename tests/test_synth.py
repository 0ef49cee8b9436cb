"""The seeded generator: determinism, counter addressing and the distributions
the workloads ask for (host only; no method arithmetic lives here)."""
import numpy as np

import synth


def test_rounding_matches_numpy_half():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 0.05, 5000), rng.normal(0, 1e-5, 5000), [65504, 65519.9, 65520, 2 ** -24,
                        2 ** -25, 2 ** -25 * 1.0001, -0.0, 0.0]])
    ours = np.array([synth.f16_bits(x) for x in v], dtype=np.uint16)
    np.testing.assert_array_equal(ours, v.astype(np.float16).view(np.uint16))


def test_bf16_rounding_is_nearest_even():
    assert synth.bf16_bits(1.0) == 0x3F80
    assert synth.bf16_bits(1.0 + 2 ** -8) == 0x3F80           # tie -> even
    assert synth.bf16_bits(1.0 + 3 * 2 ** -8) == 0x3F82       # tie -> even (up)
    assert synth.bf16_bits(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert synth.bf16_bits(-3.0) == 0xC040


def test_blobs_are_counter_addressed():
    a = synth.expert_blobs(0, 3, 10, 4, 64, 256, 128, 0.05)
    for i in range(4):
        np.testing.assert_array_equal(a[i], synth.expert_blob(0, 3, 10 + i, 64, 256, 128, 0.05))
    assert not np.array_equal(a[0], a[1])
    assert not np.array_equal(synth.expert_blob(1, 3, 10, 64, 256, 128, 0.05), a[0])


def test_scale_and_code_distributions():
    b = synth.expert_blob(0, 0, 0, 32, 512, 256, 0.02)
    nb = 256 * 512 // 32
    codes = b[:nb * 16]
    scales = b[nb * 16: nb * 18].view(np.float16).astype(np.float64)
    nib = np.concatenate([codes & 15, codes >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * nib.size / 16
    assert np.all(scales >= 0)
    assert abs(np.sqrt(np.mean(scales ** 2)) - 0.02) < 0.001     # |N(0, sigma)| has rms sigma


def test_zipf_logits_follow_popularity():
    E, T = 512, 4000
    rank = synth.popularity_rank(0, 5, E)
    assert sorted(rank) == list(range(E))
    l = synth.logits(0, 5, 0, T, E, 1.0)
    top = np.argsort(-l, axis=1, kind="stable")[:, :10]
    hot = int(np.argmin(rank))
    assert (top == hot).any(1).mean() > 0.7
    # a plain N(0,1) draw when s = 0
    l0 = synth.logits(0, 5, 0, 1000, 8, 0.0)
    assert abs(l0.std() - 1) < 0.05
    assert not np.array_equal(synth.logits(0, 5, 1, 4, E, 1.0), synth.logits(0, 5, 0, 4, E, 1.0))
