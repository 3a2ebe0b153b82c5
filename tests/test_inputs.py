"""Seeded input generators: determinism, shapes and format conversions."""
import numpy as np

import palu_inputs as PI


def test_deterministic_and_independent_streams():
    wl = PI.scaled("llama2_7b", batch=2, max_len=64)
    a = PI.latent(wl, "k", 1, 3)
    b = PI.latent(wl, "k", 1, 3)
    np.testing.assert_array_equal(a, b)
    assert a.dtype == np.float16 and a.shape == (64, 256)
    assert not np.array_equal(PI.latent(wl, "k", 1, 3), PI.latent(wl, "v", 1, 3))
    assert not np.array_equal(PI.latent(wl, "k", 0, 3), PI.latent(wl, "k", 1, 3))
    # a prefix of the stream does not depend on how many rows are drawn
    np.testing.assert_array_equal(PI.latent_f32(wl, "k", 0, 0, n=10), PI.latent_f32(wl, "k", 0, 0, n=64)[:10])


def test_ranks_and_lengths():
    wl = PI.workload("gqa_rope")
    r = PI.ranks(wl)
    assert r.shape == (4,) and set(r.tolist()) <= {128, 192, 256, 320}
    np.testing.assert_array_equal(r, PI.ranks(wl))
    wl = PI.workload("long_b4")
    L = PI.lengths(wl)
    assert L.shape == (4,) and L.min() >= 16384 and L.max() <= 32768
    assert PI.lengths(PI.workload("llama2_7b")).tolist() == [4096] * 16


def test_bf16_rounding():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    bits = PI.to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0); 1 + 3*2^-8 rounds up to 1 + 2^-6
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1 + 2 ** -6)
    assert back[3] == -2.5
    assert abs(back[4] - 3.0e38) / 3.0e38 < 2 ** -8


def test_factor_scale():
    wl = PI.workload("llama2_7b")
    B = PI.factor(wl, "Bk", 0).astype(np.float64)
    assert B.shape == (256, 512)
    assert abs(B.std() - 1 / 16) < 0.002
