"""CPU check of the low-rank-aware int4 reading (rotated chunks), in the
oracle only.  With a factorisation W = (U S)(V^T) the latents z = x U S carry
channel energy that decays along the rank while B = V^T has orthonormal rows,
so the error of a rebuilt key row, (z_hat - z) B, has the norm of the latent
error.  A plain int4 chunk's step is set by its largest channel; the rotated
chunk's by the chunk's total energy spread over 32 elements.  So: on latents
with decaying channel energy the rotated int4 cache rebuilds keys with a
smaller error than the plain one; on latents of equal channel energy the two
are about the same.  This states why the reading was adopted; correctness of
each function is pinned in test_oracle_pins.py."""
import numpy as np

import oracle as O


def _key_errors(decay, n=2000, r=160, w=256, seed=3):
    rng = np.random.default_rng(seed)
    sig = np.exp(-np.arange(r) / decay) if decay else np.ones(r)
    z = (rng.standard_normal((n, r)) * sig).astype(np.float32)
    V, _ = np.linalg.qr(rng.standard_normal((w, r)))
    B = V.T                                              # orthonormal rows
    K = z.astype(np.float64) @ B
    c, s = O.quant_int4(z)
    e_plain = O.dequant_int4(c, s) @ B - K
    c, s = O.quant_int4_rotated(z)
    B2 = O.fold_rotation(np.zeros((1, r)), B)[1]
    e_rot = O.dequant_int4(c, s) @ B2 - K
    return float(np.mean(e_plain ** 2)), float(np.mean(e_rot ** 2))


def test_rotation_helps_decaying_channel_energy():
    plain, rot = _key_errors(decay=16.0)
    assert rot < 0.6 * plain, (plain, rot)


def test_rotation_about_neutral_on_equal_channel_energy():
    plain, rot = _key_errors(decay=0)
    assert 0.7 * plain < rot < 1.3 * plain, (plain, rot)
