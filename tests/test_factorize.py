"""Host-side low-rank factorisation helper (rank_decode_attention_amd.factorize),
pinned against matrices of known singular values (the best rank-r
approximation and its error are then known in closed form: Eckart-Young) and
the rank allocation against brute force."""
import itertools

import numpy as np
import pytest

from rank_decode_attention_amd import factorize as F


def _known(d, w, s, seed):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((d, len(s))))
    V, _ = np.linalg.qr(rng.standard_normal((w, len(s))))
    return U, np.asarray(s, dtype=np.float64), V


@pytest.mark.parametrize("r", [1, 5, 17, 32])
def test_truncation_is_the_known_best_approximation(r):
    s = np.linspace(9.0, 0.5, 32)             # distinct singular values
    U, s, V = _known(96, 64, s, seed=r)
    W = (U * s) @ V.T
    A, B, err = F.factorize_group(W, r)
    best = (U[:, :r] * s[:r]) @ V[:, :r].T
    assert np.allclose(A @ B, best, atol=1e-10)
    assert abs(err - np.sqrt(np.sum(s[r:] ** 2) / np.sum(s ** 2))) < 1e-12
    assert np.allclose(B @ B.T, np.eye(r), atol=1e-12)          # orthonormal rows
    x = np.random.default_rng(1).standard_normal((5, 96))
    assert np.allclose((x @ A) @ B, x @ best, atol=1e-10)        # K = (x A) B = x W_r


def test_full_rank_is_exact():
    W = np.random.default_rng(2).standard_normal((40, 24))
    A, B, err = F.factorize_group(W, 24)
    assert np.allclose(A @ B, W, atol=1e-12) and err < 1e-14


def test_rejects_bad_rank():
    with pytest.raises(ValueError):
        F.factorize_group(np.ones((4, 3)), 4)


def test_allocation_hand_worked():
    """Chunks of 2: group 0 energies per chunk 200, 2; group 1: 50, 50, 0."""
    s0 = np.array([10, 10, 1, 1], dtype=np.float64)
    s1 = np.array([5, 5, 5, 5, 0, 0], dtype=np.float64)
    assert F.allocate_ranks([s0, s1], budget=2, granularity=2) == [2, 0]
    assert F.allocate_ranks([s0, s1], budget=6, granularity=2) == [2, 4]
    assert F.allocate_ranks([s0, s1], budget=8, granularity=2) == [4, 4]
    assert F.allocate_ranks([s0, s1], budget=100, granularity=2) == [4, 6]   # capped by the spectra
    assert F.allocate_ranks([s0, s1], budget=6, granularity=2, min_rank=2) == [2, 4]


def test_allocation_is_optimal_by_brute_force():
    """Sorted spectra make chunk energies non-increasing per group, so the
    greedy allocation captures the most energy of any allocation."""
    rng = np.random.default_rng(7)
    spectra = [np.sort(rng.uniform(0, 3, n))[::-1] for n in (8, 12, 6)]
    g = 2
    for budget in range(0, 27, 2):
        got = F.allocate_ranks(spectra, budget, granularity=g)
        cap = lambda s: (len(s) // g) * g
        best = -1.0
        for alloc in itertools.product(*[range(0, cap(s) + 1, g) for s in spectra]):
            if sum(alloc) <= budget:
                best = max(best, sum(float(np.sum(s[:a] ** 2)) for s, a in zip(spectra, alloc)))
        mine = sum(float(np.sum(s[:a] ** 2)) for s, a in zip(spectra, got))
        assert abs(mine - best) < 1e-9 and sum(got) <= budget and all(a % g == 0 for a in got)


def test_factorize_layer_matches_groups():
    rng = np.random.default_rng(3)
    Ws = [rng.standard_normal((64, 32)) for _ in range(3)]
    As, Bs, errs = F.factorize_layer(Ws, [8, 16, 32])
    for W, A, B, e, r in zip(Ws, As, Bs, errs, [8, 16, 32]):
        assert A.shape == (64, r) and B.shape == (r, 32)
        assert abs(np.linalg.norm(W - A @ B) / np.linalg.norm(W) - e) < 1e-12
