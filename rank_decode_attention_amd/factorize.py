"""Low-rank factorisation of per-head-group projection weights (offline,
host side; not part of the decode hot path).

The method replaces a key or value projection W (d_model x w for a head-group
of w = n_g * d_h columns) by W ~ A B with A in R^{d_model x r} and B in
R^{r x w} ("PALU low-rank projection decomposition" page, section "Low-rank
projection decomposition", formula block; arXiv 2407.21118v2 abstract:
medium-grained, per head-group).  The pages do not say how A and B are
obtained; this module takes the plain reading:

* factorisation: the truncated SVD W = U S V^T, A = U_r S_r, B = V_r^T (the
  best rank-r approximation in the Frobenius and spectral norms,
  Eckart-Young); B then has orthonormal rows, so the rebuilt keys and values
  K = z B keep the scale of the latents z = x A;
* rank allocation (optional): a total rank budget is spent in chunks of
  `granularity` ranks, each chunk going to the group whose next chunk of
  singular values carries the most energy (sum of squares), i.e. greedily
  minimising the total squared Frobenius error.  The pages' own rank search
  is not described there; this is an energy heuristic, not theirs.

Uses numpy's LAPACK SVD on the host.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

__all__ = ["factorize_group", "allocate_ranks", "factorize_layer", "fold_rotation"]


def factorize_group(W: np.ndarray, rank: int) -> Tuple[np.ndarray, np.ndarray, float]:
    """Rank-`rank` factorisation of one head-group's weight W [d_model][w]:
    returns (A [d_model][rank], B [rank][w], relative Frobenius error
    ||W - A B||_F / ||W||_F), in float64."""
    W = np.asarray(W, dtype=np.float64)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    if not 0 < rank <= min(W.shape):
        raise ValueError(f"rank must be in [1, {min(W.shape)}]")
    U, s, Vt = np.linalg.svd(W, full_matrices=False)
    A = U[:, :rank] * s[:rank]
    B = Vt[:rank]
    total = float(np.sum(s * s))
    err = float(np.sqrt(np.sum(s[rank:] ** 2) / total)) if total > 0 else 0.0
    return A, B, err


def allocate_ranks(spectra: Sequence[np.ndarray], budget: int, granularity: int = 32,
                   min_rank: int = 0) -> List[int]:
    """Split a total rank `budget` over groups with singular values
    `spectra[j]` (descending): every group starts at `min_rank` (rounded up to
    the granularity), then chunks of `granularity` ranks go one at a time to
    the group whose next chunk holds the largest squared singular values.
    Returns the ranks (multiples of the granularity, each <= its spectrum's
    length rounded down to the granularity, summing to at most the budget)."""
    if granularity <= 0 or budget < 0:
        raise ValueError("granularity must be positive and budget non-negative")
    sq = [np.asarray(s, dtype=np.float64) ** 2 for s in spectra]
    caps = [(len(s) // granularity) * granularity for s in sq]
    start = -(-min_rank // granularity) * granularity
    ranks = [min(start, c) for c in caps]
    left = budget - sum(ranks)
    if left < 0:
        raise ValueError("budget below the minimum ranks")

    def gain(j: int) -> float:
        r = ranks[j]
        return float(np.sum(sq[j][r:r + granularity])) if r + granularity <= caps[j] else -1.0

    while left >= granularity:
        j = max(range(len(sq)), key=gain)
        if gain(j) < 0:
            break
        ranks[j] += granularity
        left -= granularity
    return ranks


def factorize_layer(W_groups: Sequence[np.ndarray], ranks: Sequence[int]):
    """Factorise every head-group's weight at its rank: returns
    ([A_j], [B_j], [relative error_j])."""
    out = [factorize_group(W, int(r)) for W, r in zip(W_groups, ranks)]
    return [o[0] for o in out], [o[1] for o in out], [o[2] for o in out]


def _sylvester(n: int) -> np.ndarray:
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.vstack([np.hstack([H, H]), np.hstack([H, -H])])
    return H


def fold_rotation(A: np.ndarray, B: np.ndarray, chunk: int = 32) -> Tuple[np.ndarray, np.ndarray]:
    """Factors for latents quantised with palu_quant_latent_rotated: A' = A H
    and B' = H B / chunk on every full `chunk`-row block of the rank (H the
    Sylvester Hadamard matrix, entries +-1, H H^T = chunk I; a trailing
    partial block is left as is), so that (x A') B' = x A B and x A' is the
    chunk-rotated latent.  float64."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    r = A.shape[1]
    if B.shape[0] != r:
        raise ValueError("A and B ranks differ")
    H = _sylvester(chunk)
    A2, B2 = A.copy(), B.copy()
    for c in range(r // chunk):
        sl = slice(c * chunk, (c + 1) * chunk)
        A2[:, sl] = A[:, sl] @ H
        B2[sl] = (H @ B[sl]) / chunk
    return A2, B2
