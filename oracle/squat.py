"""Plain fp64 reference of the SQuat-style key coder's set-up: the query
subspace and the update coefficients.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the GPU library never imports it.

Source: the SQuat explainer page (aibr.jp, "SQuat"), section 3
中核となる技術的要素, read as follows (the page gives the steps in prose only):
  1. the query subspace is spanned by the principal directions of the past
     queries: here the r eigenvectors of C = sum_q q q^T (the queries of the
     query heads that read the KV head) with the largest eigenvalues;
  2. keys are quantized element by element, and after each element the
     elements not yet quantized take the closed-form optimal correction. The
     objective read here is E(e) = ||U^T e||^2 + lambda ||e||^2 for the error e
     of the key (U the orthonormal subspace basis; lambda > 0 keeps the
     correction finite once fewer free elements remain than the subspace has
     dimensions). Minimising E over the free elements after fixing element c
     is the optimal-brain-surgeon step: with Hinv = (U U^T + lambda I)^-1 and
     T its upper Cholesky factor (Hinv = T^T T), element j > c moves by
     -delta * T[c][j] / T[c][c]; g[c][j] = T[c][j] / T[c][c] are the update
     coefficients (the codes themselves are decided in fp32 by the C oracle,
     or_squat_token).
"""

from __future__ import annotations

import numpy as np


def subspace(queries, rank: int) -> np.ndarray:
    """Orthonormal basis [d, rank] of the top-`rank` eigenvectors of
    sum_q q q^T over the rows of `queries` ([n, d], any float dtype), in fp64."""
    q = np.asarray(queries, dtype=np.float64)
    d = q.shape[1]
    if rank == 0:
        return np.zeros((d, 0))
    c = q.T @ q
    w, v = np.linalg.eigh(c)  # ascending eigenvalues
    return v[:, ::-1][:, :rank].copy()


def inverse_objective(u: np.ndarray, lam: float) -> np.ndarray:
    """(U U^T + lambda I)^-1 for an orthonormal U: 1/lambda off the subspace,
    1/(1 + lambda) on it."""
    d = u.shape[0]
    p = u @ u.T
    return (np.eye(d) - p) / lam + p / (1.0 + lam)


def coefficients(u: np.ndarray, lam: float) -> np.ndarray:
    """Update coefficients g[c][j] = T[c][j] / T[c][c] for j > c (0 elsewhere),
    T the upper Cholesky factor of (U U^T + lambda I)^-1, in fp64."""
    hinv = inverse_objective(u, lam)
    t = np.linalg.cholesky(hinv).T  # numpy returns the lower factor L = T^T
    g = t / np.diag(t)[:, None]
    return np.triu(g, k=1)


def unit_coefficients(q_unit, rank: int, lam: float) -> np.ndarray:
    """g as fp32 (the precision the coder uses) from one unit's past queries."""
    return coefficients(subspace(q_unit, rank), lam).astype(np.float32)
