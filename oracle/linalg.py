"""Dense linear-algebra building blocks of the oracle (fp64, CPU).

* ``jacobi_svd`` -- one-sided (Hestenes) Jacobi SVD written out here, so the
  polar factor UV^T that Newton-Schulz must approach has a source independent
  of any library SVD. Pinned against ``numpy.linalg.svd`` in the tests.
* ``polar_svd`` -- UV^T, the polar factor of "SOAP, Muon, and Beyond",
  section 2-1 (Muon approximates the polar factor of the momentum).
* ``qr_positive`` -- QR with diag(R) >= 0 (LAPACK Householder through
  ``numpy.linalg.qr``, then column signs fixed). For a full-rank input that Q
  is unique. Pinned by its defining properties in the tests.
* ``eigh_descending`` -- eigenvectors of a symmetric matrix ordered by
  descending eigenvalue, column signs aligned with a reference basis (LAPACK
  through ``numpy.linalg.eigh``, then reordered). Pinned against the oracle's
  own Jacobi SVD (eigenvalues of a PSD matrix) and against the limit of
  repeated QR power iterations in the tests.
* ``sym_inv_root`` / ``shampoo_polar`` -- Shampoo's (G G^T)^{-1/4} G
  (G^T G)^{-1/4} ("SOAP, Muon, and Beyond", section 1-1 and the identity of
  section 2-1; picx.dev summary, theoretical foundation), with Moore-Penrose
  roots so that singular factors of a rectangular G are handled.
"""
from __future__ import annotations

import numpy as np


def jacobi_svd(a: np.ndarray, tol: float = 1e-15, max_sweeps: int = 100):
    """Thin SVD a = U diag(s) V^T by one-sided Jacobi rotations.

    Columns of a working copy are rotated pairwise until every pair is
    orthogonal to ``tol`` (relative); singular values are the final column
    norms. For a wide input the tall transpose is factored instead.
    Returns U (m x k), s (k), Vt (k x n) with k = min(m, n), s descending.
    """
    a = np.asarray(a, dtype=np.float64)
    m, n = a.shape
    if m < n:
        u, s, vt = jacobi_svd(a.T, tol, max_sweeps)
        return vt.T, s, u.T
    x = a.copy()
    v = np.eye(n)
    for _ in range(max_sweeps):
        rotated = False
        for p in range(n - 1):
            for q in range(p + 1, n):
                alpha = float(x[:, p] @ x[:, p])
                beta = float(x[:, q] @ x[:, q])
                gamma = float(x[:, p] @ x[:, q])
                if abs(gamma) <= tol * np.sqrt(alpha * beta) or gamma == 0.0:
                    continue
                rotated = True
                zeta = (beta - alpha) / (2.0 * gamma)
                t = np.sign(zeta) / (abs(zeta) + np.sqrt(1.0 + zeta * zeta)) if zeta != 0 else 1.0
                c = 1.0 / np.sqrt(1.0 + t * t)
                s_ = c * t
                xp, xq = x[:, p].copy(), x[:, q].copy()
                x[:, p] = c * xp - s_ * xq
                x[:, q] = s_ * xp + c * xq
                vp, vq = v[:, p].copy(), v[:, q].copy()
                v[:, p] = c * vp - s_ * vq
                v[:, q] = s_ * vp + c * vq
        if not rotated:
            break
    s = np.sqrt(np.sum(x * x, axis=0))
    order = np.argsort(-s)
    s = s[order]
    x = x[:, order]
    v = v[:, order]
    u = np.zeros_like(x)
    nz = s > 0
    u[:, nz] = x[:, nz] / s[nz]
    return u, s, v.T


def polar_svd(a: np.ndarray, rank_tol: float = 1e-12) -> np.ndarray:
    """U_r V_r^T over the singular values above ``rank_tol * s_max`` (the
    polar factor; for a rank-deficient input its partial isometry)."""
    u, s, vt = jacobi_svd(a)
    keep = s > rank_tol * (s[0] if s.size else 0.0)
    return u[:, keep] @ vt[keep, :]


def qr_positive(p: np.ndarray):
    """Householder QR of a square (or tall) matrix with diag(R) >= 0."""
    q, r = np.linalg.qr(np.asarray(p, dtype=np.float64))
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d[None, :], r * d[:, None]


def eigh_descending(s: np.ndarray, ref: np.ndarray | None = None):
    """(lam, Q): S = Q diag(lam) Q^T with lam descending; where ``ref`` is given,
    column j of Q is negated when q_j . ref_j < 0 (the sign of an eigenvector
    is free)."""
    w, q = np.linalg.eigh(np.asarray(s, dtype=np.float64))
    order = np.argsort(-w, kind="stable")
    w, q = w[order], q[:, order]
    if ref is not None:
        d = np.sign(np.sum(q * np.asarray(ref, dtype=np.float64), axis=0))
        d[d == 0] = 1.0
        q = q * d[None, :]
    return w, q


def sym_inv_root(s: np.ndarray, power: float, rel_floor: float = 1e-10) -> np.ndarray:
    """Moore-Penrose S^{-power} of a symmetric PSD matrix: eigenvalues below
    ``rel_floor * lambda_max`` are treated as zero and stay zero."""
    w, q = np.linalg.eigh(np.asarray(s, dtype=np.float64))
    cut = rel_floor * max(float(w.max()), 0.0)
    inv = np.zeros_like(w)
    keep = w > cut
    inv[keep] = w[keep] ** (-power)
    return (q * inv[None, :]) @ q.T


def shampoo_polar(g: np.ndarray) -> np.ndarray:
    """Shampoo's update with both EMAs switched off:
    (G G^T)^{-1/4} G (G^T G)^{-1/4}. Equal to UV^T (the pages' identity)."""
    g = np.asarray(g, dtype=np.float64)
    return sym_inv_root(g @ g.T, 0.25) @ g @ sym_inv_root(g.T @ g, 0.25)
