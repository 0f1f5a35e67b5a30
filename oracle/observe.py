"""Observability quantities of the optimizer step (fp64, CPU; test infrastructure).

Sources:

* "SOAP, Muon, and Beyond" review, section 2-1: the update RMS that update
  scales are matched by, the Frobenius norm of the update divided by the
  square root of the number of entries; section 7-2, item 4: an optimizer log
  should carry the layer-wise update RMS, the Newton-Schulz residual, the SOAP
  factor condition number and the basis update age.
* "Factored One-sided Adam-Moment for Practical and Scalable SOAP" review,
  section 3: the rank-1 share of the rotated second moment (about 0.84 in
  FOAM's input-only basis) as the reason to factor after rotating.

The pages name the last four quantities without formulas. Readings:

* Newton-Schulz residual: ||X X^T - I||_F / sqrt(a) for the iteration's
  output X taken on its wide orientation (a = min(rows, cols)), i.e. the RMS
  of s_i^2 - 1 over the singular values of X; zero exactly at the polar
  factor the iteration approaches (section 2-1).
* Factor condition number: max_i d_i / min_i d_i with d_i = q_i^T F q_i, the
  Rayleigh quotients of the factor F in its current basis Q (the basis the
  power iteration maintains); equal to cond(F) when Q diagonalises F.
* Rank-1 share: s_1(V)^2 / ||V||_F^2, the fraction of the squared Frobenius
  mass that the best rank-1 approximation keeps (Eckart-Young).
* Basis age: steps since the basis was last refreshed, 0 on a refreshing
  step.

Parity status: every function here is pinned in tests/test_oracle_pins.py
against closed forms (constant and one-entry matrices, matrices built from
known singular values and orthonormal bases, diagonal and rank-1 inputs).
"""
from __future__ import annotations

import numpy as np


def matrix_rms(x: np.ndarray) -> float:
    """||x||_F / sqrt(number of entries)."""
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.sum(x * x) / x.size))


def ns_residual(o: np.ndarray, scale: float = 1.0) -> float:
    """||X X^T - I||_F / sqrt(a) with X = scale * o on its wide orientation."""
    x = scale * np.asarray(o, dtype=np.float64)
    if x.shape[0] > x.shape[1]:
        x = x.T
    a = x.shape[0]
    e = x @ x.T - np.eye(a)
    return float(np.sqrt(np.sum(e * e) / a))


def rayleigh(f: np.ndarray, q: np.ndarray):
    """(d, kappa): d_i = q_i^T f q_i for every column q_i of q, and
    kappa = max d / min d (inf when min d <= 0)."""
    f = np.asarray(f, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    d = np.array([q[:, i] @ (f @ q[:, i]) for i in range(q.shape[1])])
    kappa = float(d.max() / d.min()) if d.min() > 0 else float("inf")
    return d, kappa


def rank1_share(v: np.ndarray) -> float:
    """s_1(v)^2 / ||v||_F^2 (0 for a zero matrix)."""
    v = np.asarray(v, dtype=np.float64)
    mass = float(np.sum(v * v))
    if mass == 0.0:
        return 0.0
    s1 = np.linalg.svd(v, compute_uv=False)[0]
    return float(s1 * s1 / mass)


def basis_ages(refreshed) -> list:
    """Age after each step given whether that step refreshed the basis
    (starting from age 0 before the first step)."""
    ages, age = [], 0
    for r in refreshed:
        age = 0 if r else age + 1
        ages.append(age)
    return ages
