"""Muon and Muon+ step, fp64 (oracle; test infrastructure).

Follows "Muon+: Towards Better Muon via One Additional Normalization Step"
(gist.science), section 2, and the Muon recipe of "SOAP, Muon, and Beyond",
section 3-2 (2):

1. momentum  M_t = mu M_{t-1} + (1 - mu) G_t        (no Nesterov, no bias
   correction: the pages give neither; Newton-Schulz is scale-invariant)
2. O_t = Ortho(M_t), a Newton-Schulz approximation of the polar factor UV^T
   ("SOAP, Muon, and Beyond", section 2-1)
3. Muon+ only: O_t = Norm^(d)(O_t), d in {col, row, col-row, row-col}
4. W_t = W_{t-1} - lr (wd W_{t-1} + sqrt(m/n) O_t)   (decoupled weight decay
   0.1 from the recipe of section 3-2 (2); sqrt(m/n) from the Muon+ page,
   m = rows, n = cols of W as stored)

Readings where the pages leave a step open (each listed in the design notes):

* Input scaling before the iteration: X_0 = M / (||M||_F + eps), eps = 1e-7
  (the recipe's numerical epsilon). ||X_0||_2 <= 1 keeps every singular value
  inside the iteration's basin.
* The iteration runs on the wide orientation (rows <= cols) and transposes
  back; exact, because X p(X^T X) = p(X X^T) X.
* Iteration k: A = X X^T, B = b_k A + c_k A A, X <- a_k X + B X. The pages
  name coefficient families without printing them; the default is the
  classical Newton-Schulz quintic (15/8, -10/8, 3/8) for every k, i.e. the
  degree-2 Taylor polynomial of (1 - z)^{-1/2} at z = 1 - sigma^2, which
  fixes sigma = 1 with p'(1) = p''(1) = 0. A per-iteration table overrides it.
* Norm^(d) is not defined on the page. Reading: scale-preserving
  equalisation. col: every column j is rescaled to the RMS column norm
  ||O||_F / sqrt(n); row: every row i to ||O||_F / sqrt(m). Each pass keeps
  ||O||_F (up to eps), so the update scale -- and the learning rate -- stay
  those of Muon, as the page says Muon+ needs no re-tuning. col-row applies
  col first. eps = 1e-7 in the denominators.

Parity: pinned (Jacobi-SVD polar factor, Shampoo identity, transpose
symmetry, closed forms at ns_steps = 0 and step 1, Muon+ invariants).
"""
from __future__ import annotations

import numpy as np

CLASSICAL_QUINTIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)

NORM_MODES = {"none": 0, "row": 1, "col": 2, "col_row": 3, "row_col": 4}


def newton_schulz(m: np.ndarray, steps: int, coeffs=None, eps: float = 1e-7) -> np.ndarray:
    """Ortho(M): ``steps`` Newton-Schulz quintic iterations from
    X_0 = M / (||M||_F + eps) on the wide orientation."""
    x = np.asarray(m, dtype=np.float64)
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T
    x = x / (np.linalg.norm(x) + eps)
    for k in range(steps):
        a, b, c = (coeffs[k] if coeffs is not None else CLASSICAL_QUINTIC)
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x.T if transposed else x


def muon_plus_normalize(o: np.ndarray, mode: str, eps: float = 1e-7) -> np.ndarray:
    """Norm^(d)(O) on O in W's orientation (m x n)."""
    o = np.asarray(o, dtype=np.float64)
    m, n = o.shape

    def col(x):
        target = np.linalg.norm(x) / np.sqrt(n)
        norms = np.sqrt(np.sum(x * x, axis=0))
        return x * (target / (norms + eps))[None, :]

    def row(x):
        target = np.linalg.norm(x) / np.sqrt(m)
        norms = np.sqrt(np.sum(x * x, axis=1))
        return x * (target / (norms + eps))[:, None]

    if mode == "none":
        return o
    if mode == "col":
        return col(o)
    if mode == "row":
        return row(o)
    if mode == "col_row":
        return row(col(o))
    if mode == "row_col":
        return col(row(o))
    raise ValueError(mode)


def muon_update_direction(m: np.ndarray, ns_steps: int, coeffs=None, norm_mode: str = "none",
                          eps: float = 1e-7, norm_eps: float = 1e-7) -> np.ndarray:
    """sqrt(m/n) * Norm^(d)(Ortho(M)): the update before the learning rate."""
    rows, cols = m.shape
    o = newton_schulz(m, ns_steps, coeffs, eps)
    o = muon_plus_normalize(o, norm_mode, norm_eps)
    return np.sqrt(rows / cols) * o


def muon_step(w: np.ndarray, g: np.ndarray, mom: np.ndarray, *, lr: float, mu: float,
              weight_decay: float, ns_steps: int, coeffs=None, norm_mode: str = "none",
              eps: float = 1e-7, norm_eps: float = 1e-7):
    """One Muon(+) step. Returns (W_new, M_new, update) with
    update = sqrt(m/n) Norm(Ortho(M_new)) (before the learning rate)."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    mom_new = mu * np.asarray(mom, dtype=np.float64) + (1.0 - mu) * g
    upd = muon_update_direction(mom_new, ns_steps, coeffs, norm_mode, eps, norm_eps)
    w_new = w - lr * (weight_decay * w + upd)
    return w_new, mom_new, upd
