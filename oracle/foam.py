"""FOAM step (input-only rotation, factored Adam moment), fp64 (oracle; test
infrastructure).

Source: "Factored One-sided Adam-Moment for Practical and Scalable SOAP"
review, section 1 (input-only preconditioning G_rot = G Q_R; factored moment
from EMAs of the row mean r in R^m and column mean c in R^n of the rotated
squared gradient, reconstructed as tau r_hat c_hat^T with
tau = tr(R) / (||r_hat||_1 ||c_hat||_1); exact under K-FAC with a diagonal
output side) and section 3 (state mn + 2n^2 + m + n; R's EMA, refresh only
when the adaptive-tolerance criterion with pf = 10, tol = 0.1 fires, then a
bias-corrected Adam step in the rotated space).

Step t (1-based):

1. M = b1 M + (1-b1) G;  R = b2 R + (1-b2) G^T G
2. if (t-1) mod pf == 0: D = Q_R^T R Q_R, rho = ||D - diag D||_F / ||D||_F;
   if rho > tol: Q_R = qr(R Q_R) (diag >= 0)
3. G_rot = G Q_R;  M_rot = M Q_R
4. r = b2 r + (1-b2) rowmean(G_rot^2);  c = b2 c + (1-b2) colmean(G_rot^2)
5. r_hat = r/(1-b2^t), c_hat = c/(1-b2^t), R_hat = R/(1-b2^t),
   tau = tr(R_hat) / (||r_hat||_1 ||c_hat||_1)   (0 when r = c = 0)
6. N = (M_rot/(1-b1^t)) / (sqrt(tau r_hat c_hat^T) + eps)
7. U = N Q_R^T;  W = W - lr (wd W + U)

Readings (listed in the design notes): the refresh criterion is not defined
on the page; the reading above checks the off-diagonal mass of R in the
current basis every pf steps and refreshes by the same one-step QR power
iteration SOAP uses. tau takes the bias-corrected trace tr(R_hat): with the
plain trace the reconstruction is off by 1/(1-b2^t) and the page's exactness
claim fails. eps = 1e-8.

``q_override`` / ``refresh_override`` let a teacher-forced test finish the
step with the other side's basis and refresh decision.

Refresh by full eigendecomposition (``refresh="eigh"``): the review's section
1 describes FOAM's basis as the eigenvectors of R, recomputed periodically,
and its section 3 counts the eigendecompositions it saves. With this variant a
triggered refresh sets Q_R to the eigenvectors of R itself (not one power
step). Readings: the columns are ordered by descending eigenvalue -- the order
the QR power step converges to, so both refreshes name the same basis in the
limit -- ties kept in LAPACK's order; each column's sign follows the previous
basis (q_new . q_old >= 0; the update does not depend on signs).

Output-only variant (``side="output"``): the review's section 3 ablation
keeps the basis on the output side instead. Reading: the mirror of the
steps above with the factor L = b2 L + (1-b2) G G^T (m x m) and its basis
Q_L in place of R and Q_R; G_rot = Q_L^T G, M_rot = Q_L^T M; r and c stay the
row and column means of G_rot^2 (lengths m and n); tau = tr(L_hat) /
(||r_hat||_1 ||c_hat||_1); U = Q_L N. The state fields R and QR then hold L
and Q_L.

Parity: pinned (exact reconstruction of SOAP's dense rotated moment on
Rademacher K-FAC gradients, on either side; mass invariant
sum(tau r c^T) = tr(R_hat); rho = 0 in R's eigenbasis and no refresh at
rho = tol; the refresh as one orthogonal-iteration step: with b2 = 0 and a
fixed G, k refreshes give qr(R^k) and rho converges to 0; the eigh refresh
diagonalises R with the oracle's Jacobi-SVD eigenvalues in descending order,
equals the limit of repeated QR refreshes and leaves rho at 0; the output variant
equals the input variant on the transposed problem; state size
mn + 2n^2 + m + n).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .linalg import eigh_descending, qr_positive


@dataclass
class FoamState:
    M: np.ndarray
    R: np.ndarray
    QR: np.ndarray
    r: np.ndarray
    c: np.ndarray

    def copy(self) -> "FoamState":
        return FoamState(*(x.copy() for x in (self.M, self.R, self.QR, self.r, self.c)))


def foam_init(m: int, n: int, side: str = "input") -> FoamState:
    k = m if side == "output" else n
    return FoamState(np.zeros((m, n)), np.zeros((k, k)), np.eye(k), np.zeros(m), np.zeros(n))


def offdiag_ratio(d: np.ndarray) -> float:
    """||D - diag(D)||_F / ||D||_F (0 for D = 0)."""
    d = np.asarray(d, dtype=np.float64)
    total = np.linalg.norm(d)
    if total == 0.0:
        return 0.0
    off = d - np.diag(np.diag(d))
    return float(np.linalg.norm(off) / total)


def foam_checks(t: int, pf: int) -> bool:
    return (t - 1) % pf == 0


def foam_step(w, g, state: FoamState, t: int, *, lr: float, beta1: float, beta2: float,
              eps: float = 1e-8, weight_decay: float = 0.0, pf: int = 10, tol: float = 0.1,
              q_override=None, refresh_override=None, side: str = "input",
              refresh: str = "qr"):
    """One FOAM step. Returns (W_new, new_state, U, info); ``info`` holds rho,
    the refresh decision, P = R Q_R (QR refresh) or the eigenvalues (eigh
    refresh) when checked, tau and N. ``side``: "input" (the review's FOAM) or
    "output" (its output-only ablation). ``refresh``: "qr" (one power step)
    or "eigh" (full eigendecomposition)."""
    if side not in ("input", "output"):
        raise ValueError(side)
    if refresh not in ("qr", "eigh"):
        raise ValueError(refresh)
    out_side = side == "output"
    refresh_mode_eigh = refresh == "eigh"
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    s = state.copy()
    s.M = beta1 * s.M + (1.0 - beta1) * g
    s.R = beta2 * s.R + (1.0 - beta2) * ((g @ g.T) if out_side else (g.T @ g))
    info = {"checked": False, "refreshed": False}
    if foam_checks(t, pf):
        d = s.QR.T @ s.R @ s.QR
        rho = offdiag_ratio(d)
        refresh = rho > tol
        if refresh_override is not None:
            refresh = bool(refresh_override)
        info.update(checked=True, rho=rho, refreshed=refresh)
        if refresh and refresh_mode_eigh:
            info["eigenvalues"], s.QR = eigh_descending(s.R, ref=s.QR)
        elif refresh:
            info["P"] = s.R @ s.QR
            s.QR = qr_positive(info["P"])[0]
    if q_override is not None:
        s.QR = np.asarray(q_override, dtype=np.float64)
    if out_side:
        g_rot = s.QR.T @ g
        m_rot = s.QR.T @ s.M
    else:
        g_rot = g @ s.QR
        m_rot = s.M @ s.QR
    sq = g_rot * g_rot
    s.r = beta2 * s.r + (1.0 - beta2) * sq.mean(axis=1)
    s.c = beta2 * s.c + (1.0 - beta2) * sq.mean(axis=0)
    b1 = 1.0 - beta1 ** t
    b2 = 1.0 - beta2 ** t
    r_hat = s.r / b2
    c_hat = s.c / b2
    denom = r_hat.sum() * c_hat.sum()
    tau = float(np.trace(s.R / b2) / denom) if denom > 0 else 0.0
    v_hat = tau * np.outer(r_hat, c_hat)
    n_rot = (m_rot / b1) / (np.sqrt(v_hat) + eps)
    upd = (s.QR @ n_rot) if out_side else (n_rot @ s.QR.T)
    w_new = w - lr * (weight_decay * w + upd)
    info.update(tau=tau, N=n_rot, g_rot=g_rot, v_hat=v_hat)
    return w_new, s, upd, info


def foam_state_bytes(m: int, n: int, bytes_per_elem: int = 4, side: str = "input") -> int:
    """{M, R, Q_R, r, c}: mn + 2n^2 + m + n elements (FOAM review, section 3);
    the output variant keeps m x m factors instead."""
    k = m if side == "output" else n
    return bytes_per_elem * (m * n + 2 * k * k + m + n)
