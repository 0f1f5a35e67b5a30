"""SOAP step with the real-time eigenbasis refresh, fp64 (oracle; test
infrastructure).

Sources: "SOAP, Muon, and Beyond", section 1-1 (factor EMAs
L = b2 L + (1-b2) G G^T, R = b2 R + (1-b2) G^T G), section 3-2 (3) (rotate
the momentum by Q_L^T . Q_R, Adam in that basis, rotate back with Q_L . Q_R^T;
rotations keep the Frobenius norm) and section 3-2 (4) (real-time update:
factors take the current gradient first, then the basis is refreshed and
re-orthogonalised by QR, then the same step's momentum is preconditioned);
picx.dev summary Eq. (1) u = Q_L Adam(Q_L^T m Q_R) Q_R^T. The refresh is one
power-iteration step Q <- qr(F Q) per factor F.

Step t (1-based), in the pages' order:

1. M = b1 M + (1-b1) G                      (momentum in the original space)
2. L = b2 L + (1-b2) G G^T,  R = b2 R + (1-b2) G^T G   (current G included)
3. if the step refreshes: Q_L = qr(L Q_L), Q_R = qr(R Q_R), diag(R) >= 0
4. G~ = Q_L^T G Q_R,  M~ = Q_L^T M Q_R       (with the refreshed basis)
5. V = b2 V + (1-b2) G~ * G~                 (rotated second moment)
6. N = (M~ / (1-b1^t)) / (sqrt(V / (1-b2^t)) + eps)
7. U = Q_L N Q_R^T;  W = W - lr (wd W + U)

Readings where the pages are silent (listed in the design notes): Adam
eps = 1e-8 after the square root; the same b2 for the factors and for V; no
eigenvalue sorting or column permutation after QR; V is not re-projected
when the basis moves; Q_L = I, Q_R = I and all other state zero at t = 1;
``refresh_every`` = 1 refreshes every step, k > 1 at t = 1, k+1, ..., and 0
freezes the basis.

``q_override`` hands the step an externally computed refreshed basis
(teacher-forced parity: the step is finished with the other side's Q).

Parity: pinned (t = 1 closed form N = G~/(|G~|+eps); frozen basis == AdamW;
b1 = b2 = 0 with a converged basis == UV^T; rotation norm preservation;
state size 2mn + 2m^2 + 2n^2).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .linalg import qr_positive


@dataclass
class SoapState:
    M: np.ndarray
    V: np.ndarray
    L: np.ndarray
    R: np.ndarray
    QL: np.ndarray
    QR: np.ndarray

    def copy(self) -> "SoapState":
        return SoapState(*(x.copy() for x in (self.M, self.V, self.L, self.R, self.QL, self.QR)))


def soap_init(m: int, n: int) -> SoapState:
    return SoapState(np.zeros((m, n)), np.zeros((m, n)), np.zeros((m, m)), np.zeros((n, n)),
                     np.eye(m), np.eye(n))


def soap_refreshes(t: int, refresh_every: int) -> bool:
    return refresh_every > 0 and (t - 1) % refresh_every == 0


def soap_step(w, g, state: SoapState, t: int, *, lr: float, beta1: float, beta2: float,
              eps: float = 1e-8, weight_decay: float = 0.0, refresh_every: int = 1,
              q_override=None):
    """One SOAP step. Returns (W_new, new_state, U, info); ``info`` holds the
    power-iteration products P_L = L Q_L, P_R = R Q_R (before QR), the
    rotated gradient and N."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    s = state.copy()
    s.M = beta1 * s.M + (1.0 - beta1) * g
    s.L = beta2 * s.L + (1.0 - beta2) * (g @ g.T)
    s.R = beta2 * s.R + (1.0 - beta2) * (g.T @ g)
    info = {}
    if soap_refreshes(t, refresh_every):
        info["PL"] = s.L @ s.QL
        info["PR"] = s.R @ s.QR
        s.QL = qr_positive(info["PL"])[0]
        s.QR = qr_positive(info["PR"])[0]
    if q_override is not None:
        s.QL = np.asarray(q_override[0], dtype=np.float64)
        s.QR = np.asarray(q_override[1], dtype=np.float64)
    g_rot = s.QL.T @ g @ s.QR
    m_rot = s.QL.T @ s.M @ s.QR
    s.V = beta2 * s.V + (1.0 - beta2) * g_rot * g_rot
    b1 = 1.0 - beta1 ** t
    b2 = 1.0 - beta2 ** t
    n_rot = (m_rot / b1) / (np.sqrt(s.V / b2) + eps)
    upd = s.QL @ n_rot @ s.QR.T
    w_new = w - lr * (weight_decay * w + upd)
    info.update(g_rot=g_rot, m_rot=m_rot, N=n_rot)
    return w_new, s, upd, info


def soap_state_bytes(m: int, n: int, bytes_per_elem: int = 4) -> int:
    """{M, V, L, R, Q_L, Q_R}: 2mn + 2m^2 + 2n^2 elements (FOAM review,
    section 1)."""
    return bytes_per_elem * (2 * m * n + 2 * m * m + 2 * n * n)
