"""AdamW on a flat parameter, fp64 (oracle; test infrastructure).

"SOAP, Muon, and Beyond", section 1-1: coordinate-wise first and second
moments m = b1 m + (1-b1) g, v = b2 v + (1-b2) g*g, update m/(sqrt(v)+eps).
Readings: bias correction m_hat = m/(1-b1^t), v_hat = v/(1-b2^t) (the standard
form; the FOAM review's "bias-corrected Adam step" uses it too), eps = 1e-8
added after the square root as printed, and decoupled weight decay
W <- W - lr (wd W + u). Used for the tied embedding of the FOAM workload,
which the FOAM review says stays on AdamW (section 4).

Parity: pinned (step-1 closed form u = g/(|g|+eps); constant-gradient
closed form).
"""
from __future__ import annotations

import numpy as np


def adamw_step(w, g, m, v, t: int, *, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float):
    """Returns (W_new, m_new, v_new, update) with update = m_hat/(sqrt(v_hat)+eps)."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m_new = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v_new = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    b1 = 1.0 - beta1 ** t
    b2 = 1.0 - beta2 ** t
    upd = (m_new / b1) / (np.sqrt(v_new / b2) + eps)
    w_new = w - lr * (weight_decay * w + upd)
    return w_new, m_new, v_new, upd
