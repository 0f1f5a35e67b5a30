"""Facts about the seeded synthetic inputs that the GPU parity tests rely on
(CPU, fp64)."""
import numpy as np

import synth
from synth import bf16_round


def test_llama8b_o_factor_is_numerically_rank_deficient_at_step_one():
    """The Kronecker gradients of the 8B layer's O projection (4096 x 4096,
    row and column covariance spectra proportional to 1/k) give a step-1
    factor L_1 = (1 - b2) G_1 G_1^T of full exact rank but condition number
    above 2^24 (directions fp32 cannot resolve), and a step-2 factor below
    it. The full-size SOAP parity test gates O from t0 = t_f + 2 = 4 for that
    reason."""
    sp = [s for s in synth.specs("c3") if s.name == "o"][0]
    L = np.zeros((sp.rows, sp.rows))
    kappas = []
    for t in (1, 2):
        g = bf16_round(synth.gradient("c3", sp, t)).astype(np.float64)
        L = 0.95 * L + 0.05 * g @ g.T
        w = np.linalg.eigvalsh(L)
        kappas.append(w[-1] / w[0])
    assert kappas[0] * 2.0 ** -24 > 1e3
    assert kappas[1] * 2.0 ** -24 < 1e-2
