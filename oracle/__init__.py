"""fp64 CPU oracle for the matrix-aware optimizer step (test infrastructure).

This package is the plain, slow, obviously-correct reference the HIP library
is checked against. It is test infrastructure: only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it. The
product path never calls it, and it shares no code with the HIP sources.

Everything is NumPy float64. Library primitives (matmul, ``numpy.linalg.qr``,
``numpy.linalg.eigh``) serve as single steps; every other step is written out
in the order the pages give it.

Sources (page title, then section / equation):

* "SOAP, Muon, and Beyond" review (dimensionstp.github.io), section 1-1
  (AdamW and Shampoo factor EMAs), section 2-1 (polar factor, Shampoo/polar
  identity), section 3-2 (Muon recipe, SOAP rotation, real-time eigenbasis
  update with the current gradient and per-step QR).
* picx.dev summary of the same paper, Eq. (1) (SOAP update), Eq. (2).
* "Factored One-sided Adam-Moment for Practical and Scalable SOAP" review,
  sections 1 and 3 (FOAM: input-only rotation, factored second moment,
  trace normalisation, adaptive-tolerance refresh, state sizes).
* "Muon+: Towards Better Muon via One Additional Normalization Step"
  (gist.science), section 2 (momentum, orthogonalisation, normalisation,
  sqrt(m/n) update).
* Observability ("SOAP, Muon, and Beyond", sections 2-1 and 7-2; FOAM
  review, section 3): update RMS, Newton-Schulz residual, factor Rayleigh
  quotients, rank-1 share, basis age.

Parity status of each function is stated in its module header.
"""
from .linalg import (eigh_descending, jacobi_svd, polar_svd, qr_positive, shampoo_polar,
                     sym_inv_root)
from .muon import (CLASSICAL_QUINTIC, muon_plus_normalize, muon_step,
                   muon_update_direction, newton_schulz)
from .adamw import adamw_step
from .soap import SoapState, soap_init, soap_step, soap_state_bytes
from .foam import FoamState, foam_init, foam_step, foam_state_bytes, offdiag_ratio
from .observe import basis_ages, matrix_rms, ns_residual, rank1_share, rayleigh

__all__ = [
    "jacobi_svd", "polar_svd", "qr_positive", "eigh_descending", "shampoo_polar",
    "sym_inv_root",
    "CLASSICAL_QUINTIC", "newton_schulz", "muon_plus_normalize", "muon_update_direction",
    "muon_step", "adamw_step", "SoapState", "soap_init", "soap_step", "soap_state_bytes",
    "FoamState", "foam_init", "foam_step", "foam_state_bytes", "offdiag_ratio",
    "matrix_rms", "ns_residual", "rayleigh", "rank1_share", "basis_ages",
]
