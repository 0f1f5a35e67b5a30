"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the fact it checks. None of them re-types the oracle's own
formula: they use an independent routine (Jacobi SVD vs LAPACK SVD, AdamW vs
SOAP with a frozen basis), a closed form, an invariant, or a number printed
on the pages.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import foam as ofoam
from oracle import soap as osoap
from synth import rademacher_kfac_gradient, specs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY_SHAPES = [(4, 6), (6, 4), (5, 5), (3, 8), (8, 3)]


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# linear-algebra building blocks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_jacobi_svd_matches_lapack(shape):
    a = _rng(1).standard_normal(shape)
    u, s, vt = oracle.jacobi_svd(a)
    s_ref = np.linalg.svd(a, compute_uv=False)
    assert np.allclose(s, s_ref, rtol=1e-12, atol=1e-13)
    assert rel(u @ np.diag(s) @ vt, a) < 1e-13
    k = min(shape)
    assert np.allclose(u.T @ u, np.eye(k), atol=1e-13)
    assert np.allclose(vt @ vt.T, np.eye(k), atol=1e-13)


@pytest.mark.parametrize("n", [1, 5, 33])
def test_qr_positive_defining_properties(n):
    p = _rng(2).standard_normal((n, n))
    q, r = oracle.qr_positive(p)
    assert np.allclose(q.T @ q, np.eye(n), atol=1e-13)
    assert np.allclose(np.tril(r, -1), 0.0)
    assert np.all(np.diag(r) >= 0)
    assert rel(q @ r, p) < 1e-13
    # uniqueness: Gram-Schmidt on the columns gives the same Q
    g = np.zeros_like(p)
    for j in range(n):
        v = p[:, j] - g[:, :j] @ (g[:, :j].T @ p[:, j])
        v = v - g[:, :j] @ (g[:, :j].T @ v)
        g[:, j] = v / np.linalg.norm(v)
    assert rel(q, g) < 1e-10


def test_qr_positive_rank_deficient_stays_orthonormal():
    a = _rng(3).standard_normal((12, 4))
    p = a @ a.T  # rank 4 of 12
    q, r = oracle.qr_positive(p)
    assert np.allclose(q.T @ q, np.eye(12), atol=1e-12)
    assert rel(q @ r, p) < 1e-13


@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_shampoo_identity_equals_polar(shape):
    """(G G^T)^{-1/4} G (G^T G)^{-1/4} = U V^T with both EMAs off
    ("SOAP, Muon, and Beyond", section 2-1; picx.dev summary)."""
    g = _rng(4).standard_normal(shape)
    assert rel(oracle.shampoo_polar(g), oracle.polar_svd(g)) < 1e-12


# ---------------------------------------------------------------------------
# Muon / Muon+
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_newton_schulz_converges_to_jacobi_polar(shape):
    """Newton-Schulz output approaches UV^T from the Jacobi SVD."""
    m = _rng(5).standard_normal(shape)
    target = oracle.polar_svd(m)
    errs = [rel(oracle.newton_schulz(m, k), target) for k in (2, 5, 10, 30)]
    assert errs[-1] < 1e-12
    assert errs[0] > errs[1] > errs[2] or errs[2] < 1e-12


def test_newton_schulz_rank_deficient_converges_to_partial_isometry():
    a = _rng(6).standard_normal((6, 2))
    b = _rng(7).standard_normal((2, 9))
    m = a @ b  # rank 2
    # roundoff in the null space grows by 15/8 per iteration, so stop at 20
    assert rel(oracle.newton_schulz(m, 20), oracle.polar_svd(m, 1e-10)) < 1e-8


def test_newton_schulz_transpose_symmetry_square():
    m = _rng(8).standard_normal((7, 7))
    assert rel(oracle.newton_schulz(m.T, 5), oracle.newton_schulz(m, 5).T) < 1e-13


def test_newton_schulz_zero_steps_is_normalised_input():
    m = _rng(9).standard_normal((5, 9))
    o = oracle.newton_schulz(m, 0)
    assert np.allclose(o, m / (math.sqrt(float((m * m).sum())) + 1e-7), rtol=1e-15)


def test_newton_schulz_rank_one_is_fixed_point():
    """A rank-one unit-Frobenius X has its only singular value at 1, which the
    quintic keeps fixed (p(1) = 1): Ortho(u v^T) = u v^T / |u||v| (brute force
    on the 1 x n case too)."""
    u = _rng(10).standard_normal(6)
    v = _rng(11).standard_normal(9)
    m = np.outer(u, v)
    expect = m / (np.linalg.norm(u) * np.linalg.norm(v))
    assert rel(oracle.newton_schulz(m, 5, eps=0.0), expect) < 1e-14
    row = v[None, :]
    assert rel(oracle.newton_schulz(row, 3, eps=0.0), row / np.linalg.norm(v)) < 1e-14


def test_newton_schulz_coefficient_table_is_used():
    m = _rng(12).standard_normal((4, 6))
    o_default = oracle.newton_schulz(m, 3)
    table = [(1.0, 0.0, 0.0)] * 3  # identity polynomial: X stays X_0
    o_id = oracle.newton_schulz(m, 3, coeffs=table)
    assert rel(o_id, m / (np.linalg.norm(m) + 1e-7)) < 1e-15
    assert rel(o_default, o_id) > 1e-3


def test_muon_step_one_closed_form():
    """Step 1 from zero momentum: M_1 = (1-mu) G; with 0 iterations the update
    is sqrt(m/n) M_1/(|M_1|_F+eps); W moves by -lr (wd W + update)."""
    r = _rng(13)
    w = r.standard_normal((6, 10))
    g = r.standard_normal((6, 10))
    mu, lr, wd = 0.95, 1e-3, 0.1
    w1, m1, upd = oracle.muon_step(w, g, np.zeros_like(g), lr=lr, mu=mu, weight_decay=wd,
                                   ns_steps=0)
    assert np.allclose(m1, 0.05 * g, rtol=1e-15)
    expect_upd = math.sqrt(6 / 10) * m1 / (np.linalg.norm(m1) + 1e-7)
    assert rel(upd, expect_upd) < 1e-14
    assert rel(w1, w - lr * wd * w - lr * expect_upd) < 1e-14


def test_muon_momentum_is_an_exponential_average_of_the_gradients():
    """M_t = mu M_{t-1} + (1-mu) G_t from M_0 = 0 unrolls to
    sum_s (1-mu) mu^(t-s) G_s (Muon+ page, section 2, step 1); with 0
    iterations the update is sqrt(m/n) M_t / (|M_t|_F + eps)."""
    r = _rng(33)
    mu = 0.9
    gs = [r.standard_normal((4, 6)) for _ in range(6)]
    mom = np.zeros((4, 6))
    w = np.zeros((4, 6))
    for t, g in enumerate(gs, start=1):
        w, mom, upd = oracle.muon_step(w, g, mom, lr=0.0, mu=mu, weight_decay=0.0, ns_steps=0)
        unrolled = sum((1 - mu) * mu ** (t - s) * gs[s - 1] for s in range(1, t + 1))
        assert rel(mom, unrolled) < 1e-14
        assert rel(upd, math.sqrt(4 / 6) * unrolled / (np.linalg.norm(unrolled) + 1e-7)) < 1e-13


def test_muon_zero_gradient_only_decays():
    w = _rng(14).standard_normal((4, 4))
    w1, m1, upd = oracle.muon_step(w, np.zeros((4, 4)), np.zeros((4, 4)), lr=0.01, mu=0.9,
                                   weight_decay=0.1, ns_steps=5)
    assert np.all(upd == 0) and np.all(m1 == 0)
    assert np.allclose(w1, 0.999 * w, rtol=1e-15)


def test_muon_converged_update_is_scaled_polar():
    m = _rng(15).standard_normal((5, 8))
    upd = oracle.muon_update_direction(m, 40)
    assert rel(upd, math.sqrt(5 / 8) * oracle.polar_svd(m)) < 1e-12


@pytest.mark.parametrize("mode", ["col", "row", "col_row", "row_col"])
def test_muon_plus_keeps_frobenius_norm(mode):
    o = _rng(16).standard_normal((7, 11))
    out = oracle.muon_plus_normalize(o, mode, eps=0.0)
    assert abs(np.linalg.norm(out) - np.linalg.norm(o)) < 1e-12 * np.linalg.norm(o)


def test_muon_plus_equalises_and_is_idempotent():
    o = _rng(17).standard_normal((7, 11))
    c = oracle.muon_plus_normalize(o, "col", eps=0.0)
    cn = np.linalg.norm(c, axis=0)
    assert np.allclose(cn, cn[0], rtol=1e-13)
    assert rel(oracle.muon_plus_normalize(c, "col", eps=0.0), c) < 1e-14
    cr = oracle.muon_plus_normalize(o, "col_row", eps=0.0)
    rn = np.linalg.norm(cr, axis=1)
    assert np.allclose(rn, rn[0], rtol=1e-13)
    # the pass applied last decides which norms come out equal: col-row ends
    # on rows, row-col on columns (and they are different operators)
    assert np.std(np.linalg.norm(cr, axis=0)) > 1e-3
    rc = oracle.muon_plus_normalize(o, "row_col", eps=0.0)
    cn2 = np.linalg.norm(rc, axis=0)
    assert np.allclose(cn2, cn2[0], rtol=1e-13)
    assert np.std(np.linalg.norm(rc, axis=1)) > 1e-3
    assert rel(rc, cr) > 1e-3


def test_muon_plus_identity_on_exact_polar_factor():
    """Rows of an exact wide polar factor are orthonormal, so row mode leaves
    it unchanged; the tall case likewise for col mode."""
    p = oracle.polar_svd(_rng(18).standard_normal((4, 9)))
    assert rel(oracle.muon_plus_normalize(p, "row", eps=0.0), p) < 1e-13
    pt = p.T
    assert rel(oracle.muon_plus_normalize(pt, "col", eps=0.0), pt) < 1e-13


def test_muon_plus_zero_column_stays_zero():
    o = _rng(19).standard_normal((5, 6))
    o[:, 2] = 0.0
    out = oracle.muon_plus_normalize(o, "col_row")
    assert np.all(out[:, 2] == 0.0)
    assert np.all(np.isfinite(out))


# ---------------------------------------------------------------------------
# AdamW
# ---------------------------------------------------------------------------

def test_adamw_first_step_is_sign_like():
    g = _rng(20).standard_normal(50)
    _, _, _, upd = oracle.adamw_step(np.zeros(50), g, np.zeros(50), np.zeros(50), 1, lr=1e-3,
                                     beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)
    assert np.allclose(upd, g / (np.abs(g) + 1e-8), rtol=1e-14)


def test_adamw_constant_gradient_bias_correction_exact():
    g = _rng(21).standard_normal(20)
    m = np.zeros(20)
    v = np.zeros(20)
    w = np.zeros(20)
    for t in range(1, 8):
        w, m, v, upd = oracle.adamw_step(w, g, m, v, t, lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8,
                                         weight_decay=0.0)
        assert np.allclose(upd, g / (np.abs(g) + 1e-8), rtol=1e-12)


# ---------------------------------------------------------------------------
# SOAP
# ---------------------------------------------------------------------------

SOAP_HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def test_soap_first_step_closed_form():
    """At t = 1 the bias-corrected Adam step in the eigenbasis is
    N = G~/(|G~|+eps), with G~ rotated by the refreshed basis
    qr((1-b2) G G^T), qr((1-b2) G^T G)."""
    r = _rng(22)
    g = r.standard_normal((6, 6))
    w = r.standard_normal((6, 6))
    st = oracle.soap_init(6, 6)
    w1, s1, upd, info = oracle.soap_step(w, g, st, 1, **SOAP_HP)
    ql = oracle.qr_positive(0.05 * g @ g.T)[0]
    qr = oracle.qr_positive(0.05 * g.T @ g)[0]
    gt = ql.T @ g @ qr
    assert rel(info["N"], gt / (np.abs(gt) + 1e-8)) < 1e-10
    assert rel(upd, ql @ (gt / (np.abs(gt) + 1e-8)) @ qr.T) < 1e-10
    assert np.allclose(s1.M, 0.1 * g)


def test_soap_frozen_basis_equals_adamw():
    r = _rng(23)
    m, n = 5, 7
    st = oracle.soap_init(m, n)
    w = r.standard_normal((m, n))
    wa, ma, va = w.copy(), np.zeros(m * n), np.zeros(m * n)
    for t in range(1, 6):
        g = r.standard_normal((m, n))
        w, st, upd, _ = oracle.soap_step(w, g, st, t, refresh_every=0, **SOAP_HP)
        wa_flat, ma, va, upd_a = oracle.adamw_step(wa.ravel(), g.ravel(), ma, va, t, **SOAP_HP)
        wa = wa_flat.reshape(m, n)
        assert rel(upd, upd_a.reshape(m, n)) < 1e-13
        assert rel(w, wa) < 1e-13


def test_soap_rotation_keeps_frobenius_norm():
    r = _rng(24)
    st = oracle.soap_init(6, 9)
    w = np.zeros((6, 9))
    for t in range(1, 4):
        g = r.standard_normal((6, 9))
        w, st, upd, info = oracle.soap_step(w, g, st, t, **SOAP_HP)
        assert abs(np.linalg.norm(info["g_rot"]) - np.linalg.norm(g)) < 1e-12 * np.linalg.norm(g)
        assert np.allclose(st.QL.T @ st.QL, np.eye(6), atol=1e-12)
        assert np.allclose(st.QR.T @ st.QR, np.eye(9), atol=1e-12)


def test_soap_no_ema_converged_basis_gives_polar_factor():
    """b1 = b2 = 0 on a fixed square full-rank G: L = G G^T, R = G^T G, the
    power iteration converges to their eigenvectors, and the update becomes
    U V^T -- the Shampoo / SOAP / Muon family limit ("SOAP, Muon, and
    Beyond", section 2-1)."""
    r = _rng(25)
    n = 6
    u = oracle.qr_positive(r.standard_normal((n, n)))[0]
    v = oracle.qr_positive(r.standard_normal((n, n)))[0]
    s = 2.0 ** -np.arange(n)
    g = u @ np.diag(s) @ v.T
    st = oracle.soap_init(n, n)
    w = np.zeros((n, n))
    # eps stays well above the roundoff left off the diagonal of G~ (N is a
    # sign function there) and well below the smallest singular value
    # (error ~ eps / s_min + roundoff / eps, about 3e-7 here)
    hp = dict(SOAP_HP, beta1=0.0, beta2=0.0, eps=1e-8)
    for t in range(1, 80):
        w, st, upd, _ = oracle.soap_step(w, g, st, t, **hp)
    assert rel(upd, oracle.polar_svd(g)) < 1e-6


def test_soap_factors_are_exponential_averages_with_equal_trace():
    """L and R are EMAs of G G^T and G^T G ("SOAP, Muon, and Beyond", section
    1-1): from zero they unroll to sum_s (1-b2) b2^(t-s) G_s G_s^T (and
    G_s^T G_s), and because tr(G G^T) = tr(G^T G) = |G|_F^2 the two factors
    always carry the same trace. (The refresh is scale-invariant, so nothing
    downstream would notice a wrong factor scale.)"""
    r = _rng(34)
    m, n = 5, 8
    st = oracle.soap_init(m, n)
    w = np.zeros((m, n))
    gs = []
    for t in range(1, 6):
        g = r.standard_normal((m, n))
        gs.append(g)
        w, st, _, _ = oracle.soap_step(w, g, st, t, **SOAP_HP)
        wts = [(1 - 0.95) * 0.95 ** (t - s) for s in range(1, t + 1)]
        assert rel(st.L, sum(c * x @ x.T for c, x in zip(wts, gs))) < 1e-14
        assert rel(st.R, sum(c * x.T @ x for c, x in zip(wts, gs))) < 1e-14
        mass = sum(c * np.sum(x * x) for c, x in zip(wts, gs))
        assert abs(np.trace(st.L) - mass) < 1e-13 * mass
        assert abs(np.trace(st.R) - mass) < 1e-13 * mass


def test_soap_periodic_refresh_schedule():
    """refresh_every = k refreshes at t = 1, k+1, 2k+1, ... (the basis is
    needed from the first step; standard SOAP refreshes every k steps,
    picx.dev summary, SOAP instability diagnosis): the basis is bitwise
    unchanged on the other steps, and on a refreshing step it is the positive
    QR of F Q_prev, checked through its defining properties."""
    r = _rng(35)
    m, n, k = 4, 6, 3
    st = oracle.soap_init(m, n)
    w = np.zeros((m, n))
    for t in range(1, 11):
        g = r.standard_normal((m, n))
        prev = st.copy()
        w, st, _, _ = oracle.soap_step(w, g, st, t, refresh_every=k, **SOAP_HP)
        if t in (1, 4, 7, 10):
            for f, q0, q1 in ((st.L, prev.QL, st.QL), (st.R, prev.QR, st.QR)):
                tri = q1.T @ (f @ q0)
                assert np.abs(np.tril(tri, -1)).max() < 1e-10 * np.abs(tri).max()
                assert np.all(np.diag(tri) >= -1e-12)
                assert np.allclose(q1.T @ q1, np.eye(q1.shape[0]), atol=1e-12)
            assert not np.array_equal(st.QL, prev.QL)
        else:
            assert np.array_equal(st.QL, prev.QL) and np.array_equal(st.QR, prev.QR)


def test_soap_state_size_ratio_on_760m_shapes():
    """2mn + 2m^2 + 2n^2 over AdamW's 2mn on the 760M matrix set is 4.5
    (FOAM review, section 1)."""
    gold = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    soap = sum(oracle.soap_state_bytes(s.rows, s.cols) for s in specs("c5"))
    adamw = sum(4 * 2 * s.rows * s.cols for s in specs("c5"))
    assert soap / adamw == pytest.approx(gold["soap_over_adamw_state"]["value"], abs=1e-12)


# ---------------------------------------------------------------------------
# FOAM
# ---------------------------------------------------------------------------

FOAM_HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def test_foam_factored_moment_exact_under_kfac():
    """With a fixed basis Q and G = (D_a Z D_b) Q^T, Z = +-1, the rotated
    squared gradient is exactly a_i^2 b_j^2, so tau r_hat c_hat^T reproduces
    SOAP's dense rotated moment (Q_L = I, Q_R = Q) and the two updates agree
    (FOAM review, sections 1 and 3)."""
    r = _rng(26)
    m, n = 6, 9
    q = oracle.qr_positive(r.standard_normal((n, n)))[0]
    alpha = np.exp(r.standard_normal(m))
    beta = np.exp(r.standard_normal(n))
    fs = oracle.foam_init(m, n)
    fs.QR = q.copy()
    ss = oracle.soap_init(m, n)
    ss.QR = q.copy()
    wf = ws = np.zeros((m, n))
    for t in range(1, 8):
        g = rademacher_kfac_gradient(alpha, beta, q, seed=1, step=t)
        wf, fs, uf, fi = oracle.foam_step(wf, g, fs, t, tol=np.inf, **FOAM_HP)
        ws, ss, us, si = oracle.soap_step(ws, g, ss, t, refresh_every=0, **FOAM_HP)
        v_dense = ss.V / (1 - 0.95 ** t)
        assert rel(fi["v_hat"], v_dense) < 1e-12
        assert rel(uf, us) < 1e-10


def test_foam_output_side_exact_under_kfac():
    """Output-only FOAM (the review's section 3 ablation): with the basis Q on
    the output side and G = Q (D_a Z D_b), Z = +-1, Q^T G is exactly
    a_i b_j Z_ij, so tau r_hat c_hat^T reproduces SOAP's dense rotated moment
    with Q_L = Q, Q_R = I, and the updates agree."""
    r = _rng(30)
    m, n = 7, 5
    q = oracle.qr_positive(r.standard_normal((m, m)))[0]
    alpha = np.exp(r.standard_normal(m))
    beta = np.exp(r.standard_normal(n))
    fs = oracle.foam_init(m, n, side="output")
    assert fs.R.shape == (m, m) and fs.QR.shape == (m, m)
    fs.QR = q.copy()
    ss = oracle.soap_init(m, n)
    ss.QL = q.copy()
    wf = ws = np.zeros((m, n))
    for t in range(1, 8):
        g = rademacher_kfac_gradient(beta, alpha, q, seed=2, step=t).T
        wf, fs, uf, fi = oracle.foam_step(wf, g, fs, t, tol=np.inf, side="output", **FOAM_HP)
        ws, ss, us, si = oracle.soap_step(ws, g, ss, t, refresh_every=0, **FOAM_HP)
        v_dense = ss.V / (1 - 0.95 ** t)
        assert rel(fi["v_hat"], v_dense) < 1e-12
        assert rel(uf, us) < 1e-10
        assert abs(fi["v_hat"].sum() - np.trace(fs.R) / (1 - 0.95 ** t)) < 1e-10 * np.trace(fs.R)


def test_foam_output_side_is_input_side_of_the_transpose():
    """Stepping W with the output-side basis equals stepping W^T with the
    input-side basis (r and c trade places), refreshes included."""
    r = _rng(31)
    m, n = 9, 4
    so = oracle.foam_init(m, n, side="output")
    si = oracle.foam_init(n, m)
    wo = r.standard_normal((m, n))
    wi = wo.T.copy()
    for t in range(1, 9):
        g = r.standard_normal((m, n)) * np.exp(r.standard_normal((m, 1)))
        wo, so, uo, io = oracle.foam_step(wo, g, so, t, pf=3, tol=0.05, side="output", **FOAM_HP)
        wi, si, ui, ii = oracle.foam_step(wi, g.T, si, t, pf=3, tol=0.05, **FOAM_HP)
        assert io["checked"] == ii["checked"] and io["refreshed"] == ii["refreshed"]
        assert rel(uo, ui.T) < 1e-12 and rel(wo, wi.T) < 1e-12
        assert rel(so.r, si.c) < 1e-12 and rel(so.c, si.r) < 1e-12
        assert rel(so.QR, si.QR) < 1e-12 and rel(so.M, si.M.T) < 1e-12


def test_foam_mass_invariant_and_refresh_rule():
    r = _rng(27)
    m, n = 7, 5
    fs = oracle.foam_init(m, n)
    w = np.zeros((m, n))
    for t in range(1, 14):
        g = r.standard_normal((m, n))
        w, fs, upd, info = oracle.foam_step(w, g, fs, t, pf=4, tol=0.1, **FOAM_HP)
        assert abs(info["v_hat"].sum() - np.trace(fs.R) / (1 - 0.95 ** t)) < 1e-10 * np.trace(fs.R)
        assert info["checked"] == ((t - 1) % 4 == 0)
        assert np.allclose(fs.QR.T @ fs.QR, np.eye(n), atol=1e-12)


def _fixed_spectrum_gradient(r, m, n, ratio):
    """G = U diag(s) V^T with s_i = ratio^i (distinct, well separated)."""
    u = oracle.qr_positive(r.standard_normal((m, m)))[0][:, :min(m, n)]
    v = oracle.qr_positive(r.standard_normal((n, n)))[0][:, :min(m, n)]
    s = ratio ** np.arange(min(m, n))
    return (u * s[None, :]) @ v.T


def test_foam_refresh_is_one_power_iteration_step():
    """The refresh is one step of orthogonal (subspace) iteration on R (FOAM
    review, section 3, with the QR power step SOAP uses). With b2 = 0 and a
    fixed G the factor is R = G^T G at every step, so after k refreshes from
    Q_R = I the basis is qr(R^k) (R^k = Q_k (R_k ... R_1) with positive
    triangular factors), and repeated refreshes converge to R's eigenbasis,
    which drives rho to zero. A refresh that factors R alone, or Q_R^T R,
    stalls at one basis and fails both checks."""
    r = _rng(32)
    m, n = 7, 5
    g = _fixed_spectrum_gradient(r, m, n, 0.8)
    hp = dict(FOAM_HP, beta2=0.0)
    fs = oracle.foam_init(m, n)
    w = np.zeros((m, n))
    rr = g.T @ g
    for k in range(1, 5):
        w, fs, _, info = oracle.foam_step(w, g, fs, k, pf=1, tol=0.0, **hp)
        assert info["refreshed"]
        q_k = np.linalg.qr(np.linalg.matrix_power(rr, k))[0]
        q_k = q_k * np.sign(np.diag(q_k.T @ fs.QR))[None, :]
        assert np.abs(fs.QR - q_k).max() < 1e-9
        assert np.all(np.diag(fs.QR.T @ rr @ fs.QR) > 0)
    rhos = []
    for t in range(5, 120):
        w, fs, _, info = oracle.foam_step(w, g, fs, t, pf=1, tol=0.0, **hp)
        rhos.append(info["rho"])
    assert rhos[0] > 1e-3 and rhos[-1] < 1e-10
    lam = np.linalg.eigvalsh(rr)[::-1]
    d = np.diag(fs.QR.T @ rr @ fs.QR)
    assert np.abs(d - lam).max() < 1e-12 * lam[0]


def test_foam_eigh_refresh_diagonalises_r_in_descending_order():
    """The eigendecomposition refresh (FOAM review, sections 1 and 3) leaves
    Q_R^T R Q_R diagonal, with the diagonal equal to R's eigenvalues from the
    oracle's own Jacobi SVD (R is PSD, so its singular values are its
    eigenvalues) in descending order, and the criterion then reads rho = 0."""
    r = _rng(36)
    m, n = 9, 6
    fs = oracle.foam_init(m, n)
    w = np.zeros((m, n))
    for t in range(1, 4):
        g = r.standard_normal((m, n)) * np.exp(r.standard_normal((1, n)))
        w, fs, _, info = oracle.foam_step(w, g, fs, t, pf=1, tol=0.0, refresh="eigh", **FOAM_HP)
        assert info["refreshed"]
        d = fs.QR.T @ fs.R @ fs.QR
        s_ref = oracle.jacobi_svd(fs.R)[1]
        assert np.abs(d - np.diag(np.diag(d))).max() < 1e-12 * s_ref[0]
        assert np.abs(np.diag(d) - s_ref).max() < 1e-12 * s_ref[0]
        assert np.all(np.diff(np.diag(d)) <= 1e-12 * s_ref[0])
        assert np.allclose(fs.QR.T @ fs.QR, np.eye(n), atol=1e-12)
    g = r.standard_normal((m, n))
    _, _, _, info = oracle.foam_step(w, 0.0 * g, fs, 4, pf=1, tol=0.0, refresh="eigh",
                                     **dict(FOAM_HP, beta2=0.999999))
    assert info["rho"] < 1e-6


def test_foam_eigh_refresh_is_the_limit_of_qr_refreshes():
    """With b2 = 0 and a fixed G, repeated QR power-step refreshes converge to
    R's eigenbasis (orthogonal iteration); one eigh refresh lands there at
    once, with the same column order and, after sign alignment, the same
    columns."""
    r = _rng(37)
    m, n = 7, 5
    g = _fixed_spectrum_gradient(r, m, n, 0.8)
    hp = dict(FOAM_HP, beta2=0.0)
    fq = oracle.foam_init(m, n)
    fe = oracle.foam_init(m, n)
    w = np.zeros((m, n))
    for t in range(1, 150):
        _, fq, _, _ = oracle.foam_step(w, g, fq, t, pf=1, tol=0.0, **hp)
    _, fe, _, info = oracle.foam_step(w, g, fe, 1, pf=1, tol=0.0, refresh="eigh", **hp)
    signs = np.sign(np.sum(fq.QR * fe.QR, axis=0))
    assert np.abs(fq.QR - fe.QR * signs[None, :]).max() < 1e-9
    assert np.all(np.diff(info["eigenvalues"]) < 0)


def test_foam_refresh_needs_rho_strictly_above_tol():
    """The criterion refreshes only when rho exceeds tol: with an exactly
    diagonal R in the current basis (G with orthogonal columns, Q_R = I),
    rho is exactly 0 and tol = 0 keeps the basis."""
    g = np.zeros((6, 4))
    g[0, 0], g[1, 1], g[2, 2], g[3, 3], g[4, 0] = 2.0, 1.5, 0.5, 0.25, 1.0
    fs = oracle.foam_init(6, 4)
    _, fs2, _, info = oracle.foam_step(np.zeros((6, 4)), g, fs, 1, pf=1, tol=0.0, **FOAM_HP)
    assert info["checked"] and info["rho"] == 0.0 and not info["refreshed"]
    assert np.array_equal(fs2.QR, np.eye(4))


def test_offdiag_ratio_values():
    assert oracle.offdiag_ratio(np.array([[1.0, 1.0], [1.0, 1.0]])) == pytest.approx(math.sqrt(0.5))
    assert oracle.offdiag_ratio(np.diag([3.0, 1.0])) == 0.0
    assert oracle.offdiag_ratio(np.zeros((3, 3))) == 0.0
    a = _rng(28).standard_normal((6, 6))
    s = a @ a.T
    _, q = np.linalg.eigh(s)
    assert oracle.offdiag_ratio(q.T @ s @ q) < 1e-13


def test_foam_no_refresh_when_basis_is_eigenbasis():
    r = _rng(29)
    g = r.standard_normal((4, 6))
    fs = oracle.foam_init(4, 6)
    rr = 0.05 * g.T @ g
    _, q = np.linalg.eigh(rr)
    fs.QR = q
    _, fs2, _, info = oracle.foam_step(np.zeros((4, 6)), g, fs, 1, **FOAM_HP)
    assert info["checked"] and not info["refreshed"] and info["rho"] < 1e-12
    assert np.array_equal(fs2.QR, q)


def test_foam_vs_soap_state_on_760m_shapes():
    """FOAM's matrix-parameter state is about half of SOAP's at 760M: 11.87 vs
    23.73 GiB on the page (FOAM review, section 3)."""
    gold = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))["foam_vs_soap_state_gib_760m"]
    soap = sum(oracle.soap_state_bytes(s.rows, s.cols) for s in specs("c5"))
    foam = sum(oracle.foam_state_bytes(s.rows, s.cols) for s in specs("c5"))
    assert soap / foam == pytest.approx(gold["soap"] / gold["foam"], rel=2e-3)
    assert soap / 2**30 == pytest.approx(gold["soap"], rel=0.05)
    assert foam / 2**30 == pytest.approx(gold["foam"], rel=0.05)


def test_pages_arithmetic():
    gold = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    c = gold["momentum_correction_beta1_0p9"]
    assert math.sqrt((1 - c["beta1"]) / (1 + c["beta1"])) == pytest.approx(c["value"], abs=0.03)
    e = gold["moe_effective_batch_ratio"]
    assert e["k"] / e["n"] == e["value"]
    p = gold["bf16_fp32_machine_precision"]
    assert 2.0 ** -7 == p["bf16"]
    assert 2.0 ** -23 == pytest.approx(p["fp32"], rel=1e-2)
    bf16_eps = float(np.finfo(np.float32).eps) * 2 ** 16
    assert bf16_eps == p["bf16"]


# ---- observability ("SOAP, Muon, and Beyond" sections 2-1 and 7-2; FOAM
# review section 3) --------------------------------------------------------


def _dct_rows(n):
    """Orthonormal DCT-II matrix (rows orthonormal), closed form."""
    k = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    c = np.sqrt(2.0 / n) * np.cos(np.pi * (2 * j + 1) * k / (2 * n))
    c[0, :] = np.sqrt(1.0 / n)
    return c


def test_matrix_rms_closed_forms():
    assert oracle.matrix_rms(np.full((7, 13), -0.25)) == pytest.approx(0.25, rel=1e-15)
    x = np.zeros((4, 9))
    x[2, 5] = 3.0
    assert oracle.matrix_rms(x) == pytest.approx(3.0 / 6.0, rel=1e-15)


def test_ns_residual_from_known_singular_values():
    a, b = 6, 10
    u = _dct_rows(a).T                     # a x a orthonormal
    v = _dct_rows(b)[:a].T                 # b x a, orthonormal columns
    s = np.array([1.0, 0.9, 1.1, 0.5, 1.0, 0.0])
    x = u @ np.diag(s) @ v.T               # a x b with singular values s
    want = math.sqrt(np.mean((s * s - 1.0) ** 2))
    assert oracle.ns_residual(x) == pytest.approx(want, rel=1e-12)
    assert oracle.ns_residual(x.T) == pytest.approx(want, rel=1e-12)     # tall: its wide view
    assert oracle.ns_residual(2.0 * x, 0.5) == pytest.approx(want, rel=1e-12)
    assert oracle.ns_residual(u @ v.T) < 1e-14                           # orthonormal rows


def test_rayleigh_quotients_in_an_eigenbasis():
    n = 8
    q = _dct_rows(n).T
    lam = np.array([4.0, 0.5, 2.0, 1.0, 8.0, 0.25, 3.0, 1.5])
    f = q @ np.diag(lam) @ q.T
    d, kappa = oracle.rayleigh(f, q)
    assert np.allclose(d, lam, rtol=1e-12, atol=1e-14)
    assert kappa == pytest.approx(8.0 / 0.25, rel=1e-12)
    d_id, _ = oracle.rayleigh(f, np.eye(n))
    assert np.allclose(d_id, np.diag(f), rtol=0, atol=0)
    # any orthonormal basis: every quotient lies in [lambda_min, lambda_max],
    # so the estimate never exceeds cond(f)
    w = oracle.qr_positive(_rng(3).standard_normal((n, n)))[0]
    d_w, k_w = oracle.rayleigh(f, w)
    assert d_w.min() >= 0.25 - 1e-12 and d_w.max() <= 8.0 + 1e-12
    assert k_w <= 32.0 + 1e-9
    _, k_neg = oracle.rayleigh(-f, q)
    assert k_neg == float("inf")


def test_rank1_share_closed_forms():
    r = _rng(4)
    a, b = np.abs(r.standard_normal(9)), np.abs(r.standard_normal(5))
    assert oracle.rank1_share(np.outer(a, b)) == pytest.approx(1.0, rel=1e-12)
    s = np.array([3.0, 1.0, 2.0])
    v = np.zeros((5, 3))
    v[[0, 1, 2], [0, 1, 2]] = s
    assert oracle.rank1_share(v) == pytest.approx(9.0 / 14.0, rel=1e-12)
    # two disjoint rank-1 blocks: the larger block's mass over the total
    blk = np.zeros((6, 6))
    blk[:3, :3] = 2.0
    blk[3:, 3:] = 1.0
    assert oracle.rank1_share(blk) == pytest.approx(36.0 / 45.0, rel=1e-12)
    assert oracle.rank1_share(np.zeros((3, 4))) == 0.0


def test_basis_age_recurrence():
    assert oracle.basis_ages([1, 0, 0, 1, 0, 0, 0]) == [0, 1, 2, 0, 1, 2, 3]
    assert oracle.basis_ages([0, 0]) == [1, 2]
