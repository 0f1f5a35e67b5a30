"""SOAP, FOAM and AdamW parity against the fp64 oracle (GPU).

SOAP and FOAM are checked teacher-forced: at every step the oracle starts from
the GPU's state after the previous step and the same gradient, so each step is
judged on its own. The refreshed basis is checked by what defines it
(orthonormal columns, Q^T P upper triangular with a non-negative diagonal, and
agreement with the oracle's Q where P is well conditioned); the oracle then
finishes the step with the GPU's basis and V, U must match to 1e-4 (fp32).
Before the factors have been full rank for two steps the basis completion is
arbitrary and the elementwise Adam step is not rotation-equivariant, so those
steps are reported, not gated (t < ceil(b/a) + 2). With the forward rotations
as bf16x3 products (about 2^-17 relative per product instead of 2^-24) the
first full-rank step divides that rounding by the smallest Adam denominators
the factors will have: an fp64 emulation of the split arithmetic puts the
update error there at 7e-5 to 1e-4 (Llama-8B O projection 9.0e-5), and
4e-5 or less from the next step on. That step is held to the bf16-MFMA
rotation tolerance (2e-2), the later ones to 1e-4; V and the basis are
gated at every step as for fp32.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import bf16_round
from tests.helpers import PRODUCT_EPS, log, rel, to_dev, to_host, w_bound

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _soap_state_dev(m, n):
    import torch
    z = lambda r, c: torch.zeros((r, c), dtype=torch.float32, device="cuda")
    return {"M": z(m, n), "V": z(m, n), "L": z(m, m), "R": z(n, n),
            "QL": torch.eye(m, dtype=torch.float32, device="cuda"),
            "QR": torch.eye(n, dtype=torch.float32, device="cuda")}


def _host_soap(st):
    return oracle.SoapState(*(to_host(st[k]) for k in ("M", "V", "L", "R", "QL", "QR")))


def _check_basis(q, p, q_ref, tag, prod="f32"):
    """q: GPU basis; p: the oracle's power-iteration product; q_ref: its QR.
    The forward error of q is gated where the QR's condition-number bound
    (kappa times the product's relative error) leaves it meaningful: below
    1e-4 for an fp32 product with kappa * 2^-24 <= 1e-5; below 16 kappa eps
    for a bf16x3 product where that is under 1e-2."""
    n = q.shape[0]
    orth = np.abs(q.T @ q - np.eye(n)).max()
    assert orth < 1e-4, f"{tag}: orthogonality {orth}"
    rr = q.T @ p
    scale = np.linalg.norm(p)
    assert np.linalg.norm(np.tril(rr, -1)) <= 1e-4 * scale, f"{tag}: Q^T P not triangular"
    assert np.all(np.diag(rr) >= -1e-5 * scale), f"{tag}: negative diagonal"
    s = np.linalg.svd(p, compute_uv=False)
    kappa = s[0] / s[-1] if s[-1] > 0 else np.inf
    eps = PRODUCT_EPS[prod]
    if prod == "f32" and kappa * eps <= 1e-5:
        fe = rel(q, q_ref)
        assert fe < 1e-4, f"{tag}: forward error {fe} at kappa {kappa:.1e}"
    elif prod != "f32" and 16 * kappa * eps <= 1e-2:
        fe = rel(q, q_ref)
        log(f"  {tag}: forward error {fe:.2e} at kappa {kappa:.1e} (bound {16 * kappa * eps:.1e})")
        assert fe < max(1e-4, 16 * kappa * eps), f"{tag}: forward error {fe} at kappa {kappa:.1e}"


def _run_soap(gpu_lib, m, n, steps, grad, dtype="f32", refresh_every=1, back="f32", fwd="f32",
              prod="f32"):
    import torch
    W = to_dev(synth.init_weight("c1", synth.MatrixSpec("w", m, n, 7)), dtype)
    st = _soap_state_dev(m, n)
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    t0 = math.ceil(max(m, n) / min(m, n)) + 2
    t1 = t0 + 1 if fwd == "bf16x3" else t0  # first step held to 1e-4
    free_w = to_host(W)
    free_state = oracle.soap_init(m, n)
    for t in range(1, steps + 1):
        g = grad(t)
        if dtype == "bf16":
            g = bf16_round(g)
        prev = _host_soap(st)
        w_prev = to_host(W)
        gpu_lib.soap_step(W, to_dev(g, dtype), st, t, update_out=out, refresh_every=refresh_every,
                          back_rot_dtype=back, fwd_rot=fwd, refresh_prod=prod, **HP)
        torch.cuda.synchronize()
        new = _host_soap(st)
        # EMAs from the GPU's previous state
        _, ref, _, info = oracle.soap_step(w_prev, g, prev, t, refresh_every=refresh_every, **HP)
        assert rel(new.M, ref.M) < 1e-5 and rel(new.L, ref.L) < 1e-5 and rel(new.R, ref.R) < 1e-5
        if "PL" in info:
            _check_basis(new.QL, info["PL"], ref.QL, f"t={t} QL", prod)
            _check_basis(new.QR, info["PR"], ref.QR, f"t={t} QR", prod)
        else:  # not a refreshing step: the basis is left exactly as it was
            assert np.array_equal(new.QL, prev.QL) and np.array_equal(new.QR, prev.QR)
        # finish the step with the GPU's basis
        w_ref, ref2, upd_ref, _ = oracle.soap_step(w_prev, g, prev, t, refresh_every=0,
                                                   q_override=(new.QL, new.QR), **HP)
        eu = rel(to_host(out), upd_ref)
        ev = rel(new.V, ref2.V)
        free_w, free_state, free_upd, _ = oracle.soap_step(free_w, g, free_state, t,
                                                           refresh_every=refresh_every, **HP)
        log(f"  soap t={t}: update {eu:.2e}  V {ev:.2e}  (free-running {rel(to_host(out), free_upd):.2e})")
        if t >= t0:
            # the bf16 back rotation rounds N and the bases to bf16: the update
            # is held to the bf16-MFMA tolerance, V (fp32-accurate forward
            # path) to 1e-4
            tol = 2e-2 if back == "bf16" or t < t1 else 1e-4
            assert eu < tol and ev < 1e-4, f"t={t}: update {eu}, V {ev}"
            if dtype == "f32" and back == "f32":
                assert rel(to_host(W), w_ref) < 1e-5


def test_soap_c1_teacher_forced(gpu_lib):
    """256x512 fp32, Q_L = Q_R = I at t = 1, refresh every step, 10 steps."""
    log("soap c1")
    spec = synth.specs("c1")[0]
    _run_soap(gpu_lib, 256, 512, 10, lambda t: synth.gradient("c1", spec, t))


def test_soap_kronecker_ragged(gpu_lib):
    """Kronecker-structured gradients (k^-1 spectra) on a ragged tall shape."""
    log("soap kronecker 328x200")
    spec = synth.MatrixSpec("k", 328, 200, 3)
    _run_soap(gpu_lib, 328, 200, 6, lambda t: synth.kronecker_gradient("c3", spec, t))


def test_soap_bf16_gradient_and_frozen_basis(gpu_lib):
    log("soap bf16 frozen")
    spec = synth.MatrixSpec("k", 96, 160, 4)
    _run_soap(gpu_lib, 96, 160, 4, lambda t: synth.kronecker_gradient("c3", spec, t),
              dtype="bf16", refresh_every=0)


def test_soap_bf16_gradient_refreshing_ragged(gpu_lib):
    """bf16 gradients (factor EMAs on the bf16 MFMA path, in place) with a
    refresh every step on a shape of several 256-tiles with ragged edges."""
    log("soap bf16 refreshing 296x520")
    spec = synth.MatrixSpec("k", 296, 520, 6)
    _run_soap(gpu_lib, 296, 520, 6, lambda t: synth.kronecker_gradient("c3", spec, t),
              dtype="bf16", refresh_every=1)


# ---------------------------------------------------------------------------

def _foam_state_dev(m, n, side="input"):
    import torch
    k = m if side == "output" else n
    return {"M": torch.zeros((m, n), dtype=torch.float32, device="cuda"),
            "R": torch.zeros((k, k), dtype=torch.float32, device="cuda"),
            "QR": torch.eye(k, dtype=torch.float32, device="cuda"),
            "r": torch.zeros(m, dtype=torch.float32, device="cuda"),
            "c": torch.zeros(n, dtype=torch.float32, device="cuda"),
            "aux": torch.zeros(8, dtype=torch.float32, device="cuda")}


def _host_foam(st):
    return oracle.FoamState(to_host(st["M"]), to_host(st["R"]), to_host(st["QR"]),
                            to_host(st["r"]), to_host(st["c"]))


@pytest.mark.parametrize("m,n,pf,side,gdt,fwd,prod", [
    (160, 96, 3, "input", "f32", "f32", "f32"), (96, 264, 4, "input", "f32", "f32", "f32"),
    (160, 96, 3, "output", "f32", "f32", "f32"), (264, 96, 4, "output", "f32", "f32", "f32"),
    (96, 160, 3, "input", "bf16", "f32", "f32"), (160, 96, 3, "output", "bf16", "f32", "f32"),
    # forward rotations and criterion products as bf16x3 products on bf16 MFMA
    (328, 136, 3, "input", "f32", "bf16x3", "f32"), (96, 264, 4, "input", "bf16", "bf16x3", "f32"),
    (136, 328, 3, "output", "f32", "bf16x3", "f32"),
    (264, 96, 4, "output", "bf16", "bf16x3", "f32"),
    (328, 136, 2, "input", "f32", "f32", "bf16x3"),
    (136, 328, 2, "output", "bf16", "bf16x3", "bf16x3")])
def test_foam_teacher_forced(gpu_lib, m, n, pf, side, gdt, fwd, prod):
    """FOAM (input side) and its output-only ablation ([FOAM] section 3),
    teacher-forced against the oracle, with fp32 and bf16 gradients."""
    import torch
    log(f"foam {side} {m}x{n} pf={pf} {gdt} gradient, {fwd} forward rotation, {prod} criterion")
    spec = synth.MatrixSpec("f", m, n, 5)
    W = to_dev(synth.init_weight("c5", spec))
    st = _foam_state_dev(m, n, side)
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    t0 = math.ceil(max(m, n) / min(m, n)) + 2
    t1 = t0 + 1 if fwd == "bf16x3" else t0  # first step held to 1e-4
    for t in range(1, 10):
        g = synth.kronecker_gradient("c5", spec, t)
        if gdt == "bf16":
            g = bf16_round(g)
        prev = _host_foam(st)
        w_prev = to_host(W)
        gpu_lib.foam_step(W, to_dev(g, gdt), st, t, update_out=out, pf=pf, tol=0.1, side=side,
                          fwd_rot=fwd, refresh_prod=prod, **HP)
        torch.cuda.synchronize()
        new = _host_foam(st)
        aux = to_host(st["aux"])
        _, ref, _, info = oracle.foam_step(w_prev, g, prev, t, pf=pf, tol=0.1, side=side, **HP)
        assert bool(aux[3]) == info["checked"]
        assert rel(new.M, ref.M) < 1e-5 and rel(new.R, ref.R) < 1e-5
        decision = info["refreshed"]
        if info["checked"]:
            assert abs(aux[0] - info["rho"]) < 1e-4
            if abs(info["rho"] - 0.1) > 1e-4:
                assert bool(aux[1]) == info["refreshed"]
            decision = bool(aux[1])
            if decision:
                _check_basis(new.QR, info["P"], ref.QR, f"t={t} QR", prod)
        if not decision:
            assert np.array_equal(new.QR, prev.QR)
        w_ref, ref2, upd_ref, info2 = oracle.foam_step(w_prev, g, prev, t, pf=pf, tol=0.1,
                                                       q_override=new.QR,
                                                       refresh_override=decision, side=side,
                                                       **HP)
        eu = rel(to_host(out), upd_ref)
        er, ec = rel(new.r, ref2.r), rel(new.c, ref2.c)
        log(f"  foam t={t}: update {eu:.2e} r {er:.2e} c {ec:.2e} rho {aux[0]:.3f} refresh {decision}")
        if t >= t0:
            assert eu < (1e-4 if t >= t1 else 2e-2) and er < 1e-4 and ec < 1e-4
            assert abs(aux[2] - info2["tau"]) <= 1e-4 * abs(info2["tau"])
            assert rel(to_host(W), w_ref) < 1e-5


# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_adamw_flat_ragged(gpu_lib, wdt):
    import torch
    n = 1_000_003
    r = np.random.default_rng(17)
    w = (0.02 * r.standard_normal(n)).astype(np.float32)
    if wdt == "bf16":
        w = bf16_round(w)
    W = to_dev(w, wdt)
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    mr, vr = np.zeros(n), np.zeros(n)
    for t in range(1, 4):
        g = r.standard_normal(n).astype(np.float32)
        w_prev = to_host(W)
        gpu_lib.adamw_step(W, to_dev(g), m, v, t, update_out=out, **HP)
        torch.cuda.synchronize()
        w_ref, mr, vr, u_ref = oracle.adamw_step(w_prev, g, mr, vr, t, **HP)
        assert rel(to_host(out), u_ref) < 1e-5
        assert rel(to_host(m), mr) < 1e-6 and rel(to_host(v), vr) < 1e-6
        if wdt == "bf16":
            lr_term = HP["lr"] * (HP["weight_decay"] * w_prev + to_host(out))
            w_expect = w_prev - lr_term
            assert np.all(np.abs(to_host(W) - bf16_round(w_expect.astype(np.float32))) <=
                          w_bound(w_expect, w_prev, lr_term))
        else:
            assert rel(to_host(W), w_ref) < 1e-6


# ---- many matrices per call ------------------------------------------------

MANY_SHAPES = [(200, 328), (328, 200), (200, 328), (96, 96), (72, 264)]


def _many_inputs(shapes, steps, seed):
    r = np.random.default_rng(seed)
    ws = [(0.02 * r.standard_normal((m, n))).astype(np.float32) for m, n in shapes]
    gs = [[(r.standard_normal((m, n)) * np.exp(0.5 * r.standard_normal((m, 1)))).astype(np.float32)
           for _ in range(steps)] for m, n in shapes]
    return ws, gs


def _close(a, b, tag, tol=1e-5):
    e = rel(to_host(a), to_host(b))
    assert e <= tol, f"{tag}: {e}"


@pytest.mark.parametrize("refresh_every", [1, 2])
def test_soap_many_matches_separate_calls(gpu_lib, refresh_every):
    """soap_step_many on matrices of several shapes (QR sizes shared across
    matrices and sides: batched groups of 2-3 factors) gives the states and
    updates of separate soap_step calls."""
    import torch
    log(f"soap many vs single, refresh every {refresh_every}")
    steps = 3
    ws, gs = _many_inputs(MANY_SHAPES, steps, 41)
    Ws1 = [to_dev(w) for w in ws]
    Ws2 = [to_dev(w) for w in ws]
    st1 = [_soap_state_dev(m, n) for m, n in MANY_SHAPES]
    st2 = [_soap_state_dev(m, n) for m, n in MANY_SHAPES]
    o1 = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in MANY_SHAPES]
    o2 = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in MANY_SHAPES]
    for t in range(1, steps + 1):
        G = [to_dev(g[t - 1]) for g in gs]
        for i in range(len(MANY_SHAPES)):
            gpu_lib.soap_step(Ws1[i], G[i], st1[i], t, update_out=o1[i],
                              refresh_every=refresh_every, **HP)
        gpu_lib.soap_step_many([(Ws2[i], G[i], st2[i]) for i in range(len(MANY_SHAPES))], t,
                               update_out=o2, refresh_every=refresh_every, **HP)
        torch.cuda.synchronize()
        for i in range(len(MANY_SHAPES)):
            for k in ("M", "V", "L", "R", "QL", "QR"):
                _close(st2[i][k], st1[i][k], f"t={t} matrix {i} {k}")
            _close(o2[i], o1[i], f"t={t} matrix {i} update")
            _close(Ws2[i], Ws1[i], f"t={t} matrix {i} W", 1e-6)


def _foam_state_dev_many(m, n, side="input"):
    import torch
    k = m if side == "output" else n
    return {"M": torch.zeros((m, n), dtype=torch.float32, device="cuda"),
            "R": torch.zeros((k, k), dtype=torch.float32, device="cuda"),
            "QR": torch.eye(k, dtype=torch.float32, device="cuda"),
            "r": torch.zeros(m, dtype=torch.float32, device="cuda"),
            "c": torch.zeros(n, dtype=torch.float32, device="cuda"),
            "aux": torch.zeros(4, dtype=torch.float32, device="cuda")}


@pytest.mark.parametrize("pf,tol,side", [(1, 0.0, "input"), (2, 0.1, "input"), (1, 0.5, "input"),
                                         (1, 0.0, "output"), (2, 0.1, "output")])
def test_foam_many_matches_separate_calls(gpu_lib, pf, tol, side):
    """foam_step_many against separate foam_step calls, with the criterion
    every step and a refresh every time (tol 0), every other step, and a
    tolerance under which some matrices refresh and others do not (the
    batched QR skips a job on its own device flag)."""
    import torch
    log(f"foam many vs single, pf={pf} tol={tol} side={side}")
    steps = 4
    ws, gs = _many_inputs(MANY_SHAPES, steps, 43)
    Ws1 = [to_dev(w) for w in ws]
    Ws2 = [to_dev(w) for w in ws]
    st1 = [_foam_state_dev_many(m, n, side) for m, n in MANY_SHAPES]
    st2 = [_foam_state_dev_many(m, n, side) for m, n in MANY_SHAPES]
    o1 = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in MANY_SHAPES]
    o2 = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in MANY_SHAPES]
    refreshed = set()
    for t in range(1, steps + 1):
        G = [to_dev(g[t - 1]) for g in gs]
        for i in range(len(MANY_SHAPES)):
            gpu_lib.foam_step(Ws1[i], G[i], st1[i], t, update_out=o1[i], pf=pf, tol=tol,
                              side=side, **HP)
        gpu_lib.foam_step_many([(Ws2[i], G[i], st2[i]) for i in range(len(MANY_SHAPES))], t,
                               update_out=o2, pf=pf, tol=tol, side=side, **HP)
        torch.cuda.synchronize()
        for i in range(len(MANY_SHAPES)):
            a1, a2 = to_host(st1[i]["aux"]), to_host(st2[i]["aux"])
            assert a1[1] == a2[1] and a1[3] == a2[3], f"t={t} matrix {i} aux {a1} {a2}"
            refreshed.add(bool(a2[1]))
            for k in ("M", "R", "QR", "r", "c"):
                _close(st2[i][k], st1[i][k], f"t={t} matrix {i} {k}")
            _close(o2[i], o1[i], f"t={t} matrix {i} update")
    if tol == 0.0:
        assert refreshed == {True}


# Enough equal shapes that a phase's grouped products fill the 256 x 256
# streamed kernel from one pointer-table batch, while the separate calls run
# each product alone on smaller tiles: the K sums are ordered differently,
# hence 1e-4. The factors must be well conditioned for the refreshed bases to
# be determined to that accuracy (a rank-deficient factor leaves part of its
# basis to rounding): FOAM's factor is G^T G of a tall gradient (or G G^T of
# a wide one, output side), SOAP's square gradients have singular values in
# [1, 2], so both of its factors have condition number <= 4 at every step.
def _square_gradients(count, n, steps, seed):
    r = np.random.default_rng(seed)
    s = np.linspace(1.0, 2.0, n)
    out = []
    for _ in range(count):
        gs = []
        for _ in range(steps):
            u = np.linalg.qr(r.standard_normal((n, n)))[0]
            v = np.linalg.qr(r.standard_normal((n, n)))[0]
            gs.append(((u * s) @ v.T).astype(np.float32))
        out.append(gs)
    return out


@pytest.mark.parametrize("opt,side,gdt", [("foam", "input", "f32"), ("foam", "output", "f32"),
                                          ("soap", None, "f32"), ("soap", None, "bf16")])
def test_many_large_batches_match_separate_calls(gpu_lib, opt, side, gdt):
    import torch
    log(f"{opt} many (grouped 256-tile batches) vs single, side={side} g={gdt}")
    steps = 2
    if opt == "foam":
        shapes = [(2600, 1040) if side == "input" else (1040, 2600)] * 6
        ws, gs = _many_inputs(shapes, steps, 47)
    else:
        shapes = [(1040, 1040)] * 6
        ws = _many_inputs(shapes, 1, 47)[0]
        gs = _square_gradients(len(shapes), 1040, steps, 48)
    Ws1 = [to_dev(w) for w in ws]
    Ws2 = [to_dev(w) for w in ws]
    if opt == "foam":
        st1 = [_foam_state_dev_many(m, n, side) for m, n in shapes]
        st2 = [_foam_state_dev_many(m, n, side) for m, n in shapes]
        keys, kw = ("M", "R", "QR", "r", "c"), dict(pf=1, tol=0.0, side=side)
    else:
        st1 = [_soap_state_dev(m, n) for m, n in shapes]
        st2 = [_soap_state_dev(m, n) for m, n in shapes]
        keys, kw = ("M", "V", "L", "R", "QL", "QR"), dict(refresh_every=1)
    hp = dict(HP)
    if opt == "soap":
        # Adam's first step divides G~ by |G~| + eps, a sign function at
        # eps = 1e-8: an entry of G~ within rounding of zero flips between two
        # valid summation orders, a rank-1 change of the update. eps = 1e-2
        # (entries of G~ are ~0.05 here) keeps the division smooth; the states
        # do not depend on eps.
        hp["eps"] = 1e-2
    o1 = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    o2 = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    single = gpu_lib.foam_step if opt == "foam" else gpu_lib.soap_step
    many = gpu_lib.foam_step_many if opt == "foam" else gpu_lib.soap_step_many
    for t in range(1, steps + 1):
        G = [to_dev(bf16_round(g[t - 1]) if gdt == "bf16" else g[t - 1], gdt) for g in gs]
        for i in range(len(shapes)):
            single(Ws1[i], G[i], st1[i], t, update_out=o1[i], **kw, **hp)
        many([(Ws2[i], G[i], st2[i]) for i in range(len(shapes))], t, update_out=o2, **kw, **hp)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            for k in keys:
                _close(st2[i][k], st1[i][k], f"t={t} matrix {i} {k}", 1e-4)
            _close(o2[i], o1[i], f"t={t} matrix {i} update", 1e-4)


def test_foam_many_more_shape_groups_than_one_launch_holds(gpu_lib):
    """Ten distinct shapes (two of them repeated): a phase's grouped products
    split over two launches of at most eight batches each; the states and
    updates equal those of separate calls."""
    import torch
    shapes = [(64 + 8 * i, 72 + 16 * i) for i in range(10)] + [(64, 72), (136, 216)]
    log(f"foam many over {len(shapes)} matrices, 10 distinct shapes")
    steps = 2
    ws, gs = _many_inputs(shapes, steps, 53)
    Ws1 = [to_dev(w) for w in ws]
    Ws2 = [to_dev(w) for w in ws]
    st1 = [_foam_state_dev_many(m, n) for m, n in shapes]
    st2 = [_foam_state_dev_many(m, n) for m, n in shapes]
    o1 = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    o2 = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, steps + 1):
        G = [to_dev(g[t - 1]) for g in gs]
        for i in range(len(shapes)):
            gpu_lib.foam_step(Ws1[i], G[i], st1[i], t, update_out=o1[i], pf=1, tol=0.0, **HP)
        gpu_lib.foam_step_many([(Ws2[i], G[i], st2[i]) for i in range(len(shapes))], t,
                               update_out=o2, pf=1, tol=0.0, **HP)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            for k in ("M", "R", "QR", "r", "c"):
                _close(st2[i][k], st1[i][k], f"t={t} matrix {i} {k}")
            _close(o2[i], o1[i], f"t={t} matrix {i} update")


# ---- many-matrix calls against the oracle ----------------------------------

def _teacher_force_soap_many(gpu_lib, shapes, grads, steps, refresh_every, gated_tol=1e-4):
    """soap_step_many over all matrices each step; every matrix teacher-forced
    against the oracle (EMAs 1e-5, bases by their defining properties, update
    and V gated from t0 = ceil(b/a) + 2)."""
    import torch
    Ws = [to_dev(synth.init_weight("c1", synth.MatrixSpec("w", m, n, 20 + i)))
          for i, (m, n) in enumerate(shapes)]
    sts = [_soap_state_dev(m, n) for m, n in shapes]
    outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, steps + 1):
        prevs = [_host_soap(st) for st in sts]
        w_prevs = [to_host(W) for W in Ws]
        G = [to_dev(grads[i][t - 1]) for i in range(len(shapes))]
        gpu_lib.soap_step_many([(Ws[i], G[i], sts[i]) for i in range(len(shapes))], t,
                               update_out=outs, refresh_every=refresh_every, **HP)
        torch.cuda.synchronize()
        worst_u = worst_v = 0.0
        for i, (m, n) in enumerate(shapes):
            t0 = math.ceil(max(m, n) / min(m, n)) + 2
            new = _host_soap(sts[i])
            g = grads[i][t - 1].astype(np.float64)
            _, ref, _, info = oracle.soap_step(w_prevs[i], g, prevs[i], t,
                                               refresh_every=refresh_every, **HP)
            assert rel(new.M, ref.M) < 1e-5 and rel(new.L, ref.L) < 1e-5
            assert rel(new.R, ref.R) < 1e-5
            if "PL" in info:
                _check_basis(new.QL, info["PL"], ref.QL, f"t={t} matrix {i} QL")
                _check_basis(new.QR, info["PR"], ref.QR, f"t={t} matrix {i} QR")
            else:
                assert np.array_equal(new.QL, prevs[i].QL) and np.array_equal(new.QR, prevs[i].QR)
            _, ref2, upd, _ = oracle.soap_step(w_prevs[i], g, prevs[i], t, refresh_every=0,
                                               q_override=(new.QL, new.QR), **HP)
            eu, ev = rel(to_host(outs[i]), upd), rel(new.V, ref2.V)
            if t >= t0:
                assert eu < gated_tol and ev < gated_tol, f"t={t} matrix {i}: {eu} {ev}"
                worst_u, worst_v = max(worst_u, eu), max(worst_v, ev)
        log(f"  soap many t={t}: worst gated update {worst_u:.2e}, V {worst_v:.2e}")


def test_soap_many_grouped_batches_match_oracle(gpu_lib):
    """soap_step_many on six 1040 x 1040 matrices (each phase's products one
    pointer-table batch on the 256 x 256 kernel, the six QRs of each side one
    batched QR), eps = 1e-8, teacher-forced against the oracle: the many-matrix
    path itself held to the oracle, not only to separate calls."""
    log("soap many (grouped 256-tile batches) vs oracle")
    shapes = [(1040, 1040)] * 6
    grads = _square_gradients(len(shapes), 1040, 4, 61)
    _teacher_force_soap_many(gpu_lib, shapes, grads, 4, refresh_every=1)


@pytest.mark.parametrize("refresh_every,steps", [(2, 6), (10, 12)])
def test_soap_periodic_refresh_teacher_forced(gpu_lib, refresh_every, steps):
    """Standard SOAP's periodic refresh (every k steps, at t = 1, k+1, ...),
    single calls on a Kronecker ragged shape, teacher-forced: the basis is
    refreshed exactly on the scheduled steps and frozen bitwise in between."""
    log(f"soap refresh every {refresh_every}, {steps} steps")
    spec = synth.MatrixSpec("k", 200, 328, 8)
    _run_soap(gpu_lib, 200, 328, steps, lambda t: synth.kronecker_gradient("c3", spec, t),
              refresh_every=refresh_every)


def test_soap_many_periodic_refresh_matches_oracle(gpu_lib):
    """soap_step_many with refresh_every = 2 over the mixed small shapes (QR
    sizes shared across matrices and sides), teacher-forced."""
    log("soap many refresh every 2 vs oracle")
    ws, gs = _many_inputs(MANY_SHAPES, 6, 63)
    _teacher_force_soap_many(gpu_lib, MANY_SHAPES, gs, 6, refresh_every=2)


@pytest.mark.parametrize("side", ["input", "output"])
def test_foam_many_grouped_batches_match_oracle(gpu_lib, side):
    """foam_step_many on six 2600 x 1040 matrices (1040 x 2600 on the output
    side), criterion and refresh every step, teacher-forced against the oracle
    through t0 = 5."""
    import torch
    log(f"foam many (grouped 256-tile batches) vs oracle, side={side}")
    shapes = [(2600, 1040) if side == "input" else (1040, 2600)] * 6
    steps = 5
    ws, gs = _many_inputs(shapes, steps, 67)
    Ws = [to_dev(w) for w in ws]
    sts = [_foam_state_dev_many(m, n, side) for m, n in shapes]
    outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, steps + 1):
        prevs = [_host_foam(st) for st in sts]
        w_prevs = [to_host(W) for W in Ws]
        G = [to_dev(g[t - 1]) for g in gs]
        gpu_lib.foam_step_many([(Ws[i], G[i], sts[i]) for i in range(len(shapes))], t,
                               update_out=outs, pf=1, tol=0.0, side=side, **HP)
        torch.cuda.synchronize()
        worst = 0.0
        for i, (m, n) in enumerate(shapes):
            t0 = math.ceil(max(m, n) / min(m, n)) + 2
            new = _host_foam(sts[i])
            aux = to_host(sts[i]["aux"])
            g = gs[i][t - 1].astype(np.float64)
            _, ref, _, info = oracle.foam_step(w_prevs[i], g, prevs[i], t, pf=1, tol=0.0,
                                               side=side, **HP)
            assert rel(new.M, ref.M) < 1e-5 and rel(new.R, ref.R) < 1e-5
            assert aux[3] == 1.0 and abs(aux[0] - info["rho"]) < 1e-4
            assert bool(aux[1]) == info["refreshed"]
            if info["refreshed"]:
                _check_basis(new.QR, info["P"], ref.QR, f"t={t} matrix {i} QR")
            _, ref2, upd, info2 = oracle.foam_step(w_prevs[i], g, prevs[i], t, pf=1, tol=0.0,
                                                   q_override=new.QR,
                                                   refresh_override=bool(aux[1]), side=side,
                                                   **HP)
            eu = rel(to_host(outs[i]), upd)
            er, ec = rel(new.r, ref2.r), rel(new.c, ref2.c)
            if t >= t0:
                assert eu < 1e-4 and er < 1e-4 and ec < 1e-4, f"t={t} matrix {i}: {eu} {er} {ec}"
                assert abs(aux[2] - info2["tau"]) <= 1e-4 * abs(info2["tau"])
                worst = max(worst, eu)
        log(f"  foam many t={t}: worst gated update {worst:.2e}")


# ---- rotation back in bf16 (back_rot_dtype) ---------------------------------

@pytest.mark.parametrize("shape", [(328, 200), (200, 520)])
def test_soap_bf16_back_rotation_teacher_forced(gpu_lib, shape):
    """U = Q_L N Q_R^T on bf16 MFMA ("SOAP, Muon, and Beyond", section 3-2
    (3): the rotation back may run in reduced precision): update within the
    bf16 tolerance, V exact to fp32."""
    m, n = shape
    log(f"soap bf16 back rotation {m}x{n}")
    spec = synth.MatrixSpec("k", m, n, 12)
    _run_soap(gpu_lib, m, n, 6, lambda t: synth.kronecker_gradient("c3", spec, t), back="bf16")


@pytest.mark.parametrize("side", ["input", "output"])
def test_foam_bf16_back_rotation_teacher_forced(gpu_lib, side):
    import torch
    m, n = (328, 136) if side == "input" else (136, 328)
    log(f"foam bf16 back rotation {side} {m}x{n}")
    spec = synth.MatrixSpec("f", m, n, 13)
    W = to_dev(synth.init_weight("c5", spec))
    st = _foam_state_dev(m, n, side)
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    t0 = math.ceil(max(m, n) / min(m, n)) + 2
    for t in range(1, 8):
        g = synth.kronecker_gradient("c5", spec, t)
        prev, w_prev = _host_foam(st), to_host(W)
        gpu_lib.foam_step(W, to_dev(g), st, t, update_out=out, pf=3, tol=0.1, side=side,
                          back_rot_dtype="bf16", **HP)
        torch.cuda.synchronize()
        new, aux = _host_foam(st), to_host(st["aux"])
        decision = bool(aux[1])
        _, ref2, upd, _ = oracle.foam_step(w_prev, g, prev, t, pf=3, tol=0.1, q_override=new.QR,
                                           refresh_override=decision, side=side, **HP)
        eu, er, ec = rel(to_host(out), upd), rel(new.r, ref2.r), rel(new.c, ref2.c)
        log(f"  foam bf16 back t={t}: update {eu:.2e} r {er:.2e} c {ec:.2e}")
        if t >= t0:
            assert eu < 2e-2 and er < 1e-4 and ec < 1e-4


def test_many_bf16_back_rotation_matches_oracle(gpu_lib):
    """soap_step_many and foam_step_many with the bf16 rotation back (grouped
    bf16 products), teacher-forced."""
    import torch
    log("soap many bf16 back")
    shapes = [(1040, 1040)] * 3
    grads = _square_gradients(len(shapes), 1040, 4, 71)
    Ws = [to_dev(synth.init_weight("c1", synth.MatrixSpec("w", m, n, 40 + i)))
          for i, (m, n) in enumerate(shapes)]
    sts = [_soap_state_dev(m, n) for m, n in shapes]
    outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, 5):
        prevs, wps = [_host_soap(x) for x in sts], [to_host(W) for W in Ws]
        gpu_lib.soap_step_many([(Ws[i], to_dev(grads[i][t - 1]), sts[i]) for i in range(3)], t,
                               update_out=outs, back_rot_dtype="bf16", **HP)
        torch.cuda.synchronize()
        for i in range(3):
            new = _host_soap(sts[i])
            _, ref2, upd, _ = oracle.soap_step(wps[i], grads[i][t - 1].astype(np.float64),
                                               prevs[i], t, refresh_every=0,
                                               q_override=(new.QL, new.QR), **HP)
            eu, ev = rel(to_host(outs[i]), upd), rel(new.V, ref2.V)
            if t >= 3:
                assert eu < 2e-2 and ev < 1e-4, f"t={t} matrix {i}: {eu} {ev}"
        log(f"  soap many bf16 back t={t} ok")
    log("foam many bf16 back")
    shapes = [(2600, 1040)] * 3
    ws, gs = _many_inputs(shapes, 5, 73)
    Ws = [to_dev(w) for w in ws]
    sts = [_foam_state_dev_many(m, n) for m, n in shapes]
    outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, 6):
        prevs, wps = [_host_foam(x) for x in sts], [to_host(W) for W in Ws]
        gpu_lib.foam_step_many([(Ws[i], to_dev(gs[i][t - 1]), sts[i]) for i in range(3)], t,
                               update_out=outs, pf=1, tol=0.0, back_rot_dtype="bf16", **HP)
        torch.cuda.synchronize()
        for i in range(3):
            new, aux = _host_foam(sts[i]), to_host(sts[i]["aux"])
            _, ref2, upd, _ = oracle.foam_step(wps[i], gs[i][t - 1].astype(np.float64), prevs[i],
                                               t, pf=1, tol=0.0, q_override=new.QR,
                                               refresh_override=bool(aux[1]), **HP)
            if t >= 5:
                assert rel(to_host(outs[i]), upd) < 2e-2
                assert rel(new.r, ref2.r) < 1e-4 and rel(new.c, ref2.c) < 1e-4


# ---- forward rotations as bf16x3 products (fwd_rot) --------------------------

@pytest.mark.parametrize("shape,gdt", [((328, 200), "f32"), ((296, 520), "bf16"),
                                       ((200, 520), "f32")])
def test_soap_bf16x3_forward_rotation_teacher_forced(gpu_lib, shape, gdt):
    """Q_L^T G Q_R and Q_L^T M Q_R as three bf16 products per fp32 product
    (hi.hi + lo.hi + hi.lo): the update and V are held to the fp32 tolerance."""
    m, n = shape
    log(f"soap bf16x3 forward rotation {m}x{n} {gdt} gradient")
    spec = synth.MatrixSpec("k", m, n, 14)
    _run_soap(gpu_lib, m, n, 7, lambda t: synth.kronecker_gradient("c3", spec, t), dtype=gdt,
              fwd="bf16x3")


def test_soap_bf16x3_forward_with_bf16_back_rotation(gpu_lib):
    """Both rotation options together (the configuration timed for the 8B
    layer): V at the fp32 tolerance, the update at the bf16 one."""
    log("soap bf16x3 forward + bf16 back 328x200")
    spec = synth.MatrixSpec("k", 328, 200, 15)
    _run_soap(gpu_lib, 328, 200, 7, lambda t: synth.kronecker_gradient("c3", spec, t),
              dtype="bf16", back="bf16", fwd="bf16x3")


def test_many_bf16x3_forward_rotation_matches_oracle(gpu_lib):
    """soap_step_many and foam_step_many with bf16x3 forward rotations (grouped
    bf16 products over split operands), teacher-forced at the fp32 tolerance."""
    import torch
    log("soap many bf16x3 forward")
    shapes = [(1040, 1040)] * 3
    grads = _square_gradients(len(shapes), 1040, 4, 75)
    Ws = [to_dev(synth.init_weight("c1", synth.MatrixSpec("w", m, n, 50 + i)))
          for i, (m, n) in enumerate(shapes)]
    sts = [_soap_state_dev(m, n) for m, n in shapes]
    outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, 5):
        prevs, wps = [_host_soap(x) for x in sts], [to_host(W) for W in Ws]
        gpu_lib.soap_step_many([(Ws[i], to_dev(grads[i][t - 1], "bf16"), sts[i])
                                for i in range(3)], t, update_out=outs, fwd_rot="bf16x3", **HP)
        torch.cuda.synchronize()
        for i in range(3):
            new = _host_soap(sts[i])
            g = bf16_round(grads[i][t - 1].astype(np.float64))
            _, ref2, upd, _ = oracle.soap_step(wps[i], g, prevs[i], t, refresh_every=0,
                                               q_override=(new.QL, new.QR), **HP)
            eu, ev = rel(to_host(outs[i]), upd), rel(new.V, ref2.V)
            if t >= 4:  # square: t0 = 3, bf16x3 forward rotations gated from t0 + 1
                assert eu < 1e-4 and ev < 1e-4, f"t={t} matrix {i}: {eu} {ev}"
        log(f"  soap many bf16x3 forward t={t} ok")
    log("foam many bf16x3 forward")
    for side in ("input", "output"):
        shapes = [(2600, 1040)] * 2 if side == "input" else [(1040, 2600)] * 2
        ws, gs = _many_inputs(shapes, 6, 77)
        Ws = [to_dev(w) for w in ws]
        sts = [_foam_state_dev_many(m, n, side) for m, n in shapes]
        outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
        for t in range(1, 7):
            prevs, wps = [_host_foam(x) for x in sts], [to_host(W) for W in Ws]
            gpu_lib.foam_step_many([(Ws[i], to_dev(gs[i][t - 1]), sts[i]) for i in range(2)], t,
                                   update_out=outs, pf=1, tol=0.0, side=side, fwd_rot="bf16x3",
                                   **HP)
            torch.cuda.synchronize()
            for i in range(2):
                new, aux = _host_foam(sts[i]), to_host(sts[i]["aux"])
                _, ref2, upd, _ = oracle.foam_step(wps[i], gs[i][t - 1].astype(np.float64),
                                                   prevs[i], t, pf=1, tol=0.0, q_override=new.QR,
                                                   refresh_override=bool(aux[1]), side=side, **HP)
                if t >= 6:  # t0 = ceil(2600 / 1040) + 2 = 5, plus one for bf16x3
                    eu = rel(to_host(outs[i]), upd)
                    assert eu < 1e-4, f"{side} t={t} matrix {i}: {eu}"
                    assert rel(new.r, ref2.r) < 1e-4 and rel(new.c, ref2.c) < 1e-4
            log(f"  foam many bf16x3 forward {side} t={t} ok")


# ---- power-iteration products as bf16x3 (refresh_prod) -----------------------

@pytest.mark.parametrize("shape,gdt", [((328, 200), "f32"), ((296, 520), "bf16")])
def test_soap_bf16x3_refresh_products_teacher_forced(gpu_lib, shape, gdt):
    """L Q_L and R Q_R (the QR inputs) as bf16x3 products: the basis is checked
    by its defining properties and by a forward-error bound from the
    product's accuracy; the update and V at the fp32 tolerance."""
    m, n = shape
    log(f"soap bf16x3 refresh products {m}x{n} {gdt} gradient")
    spec = synth.MatrixSpec("k", m, n, 16)
    _run_soap(gpu_lib, m, n, 7, lambda t: synth.kronecker_gradient("c3", spec, t), dtype=gdt,
              fwd="bf16x3", prod="bf16x3")


def test_many_bf16x3_refresh_products_match_oracle(gpu_lib):
    """soap_step_many with bf16x3 refresh products over two size groups (the
    groups share one region of operand splits and run one after another):
    the bases are orthonormal, triangularise the oracle's product, and the
    update and V match the oracle teacher-forced."""
    import torch
    log("soap many bf16x3 refresh products")
    shapes = [(520, 328), (328, 520), (520, 328)]
    specs = [synth.MatrixSpec("k", m, n, 60 + i) for i, (m, n) in enumerate(shapes)]
    Ws = [to_dev(synth.init_weight("c1", sp)) for sp in specs]
    sts = [_soap_state_dev(m, n) for m, n in shapes]
    outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, 7):
        gs = [synth.kronecker_gradient("c3", sp, t) for sp in specs]
        prevs, wps = [_host_soap(x) for x in sts], [to_host(W) for W in Ws]
        gpu_lib.soap_step_many([(Ws[i], to_dev(gs[i]), sts[i]) for i in range(3)], t,
                               update_out=outs, fwd_rot="bf16x3", refresh_prod="bf16x3", **HP)
        torch.cuda.synchronize()
        for i, (m, n) in enumerate(shapes):
            new = _host_soap(sts[i])
            _, ref, _, info = oracle.soap_step(wps[i], gs[i], prevs[i], t, **HP)
            _check_basis(new.QL, info["PL"], ref.QL, f"t={t} matrix {i} QL", "bf16x3")
            _check_basis(new.QR, info["PR"], ref.QR, f"t={t} matrix {i} QR", "bf16x3")
            _, ref2, upd, _ = oracle.soap_step(wps[i], gs[i], prevs[i], t, refresh_every=0,
                                               q_override=(new.QL, new.QR), **HP)
            eu, ev = rel(to_host(outs[i]), upd), rel(new.V, ref2.V)
            t0 = math.ceil(max(m, n) / min(m, n)) + 2
            if t >= t0:  # bf16x3 forward rotations: 1e-4 from t0 + 1
                assert eu < (1e-4 if t > t0 else 2e-2) and ev < 1e-4, f"t={t} matrix {i}: {eu} {ev}"
            log(f"  soap many bf16x3 refresh t={t} matrix {i}: update {eu:.2e} V {ev:.2e}")
    log("foam many bf16x3 criterion products")
    shapes = [(328, 200), (200, 328), (328, 200)]
    ws_, gs_ = _many_inputs(shapes, 5, 79)
    Ws = [to_dev(w) for w in ws_]
    sts = [_foam_state_dev_many(m, n) for m, n in shapes]
    outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, 6):
        prevs, wps = [_host_foam(x) for x in sts], [to_host(W) for W in Ws]
        gpu_lib.foam_step_many([(Ws[i], to_dev(gs_[i][t - 1]), sts[i]) for i in range(3)], t,
                               update_out=outs, pf=1, tol=0.0, refresh_prod="bf16x3", **HP)
        torch.cuda.synchronize()
        for i, (m, n) in enumerate(shapes):
            new, aux = _host_foam(sts[i]), to_host(sts[i]["aux"])
            g = gs_[i][t - 1].astype(np.float64)
            _, ref, _, info = oracle.foam_step(wps[i], g, prevs[i], t, pf=1, tol=0.0, **HP)
            assert abs(aux[0] - info["rho"]) < 1e-4
            if bool(aux[1]):
                _check_basis(new.QR, info["P"], ref.QR, f"t={t} matrix {i} QR", "bf16x3")
            _, ref2, upd, _ = oracle.foam_step(wps[i], g, prevs[i], t, pf=1, tol=0.0,
                                               q_override=new.QR, refresh_override=bool(aux[1]),
                                               **HP)
            if t >= math.ceil(max(m, n) / min(m, n)) + 2:  # fp32 forward rotations
                assert rel(to_host(outs[i]), upd) < 1e-4
        log(f"  foam many bf16x3 criterion t={t} ok")
