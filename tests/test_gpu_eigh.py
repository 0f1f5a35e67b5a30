"""The block-Jacobi eigensolver (mao_eigh) and FOAM's eigendecomposition
refresh against the fp64 oracle (GPU).

The eigenvalues must match the oracle's (descending) to 2e-5 of the largest;
the basis is checked by what defines it -- orthonormal columns, Q^T F Q
diagonal, residuals ||F q_j - lambda_j q_j|| small -- and each column against
the oracle's eigenvector through the Davis-Kahan bound sin(angle) <=
||residual|| / gap, which holds for any eigenvector approximation (several
bases are correct where eigenvalues coincide)."""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import bf16_round
from tests.helpers import log, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _check_eigh(q, lam, f, tag, evals_tol=2e-5, orth_tol=2e-5, off_tol=1e-4, lam_ref=None):
    """q, lam: the GPU's eigenvectors (columns) and eigenvalues; f: fp64 F.
    With lam_ref given (the oracle's eigenvalues, computed already) the
    per-column Davis-Kahan comparison is skipped."""
    n = f.shape[0]
    q_ref = None
    if lam_ref is None:
        lam_ref, q_ref = oracle.eigh_descending(f)
    top = max(abs(lam_ref[0]), abs(lam_ref[-1]), 1e-30)
    assert np.abs(lam - lam_ref).max() <= evals_tol * top, f"{tag}: eigenvalues"
    orth = np.abs(q.T @ q - np.eye(n)).max()
    assert orth <= orth_tol, f"{tag}: orthogonality {orth}"
    d = q.T @ f @ q
    off = np.linalg.norm(d - np.diag(np.diag(d))) / max(np.linalg.norm(f), 1e-300)
    assert off <= off_tol, f"{tag}: off-diagonal ratio {off}"
    assert np.abs(np.diag(d) - lam).max() <= evals_tol * top
    # Davis-Kahan per column: sin(angle(q_j, q_ref_j)) <= |F q_j - l_j q_j| / gap_j
    res = np.linalg.norm(f @ q - q * lam[None, :], axis=0)
    assert res.max() <= 1e-4 * top, f"{tag}: residual {res.max() / top}"
    if q_ref is None:
        return off, orth, np.abs(lam - lam_ref).max() / top
    gaps = np.full(n, np.inf)
    if n > 1:
        dl = np.abs(np.diff(lam_ref))
        gaps[:-1] = np.minimum(gaps[:-1], dl)
        gaps[1:] = np.minimum(gaps[1:], dl)
    cos = np.abs(np.sum(q * q_ref, axis=0)) / np.linalg.norm(q, axis=0)
    sin = np.sqrt(np.maximum(0.0, 1.0 - cos ** 2))
    ok = gaps > 1e-3 * top
    bound = res / np.maximum(gaps - res, 1e-300) + 1e-5
    assert np.all(sin[ok] <= bound[ok]), f"{tag}: eigenvector outside its Davis-Kahan bound"
    return off, orth, np.abs(lam - lam_ref).max() / top


def _spd(n, seed, decay=None):
    r = np.random.default_rng(seed)
    if decay == "k^-1":  # the Kronecker factors' spectrum, in a random basis
        u = np.linalg.qr(r.standard_normal((n, n)))[0]
        return (u * (1.0 / np.arange(1, n + 1))[None, :]) @ u.T
    g = r.standard_normal((n + 7, n)) * np.exp(r.standard_normal(n))[None, :]
    return g.T @ g / n


@pytest.mark.parametrize("n", [1, 5, 64, 100, 128, 200, 300, 520])
def test_eigh_matches_oracle(gpu_lib, n):
    import torch
    log(f"eigh n={n}")
    f = _spd(n, 400 + n).astype(np.float32)
    ev = torch.empty(n, dtype=torch.float32, device="cuda")
    info = torch.empty(13, dtype=torch.float32, device="cuda")
    Q = gpu_lib.eigh(to_dev(f), evals=ev, info=info)
    torch.cuda.synchronize()
    off, orth, el = _check_eigh(to_host(Q), to_host(ev), f.astype(np.float64), f"n={n}")
    inf = to_host(info)
    log(f"  sweeps {int(inf[12])}, off {off:.1e}, orth {orth:.1e}, eig {el:.1e}, "
        f"ratios {' '.join('%.1e' % x for x in inf[:int(inf[12])])}")


@pytest.mark.parametrize("n", [1536, 2100])
def test_eigh_kronecker_spectrum(gpu_lib, n):
    """The k^-1 spectrum of the Kronecker factors at the 760M width (and a
    ragged size): many close small eigenvalues."""
    import torch
    log(f"eigh k^-1 n={n}")
    f = _spd(n, 500 + n, "k^-1").astype(np.float32)
    ev = torch.empty(n, dtype=torch.float32, device="cuda")
    info = torch.empty(13, dtype=torch.float32, device="cuda")
    Q = gpu_lib.eigh(to_dev(f), evals=ev, info=info)
    torch.cuda.synchronize()
    off, orth, el = _check_eigh(to_host(Q), to_host(ev), f.astype(np.float64), f"n={n}")
    log(f"  sweeps {int(to_host(info)[12])}, off {off:.1e}, orth {orth:.1e}, eig {el:.1e}")


def test_eigh_degenerate_and_zero(gpu_lib):
    """Repeated eigenvalues (any orthonormal basis of the eigenspace is
    correct) and the zero matrix (Q = I, nothing to rotate)."""
    import torch
    n = 200
    r = np.random.default_rng(9)
    u = np.linalg.qr(r.standard_normal((n, n)))[0]
    lam = np.repeat([3.0, 1.0, 0.0, -0.5], n // 4)
    f = ((u * lam[None, :]) @ u.T).astype(np.float32)
    ev = torch.empty(n, dtype=torch.float32, device="cuda")
    Q = gpu_lib.eigh(to_dev(f), evals=ev)
    torch.cuda.synchronize()
    q, l = to_host(Q), to_host(ev)
    assert np.abs(q.T @ q - np.eye(n)).max() < 2e-5
    assert np.abs(l - np.sort(lam)[::-1]).max() < 2e-5 * 3.0
    d = q.T @ f.astype(np.float64) @ q
    assert np.linalg.norm(d - np.diag(np.diag(d))) < 1e-4 * np.linalg.norm(f)
    Z = gpu_lib.eigh(torch.zeros((70, 70), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(Z), np.eye(70))


# ---- FOAM with the eigendecomposition refresh ------------------------------

def _foam_state_dev(m, n, side="input"):
    import torch
    k = m if side == "output" else n
    return {"M": torch.zeros((m, n), dtype=torch.float32, device="cuda"),
            "R": torch.zeros((k, k), dtype=torch.float32, device="cuda"),
            "QR": torch.eye(k, dtype=torch.float32, device="cuda"),
            "r": torch.zeros(m, dtype=torch.float32, device="cuda"),
            "c": torch.zeros(n, dtype=torch.float32, device="cuda"),
            "aux": torch.zeros(4, dtype=torch.float32, device="cuda")}


def _host_foam(st):
    return oracle.FoamState(to_host(st["M"]), to_host(st["R"]), to_host(st["QR"]),
                            to_host(st["r"]), to_host(st["c"]))


def _foam_eigh_step_check(st, prev, w_prev, g, t, out, pf, tol, side, tag, gate, full=False):
    new = _host_foam(st)
    aux = to_host(st["aux"])
    _, ref, _, info = oracle.foam_step(w_prev, g, prev, t, pf=pf, tol=tol, side=side,
                                       refresh="eigh", **HP)
    assert bool(aux[3]) == info["checked"]
    assert rel(new.M, ref.M) < 1e-5 and rel(new.R, ref.R) < 1e-5
    decision = info["refreshed"]
    if info["checked"]:
        assert abs(aux[0] - info["rho"]) < 1e-4
        if abs(info["rho"] - tol) > 1e-4:
            assert bool(aux[1]) == info["refreshed"]
        decision = bool(aux[1])
        if decision:  # the new basis: eigenvectors of the GPU's own R
            lam = np.diag(new.QR.T @ new.R @ new.QR)
            _check_eigh(new.QR, lam, new.R, f"{tag} t={t}",
                        lam_ref=info["eigenvalues"] if full else None)
    if not decision:
        assert np.array_equal(new.QR, prev.QR)
    _, ref2, upd, info2 = oracle.foam_step(w_prev, g, prev, t, pf=pf, tol=tol,
                                           q_override=new.QR, refresh_override=decision,
                                           side=side, **HP)
    eu = rel(to_host(out), upd)
    er, ec = rel(new.r, ref2.r), rel(new.c, ref2.c)
    log(f"  {tag} t={t}: update {eu:.2e} r {er:.2e} c {ec:.2e} rho {aux[0]:.3f} refresh {decision}")
    if gate:
        assert eu < 1e-4 and er < 1e-4 and ec < 1e-4
        assert abs(aux[2] - info2["tau"]) <= 1e-4 * abs(info2["tau"])


@pytest.mark.parametrize("m,n,side", [(300, 200, "input"), (200, 304, "output"),
                                      (136, 264, "input")])
def test_foam_eigh_refresh_teacher_forced(gpu_lib, m, n, side):
    import torch
    log(f"foam eigh refresh {side} {m}x{n}")
    spec = synth.MatrixSpec("f", m, n, 9)
    W = to_dev(synth.init_weight("c5", spec))
    st = _foam_state_dev(m, n, side)
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    t0 = math.ceil(max(m, n) / min(m, n)) + 2
    for t in range(1, 9):
        g = synth.kronecker_gradient("c5", spec, t)
        prev, w_prev = _host_foam(st), to_host(W)
        gpu_lib.foam_step(W, to_dev(g), st, t, update_out=out, pf=3, tol=0.05, side=side,
                          refresh="eigh", **HP)
        torch.cuda.synchronize()
        _foam_eigh_step_check(st, prev, w_prev, g, t, out, 3, 0.05, side, "foam eigh", t >= t0)


def test_foam_many_eigh_refresh_teacher_forced(gpu_lib):
    """foam_step_many with the eigh refresh over mixed shapes (batched
    eigendecompositions of two sizes), criterion every step, teacher-forced."""
    import torch
    shapes = [(300, 200), (264, 136), (300, 200), (200, 136)]
    log("foam many eigh refresh")
    W = [to_dev(synth.init_weight("c5", synth.MatrixSpec("f", m, n, 30 + i)))
         for i, (m, n) in enumerate(shapes)]
    st = [_foam_state_dev(m, n) for m, n in shapes]
    outs = [torch.empty((m, n), dtype=torch.float32, device="cuda") for m, n in shapes]
    for t in range(1, 6):
        gs = [synth.kronecker_gradient("c5", synth.MatrixSpec("f", m, n, 30 + i), t)
              for i, (m, n) in enumerate(shapes)]
        prevs, wps = [_host_foam(s) for s in st], [to_host(w) for w in W]
        gpu_lib.foam_step_many([(W[i], to_dev(gs[i]), st[i]) for i in range(len(shapes))], t,
                               update_out=outs, pf=1, tol=0.0, refresh="eigh", **HP)
        torch.cuda.synchronize()
        for i, (m, n) in enumerate(shapes):
            t0 = math.ceil(max(m, n) / min(m, n)) + 2
            _foam_eigh_step_check(st[i], prevs[i], wps[i], gs[i], t, outs[i], 1, 0.0, "input",
                                  f"many {i}", t >= t0)


@pytest.mark.parametrize("name", ["l0.q", "l0.fc", "l0.proj"])
def test_foam_eigh_full_size_gpt2_layer(gpu_lib, name):
    """The eigh refresh at the 760M set's factor sizes (1536 for Q and FC,
    6144 for PROJ) at t = 1 (criterion evaluated, refresh triggered from
    Q_R = I), teacher-forced."""
    import torch
    sp = [s for s in synth.specs("c5") if s.name == name][0]
    m, n = sp.rows, sp.cols
    log(f"foam eigh full size {name} {m}x{n}")
    w = synth.init_weight("c5", sp)
    g = synth.gradient("c5", sp, 1)
    W = to_dev(w)
    st = _foam_state_dev(m, n)
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    gpu_lib.foam_step(W, to_dev(g), st, 1, update_out=out, pf=10, tol=0.1, refresh="eigh", **HP)
    torch.cuda.synchronize()
    prev = oracle.foam_init(m, n)
    _foam_eigh_step_check(st, prev, w.astype(np.float64), g, 1, out, 10, 0.1, "input",
                          f"full {name}", n <= m, full=True)
