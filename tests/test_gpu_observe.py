"""Observability reductions through the C ABI against the fp64 oracle (GPU).

Each call is compared with the oracle on the same inputs (the buffers a step
holds: an update, a Newton-Schulz output, a factor and its basis, a second
moment). Tolerances follow from the arithmetic: fp64 accumulation of exact
fp32/bf16 inputs for the RMS (1e-6 relative); for the residual and the
Rayleigh quotients the fp32 MFMA products bound the error (stated per test);
the rank-1 share by power iteration converges to fp32 rounding on inputs with
a spectral gap.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import bf16_round
from tests.helpers import log, to_dev, to_host

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _dct_rows(n):
    k = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    c = np.sqrt(2.0 / n) * np.cos(np.pi * (2 * j + 1) * k / (2 * n))
    c[0, :] = np.sqrt(1.0 / n)
    return c


@pytest.mark.parametrize("dtype,shape", [("f32", (3, 130, 70)), ("bf16", (2, 37, 1000)),
                                         ("f32", (1, 1000, 777)), ("f32", (1, 1, 1))])
def test_matrix_rms(gpu_lib, dtype, shape):
    import torch
    log(f"matrix rms {dtype} {shape}")
    r = np.random.default_rng(41)
    x = (r.standard_normal(shape) * np.exp(r.standard_normal((shape[0], 1, 1)))).astype(np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    out = gpu_lib.matrix_rms(to_dev(x, dtype))
    torch.cuda.synchronize()
    got = to_host(out)
    for b in range(shape[0]):
        want = oracle.matrix_rms(x[b])
        assert abs(got[b] - want) <= 1e-6 * want, (b, got[b], want)
    again = gpu_lib.matrix_rms(to_dev(x, dtype))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(again), got)


def _residual_tol(ref):
    # fp32 products of near-unit rows: entry errors ~sqrt(K) u; the
    # residual moves by at most ||dA||_F / sqrt(a)
    return 1e-3 * ref + 2e-4


@pytest.mark.parametrize("count,m,n", [(3, 96, 160), (2, 160, 96), (1, 256, 512), (1, 300, 1)])
def test_ns_residual_on_muon_updates(gpu_lib, count, m, n):
    """The residual of the Newton-Schulz output recovered from muon_step's
    update (scale = sqrt(n / m)), per matrix of a batch, wide and tall."""
    import torch
    log(f"ns residual {count}x{m}x{n}")
    r = np.random.default_rng(42)
    g = r.standard_normal((count, m, n)).astype(np.float32)
    W, G, M = to_dev(np.zeros_like(g)), to_dev(g), to_dev(np.zeros_like(g))
    out = to_dev(np.zeros((count, m, n), np.float32))
    gpu_lib.muon_step_batched([(W, G, M)], update_out=[out], lr=0.0, mu=0.95, weight_decay=0.0,
                              ns_steps=5, ns_dtype="f32")
    torch.cuda.synchronize()
    scale = math.sqrt(n / m)
    res = to_host(gpu_lib.ns_residual(out, scale))
    o = to_host(out)
    for b in range(count):
        want = oracle.ns_residual(o[b], scale)
        log(f"  matrix {b}: residual {res[b]:.4e} (oracle {want:.4e})")
        assert abs(res[b] - want) <= _residual_tol(want)


def test_ns_residual_orthonormal_rows_is_zero(gpu_lib):
    import torch
    log("ns residual of orthonormal rows")
    x = _dct_rows(320)[:200].astype(np.float32)          # 200 x 320, orthonormal rows
    res = to_host(gpu_lib.ns_residual(to_dev(3.0 * x), 1.0 / 3.0))
    res_t = to_host(gpu_lib.ns_residual(to_dev(np.ascontiguousarray(x.T))))
    torch.cuda.synchronize()
    assert res[0] <= 2e-4 and res_t[0] <= 2e-4
    s = np.linspace(0.2, 1.3, 200)
    y = (np.diag(s) @ x).astype(np.float32)              # singular values s
    want = math.sqrt(np.mean((s * s - 1.0) ** 2))
    got = to_host(gpu_lib.ns_residual(to_dev(y)))[0]
    assert abs(got - want) <= _residual_tol(want)


@pytest.mark.parametrize("n", [1, 65, 300])
def test_rayleigh_quotients_of_a_factor(gpu_lib, n):
    """d_i = q_i^T F q_i for a SOAP-like factor F = G G^T / m + 1e-3 I and an
    orthonormal basis; error bound of the two fp32 products stated inline."""
    import torch
    log(f"rayleigh n={n}")
    r = np.random.default_rng(43)
    g = r.standard_normal((n, 2 * n + 3)) * np.exp(0.5 * r.standard_normal((n, 1)))
    f = (g @ g.T / g.shape[1] + 1e-3 * np.eye(n)).astype(np.float32)
    q = oracle.qr_positive(r.standard_normal((n, n)))[0].astype(np.float32)
    d, kappa = gpu_lib.rayleigh(to_dev(f), to_dev(q))
    torch.cuda.synchronize()
    d, kappa = to_host(d), float(to_host(kappa)[0])
    fd, qd = f.astype(np.float64), q.astype(np.float64)
    d_ref, k_ref = oracle.rayleigh(fd, qd)
    gam = n * U32 / (1 - n * U32)
    bound = 2.2 * gam * np.array([np.abs(qd[:, i]) @ np.abs(fd) @ np.abs(qd[:, i])
                                  for i in range(n)]) + 1e-7 * np.abs(d_ref)
    assert np.all(np.abs(d - d_ref) <= bound)
    assert abs(kappa - d.max() / d.min()) <= 1e-6 * kappa
    rk = bound[np.argmax(d_ref)] / d_ref.max() + bound[np.argmin(d_ref)] / d_ref.min()
    assert abs(kappa - k_ref) <= (1.01 * rk + 1e-6) * k_ref
    # in F's own eigenbasis the quotients are the eigenvalues
    lam, vec = np.linalg.eigh(fd)
    d2, k2 = gpu_lib.rayleigh(to_dev(f), to_dev(vec.astype(np.float32)))
    torch.cuda.synchronize()
    log(f"  kappa {kappa:.4e} (oracle {k_ref:.4e}); eigenbasis kappa {float(to_host(k2)[0]):.4e} "
        f"(cond {lam.max() / lam.min():.4e})")
    assert np.allclose(np.sort(to_host(d2)), lam, rtol=1e-4, atol=1e-6 * lam.max())


def _second_moment(m, n, seed):
    """A rotated-second-moment-like nonnegative matrix: the EMA of squared
    Kronecker-structured gradients (row and column scales times noise)."""
    r = np.random.default_rng(seed)
    a, b = np.exp(r.standard_normal((m, 1))), np.exp(r.standard_normal((1, n)))
    v = np.zeros((m, n))
    for _ in range(6):
        g = a * r.standard_normal((m, n)) * b
        v = 0.95 * v + 0.05 * g * g
    return v.astype(np.float32)


@pytest.mark.parametrize("m,n", [(300, 137), (1000, 700), (37, 1)])
def test_rank1_share(gpu_lib, m, n):
    import torch
    log(f"rank-1 share {m}x{n}")
    v = _second_moment(m, n, 44)
    got = float(to_host(gpu_lib.rank1_share(to_dev(v), iters=50))[0])
    torch.cuda.synchronize()
    want = oracle.rank1_share(v.astype(np.float64))
    log(f"  share {got:.6f} (oracle {want:.6f})")
    assert abs(got - want) <= 1e-5
    assert got <= want + 1e-6
    r = np.random.default_rng(45)
    one = np.outer(np.abs(r.standard_normal(m)), np.abs(r.standard_normal(n))).astype(np.float32)
    assert abs(float(to_host(gpu_lib.rank1_share(to_dev(one), iters=3))[0]) - 1.0) <= 1e-5
    zero = float(to_host(gpu_lib.rank1_share(to_dev(np.zeros((m, n), np.float32)), iters=2))[0])
    assert zero == 0.0


def test_rank1_share_of_a_signed_momentum_is_inverse_stable_rank(gpu_lib):
    """On a signed matrix built from known singular values the share is
    s_1^2 / sum s_i^2 = 1 / stable rank, the summary of the momentum's
    singular-value distribution; the all-ones start still converges."""
    import torch
    log("rank-1 share of a signed matrix with known singular values")
    r = np.random.default_rng(46)
    m, n, k = 384, 200, 200
    u = oracle.qr_positive(r.standard_normal((m, m)))[0][:, :k]
    v = oracle.qr_positive(r.standard_normal((n, n)))[0][:, :k]
    s = np.concatenate([[4.0, 2.0], np.linspace(1.0, 0.01, k - 2)])
    x = (u * s) @ v.T
    want = s[0] ** 2 / np.sum(s * s)
    assert want == pytest.approx(oracle.rank1_share(x), rel=1e-10)
    got = float(to_host(gpu_lib.rank1_share(to_dev(x.astype(np.float32)), iters=40))[0])
    torch.cuda.synchronize()
    log(f"  share {got:.6f} (1 / stable rank {want:.6f})")
    assert abs(got - want) <= 1e-5


def test_basis_age_follows_foam_refreshes(gpu_lib):
    """The device age tracks the refresh flag each foam_step writes."""
    import torch
    log("basis age over foam steps")
    m, n = 96, 160
    spec = synth.MatrixSpec("f", m, n, 5)
    z = lambda r, c: torch.zeros((r, c), dtype=torch.float32, device="cuda")
    for tol in (0.0, 0.1, 1.0):
        W = to_dev(synth.init_weight("c5", spec))
        st = {"M": z(m, n), "R": z(n, n), "QR": torch.eye(n, dtype=torch.float32, device="cuda"),
              "r": torch.zeros(m, device="cuda"), "c": torch.zeros(n, device="cuda"),
              "aux": torch.zeros(4, device="cuda")}
        age = torch.zeros(1, device="cuda")
        flags, ages = [], []
        for t in range(1, 8):
            g = synth.kronecker_gradient("c5", spec, t)
            gpu_lib.foam_step(W, to_dev(g), st, t, pf=2, tol=tol, lr=1e-3)
            gpu_lib.basis_age(st["aux"], age)
            torch.cuda.synchronize()
            flags.append(bool(to_host(st["aux"])[1]))
            ages.append(int(to_host(age)[0]))
        log(f"  tol {tol}: refreshed {flags} ages {ages}")
        assert ages == oracle.basis_ages(flags)
        if tol == 1.0:
            assert not any(flags)
        if tol == 0.0:
            assert flags[0::2] == [True] * 4 and not any(flags[1::2])
