"""Kernel-level parity of the MFMA contraction and the Householder QR against
the fp64 oracle (GPU)."""
import math

import numpy as np
import pytest

import oracle
from synth import bf16_round
from tests.helpers import log, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

GEMM_SHAPES = [(1, 1, 1), (64, 64, 64), (130, 77, 203), (300, 257, 500), (513, 129, 64),
               (1024, 1000, 1536),
               # large enough for the 256 x 256 streamed kernels, ragged in M, N, K;
               # whole tiles with K a multiple of the slice
               (4100, 2052, 1060), (2304, 4352, 8), (2048, 4096, 1024),
               # rank-k updates (k <= 64) on the fp32 256 x 256 rank kernel
               (1500, 1300, 64), (4100, 2052, 40), (1030, 1030, 1),
               # tall skinny products (the QR projections, 64-wide tiles)
               (40000, 64, 300), (33000, 40, 96)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm_nt_matches_fp64(gpu_lib, dtype, shape):
    import torch
    M, N, K = shape
    log(f"gemm {dtype} {shape}")
    r = np.random.default_rng(100 + M + N + K)
    a = r.standard_normal((M, K)).astype(np.float32)
    b = r.standard_normal((N, K)).astype(np.float32)
    c0 = r.standard_normal((M, N)).astype(np.float32)
    if dtype == "bf16":
        a, b = bf16_round(a), bf16_round(b)
    A, B, C0 = to_dev(a, dtype), to_dev(b, dtype), to_dev(c0)
    D = gpu_lib.gemm_nt(A, B, alpha=0.75, beta=-0.5, C0=C0)
    torch.cuda.synchronize()
    ref = 0.75 * (a.astype(np.float64) @ b.astype(np.float64).T) - 0.5 * c0
    assert rel(to_host(D), ref) < 1e-5


# B stored K x N (the Newton-Schulz product B X reads X this way): ragged in
# every dimension, K below one slice, K with a partial last slice, N below one
# 16-byte chunk
KMAJOR_SHAPES = [(1, 1, 1), (8, 8, 8), (64, 64, 64), (300, 520, 96), (130, 77, 203),
                 (4100, 2052, 1060), (1536, 2048, 1536), (33, 1001, 2050), (520, 6, 40)]


@pytest.mark.parametrize("shape", KMAJOR_SHAPES)
def test_gemm_b_kmajor_matches_fp64(gpu_lib, shape):
    import torch
    M, N, K = shape
    log(f"gemm bf16 B K-major {shape}")
    r = np.random.default_rng(300 + M + N + K)
    a = bf16_round(r.standard_normal((M, K)).astype(np.float32))
    b = bf16_round(r.standard_normal((K, N)).astype(np.float32))
    c0 = r.standard_normal((M, N)).astype(np.float32)
    A, B, C0 = to_dev(a, "bf16"), to_dev(b, "bf16"), to_dev(c0)
    D = gpu_lib.gemm_nt(A, B, alpha=0.75, beta=-0.5, C0=C0, b_kmajor=True)
    torch.cuda.synchronize()
    ref = 0.75 * (a.astype(np.float64) @ b.astype(np.float64)) - 0.5 * c0
    assert rel(to_host(D), ref) < 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,k", [(1, 5), (70, 33), (200, 1000), (513, 300), (4100, 1000),
                                 (4352, 96)])
def test_syrk_is_exactly_symmetric(gpu_lib, dtype, n, k):
    import torch
    log(f"syrk {dtype} {n}x{k}")
    r = np.random.default_rng(7 + n)
    a = r.standard_normal((n, k)).astype(np.float32)
    if dtype == "bf16":
        a = bf16_round(a)
    c0 = r.standard_normal((n, n)).astype(np.float32)
    c0 = c0 + c0.T
    A = to_dev(a, dtype)
    D = gpu_lib.gemm_nt(A, A, alpha=0.05, beta=0.95, C0=to_dev(c0), symmetric=True)
    torch.cuda.synchronize()
    d = to_host(D)
    assert np.array_equal(d, d.T)
    ref = 0.05 * (a.astype(np.float64) @ a.astype(np.float64).T) + 0.95 * c0
    assert rel(d, ref) < 1e-5


@pytest.mark.parametrize("n", [1, 5, 64, 65, 130, 300, 700, 1100])
def test_qr_matches_oracle(gpu_lib, n):
    import torch
    log(f"qr n={n}")
    r = np.random.default_rng(300 + n)
    # singular values inside about [0.5, 3.5]: well conditioned, so Q is unique
    # to fp32 accuracy and a forward comparison is meaningful
    p = (r.standard_normal((n, n)) / math.sqrt(n) + 2.0 * np.eye(n)).astype(np.float32)
    Q = gpu_lib.qr(to_dev(p))
    torch.cuda.synchronize()
    q = to_host(Q)
    q_ref, r_ref = oracle.qr_positive(p.astype(np.float64))
    assert np.abs(q.T @ q - np.eye(n)).max() < 1e-5
    kappa = np.linalg.cond(p.astype(np.float64))
    assert kappa * 2.0 ** -24 < 1e-4
    assert rel(q, q_ref) < 1e-4
    rr = q.T @ p.astype(np.float64)
    assert np.all(np.diag(rr) > -1e-5 * np.linalg.norm(p))


def test_qr_rank_deficient_stays_orthonormal(gpu_lib):
    """A rank-deficient PSD product (the early-step refresh case): Q must be
    orthonormal and Q^T P upper triangular; the completion is not unique."""
    import torch
    n, k = 300, 40
    r = np.random.default_rng(11)
    a = r.standard_normal((n, k))
    p = (a @ a.T).astype(np.float32)
    Q = gpu_lib.qr(to_dev(p))
    torch.cuda.synchronize()
    q = to_host(Q)
    assert np.abs(q.T @ q - np.eye(n)).max() < 1e-4
    rr = q.T @ p.astype(np.float64)
    assert np.linalg.norm(np.tril(rr, -1)) < 1e-4 * np.linalg.norm(p)
    # the leading k columns span the range of P
    qk = q[:, :k]
    proj = qk @ (qk.T @ p)
    assert rel(proj, p) < 1e-4


def test_qr_zero_matrix(gpu_lib):
    import torch
    n = 70
    Q = gpu_lib.qr(torch.zeros((n, n), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    q = to_host(Q)
    assert np.array_equal(q, np.eye(n))


def test_qr_barrier_timeout_poisons_the_basis(gpu_lib):
    """A QR whose grid barriers time out must not hand back a plausible basis:
    started with its time-out flag raised (every barrier gives up at once,
    every kernel exits), the QR writes NaN to all of Q. A normal QR on the
    same workspace right after is unaffected (the flag is reset per QR)."""
    import torch
    for n in (70, 300):
        log(f"qr abort n={n}")
        r = np.random.default_rng(17 + n)
        p = (r.standard_normal((n, n)) / math.sqrt(n) + 2.0 * np.eye(n)).astype(np.float32)
        P = to_dev(p)
        Q = gpu_lib.qr(P, dbg_flags=gpu_lib.DBG_QR_ABORT_BARRIERS)
        torch.cuda.synchronize()
        assert torch.isnan(Q).all().item()
        Q2 = gpu_lib.qr(P)
        torch.cuda.synchronize()
        q = to_host(Q2)
        assert rel(q, oracle.qr_positive(p.astype(np.float64))[0]) < 1e-4


def test_qr_cholesky_panels_run_without_fallback(gpu_lib):
    """The per-column Householder panel that a CholeskyQR breakdown falls back
    to gives the same basis, so a broken fast panel would still pass every
    other QR test (only slower). With the fallback turned into a NaN basis
    (test flag), a well-conditioned P -- Gaussian, several panels and
    workgroups per panel, a ragged last panel -- must come out finite and
    equal, bit for bit, to the ordinary call: the CholeskyQR panels factored
    every panel themselves."""
    import torch
    for n in (70, 300, 1100, 4096):
        log(f"qr no-fallback n={n}")
        r = np.random.default_rng(29 + n)
        p = r.standard_normal((n, n)).astype(np.float32)
        P = to_dev(p)
        Q1 = gpu_lib.qr(P, dbg_flags=gpu_lib.DBG_QR_NO_FALLBACK)
        Q2 = gpu_lib.qr(P)
        torch.cuda.synchronize()
        assert torch.isfinite(Q1).all().item()
        assert torch.equal(Q1, Q2)
        if n <= 300:
            assert rel(to_host(Q1), oracle.qr_positive(p.astype(np.float64))[0]) < 1e-4
