"""The C ABI on the host: the library loads, exports every entry point that
include/mao.h declares, and rejects invalid calls with the documented status
codes before touching the device.

Invalid calls use fake, never-dereferenced device addresses; every call here
is invalid, so none of them reaches a kernel launch. They are skipped when a
GPU is present, to keep a mistake in validation from ever launching a kernel
on a fake address.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import matrix_aware_optimizers_amd as mao

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mao.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_LAYOUT, E_ALIAS, E_HPARAM, E_WORKSPACE = 0, 1, 2, 3, 4, 5, 6, 7
E_UNSUPPORTED = 9
FAKE = 0x7F0000000000  # 256-aligned, never dereferenced


def _declared():
    src = open(HEADER).read()
    return re.findall(r"MAO_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_library_exports_every_declared_symbol():
    lib = mao.load()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    # the binding's table covers the same set
    assert set(names) == set(mao.EXPORTS) - set(), sorted(set(names) ^ set(mao.EXPORTS))


def test_status_strings_and_version():
    lib = mao.load()
    assert lib.mao_abi_version() == 4
    for code in range(10):
        assert lib.mao_status_string(code)
    assert lib.mao_status_string(99) == b"unknown status"


def test_workspace_queries():
    lib = mao.load()
    hp = mao.muon_hparams(ns_dtype="bf16")
    a = lib.muon_workspace_size(4096, 4096, ctypes.byref(hp))
    b = lib.muon_workspace_size(14336, 4096, ctypes.byref(hp))
    assert 0 < a < b
    hp32 = mao.muon_hparams(ns_dtype="f32")
    assert lib.muon_workspace_size(4096, 4096, ctypes.byref(hp32)) > a
    assert lib.muon_workspace_size(0, 4, ctypes.byref(hp)) == 0
    sh = mao.soap_hparams()
    assert lib.soap_workspace_size(256, 512, ctypes.byref(sh)) > 0
    fh = mao.foam_hparams()
    assert lib.foam_workspace_size(1536, 6144, ctypes.byref(fh)) > 0
    assert lib.mao_qr_workspace_size(300) > 0
    assert lib.mao_qr_workspace_size(0) == 0


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


needs_no_gpu = pytest.mark.skipif(_gpu_present(), reason="fake-address validation runs host-only")


def _mat(ptr, rows, cols, ld, dtype=mao.F32):
    return mao.Mat(ptr, rows, cols, ld, dtype)


@needs_no_gpu
def test_muon_validation_codes():
    lib = mao.load()
    hp = mao.muon_hparams(lr=1e-3, mu=0.95)
    ws_need = lib.muon_workspace_size(8, 16, ctypes.byref(hp))
    W = _mat(FAKE, 8, 16, 16, mao.BF16)
    G = _mat(FAKE + (1 << 20), 8, 16, 16, mao.BF16)
    M = _mat(FAKE + (2 << 20), 8, 16, 16)
    ws = ctypes.c_void_p(FAKE + (4 << 20))

    def call(W=W, G=G, M=M, hp=hp, ws=ws, ws_bytes=ws_need, out=None):
        return lib.muon_step(W, G, M, ctypes.byref(hp), ws, ws_bytes, out, None)

    assert call(W=_mat(None, 8, 16, 16)) == E_NULL
    assert call(G=_mat(FAKE + (1 << 20), 8, 15, 16, mao.BF16)) == E_SHAPE
    assert call(W=_mat(FAKE, 0, 16, 16)) == E_SHAPE
    assert call(W=_mat(FAKE, 8, 16, 12)) == E_LAYOUT            # ld not a multiple of 8
    assert call(W=_mat(FAKE, 8, 16, 8)) == E_LAYOUT             # ld < cols
    assert call(W=_mat(FAKE + 4, 8, 16, 16)) == E_LAYOUT        # misaligned
    assert call(M=_mat(FAKE + (2 << 20), 8, 16, 16, mao.BF16)) == E_DTYPE  # momentum must be fp32
    assert call(W=_mat(FAKE, 8, 16, 16, 7)) == E_DTYPE
    assert call(G=_mat(FAKE + 64, 8, 16, 16, mao.BF16)) == E_ALIAS
    assert call(hp=mao.muon_hparams(mu=1.0)) == E_HPARAM
    assert call(hp=mao.muon_hparams(eps=0.0)) == E_HPARAM
    assert call(hp=mao.muon_hparams(ns_steps=65)) == E_HPARAM
    assert call(hp=mao.muon_hparams(lr=float("nan"))) == E_HPARAM
    assert call(ws=None) == E_WORKSPACE
    assert call(ws_bytes=ws_need - 1) == E_WORKSPACE
    assert call(ws=ctypes.c_void_p(FAKE + (4 << 20) + 16)) == E_WORKSPACE
    assert b"workspace" in lib.mao_last_error()


@needs_no_gpu
def test_batched_validation_codes():
    lib = mao.load()
    hp = mao.muon_hparams()
    W = (mao.Batch * 1)(mao.Batch(FAKE, 3, 8, 16, 16, 8 * 16, mao.BF16))
    G = (mao.Batch * 1)(mao.Batch(FAKE + (1 << 20), 3, 8, 16, 16, 8 * 16, mao.BF16))
    M = (mao.Batch * 1)(mao.Batch(FAKE + (2 << 20), 3, 8, 16, 16, 8 * 16, mao.F32))
    need = lib.muon_batched_workspace_size(1, W, ctypes.byref(hp))
    ws = ctypes.c_void_p(FAKE + (4 << 20))
    assert lib.muon_step_batched(0, W, G, M, ctypes.byref(hp), ws, need, None, None) == E_SHAPE
    assert lib.muon_step_batched(9, W, G, M, ctypes.byref(hp), ws, need, None, None) == E_SHAPE
    Wbad = (mao.Batch * 1)(mao.Batch(FAKE, 3, 8, 16, 16, 100, mao.BF16))  # stride < rows*ld
    assert lib.muon_step_batched(1, Wbad, G, M, ctypes.byref(hp), ws, need, None, None) == E_LAYOUT
    Mbad = (mao.Batch * 1)(mao.Batch(FAKE + (2 << 20), 2, 8, 16, 16, 8 * 16, mao.F32))
    assert lib.muon_step_batched(1, W, G, Mbad, ctypes.byref(hp), ws, need, None, None) == E_SHAPE


def _alias_verdict(lib, views):
    """muon_step_batched on bf16 W views (count, rows, cols, ld, stride, offset
    in elements), each group's G and M far away, with no workspace: E_ALIAS if
    the W views are judged to overlap, else E_WORKSPACE (validation passed)."""
    hp = mao.muon_hparams()
    n = len(views)
    Ws = (mao.Batch * n)(*[mao.Batch(FAKE + 2 * off, c, r, k, ld, st, mao.BF16)
                           for c, r, k, ld, st, off in views])
    Gs = (mao.Batch * n)(*[mao.Batch(FAKE + ((8 + i) << 24), c, r, k, ld, st, mao.BF16)
                           for i, (c, r, k, ld, st, off) in enumerate(views)])
    Ms = (mao.Batch * n)(*[mao.Batch(FAKE + ((16 + i) << 24), c, r, k, ld, st, mao.F32)
                           for i, (c, r, k, ld, st, off) in enumerate(views)])
    return lib.muon_step_batched(n, Ws, Gs, Ms, ctypes.byref(hp), None, 0, None, None)


@needs_no_gpu
def test_fused_column_views_are_not_aliases():
    """Logical Q, K, V matrices as column views of one fused buffer (three
    layers, leading dimension = the fused width) pass the alias check; a view
    that takes one column of its neighbour does not."""
    lib = mao.load()
    width, rows, layers = 40, 8, 3
    st = rows * width
    q, k, v = (layers, rows, 16, width, st, 0), (layers, rows, 8, width, st, 16), \
        (layers, rows, 8, width, st, 24)
    assert _alias_verdict(lib, [q, k, v]) == E_WORKSPACE
    assert _alias_verdict(lib, [q, (layers, rows, 9, width, st, 16), (layers, rows, 8, width, st, 32)]) \
        == E_WORKSPACE
    assert _alias_verdict(lib, [(layers, rows, 17, width, st, 0), k, v]) == E_ALIAS
    assert _alias_verdict(lib, [q, (layers, rows, 8, width, st, 8), v]) == E_ALIAS


@needs_no_gpu
def test_alias_check_against_brute_force():
    """Random pairs of strided bf16 views: the library never passes a pair that
    shares a byte, and decides exactly when both views have the same pitch and
    a batch stride that is a multiple of it (brute force over the bytes)."""
    lib = mao.load()
    r = np.random.default_rng(7)
    exact_cases = 0
    for _ in range(400):
        views = []
        for _ in range(2):
            ld = 8 * int(r.integers(1, 5))
            cols = int(r.integers(1, ld + 1))
            rows = int(r.integers(1, 4))
            count = int(r.integers(1, 3))
            stride = rows * ld + 8 * int(r.integers(0, 3)) if count > 1 else 0
            off = 8 * int(r.integers(0, 12))
            views.append((count, rows, cols, ld, stride, off))
        touched = []
        for c, rr, k, ld, st, off in views:
            s = set()
            for b in range(c):
                for i in range(rr):
                    e0 = off + b * st + i * ld
                    s.update(range(2 * e0, 2 * (e0 + k)))
            touched.append(s)
        shares = bool(touched[0] & touched[1])
        got = _alias_verdict(lib, views)
        assert got in (E_ALIAS, E_WORKSPACE)
        if shares:
            assert got == E_ALIAS, views
        periodic = all(c == 1 or st % ld == 0 for c, rr, k, ld, st, off in views)
        if periodic and views[0][3] == views[1][3]:
            exact_cases += 1
            assert (got == E_ALIAS) == shares, views
    assert exact_cases > 50


@needs_no_gpu
def test_soap_foam_adamw_qr_gemm_validation_codes():
    lib = mao.load()
    m, n = 8, 16
    sh = mao.soap_hparams()
    st = mao.SoapStateC(_mat(FAKE + (1 << 20), m, n, n), _mat(FAKE + (2 << 20), m, n, n),
                        _mat(FAKE + (3 << 20), m, m, 8), _mat(FAKE + (4 << 20), n, n, n),
                        _mat(FAKE + (5 << 20), m, m, 8), _mat(FAKE + (6 << 20), n, n, n))
    W = _mat(FAKE, m, n, n)
    G = _mat(FAKE + (7 << 20), m, n, n)
    need = lib.soap_workspace_size(m, n, ctypes.byref(sh))
    ws = ctypes.c_void_p(FAKE + (16 << 20))
    assert lib.soap_step(W, G, None, 1, ctypes.byref(sh), ws, need, None, None) == E_NULL
    assert lib.soap_step(W, G, ctypes.byref(st), 0, ctypes.byref(sh), ws, need, None, None) == E_HPARAM
    bad = mao.SoapStateC(st.M, st.V, _mat(FAKE + (3 << 20), n, n, n), st.R, st.QL, st.QR)
    assert lib.soap_step(W, G, ctypes.byref(bad), 1, ctypes.byref(sh), ws, need, None, None) == E_SHAPE
    assert lib.soap_step(W, G, ctypes.byref(st), 1, ctypes.byref(mao.soap_hparams(beta2=1.0)), ws,
                         need, None, None) == E_HPARAM
    assert lib.soap_step(W, G, ctypes.byref(st), 1, ctypes.byref(sh), ws, need - 1, None,
                         None) == E_WORKSPACE

    fh = mao.foam_hparams()
    fst = mao.FoamStateC(_mat(FAKE + (1 << 20), m, n, n), _mat(FAKE + (4 << 20), n, n, n),
                         _mat(FAKE + (6 << 20), n, n, n), FAKE + (8 << 20), FAKE + (9 << 20),
                         FAKE + (10 << 20))
    fneed = lib.foam_workspace_size(m, n, ctypes.byref(fh))
    assert lib.foam_step(W, G, ctypes.byref(fst), 1, ctypes.byref(mao.foam_hparams(pf=0)), ws,
                         fneed, None, None) == E_HPARAM
    fst2 = mao.FoamStateC(fst.M, fst.R, fst.QR, None, fst.c, fst.aux)
    assert lib.foam_step(W, G, ctypes.byref(fst2), 1, ctypes.byref(fh), ws, fneed, None,
                         None) == E_NULL
    assert lib.foam_step(W, G, ctypes.byref(fst), 1, ctypes.byref(mao.foam_hparams(refresh=2)),
                         ws, 1 << 30, None, None) == E_HPARAM
    assert lib.foam_step(W, G, ctypes.byref(fst), 1,
                         ctypes.byref(mao.foam_hparams(back_rot_dtype=5)), ws, 1 << 30, None,
                         None) == E_DTYPE
    assert lib.soap_step(W, G, ctypes.byref(st), 1, ctypes.byref(mao.soap_hparams(back_rot_dtype=7)),
                         ws, 1 << 30, None, None) == E_DTYPE
    assert lib.soap_step(W, G, ctypes.byref(st), 1, ctypes.byref(mao.soap_hparams(fwd_rot=2)),
                         ws, 1 << 30, None, None) == E_HPARAM
    assert lib.foam_step(W, G, ctypes.byref(fst), 1, ctypes.byref(mao.foam_hparams(fwd_rot=-1)),
                         ws, 1 << 30, None, None) == E_HPARAM
    assert lib.soap_step(W, G, ctypes.byref(st), 1, ctypes.byref(mao.soap_hparams(refresh_prod=3)),
                         ws, 1 << 30, None, None) == E_HPARAM
    assert lib.foam_step(W, G, ctypes.byref(fst), 1,
                         ctypes.byref(mao.foam_hparams(refresh_prod=-2)), ws, 1 << 30, None,
                         None) == E_HPARAM
    # bf16x3 criterion products feed only the QR refresh
    assert lib.foam_step(W, G, ctypes.byref(fst), 1,
                         ctypes.byref(mao.foam_hparams(refresh="eigh", refresh_prod="bf16x3")),
                         ws, 1 << 30, None, None) == E_UNSUPPORTED
    # the split operands of the bf16x3 products take workspace of their own
    for f in ("soap_workspace_size", "foam_workspace_size"):
        hp_of = mao.soap_hparams if f.startswith("soap") else mao.foam_hparams
        base = getattr(lib, f)(m, n, ctypes.byref(hp_of()))
        for kw in ({"fwd_rot": "bf16x3"}, {"refresh_prod": "bf16x3"}):
            assert getattr(lib, f)(m, n, ctypes.byref(hp_of(**kw))) > base
    assert lib.foam_step(W, G, ctypes.byref(fst), 1, ctypes.byref(mao.foam_hparams(side=2)), ws,
                         fneed, None, None) == E_HPARAM
    # the output side keeps m x m factors: the n x n state is the wrong shape
    fo = mao.foam_hparams(side="output")
    oneed = lib.foam_workspace_size(m, n, ctypes.byref(fo))
    assert oneed > 0
    assert lib.foam_step(W, G, ctypes.byref(fst), 1, ctypes.byref(fo), ws, oneed, None,
                         None) == E_SHAPE
    fso = mao.FoamStateC(fst.M, _mat(FAKE + (4 << 20), m, m, 8), _mat(FAKE + (6 << 20), m, m, 8),
                         fst.r, fst.c, fst.aux)
    assert lib.foam_step(W, G, ctypes.byref(fso), 1, ctypes.byref(fo), ws, oneed - 1, None,
                         None) == E_WORKSPACE
    assert lib.foam_step_many_workspace_size(1, ctypes.byref(W), ctypes.byref(fo)) > 0

    assert lib.adamw_step(FAKE, 0, FAKE + 4096, 0, FAKE + 8192, FAKE + 12288, 0, 1, 1e-3, 0.9,
                          0.95, 1e-8, 0.0, None, None) == E_SHAPE
    assert lib.adamw_step(FAKE, 0, FAKE + 64, 0, FAKE + 8192, FAKE + 12288, 100, 1, 1e-3, 0.9,
                          0.95, 1e-8, 0.0, None, None) == E_ALIAS
    assert lib.adamw_step(FAKE, 5, FAKE + 4096, 0, FAKE + 8192, FAKE + 12288, 100, 1, 1e-3, 0.9,
                          0.95, 1e-8, 0.0, None, None) == E_DTYPE

    assert lib.mao_qr(FAKE, 12, FAKE + (1 << 20), 16, 12, ws, 1 << 30, None) == E_LAYOUT
    assert lib.mao_qr(FAKE, 16, FAKE + 64, 16, 12, ws, 1 << 30, None) == E_ALIAS
    assert lib.mao_dbg_qr(FAKE, 16, FAKE + (1 << 20), 16, 12, ws, 1 << 30, 4, None) == E_HPARAM
    assert lib.mao_eigh_workspace_size(0) == 0 and lib.mao_eigh_workspace_size(16385) == 0
    assert lib.mao_eigh_workspace_size(300) > 0
    assert lib.mao_eigh(FAKE, 20000, FAKE + (1 << 34), 20000, None, None, 20000, ws, 1 << 30,
                        None) == 9  # above the eigensolver's 16384
    assert lib.mao_eigh(FAKE, 16, FAKE + 64, 16, None, None, 12, ws, 1 << 30, None) == E_ALIAS
    assert lib.mao_eigh(FAKE, 16, FAKE + (1 << 20), 16, None, None, 12, ws, 16, None) == E_WORKSPACE
    assert lib.mao_dbg_qr(FAKE, 16, FAKE + 64, 16, 12, ws, 1 << 30, 1, None) == E_ALIAS
    assert lib.mao_gemm_nt(4, 4, 4, 1.0, FAKE, 8, FAKE + 4096, 8, 1, 0.0, None, 0, FAKE + 8192, 8,
                           1, None) == E_SHAPE  # symmetric needs A == B
    assert lib.mao_gemm_nt(4, 4, 0, 1.0, FAKE, 8, FAKE, 8, 1, 0.0, None, 0, FAKE + 8192, 8, 0,
                           None) == E_SHAPE
    assert lib.mao_gemm_nt(4, 4, 4, 1.0, FAKE, 8, FAKE + 4096, 8, 1, 0.0, None, 0, FAKE + 8192, 8,
                           4, None) == E_HPARAM  # unknown mode bit
    assert lib.mao_gemm_nt(4, 4, 4, 1.0, FAKE, 8, FAKE, 8, 1, 0.0, None, 0, FAKE + 8192, 8, 3,
                           None) == 9  # symmetric with a K x N B: unsupported
    assert lib.mao_gemm_nt(4, 4, 4, 1.0, FAKE, 8, FAKE + 4096, 8, 0, 0.0, None, 0, FAKE + 8192, 8,
                           2, None) == 9  # K x N B needs bf16
    assert lib.mao_gemm_nt(4, 12, 4, 1.0, FAKE, 8, FAKE + 4096, 8, 1, 0.0, None, 0, FAKE + 8192,
                           16, 2, None) == 4  # K x N B: ldb < N


def test_noalloc_limits_checked_before_any_hip_call():
    """muon_step_noalloc rejects a step that does not fit its static scratch
    array, and a NULL hp, before it touches the device."""
    lib = mao.load()
    assert lib.muon_step_noalloc_max_bytes() == 64 << 20
    hp = mao.muon_hparams(ns_dtype="bf16")
    big = _mat(FAKE, 4096, 4096, 4096, mao.BF16)
    m = _mat(FAKE + (1 << 30), 4096, 4096, 4096)
    assert lib.muon_step_noalloc(big, big, m, ctypes.byref(hp), None, None) == E_WORKSPACE
    assert b"static array" in lib.mao_last_error()
    assert lib.muon_step_noalloc(big, big, m, None, None, None) == E_NULL


@needs_no_gpu
def test_many_matrix_validation_codes():
    lib = mao.load()
    m, n = 8, 16
    sh = mao.soap_hparams()
    fh = mao.foam_hparams()

    def soap_st(base):
        return mao.SoapStateC(_mat(base + (1 << 20), m, n, n), _mat(base + (2 << 20), m, n, n),
                              _mat(base + (3 << 20), m, m, 8), _mat(base + (4 << 20), n, n, n),
                              _mat(base + (5 << 20), m, m, 8), _mat(base + (6 << 20), n, n, n))

    b0, b1 = FAKE, FAKE + (64 << 20)
    W = (mao.Mat * 2)(_mat(b0, m, n, n), _mat(b1, m, n, n))
    G = (mao.Mat * 2)(_mat(b0 + (7 << 20), m, n, n), _mat(b1 + (7 << 20), m, n, n))
    S = (mao.SoapStateC * 2)(soap_st(b0), soap_st(b1))
    need = lib.soap_step_many_workspace_size(2, W, ctypes.byref(sh))
    assert need > lib.soap_workspace_size(m, n, ctypes.byref(sh))
    assert lib.soap_step_many_workspace_size(0, W, ctypes.byref(sh)) == 0
    ws = ctypes.c_void_p(FAKE + (1 << 30))
    assert lib.soap_step_many(0, W, G, S, 1, ctypes.byref(sh), ws, need, None, None) == E_SHAPE
    assert lib.soap_step_many(2, None, G, S, 1, ctypes.byref(sh), ws, need, None, None) == E_NULL
    assert lib.soap_step_many(2, W, G, S, 1, ctypes.byref(sh), ws, need - 1, None,
                              None) == E_WORKSPACE
    # the second matrix's momentum on the first one's weights
    S2 = (mao.SoapStateC * 2)(soap_st(b0), soap_st(b1))
    S2[1].M = _mat(b0, m, n, n)
    assert lib.soap_step_many(2, W, G, S2, 1, ctypes.byref(sh), ws, need, None, None) == E_ALIAS
    # a shape error in the second matrix
    S3 = (mao.SoapStateC * 2)(soap_st(b0), soap_st(b1))
    S3[1].L = _mat(b1 + (3 << 20), n, n, n)
    assert lib.soap_step_many(2, W, G, S3, 1, ctypes.byref(sh), ws, need, None, None) == E_SHAPE

    def foam_st(base):
        return mao.FoamStateC(_mat(base + (1 << 20), m, n, n), _mat(base + (4 << 20), n, n, n),
                              _mat(base + (6 << 20), n, n, n), base + (8 << 20), base + (9 << 20),
                              base + (10 << 20))

    F = (mao.FoamStateC * 2)(foam_st(b0), foam_st(b1))
    fneed = lib.foam_step_many_workspace_size(2, W, ctypes.byref(fh))
    assert fneed > lib.foam_workspace_size(m, n, ctypes.byref(fh))
    assert lib.foam_step_many(2, W, G, F, 1, ctypes.byref(mao.foam_hparams(pf=0)), ws, fneed,
                              None, None) == E_HPARAM
    F2 = (mao.FoamStateC * 2)(foam_st(b0), foam_st(b1))
    F2[0].r = None
    assert lib.foam_step_many(2, W, G, F2, 1, ctypes.byref(fh), ws, fneed, None, None) == E_NULL
    assert lib.foam_step_many(4097, W, G, F, 1, ctypes.byref(fh), ws, fneed, None,
                              None) == E_SHAPE


@needs_no_gpu
def test_observability_validation_codes():
    lib = mao.load()
    X = mao.Batch(FAKE, 2, 8, 16, 16, 8 * 16, mao.F32)
    ws = ctypes.c_void_p(FAKE + (16 << 20))
    out = ctypes.c_void_p(FAKE + (8 << 20))
    need = lib.mao_matrix_rms_workspace_size(X)
    assert need > 0
    assert lib.mao_matrix_rms(X, None, ws, need, None) == E_NULL
    assert lib.mao_matrix_rms(X, ctypes.c_void_p(FAKE + 8), ws, need, None) == E_ALIAS
    assert lib.mao_matrix_rms(mao.Batch(FAKE, 70000, 1, 8, 8, 8, mao.F32), out, ws, 1 << 30,
                              None) == E_SHAPE
    assert lib.mao_matrix_rms(X, out, ws, need - 1, None) == E_WORKSPACE

    rneed = lib.mao_ns_residual_workspace_size(X)
    assert rneed > 0
    assert lib.mao_ns_residual(mao.Batch(FAKE, 2, 8, 16, 16, 8 * 16, mao.BF16), 1.0, out, ws,
                               rneed, None) == E_DTYPE
    assert lib.mao_ns_residual(X, 0.0, out, ws, rneed, None) == E_HPARAM
    assert lib.mao_ns_residual(X, float("inf"), out, ws, rneed, None) == E_HPARAM
    assert lib.mao_ns_residual(X, 1.0, out, None, rneed, None) == E_WORKSPACE

    F = _mat(FAKE, 16, 16, 16)
    Q = _mat(FAKE + (1 << 20), 16, 16, 16)
    kneed = lib.mao_rayleigh_workspace_size(16)
    assert lib.mao_rayleigh(F, _mat(FAKE + (1 << 20), 16, 8, 8), out, None, ws, kneed, None) == E_SHAPE
    assert lib.mao_rayleigh(F, Q, None, None, ws, kneed, None) == E_NULL
    assert lib.mao_rayleigh(F, _mat(FAKE + 64, 16, 16, 16), out, None, ws, kneed, None) == E_ALIAS
    assert lib.mao_rayleigh(F, Q, out, ctypes.c_void_p(FAKE + (8 << 20) + 4), ws, kneed,
                            None) == E_ALIAS
    assert lib.mao_rayleigh(_mat(FAKE, 16, 16, 16, mao.BF16), Q, out, None, ws, kneed,
                            None) == E_DTYPE

    V = _mat(FAKE, 8, 16, 16)
    sneed = lib.mao_rank1_share_workspace_size(8, 16)
    assert sneed > 0
    assert lib.mao_rank1_share(V, 0, out, ws, sneed, None) == E_HPARAM
    assert lib.mao_rank1_share(V, 1001, out, ws, sneed, None) == E_HPARAM
    assert lib.mao_rank1_share(V, 10, None, ws, sneed, None) == E_NULL
    assert lib.mao_rank1_share(V, 10, out, ws, sneed - 1, None) == E_WORKSPACE

    assert lib.mao_basis_age(None, out, None) == E_NULL
    assert lib.mao_basis_age(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 12), None) == E_ALIAS
    assert lib.mao_basis_age(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 2), None) == E_LAYOUT
