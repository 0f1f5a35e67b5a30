"""Matrix-aware optimizer steps (Muon, Muon+, SOAP, FOAM, AdamW) on AMD MI355X.

Thin ctypes binding over ``libmao.so`` (declared in ``include/mao.h``). The
binding only marshals arguments: every step runs in the library's HIP
kernels, on the current torch stream. PyTorch provides device memory and
streams; the library itself allocates nothing, so the workspace is a torch
byte tensor allocated here and cached per device.

If the library is missing, every call raises -- there is no CPU fallback.
Build it with ``python -m matrix_aware_optimizers_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmao.so")

F32, BF16 = 0, 1
NORM_MODES = {"none": 0, "row": 1, "col": 2, "col_row": 3, "row_col": 4}
MAX_GROUPS = 8


class MaoError(RuntimeError):
    """A libmao entry point returned a non-OK status."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: status {status} ({detail})")
        self.status = status


class Mat(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("rows", c_int64), ("cols", c_int64), ("ld", c_int64),
                ("dtype", c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("count", c_int64), ("rows", c_int64), ("cols", c_int64),
                ("ld", c_int64), ("stride", c_int64), ("dtype", c_int32)]


class MuonHparams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("mu", c_float), ("weight_decay", c_float), ("eps", c_float),
                ("ns_steps", c_int32), ("ns_coeffs", POINTER(c_float)), ("ns_dtype", c_int32),
                ("norm_mode", c_int32), ("norm_eps", c_float)]


class SoapHparams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("refresh_every", c_int32),
                ("back_rot_dtype", c_int32), ("fwd_rot", c_int32), ("refresh_prod", c_int32)]


class SoapStateC(ctypes.Structure):
    _fields_ = [("M", Mat), ("V", Mat), ("L", Mat), ("R", Mat), ("QL", Mat), ("QR", Mat)]


class FoamHparams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("pf", c_int32), ("tol", c_float), ("side", c_int32),
                ("refresh", c_int32), ("back_rot_dtype", c_int32), ("fwd_rot", c_int32),
                ("refresh_prod", c_int32)]


REFRESH_MODES = {"qr": 0, "eigh": 1}
ROT_MODES = {"f32": 0, "bf16x3": 1}
EIGH_MAX_SWEEPS = 12


def _rot_code(mode):
    return ROT_MODES[mode] if isinstance(mode, str) else int(mode)


class FoamStateC(ctypes.Structure):
    _fields_ = [("M", Mat), ("R", Mat), ("QR", Mat), ("r", c_void_p), ("c", c_void_p),
                ("aux", c_void_p)]


EXPORTS = {
    "muon_workspace_size": (c_size_t, [c_int64, c_int64, POINTER(MuonHparams)]),
    "muon_step": (c_int32, [Mat, Mat, Mat, POINTER(MuonHparams), c_void_p, c_size_t, c_void_p,
                            c_void_p]),
    "muon_step_noalloc_max_bytes": (c_size_t, []),
    "muon_step_noalloc": (c_int32, [Mat, Mat, Mat, POINTER(MuonHparams), c_void_p, c_void_p]),
    "muon_batched_workspace_size": (c_size_t, [c_int32, POINTER(Batch), POINTER(MuonHparams)]),
    "muon_step_batched": (c_int32, [c_int32, POINTER(Batch), POINTER(Batch), POINTER(Batch),
                                    POINTER(MuonHparams), c_void_p, c_size_t, POINTER(Batch),
                                    c_void_p]),
    "soap_workspace_size": (c_size_t, [c_int64, c_int64, POINTER(SoapHparams)]),
    "soap_step": (c_int32, [Mat, Mat, POINTER(SoapStateC), c_int64, POINTER(SoapHparams),
                            c_void_p, c_size_t, c_void_p, c_void_p]),
    "foam_workspace_size": (c_size_t, [c_int64, c_int64, POINTER(FoamHparams)]),
    "foam_step": (c_int32, [Mat, Mat, POINTER(FoamStateC), c_int64, POINTER(FoamHparams),
                            c_void_p, c_size_t, c_void_p, c_void_p]),
    "soap_step_many_workspace_size": (c_size_t, [c_int32, POINTER(Mat), POINTER(SoapHparams)]),
    "foam_step_many_workspace_size": (c_size_t, [c_int32, POINTER(Mat), POINTER(FoamHparams)]),
    "soap_step_many": (c_int32, [c_int32, POINTER(Mat), POINTER(Mat), POINTER(SoapStateC), c_int64,
                                 POINTER(SoapHparams), c_void_p, c_size_t,
                                 POINTER(c_void_p), c_void_p]),
    "foam_step_many": (c_int32, [c_int32, POINTER(Mat), POINTER(Mat), POINTER(FoamStateC), c_int64,
                                 POINTER(FoamHparams), c_void_p, c_size_t,
                                 POINTER(c_void_p), c_void_p]),
    "adamw_step": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_int64,
                             c_int64, c_float, c_float, c_float, c_float, c_float, c_void_p,
                             c_void_p]),
    "mao_gemm_nt": (c_int32, [c_int64, c_int64, c_int64, c_float, c_void_p, c_int64, c_void_p,
                              c_int64, c_int32, c_float, c_void_p, c_int64, c_void_p, c_int64,
                              c_int32, c_void_p]),
    "mao_eigh_workspace_size": (c_size_t, [c_int64]),
    "mao_eigh": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                           c_void_p, c_size_t, c_void_p]),
    "mao_qr_workspace_size": (c_size_t, [c_int64]),
    "mao_qr": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_int64, c_void_p, c_size_t,
                         c_void_p]),
    "mao_dbg_qr": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_int64, c_void_p, c_size_t,
                             c_int32, c_void_p]),
    "mao_matrix_rms_workspace_size": (c_size_t, [Batch]),
    "mao_matrix_rms": (c_int32, [Batch, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mao_ns_residual_workspace_size": (c_size_t, [Batch]),
    "mao_ns_residual": (c_int32, [Batch, c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mao_rayleigh_workspace_size": (c_size_t, [c_int64]),
    "mao_rayleigh": (c_int32, [Mat, Mat, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mao_rank1_share_workspace_size": (c_size_t, [c_int64, c_int64]),
    "mao_rank1_share": (c_int32, [Mat, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mao_basis_age": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "mao_timing_enable": (None, [c_int32]),
    "mao_timing_collect": (c_int32, [POINTER(ctypes.c_double), POINTER(c_int64),
                                     POINTER(ctypes.c_double), c_int32]),
    "mao_status_string": (ctypes.c_char_p, [c_int32]),
    "mao_last_error": (ctypes.c_char_p, []),
    "mao_abi_version": (c_int32, []),
}

_lib = None


def load(path: str | None = None):
    """Load libmao.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    # torch first: its bundled HIP runtime has the soname the library needs,
    # so both then share one runtime. Loaded the other way round, the system
    # runtime comes first and the library's launches fail ("no ROCm-capable
    # device") once torch has initialised the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m matrix_aware_optimizers_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, name: str):
    if status != 0:
        lib = load()
        detail = lib.mao_status_string(status).decode() + ": " + lib.mao_last_error().decode()
        raise MaoError(status, name, detail)


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def mat(t) -> Mat:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D row-major tensor (unit column stride)")
    return Mat(t.data_ptr(), t.shape[0], t.shape[1], t.stride(0), dtype_code(t))


def batch(t) -> Batch:
    if t.dim() == 2:
        t = t.unsqueeze(0)
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected a 3-D [count, rows, cols] tensor with unit column stride")
    return Batch(t.data_ptr(), t.shape[0], t.shape[1], t.shape[2], t.stride(1), t.stride(0),
                 dtype_code(t))


def _stream():
    torch = _torch()
    return c_void_p(torch.cuda.current_stream().cuda_stream)


_ws_cache: dict = {}


def workspace(nbytes: int, device):
    """A cached byte buffer of at least ``nbytes`` on ``device`` (256-aligned)."""
    torch = _torch()
    key = str(device)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def padded(t):
    """``t`` itself if its rows already meet the library's layout rule (unit
    column stride, leading dimension a multiple of 8, 16-byte aligned), else a
    copy into such storage (returned as a view of the original shape)."""
    torch = _torch()
    if t.dim() == 2 and t.stride(1) == 1 and t.stride(0) % 8 == 0 and t.data_ptr() % 16 == 0:
        return t
    rows, cols = t.shape
    ld = (cols + 7) // 8 * 8
    buf = torch.zeros((rows, ld), dtype=t.dtype, device=t.device)
    view = buf[:, :cols]
    view.copy_(t)
    return view


def empty_matrix(rows, cols, dtype=None, device=None):
    """An uninitialised row-major matrix whose rows meet the layout rule."""
    torch = _torch()
    ld = (cols + 7) // 8 * 8
    buf = torch.empty((rows, ld), dtype=dtype or torch.float32, device=device)
    return buf[:, :cols]


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def muon_hparams(lr=0.0, mu=0.95, weight_decay=0.0, eps=1e-7, ns_steps=5, ns_coeffs=None,
                 ns_dtype="bf16", norm_mode="none", norm_eps=1e-7):
    hp = MuonHparams()
    hp.lr, hp.mu, hp.weight_decay, hp.eps = lr, mu, weight_decay, eps
    hp.ns_steps = ns_steps
    if ns_coeffs is not None:
        flat = [float(x) for row in ns_coeffs for x in row]
        if len(flat) != 3 * ns_steps:
            raise ValueError("ns_coeffs must hold ns_steps rows of (a, b, c)")
        arr = (c_float * len(flat))(*flat)
        hp.ns_coeffs = ctypes.cast(arr, POINTER(c_float))
        hp._keep = arr
    else:
        hp.ns_coeffs = None
    hp.ns_dtype = {"bf16": BF16, "f32": F32, "fp32": F32}[ns_dtype]
    hp.norm_mode = NORM_MODES[norm_mode]
    hp.norm_eps = norm_eps
    return hp


def muon_step(W, G, M, *, update_out=None, ws=None, **hp_kw):
    """One Muon(+) step on one matrix, in place on W and M."""
    lib = load()
    hp = muon_hparams(**hp_kw)
    need = lib.muon_workspace_size(W.shape[0], W.shape[1], ctypes.byref(hp))
    buf = ws if ws is not None else workspace(need, W.device)
    _check(lib.muon_step(mat(W), mat(G), mat(M), ctypes.byref(hp), _ptr(buf), buf.numel(),
                         _ptr(update_out), _stream()), "muon_step")


def muon_step_noalloc(W, G, M, *, update_out=None, **hp_kw):
    """muon_step without a workspace: the library's static scratch array
    serves instead (no allocation here or in the library)."""
    lib = load()
    hp = muon_hparams(**hp_kw)
    _check(lib.muon_step_noalloc(mat(W), mat(G), mat(M), ctypes.byref(hp), _ptr(update_out),
                                 _stream()), "muon_step_noalloc")


def muon_step_batched(groups, *, update_out=None, ws=None, **hp_kw):
    """Muon(+) on groups of same-shape matrices. ``groups`` is a list of
    (W, G, M) 3-D tensors [count, rows, cols]; ``update_out`` an optional list
    of fp32 tensors of the same shapes."""
    lib = load()
    hp = muon_hparams(**hp_kw)
    ng = len(groups)
    Ws = (Batch * ng)(*[batch(g[0]) for g in groups])
    Gs = (Batch * ng)(*[batch(g[1]) for g in groups])
    Ms = (Batch * ng)(*[batch(g[2]) for g in groups])
    outs = None
    if update_out is not None:
        outs = (Batch * ng)(*[batch(o) for o in update_out])
    need = lib.muon_batched_workspace_size(ng, Ws, ctypes.byref(hp))
    buf = ws if ws is not None else workspace(need, groups[0][0].device)
    _check(lib.muon_step_batched(ng, Ws, Gs, Ms, ctypes.byref(hp), _ptr(buf), buf.numel(), outs,
                                 _stream()), "muon_step_batched")


def _dtype_code(d):
    return {"f32": F32, "bf16": BF16}[d] if isinstance(d, str) else int(d)


def soap_hparams(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, refresh_every=1,
                 back_rot_dtype="f32", fwd_rot="f32", refresh_prod="f32"):
    hp = SoapHparams()
    hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay = lr, beta1, beta2, eps, weight_decay
    hp.refresh_every = refresh_every
    hp.back_rot_dtype = _dtype_code(back_rot_dtype)
    hp.fwd_rot = _rot_code(fwd_rot)
    hp.refresh_prod = _rot_code(refresh_prod)
    return hp


def soap_state(M, V, L, R, QL, QR) -> SoapStateC:
    return SoapStateC(mat(M), mat(V), mat(L), mat(R), mat(QL), mat(QR))


def soap_step(W, G, state: dict, t: int, *, update_out=None, ws=None, **hp_kw):
    """One SOAP step; ``state`` holds fp32 tensors M, V, L, R, QL, QR."""
    lib = load()
    hp = soap_hparams(**hp_kw)
    st = soap_state(state["M"], state["V"], state["L"], state["R"], state["QL"], state["QR"])
    need = lib.soap_workspace_size(W.shape[0], W.shape[1], ctypes.byref(hp))
    buf = ws if ws is not None else workspace(need, W.device)
    _check(lib.soap_step(mat(W), mat(G), ctypes.byref(st), t, ctypes.byref(hp), _ptr(buf),
                         buf.numel(), _ptr(update_out), _stream()), "soap_step")


FOAM_SIDES = {"input": 0, "output": 1}


def foam_hparams(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, pf=10, tol=0.1,
                 side="input", refresh="qr", back_rot_dtype="f32", fwd_rot="f32",
                 refresh_prod="f32"):
    hp = FoamHparams()
    hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay = lr, beta1, beta2, eps, weight_decay
    hp.pf, hp.tol = pf, tol
    hp.side = FOAM_SIDES[side] if isinstance(side, str) else int(side)
    hp.refresh = REFRESH_MODES[refresh] if isinstance(refresh, str) else int(refresh)
    hp.back_rot_dtype = _dtype_code(back_rot_dtype)
    hp.fwd_rot = _rot_code(fwd_rot)
    hp.refresh_prod = _rot_code(refresh_prod)
    return hp


def foam_step(W, G, state: dict, t: int, *, update_out=None, ws=None, **hp_kw):
    """One FOAM step; ``state`` holds fp32 tensors M, R, QR, r, c, aux (4)."""
    lib = load()
    hp = foam_hparams(**hp_kw)
    st = FoamStateC(mat(state["M"]), mat(state["R"]), mat(state["QR"]), state["r"].data_ptr(),
                    state["c"].data_ptr(), state["aux"].data_ptr())
    need = lib.foam_workspace_size(W.shape[0], W.shape[1], ctypes.byref(hp))
    buf = ws if ws is not None else workspace(need, W.device)
    _check(lib.foam_step(mat(W), mat(G), ctypes.byref(st), t, ctypes.byref(hp), _ptr(buf),
                         buf.numel(), _ptr(update_out), _stream()), "foam_step")


def _many_args(items, update_out):
    n = len(items)
    Ws = (Mat * n)(*[mat(it[0]) for it in items])
    Gs = (Mat * n)(*[mat(it[1]) for it in items])
    outs = None
    if update_out is not None:
        outs = (c_void_p * n)(*[None if o is None else o.data_ptr() for o in update_out])
    return n, Ws, Gs, outs


def soap_step_many(items, t: int, *, update_out=None, ws=None, **hp_kw):
    """SOAP on several matrices in one call: ``items`` is a list of
    (W, G, state dict) as for soap_step; equal-size QR refreshes run batched."""
    lib = load()
    hp = soap_hparams(**hp_kw)
    n, Ws, Gs, outs = _many_args(items, update_out)
    sts = (SoapStateC * n)(*[soap_state(st["M"], st["V"], st["L"], st["R"], st["QL"], st["QR"])
                             for _, _, st in items])
    need = lib.soap_step_many_workspace_size(n, Ws, ctypes.byref(hp))
    buf = ws if ws is not None else workspace(need, items[0][0].device)
    _check(lib.soap_step_many(n, Ws, Gs, sts, t, ctypes.byref(hp), _ptr(buf), buf.numel(), outs,
                              _stream()), "soap_step_many")


def foam_step_many(items, t: int, *, update_out=None, ws=None, **hp_kw):
    """FOAM on several matrices in one call: ``items`` is a list of
    (W, G, state dict) as for foam_step; equal-size QR refreshes run batched."""
    lib = load()
    hp = foam_hparams(**hp_kw)
    n, Ws, Gs, outs = _many_args(items, update_out)
    sts = (FoamStateC * n)(*[FoamStateC(mat(st["M"]), mat(st["R"]), mat(st["QR"]),
                                        st["r"].data_ptr(), st["c"].data_ptr(),
                                        st["aux"].data_ptr()) for _, _, st in items])
    need = lib.foam_step_many_workspace_size(n, Ws, ctypes.byref(hp))
    buf = ws if ws is not None else workspace(need, items[0][0].device)
    _check(lib.foam_step_many(n, Ws, Gs, sts, t, ctypes.byref(hp), _ptr(buf), buf.numel(), outs,
                              _stream()), "foam_step_many")


def adamw_step(w, g, m, v, t: int, *, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0,
               update_out=None):
    """Flat AdamW over all elements of contiguous w, g, m, v."""
    lib = load()
    for x in (w, g, m, v):
        if not x.is_contiguous():
            raise ValueError("adamw_step needs contiguous tensors")
    _check(lib.adamw_step(_ptr(w), dtype_code(w), _ptr(g), dtype_code(g), _ptr(m), _ptr(v),
                          w.numel(), t, lr, beta1, beta2, eps, weight_decay, _ptr(update_out),
                          _stream()), "adamw_step")


def _as_batch(X):
    return batch(X if X.dim() == 3 else X.unsqueeze(0))


def matrix_rms(X, out=None):
    """||X_b||_F / sqrt(rows * cols) per matrix of a 2-D or 3-D [count, rows,
    cols] tensor (fp32 or bf16), as a device fp32 tensor of count values."""
    import torch
    lib = load()
    bx = _as_batch(X)
    if out is None:
        out = torch.empty(bx.count, dtype=torch.float32, device=X.device)
    buf = workspace(lib.mao_matrix_rms_workspace_size(bx), X.device)
    _check(lib.mao_matrix_rms(bx, _ptr(out), _ptr(buf), buf.numel(), _stream()), "mao_matrix_rms")
    return out


def ns_residual(O, scale=1.0, out=None):
    """||X X^T - I||_F / sqrt(a) of X = scale * O on its wide orientation, per
    matrix of a 2-D or 3-D fp32 tensor (device fp32 tensor of count values)."""
    import torch
    lib = load()
    bo = _as_batch(O)
    if out is None:
        out = torch.empty(bo.count, dtype=torch.float32, device=O.device)
    buf = workspace(lib.mao_ns_residual_workspace_size(bo), O.device)
    _check(lib.mao_ns_residual(bo, scale, _ptr(out), _ptr(buf), buf.numel(), _stream()),
           "mao_ns_residual")
    return out


def rayleigh(F, Q):
    """(d, kappa): d_i = q_i^T F q_i for the columns of Q, kappa = max d / min d
    (device fp32 tensors)."""
    import torch
    lib = load()
    n = F.shape[0]
    d = torch.empty(n, dtype=torch.float32, device=F.device)
    kappa = torch.empty(1, dtype=torch.float32, device=F.device)
    buf = workspace(lib.mao_rayleigh_workspace_size(n), F.device)
    _check(lib.mao_rayleigh(mat(F), mat(Q), _ptr(d), _ptr(kappa), _ptr(buf), buf.numel(),
                            _stream()), "mao_rayleigh")
    return d, kappa


def rank1_share(V, iters=30):
    """s_1(V)^2 / ||V||_F^2 by power iteration (device fp32 tensor of 1 value)."""
    import torch
    lib = load()
    out = torch.empty(1, dtype=torch.float32, device=V.device)
    buf = workspace(lib.mao_rank1_share_workspace_size(V.shape[0], V.shape[1]), V.device)
    _check(lib.mao_rank1_share(mat(V), iters, _ptr(out), _ptr(buf), buf.numel(), _stream()),
           "mao_rank1_share")
    return out


def basis_age(aux, age):
    """age <- 0 if the FOAM step that wrote aux refreshed its basis, else age + 1."""
    _check(load().mao_basis_age(_ptr(aux), _ptr(age), _stream()), "mao_basis_age")


TIMING_TAGS = ("ns_gram", "ns_square", "ns_apply", "other", "qr", "other_bf16", "qr_proj",
               "qr_fused", "qr_panel", "gated", "elementwise")


def timing_enable(on: bool = True):
    """Bracket every contraction launch with HIP events (benchmarking only)."""
    load().mao_timing_enable(1 if on else 0)


def timing_collect() -> dict:
    """{tag: (total_ms, launches, algorithmic_flops)} since the last collect
    (for "elementwise": algorithmic bytes in place of flops)."""
    n = len(TIMING_TAGS)
    ms = (ctypes.c_double * n)()
    cnt = (c_int64 * n)()
    fl = (ctypes.c_double * n)()
    load().mao_timing_collect(ms, cnt, fl, n)
    return {TIMING_TAGS[i]: (ms[i], cnt[i], fl[i]) for i in range(n)}


def gemm_nt(A, B, *, alpha=1.0, beta=0.0, C0=None, out=None, symmetric=False, b_kmajor=False):
    """D = alpha A B^T + beta C0 through the library's MFMA kernel (fp32 out).
    With ``b_kmajor`` B is K x N and D = alpha A B + beta C0 (bf16 only)."""
    lib = load()
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    same = A.data_ptr() == B.data_ptr() and A.shape == B.shape and A.stride() == B.stride()
    A = padded(A)
    B = A if (symmetric and same) else padded(B)
    if C0 is not None:
        C0 = padded(C0)
    n = B.shape[1] if b_kmajor else B.shape[0]
    if out is None:
        out = empty_matrix(A.shape[0], n, device=A.device)
    mode = (1 if symmetric else 0) | (2 if b_kmajor else 0)
    _check(lib.mao_gemm_nt(A.shape[0], n, A.shape[1], alpha, _ptr(A), A.stride(0),
                           _ptr(B), B.stride(0), dtype_code(A), beta, _ptr(C0),
                           C0.stride(0) if C0 is not None else 0, _ptr(out), out.stride(0),
                           mode, _stream()), "mao_gemm_nt")
    return out


def eigh(F, out=None, evals=None, info=None):
    """Eigenvectors (columns, by descending eigenvalue) of symmetric fp32 F;
    ``evals`` / ``info`` optional fp32 device tensors of n and 13 entries."""
    lib = load()
    n = F.shape[0]
    F = padded(F)
    if out is None:
        out = empty_matrix(n, n, device=F.device)
    need = lib.mao_eigh_workspace_size(n)
    buf = workspace(need, F.device)
    _check(lib.mao_eigh(_ptr(F), F.stride(0), _ptr(out), out.stride(0), _ptr(evals), _ptr(info),
                        n, _ptr(buf), buf.numel(), _stream()), "mao_eigh")
    return out


DBG_QR_ABORT_BARRIERS = 1
DBG_QR_NO_FALLBACK = 2


def qr(P, out=None, dbg_flags: int = 0):
    """Q of the Householder QR of square fp32 P with diag(R) >= 0.
    ``dbg_flags`` (tests only) goes to mao_dbg_qr: DBG_QR_ABORT_BARRIERS
    starts the QR with its barrier time-out flag raised."""
    lib = load()
    n = P.shape[0]
    P = padded(P)
    if out is None:
        out = empty_matrix(n, n, device=P.device)
    need = lib.mao_qr_workspace_size(n)
    buf = workspace(need, P.device)
    if dbg_flags:
        _check(lib.mao_dbg_qr(_ptr(P), P.stride(0), _ptr(out), out.stride(0), n, _ptr(buf),
                              buf.numel(), dbg_flags, _stream()), "mao_dbg_qr")
    else:
        _check(lib.mao_qr(_ptr(P), P.stride(0), _ptr(out), out.stride(0), n, _ptr(buf),
                          buf.numel(), _stream()), "mao_qr")
    return out
