"""Shared test utilities (no optimizer arithmetic here)."""
import numpy as np


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def to_dev(x, dtype="f32", device="cuda"):
    """Copy to the device; 2-D and 3-D arrays get rows padded to a multiple of
    8 elements (the library's leading-dimension rule), returned as a view."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    src = torch.from_numpy(x).to(tdt)
    if x.ndim < 2 or x.shape[-1] % 8 == 0:
        return src.to(device)
    cols = x.shape[-1]
    ld = (cols + 7) // 8 * 8
    buf = torch.zeros(x.shape[:-1] + (ld,), dtype=tdt, device=device)
    view = buf[..., :cols]
    view.copy_(src.to(device))
    return view


def tile_max_rel(a, b, tile: int = 256) -> float:
    """Largest relative Frobenius error over the tile x tile blocks of a 2-D
    result (ragged edge blocks included): a localised error -- one bad band
    of one output tile -- shows here even when the whole-matrix error is
    small."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    worst = 0.0
    for i in range(0, b.shape[0], tile):
        for j in range(0, b.shape[1], tile):
            bt = b[i:i + tile, j:j + tile]
            den = np.linalg.norm(bt)
            e = np.linalg.norm(a[i:i + tile, j:j + tile] - bt) / (den if den > 0 else 1.0)
            worst = max(worst, float(e))
    return worst


def zeros_dev(shape, dtype="f32", device="cuda"):
    return to_dev(np.zeros(shape, np.float32), dtype, device)


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (for |x| normal)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def w_bound(w_expect, w_prev, lr_term):
    """Elementwise bound for a weight written in bf16 after fp32 arithmetic:
    one bf16 ulp of the exact result plus fp32 rounding of the operands (the
    subtraction w - lr*(...) can cancel)."""
    return (bf16_ulp(w_expect) * 1.001 + 4 * 2.0 ** -24 * (np.abs(w_prev) + np.abs(lr_term))
            + 1e-30)


def log(msg: str):
    print(msg, flush=True)


# Relative accuracy of one product: fp32 MFMA, or bf16x3 on split operands
# (x = hi + lo in bf16; the dropped lo*lo term and the residual of each split
# are each below 2^-18 of a product term).
PRODUCT_EPS = {"f32": 2.0 ** -24, "bf16x3": 3 * 2.0 ** -18}

