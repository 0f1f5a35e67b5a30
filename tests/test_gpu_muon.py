"""Muon / Muon+ parity: the HIP path against the fp64 oracle on the same seeded
inputs (GPU). Tolerances: relative Frobenius error of the update (before the
learning rate) <= 1e-4 on the fp32 path and <= 2e-2 on the bf16-MFMA
Newton-Schulz path. The weight write is checked given the GPU's own update:
within one bf16 ulp of the rounded exact result, plus fp32 rounding of the
operands where the subtraction cancels."""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import bf16_round
from tests.helpers import log, rel, to_dev, to_host, w_bound, zeros_dev

pytestmark = pytest.mark.gpu

LR, WD = 1e-3, 0.1
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _run_steps(gpu_lib, m, n, steps, dtype, ns_dtype, norm_mode="none", seed=0, mu=0.95,
               grad=None):
    """Free-running multi-step comparison on one matrix; returns worst errors."""
    import torch
    r = np.random.default_rng(seed)
    w0 = (0.02 * r.standard_normal((m, n))).astype(np.float32)
    if dtype == "bf16":
        w0 = bf16_round(w0)
    W = to_dev(w0, dtype)
    M = zeros_dev((m, n))
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    mom_ref = np.zeros((m, n))
    worst = 0.0
    for t in range(1, steps + 1):
        g = grad(t) if grad is not None else r.standard_normal((m, n)).astype(np.float32)
        if dtype == "bf16":
            g = bf16_round(g)
        w_before = to_host(W)
        gpu_lib.muon_step(W, to_dev(g, dtype), M, update_out=out, lr=LR, mu=mu, weight_decay=WD,
                          ns_steps=5, ns_dtype=ns_dtype, norm_mode=norm_mode)
        torch.cuda.synchronize()
        w_ref, mom_ref, upd_ref = oracle.muon_step(w_before, g, mom_ref, lr=LR, mu=mu,
                                                   weight_decay=WD, ns_steps=5,
                                                   norm_mode=norm_mode)
        e = rel(to_host(out), upd_ref)
        worst = max(worst, e)
        assert rel(to_host(M), mom_ref) < 1e-6
        assert e < TOL[ns_dtype], f"step {t}: update error {e}"
        # the weight update itself, given the GPU's update
        w_gpu = to_host(W)
        lr_term = LR * (WD * w_before + to_host(out))
        w_expect = w_before - lr_term
        if dtype == "bf16":
            w_exp16 = bf16_round(w_expect.astype(np.float32))
            assert np.all(np.abs(w_gpu - w_exp16) <= w_bound(w_expect, w_before, lr_term))
        else:
            assert rel(w_gpu, w_expect) < 1e-6
            assert rel(w_gpu, w_ref) < 1e-6
    return worst


def test_muon_c1_fp32_ten_steps(gpu_lib):
    """256x512 fp32 matrix, rows scaled log-normally, 10 steps, mu = 0.95,
    5 iterations in fp32."""
    log("muon c1 fp32")
    spec = synth.specs("c1")[0]
    worst = _run_steps(gpu_lib, 256, 512, 10, "f32", "f32",
                       grad=lambda t: synth.gradient("c1", spec, t))
    log(f"  worst update error {worst:.2e}")


@pytest.mark.parametrize("m,n", [(200, 328), (328, 200), (72, 72), (8, 1000)])
def test_muon_bf16_ragged_shapes(gpu_lib, m, n):
    log(f"muon bf16 {m}x{n}")
    worst = _run_steps(gpu_lib, m, n, 3, "bf16", "bf16", seed=m * 1000 + n)
    log(f"  worst update error {worst:.2e}")


@pytest.mark.parametrize("mode", ["row", "col", "col_row", "row_col"])
def test_muon_plus_fp32_modes(gpu_lib, mode):
    log(f"muon+ fp32 {mode}")
    _run_steps(gpu_lib, 136, 264, 2, "f32", "f32", norm_mode=mode, seed=3)
    _run_steps(gpu_lib, 264, 136, 2, "f32", "f32", norm_mode=mode, seed=4)


def test_muon_zero_gradient_and_zero_steps(gpu_lib):
    import torch
    m, n = 64, 96
    W = to_dev(np.ones((m, n), np.float32))
    M = zeros_dev((m, n))
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    gpu_lib.muon_step(W, torch.zeros_like(W), M, update_out=out, lr=0.01, mu=0.9,
                      weight_decay=0.1, ns_steps=5, ns_dtype="f32")
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    assert torch.allclose(W, torch.full_like(W, 0.999))
    # zero iterations: U = sqrt(m/n) M / (|M| + eps)
    r = np.random.default_rng(5)
    g = r.standard_normal((m, n)).astype(np.float32)
    M.zero_()
    gpu_lib.muon_step(W, to_dev(g), M, update_out=out, lr=0.0, mu=0.9, weight_decay=0.0,
                      ns_steps=0, ns_dtype="f32")
    torch.cuda.synchronize()
    m1 = 0.1 * g.astype(np.float64)
    ref = math.sqrt(m / n) * m1 / (np.linalg.norm(m1) + 1e-7)
    assert rel(to_host(out), ref) < 1e-6


def test_muon_batched_matches_oracle_per_matrix(gpu_lib):
    """Grouped launch over two groups of different shapes (one tall, one wide),
    bf16, Muon+ column-then-row."""
    import torch
    log("muon batched bf16 col_row")
    r = np.random.default_rng(21)
    shapes = [(3, 96, 160), (2, 160, 96)]
    groups, host = [], []
    for cnt, m, n in shapes:
        w = bf16_round((0.02 * r.standard_normal((cnt, m, n))).astype(np.float32))
        g = bf16_round(r.standard_normal((cnt, m, n)).astype(np.float32))
        W, G = to_dev(w, "bf16"), to_dev(g, "bf16")
        M = zeros_dev((cnt, m, n))
        groups.append((W, G, M))
        host.append((w, g))
    outs = [torch.empty(W.shape, dtype=torch.float32, device="cuda") for W, _, _ in groups]
    gpu_lib.muon_step_batched(groups, update_out=outs, lr=LR, mu=0.95, weight_decay=WD,
                              ns_steps=5, ns_dtype="bf16", norm_mode="col_row")
    torch.cuda.synchronize()
    for (w, g), out in zip(host, outs):
        o = to_host(out)
        for b in range(w.shape[0]):
            _, _, upd = oracle.muon_step(w[b], g[b], np.zeros_like(w[b]), lr=LR, mu=0.95,
                                         weight_decay=WD, ns_steps=5, norm_mode="col_row")
            assert rel(o[b], upd) < TOL["bf16"]


def _batched_case(gpu_lib, shapes, seed, norm_mode="none", ns_steps=5, coeffs=None):
    import torch
    r = np.random.default_rng(seed)
    groups, host = [], []
    for cnt, m, n in shapes:
        w = bf16_round((0.02 * r.standard_normal((cnt, m, n))).astype(np.float32))
        g = bf16_round(r.standard_normal((cnt, m, n)).astype(np.float32))
        W, G = to_dev(w, "bf16"), to_dev(g, "bf16")
        M = zeros_dev((cnt, m, n))
        groups.append((W, G, M))
        host.append((w, g))
    outs = [torch.empty(W.shape, dtype=torch.float32, device="cuda") for W, _, _ in groups]
    gpu_lib.muon_step_batched(groups, update_out=outs, lr=LR, mu=0.95, weight_decay=WD,
                              ns_steps=ns_steps, ns_coeffs=coeffs, ns_dtype="bf16",
                              norm_mode=norm_mode)
    torch.cuda.synchronize()
    worst = 0.0
    for (w, g), out in zip(host, outs):
        o = to_host(out)
        for b in range(w.shape[0]):
            _, _, upd = oracle.muon_step(w[b], g[b], np.zeros_like(w[b]), lr=LR, mu=0.95,
                                         weight_decay=WD, ns_steps=ns_steps, coeffs=coeffs,
                                         norm_mode=norm_mode)
            e = rel(o[b], upd)
            worst = max(worst, e)
            assert e < TOL["bf16"], f"{w.shape} matrix {b}: {e}"
    return worst


@pytest.mark.parametrize("norm_mode", ["none", "col_row"])
def test_muon_tiled_workspaces_ragged(gpu_lib, norm_mode):
    """Batches large enough (>= 128 tiles of 256 x 256) that the Newton-Schulz
    workspaces are kept tiled, with dimensions that are not multiples of 256
    (zero pad inside the tiles), wide and tall, and a degenerate 8-row group."""
    log(f"muon tiled bf16 ragged {norm_mode}")
    worst = _batched_case(gpu_lib, [(16, 520, 1032), (16, 1032, 520), (40, 8, 1000)], 31,
                          norm_mode=norm_mode)
    log(f"  worst update error {worst:.2e}")


def test_muon_tiled_one_iteration(gpu_lib):
    """One Newton-Schulz iteration: the first product is also the last, which
    reads the tiled X0 and writes the row-major result."""
    log("muon tiled bf16 one iteration")
    _batched_case(gpu_lib, [(12, 776, 1288), (12, 1288, 776)], 32, ns_steps=1)


@pytest.mark.parametrize("family", ["tuned_quintic", "with_cubic_steps"])
def test_muon_tiled_coefficient_families(gpu_lib, family):
    """Per-iteration coefficients through the tiled path: a tuned quintic
    (every c != 0: the polynomial completed to a square), and a schedule whose
    odd iterations are cubic (c = 0: the square step reads A as C0)."""
    if family == "tuned_quintic":
        coeffs = [(3.4445, -4.7750, 2.0315)] * 5
    else:
        coeffs = [(1.5, -0.5, 0.0), (15 / 8, -10 / 8, 3 / 8)] * 2 + [(1.5, -0.5, 0.0)]
    log(f"muon tiled bf16 coefficients {family}")
    worst = _batched_case(gpu_lib, [(16, 520, 1032), (16, 1032, 520)], 33, coeffs=coeffs)
    log(f"  worst update error {worst:.2e}")


@pytest.mark.parametrize("layers,rows,q,kv", [(3, 96, 128, 40), (6, 1024, 1024, 256)])
def test_muon_fused_qkv_views_sixteen_iterations(gpu_lib, layers, rows, q, kv):
    """The logical Q, K and V matrices of a fused QKV weight, passed as
    column views (leading dimension = the fused width) of one buffer per
    layer, and 16 iterations with a per-iteration coefficient table. Each
    view is stepped as its own matrix; K and V are tall (transposed
    orientation); 8 guard columns after V stay bit-identical. The larger case
    has enough tiles to run on the tiled iterates."""
    import torch
    log(f"muon fused qkv views {layers}x{rows}x({q}+{kv}+{kv}), 16 iterations")
    coeffs = [(3.4445, -4.7750, 2.0315)] * 8 + [(15 / 8, -10 / 8, 3 / 8)] * 8
    width = q + 2 * kv + 8
    spans = [(0, q), (q, q + kv), (q + kv, q + 2 * kv)]
    r = np.random.default_rng(34)
    w = bf16_round((0.02 * r.standard_normal((layers, rows, width))).astype(np.float32))
    g = bf16_round(r.standard_normal((layers, rows, width)).astype(np.float32))
    W, G = to_dev(w, "bf16"), to_dev(g, "bf16")
    Mf = zeros_dev((layers, rows, width))
    groups = [(W[:, :, a:b], G[:, :, a:b], Mf[:, :, a:b]) for a, b in spans]
    outs = [torch.empty((layers, rows, b - a), dtype=torch.float32, device="cuda")
            for a, b in spans]
    gpu_lib.muon_step_batched(groups, update_out=outs, lr=LR, mu=0.95, weight_decay=WD,
                              ns_steps=16, ns_coeffs=coeffs, ns_dtype="bf16")
    torch.cuda.synchronize()
    w_gpu = to_host(W)
    assert np.array_equal(w_gpu[:, :, q + 2 * kv:], w[:, :, q + 2 * kv:])
    assert np.all(to_host(Mf)[:, :, q + 2 * kv:] == 0)
    worst = 0.0
    for (a, b), out in zip(spans, outs):
        o = to_host(out)
        for layer in range(layers):
            wb, gb = w[layer, :, a:b], g[layer, :, a:b]
            _, _, upd = oracle.muon_step(wb, gb, np.zeros_like(wb), lr=LR, mu=0.95,
                                         weight_decay=WD, ns_steps=16, coeffs=coeffs)
            e = rel(o[layer], upd)
            worst = max(worst, e)
            assert e < TOL["bf16"], f"columns {a}:{b} layer {layer}: {e}"
            lr_term = LR * (WD * wb + o[layer])
            w_expect = wb - lr_term
            w_exp16 = bf16_round(w_expect.astype(np.float32))
            assert np.all(np.abs(w_gpu[layer, :, a:b] - w_exp16) <= w_bound(w_expect, wb, lr_term))
    log(f"  worst update error {worst:.2e}")


def test_muon_full_size_o_projection(gpu_lib):
    """The 4096x4096 O projection of the 8B layer at full size, bf16, one step
    (the shape and launch configuration the benchmark times)."""
    import torch
    log("muon full-size 4096x4096 bf16")
    spec = synth.specs("c2")[1]
    w = bf16_round(synth.init_weight("c2", spec))
    g = bf16_round(synth.gradient("c2", spec, 1))
    W, G = to_dev(w, "bf16"), to_dev(g, "bf16")
    M = zeros_dev(W.shape)
    out = torch.empty(W.shape, dtype=torch.float32, device="cuda")
    gpu_lib.muon_step(W, G, M, update_out=out, lr=LR, mu=0.95, weight_decay=WD, ns_steps=5,
                      ns_dtype="bf16")
    torch.cuda.synchronize()
    _, _, upd = oracle.muon_step(w, g, np.zeros_like(w, dtype=np.float64), lr=LR, mu=0.95,
                                 weight_decay=WD, ns_steps=5)
    e = rel(to_host(out), upd)
    log(f"  update error {e:.2e}")
    assert e < TOL["bf16"]


def test_muon_deterministic(gpu_lib):
    import torch
    r = np.random.default_rng(9)
    g = r.standard_normal((300, 500)).astype(np.float32)
    outs = []
    for _ in range(2):
        W = zeros_dev((300, 500))
        M = zeros_dev((300, 500))
        out = torch.empty((300, 500), dtype=torch.float32, device="cuda")
        gpu_lib.muon_step(W, to_dev(g), M, update_out=out, lr=LR, mu=0.95, weight_decay=WD,
                          ns_steps=5, ns_dtype="bf16", norm_mode="col_row")
        torch.cuda.synchronize()
        outs.append(out.clone())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("norm_mode", ["none", "col_row"])
def test_timing_elementwise_tag(gpu_lib, norm_mode):
    """The benchmark instrumentation of a Muon step's memory-bound passes:
    with timing on, the EMA, the X0 cast, the Muon+ sums of squares (one read
    of the result per axis) and the update are bracketed under the
    "elementwise" tag and credited with the bytes they must move (bf16 W and
    G, fp32 M, bf16 Newton-Schulz iterates); contractions keep their tags."""
    import torch
    m, n = 384, 640
    r = np.random.default_rng(41)
    W = to_dev(bf16_round((0.02 * r.standard_normal((m, n))).astype(np.float32)), "bf16")
    G = to_dev(bf16_round(r.standard_normal((m, n)).astype(np.float32)), "bf16")
    M = zeros_dev((m, n))
    gpu_lib.timing_collect()
    gpu_lib.timing_enable(True)
    try:
        gpu_lib.muon_step(W, G, M, lr=LR, mu=0.95, weight_decay=WD, ns_steps=5, ns_dtype="bf16",
                          norm_mode=norm_mode)
        torch.cuda.synchronize()
    finally:
        gpu_lib.timing_enable(False)
    tim = gpu_lib.timing_collect()
    ms, launches, nbytes = tim["elementwise"]
    axes = 2 if norm_mode == "col_row" else 0
    expect = m * n * ((8 + 2) + (4 + 2) + 2 * axes + (2 * 2 + 2))
    assert launches == (4 if axes else 3)
    assert nbytes == expect
    assert ms > 0.0
    assert sum(tim[k][1] for k in ("ns_gram", "ns_square", "ns_apply")) == 15
