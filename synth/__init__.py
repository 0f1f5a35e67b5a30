"""Seeded synthetic inputs for the optimizer-step workloads.

This module only draws random numbers and arranges them into weight and
gradient matrices with the shapes and statistical structure of the workloads
the pages discuss. It holds none of the optimizer arithmetic, so both the
fp64 oracle and the HIP path can take their inputs from here without sharing
any computation.

Every array comes from ``numpy.random.default_rng(SeedSequence([20261203,
config, matrix, step]))``: the same (config, matrix, step) always yields the
same numbers on any machine.

Workloads (shapes are rows x cols as stored, row-major):

* ``c1`` -- one 256x512 fp32 matrix, G_t = diag(s) Z_t with Z_t ~ N(0,1)
  fresh per step and s_i = exp(N(0, 0.5^2)) drawn once.
* ``c2`` -- one Llama-style 8B layer (hidden 4096, 32 query / 8 KV heads of
  dim 128, FFN 14336): QKV 4096x6144, O 4096x4096, gate/up 14336x4096,
  down 4096x14336; G_t = Z_t + A B^T / 4 with a fixed rank-16 pair (A, B)
  per matrix (equal Frobenius energy in signal and noise).
* ``c3`` -- the same five shapes with Kronecker-structured gradients
  G_t = U_A diag(k^-1/2) Z_t diag(k^-1/2) U_B^T, U = signed, permuted,
  orthonormal DCT-II (applied by FFT, never formed).
* ``c4`` -- 128 MoE experts x {gate 1536x2048, up 1536x2048, down 2048x1536},
  G_e = sqrt(n_e / mean(n)) Z with n_e the tokens routed to expert e under a
  Zipf(1.1) load (top-8 routing of 3072 x 8192 tokens).
* ``c5`` -- GPT-2-760M-shaped set, 24 x {Q, K, V, O 1536x1536, FC 6144x1536,
  PROJ 1536x6144} with the Kronecker generator, plus the tied 50304x1536
  embedding.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import scipy.fft

ROOT_SEED = 20261203

CONFIG_IDS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5}


def rng(config: int, matrix: int, step: int) -> np.random.Generator:
    """Counter-style seeded generator for (config, matrix, step)."""
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, config, matrix, step]))


# ---------------------------------------------------------------------------
# shapes
# ---------------------------------------------------------------------------

LLAMA8B_LAYER = [
    ("qkv", 4096, 6144),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
]

MOE_EXPERTS = 128
MOE_TOPK = 8
MOE_TOKENS = 3072 * 8192  # global batch of the 8B recipe, in tokens
MOE_SHAPES = [("gate", 1536, 2048), ("up", 1536, 2048), ("down", 2048, 1536)]

GPT2_760M_WIDTH = 1536
GPT2_760M_LAYERS = 24
GPT2_760M_FFN = 6144
GPT2_VOCAB = 50304


def gpt2_760m_shapes():
    d, f = GPT2_760M_WIDTH, GPT2_760M_FFN
    out = []
    for layer in range(GPT2_760M_LAYERS):
        for name, m, n in (("q", d, d), ("k", d, d), ("v", d, d), ("o", d, d),
                           ("fc", f, d), ("proj", d, f)):
            out.append((f"l{layer}.{name}", m, n))
    return out


@dataclass
class MatrixSpec:
    name: str
    rows: int
    cols: int
    index: int
    extra: dict = field(default_factory=dict)


def specs(config: str, scale: float = 1.0) -> list[MatrixSpec]:
    """Matrix list of a workload. ``scale`` < 1 shrinks every dimension
    (rounded to a multiple of 8, ragged sizes kept) for parity tests."""

    def s(x: int) -> int:
        if scale == 1.0:
            return x
        return max(8, int(round(x * scale / 8.0)) * 8)

    if config == "c1":
        return [MatrixSpec("w", 256, 512, 0)]
    if config in ("c2", "c3"):
        return [MatrixSpec(n, s(m), s(k), i) for i, (n, m, k) in enumerate(LLAMA8B_LAYER)]
    if config == "c4":
        out = []
        for e in range(MOE_EXPERTS):
            for j, (n, m, k) in enumerate(MOE_SHAPES):
                out.append(MatrixSpec(f"e{e}.{n}", s(m), s(k), 3 * e + j, {"expert": e}))
        return out
    if config == "c5":
        return [MatrixSpec(n, s(m), s(k), i) for i, (n, m, k) in enumerate(gpt2_760m_shapes())]
    raise KeyError(config)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------

def init_weight(config: str, spec: MatrixSpec, dtype=np.float32) -> np.ndarray:
    """W0 ~ N(0, 0.02^2)."""
    g = rng(CONFIG_IDS[config], spec.index, 10**6)
    return (0.02 * g.standard_normal((spec.rows, spec.cols))).astype(dtype)


def c1_gradient(spec: MatrixSpec, step: int) -> np.ndarray:
    row_scale = np.exp(0.5 * rng(1, spec.index, 0).standard_normal(spec.rows))
    z = rng(1, spec.index, step).standard_normal((spec.rows, spec.cols))
    return (row_scale[:, None] * z).astype(np.float32)


def lowrank_gradient(config: str, spec: MatrixSpec, step: int, rank: int = 16) -> np.ndarray:
    """Z_t + A B^T / 4 (A, B fixed per matrix)."""
    cid = CONFIG_IDS[config]
    g0 = rng(cid, spec.index, 0)
    a = g0.standard_normal((spec.rows, rank), dtype=np.float32)
    b = g0.standard_normal((spec.cols, rank), dtype=np.float32)
    z = rng(cid, spec.index, step).standard_normal((spec.rows, spec.cols), dtype=np.float32)
    z += (a @ b.T) * np.float32(0.25)
    return z


def _signed_permuted_dct(x: np.ndarray, axis: int, g: np.random.Generator) -> np.ndarray:
    """Apply U = diag(sign) . Perm . C (C the orthonormal DCT-II) along ``axis``."""
    n = x.shape[axis]
    perm = g.permutation(n)
    sign = np.where(g.random(n) < 0.5, -1.0, 1.0)
    y = scipy.fft.dct(x, type=2, norm="ortho", axis=axis, workers=-1)
    y = np.take(y, perm, axis=axis)
    shape = [1, 1]
    shape[axis] = n
    return y * sign.reshape(shape)


def kronecker_gradient(config: str, spec: MatrixSpec, step: int, dtype=np.float32) -> np.ndarray:
    """U_A diag(k^-1/2) Z_t diag(k^-1/2) U_B^T: row covariance with eigenvalues
    proportional to 1/k in basis U_A, column covariance likewise in U_B."""
    cid = CONFIG_IDS[config]
    m, n = spec.rows, spec.cols
    da = 1.0 / np.sqrt(np.arange(1, m + 1, dtype=np.float64))
    db = 1.0 / np.sqrt(np.arange(1, n + 1, dtype=np.float64))
    z = rng(cid, spec.index, step).standard_normal((m, n))
    y = (da[:, None] * z) * db[None, :]
    g0 = rng(cid, spec.index, 0)
    y = _signed_permuted_dct(y, 0, g0)   # U_A Y
    y = _signed_permuted_dct(y, 1, g0)   # (U_A Y) U_B^T
    return y.astype(dtype)


def moe_token_counts() -> np.ndarray:
    """Tokens routed to each expert: top-8 of 3072x8192 tokens over 128
    experts with a Zipf(1.1) popularity whose ranks are seed-permuted."""
    g = rng(4, 10**5, 0)
    ranks = g.permutation(MOE_EXPERTS) + 1
    p = ranks.astype(np.float64) ** -1.1
    p /= p.sum()
    return np.maximum(1, np.round(MOE_TOPK * MOE_TOKENS * p)).astype(np.int64)


def moe_gradient(spec: MatrixSpec, step: int) -> np.ndarray:
    counts = moe_token_counts()
    scale = math.sqrt(counts[spec.extra["expert"]] / counts.mean())
    z = rng(4, spec.index, step).standard_normal((spec.rows, spec.cols), dtype=np.float32)
    return z * np.float32(scale)


def gradient(config: str, spec: MatrixSpec, step: int) -> np.ndarray:
    """fp32 gradient of ``spec`` at 1-based ``step`` (callers cast to bf16 where
    the workload stores gradients in bf16)."""
    if config == "c1":
        return c1_gradient(spec, step)
    if config == "c2":
        return lowrank_gradient(config, spec, step)
    if config in ("c3", "c5"):
        return kronecker_gradient(config, spec, step)
    if config == "c4":
        return moe_gradient(spec, step)
    raise KeyError(config)


def embedding_gradient(step: int, rows: int = GPT2_VOCAB, cols: int = GPT2_760M_WIDTH) -> np.ndarray:
    """Tied-embedding gradient: Gaussian rows with a heavy-tailed per-token scale
    (token frequencies), fp32."""
    g0 = rng(5, 10**4, 0)
    freq = (np.arange(1, rows + 1, dtype=np.float64) ** -1.0)[g0.permutation(rows)]
    scale = np.sqrt(freq / freq.mean()).astype(np.float32)
    z = rng(5, 10**4, step).standard_normal((rows, cols), dtype=np.float32)
    return z * scale[:, None]


def rademacher_kfac_gradient(alpha: np.ndarray, beta: np.ndarray, q_right: np.ndarray,
                             seed: int, step: int) -> np.ndarray:
    """G = (D_alpha Z D_beta) Q^T with Z i.i.d. +-1: every rotated entry
    (G Q)_{ij}^2 equals alpha_i^2 beta_j^2 exactly (K-FAC structure with a
    diagonal output side)."""
    g = rng(9, seed, step)
    z = np.where(g.random((alpha.size, beta.size)) < 0.5, -1.0, 1.0)
    return (alpha[:, None] * z * beta[None, :]) @ q_right.T


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even), returned as fp32.
    Used to hand both sides identical bf16 inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    nan = np.isnan(x)
    out = r.view(np.float32).copy()
    out[nan] = np.nan
    return out
