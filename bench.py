#!/usr/bin/env python3
"""Optimizer-step benchmark on one MI355X.

Default workload: one Muon step (momentum, 5 Newton-Schulz quintic iterations
in bf16 MFMA with fp32 accumulation, sqrt(m/n)-scaled update with decoupled
weight decay) over the weight matrices of one Llama-style 8B layer -- QKV
4096x6144, O 4096x4096, gate 14336x4096, up 14336x4096, down 4096x14336 -- in
one grouped call (one launch per Newton-Schulz stage for the whole layer).
bf16 weights and gradients, fp32 momentum, synthetic seeded gradients
(Gaussian plus a rank-16 component), a ring of two gradients per matrix so
every step reads fresh data. Inputs are resident in HBM before timing.

Prints one JSON line: steps/s of the whole job (K timed steps, no per-launch
instrumentation), the dominant kernel's roofline (the Newton-Schulz
contraction, from HIP events around every launch of a second region of K
steps), the fp64 CPU oracle's rate on a bounded sample of the workload's own
matrices, and -- under "soap8b" -- the same 8B layer under SOAP (steps/s and
the rate of its contractions against the fp32 and bf16 peaks), and under "moe"
and "foam760m" the MoE expert bank under Muon+ and the GPT-2-760M set under
FOAM (steps/s and their dominant kernel's roofline). SOAP and FOAM
workloads run their fp32-accurate products (forward rotations, power-
iteration and criterion products) as bf16x3 by default (--fwd,
--refresh-prod) and the rotation back on bf16 MFMA (--back).

Other workloads (--workload): moe (128-expert bank, batched Muon+), c1muon /
c1soap (256x512 fp32 Muon and SOAP), soap8b (the 8B layer under SOAP),
foam760m (GPT-2-760M-shaped set under FOAM plus the AdamW embedding),
foam760m_output (the same with the basis on the output side), soap760m (the
760M set under SOAP), observe8b (the observability reductions over the 8B
layer).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "optimizer steps/sec on 8B-layer matrix set; NS+rotation GEMM MFMA % of peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Fabric traffic of the Newton-Schulz contraction, from two rocprofv3 --pmc
# runs of the default workload (FETCH_SIZE, then WRITE_SIZE; KiB per
# dispatch), each scaled by what the same counter reads for a 1 GiB
# device-to-device copy (--calibrate-copy). It describes the kernel sources it
# was taken on and is reported only while they are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ns_contraction_llama8b_layer_traffic.json")
GEMM_SOURCES = [os.path.join(ROOT, "matrix_aware_optimizers_amd", "csrc", f)
                for f in ("gemm_direct.hip", "gemm.hip", "gemm.hpp", "epilogue.hpp", "tiled.hpp",
                          "common.hpp")]
NS_KERNEL = "gemm_bf16_dl_kernel"
COPY_KERNEL = "copyBuffer"


def gemm_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """Bytes per Newton-Schulz launch from the committed counter summary, or
    None when the contraction sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != gemm_source_digest():
        return None
    return rec.get("bytes_per_launch")


def write_traffic(fetch_csv: str, write_csv: str, command: str):
    """Summarise two rocprofv3 counter CSVs (FETCH_SIZE, WRITE_SIZE) of the
    default workload run with --calibrate-copy into TRAFFIC_FILE."""
    import csv

    def per_kernel(path, counter):
        ns, copy = [], []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if NS_KERNEL in r["Kernel_Name"]:
                    ns.append(v)
                elif COPY_KERNEL in r["Kernel_Name"]:
                    copy.append(v)
        if not ns or len(copy) != 1:
            raise SystemExit(f"{path}: expected Newton-Schulz dispatches and one calibration copy")
        return sum(ns) / len(ns), copy[0], len(ns)

    f_ns, f_copy, n = per_kernel(fetch_csv, "FETCH_SIZE")
    w_ns, w_copy, _ = per_kernel(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    f_scale, w_scale = gib_kib / f_copy, gib_kib / w_copy
    rec = {
        "kernel": NS_KERNEL,
        "workload": "llama8b_layer_muon_bf16",
        "dispatches": n,
        "fetch_kib_per_launch": round(f_ns, 1),
        "write_kib_per_launch": round(w_ns, 1),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "bytes_per_launch": round((f_ns * f_scale + w_ns * w_scale) * 1024.0),
        "source_sha256": gemm_source_digest(),
        "command": command,
    }
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def ns_alg_flops(m: int, n: int, k: int = 5) -> float:
    """Algorithmic flops of k quintic iterations on an m x n matrix (symmetric
    products at half cost): per iteration a^2 b (X X^T) + a^3 (A A) + 2 a^2 b
    (B X), a = min, b = max."""
    a, b = min(m, n), max(m, n)
    return k * (3.0 * a * a * b + a ** 3)


# ---------------------------------------------------------------------------
# Muon workloads
# ---------------------------------------------------------------------------

class MuonWorkload:
    def __init__(self, groups_spec, dtype="bf16", norm_mode="none", seed_config="c2",
                 ns_dtype="bf16"):
        import torch

        import matrix_aware_optimizers_amd as mao
        import synth
        self.mao = mao
        self.lib = mao.load()
        self.hp = mao.muon_hparams(lr=1e-3, mu=0.95, weight_decay=0.1, eps=1e-7, ns_steps=5,
                                   ns_dtype=ns_dtype, norm_mode=norm_mode)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.tensors = []
        self.shapes = []
        for name, specs in groups_spec:
            cnt = len(specs)
            m, n = specs[0].rows, specs[0].cols
            self.shapes.append((cnt, m, n))
            W = torch.empty((cnt, m, n), dtype=tdt, device="cuda")
            Gs = [torch.empty((cnt, m, n), dtype=tdt, device="cuda") for _ in range(2)]
            for b, sp in enumerate(specs):
                W[b].copy_(torch.from_numpy(synth.init_weight(seed_config, sp)))
                for k in range(2):
                    Gs[k][b].copy_(torch.from_numpy(synth.gradient(seed_config, sp, k + 1)))
            M = torch.zeros((cnt, m, n), dtype=torch.float32, device="cuda")
            self.tensors.append((W, Gs, M))
        ng = len(self.tensors)
        self.ng = ng
        self.Ws = (mao.Batch * ng)(*[mao.batch(W) for W, _, _ in self.tensors])
        self.Ms = (mao.Batch * ng)(*[mao.batch(M) for _, _, M in self.tensors])
        self.Gs = [(mao.Batch * ng)(*[mao.batch(Gs[k]) for _, Gs, _ in self.tensors])
                   for k in range(2)]
        need = self.lib.muon_batched_workspace_size(ng, self.Ws, ctypes.byref(self.hp))
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()

    def step(self, i: int):
        st = self.lib.muon_step_batched(self.ng, self.Ws, self.Gs[i % 2], self.Ms,
                                        ctypes.byref(self.hp), ctypes.c_void_p(self.ws.data_ptr()),
                                        self.ws.numel(), None, self.stream)
        if st != 0:
            self.mao._check(st, "muon_step_batched")

    def ns_flops(self) -> float:
        return sum(c * ns_alg_flops(m, n) for c, m, n in self.shapes)


def llama8b_groups():
    import synth
    return [(s.name, [s]) for s in synth.specs("c2")]


def moe_groups():
    import synth
    sp = synth.specs("c4")
    out = []
    for j, name in enumerate(("gate", "up", "down")):
        out.append((name, [s for s in sp if s.name.endswith("." + name)]))
    return out


def _host_description():
    """nproc, CPU model and BLAS of this host (for the baseline record)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads, blas = os.cpu_count(), "unknown"
    try:
        import threadpoolctl
        info = [d for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        if info:
            threads = max(d.get("num_threads", 1) for d in info)
            blas = ",".join(sorted({f"{d.get('internal_api')} {d.get('version')}" for d in info}))
    except Exception:  # pragma: no cover
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model, "blas": blas}, int(threads)


def cpu_baseline_muon(groups, seed_config: str, budget_s: float = 60.0):
    """The oracle (fp64, NumPy) on the workload's own matrices, one Muon step
    each (5 iterations), in the set's order, until the time budget is spent;
    the whole step's rate is the flop-weighted extrapolation from the matrices
    that ran (exact when they all ran)."""
    import oracle
    import synth
    host, threads = _host_description()
    specs = [sp for _, sps in groups for sp in sps]
    total = sum(ns_alg_flops(sp.rows, sp.cols) for sp in specs)
    done, done_fl, t_all = [], 0.0, 0.0
    for sp in specs:
        w = synth.bf16_round(synth.init_weight(seed_config, sp)).astype(np.float64)
        g = synth.bf16_round(synth.gradient(seed_config, sp, 1)).astype(np.float64)
        t0 = time.perf_counter()
        oracle.muon_step(w, g, np.zeros_like(w), lr=1e-3, mu=0.95, weight_decay=0.1, ns_steps=5)
        dt = time.perf_counter() - t0
        t_all += dt
        done_fl += ns_alg_flops(sp.rows, sp.cols)
        done.append(f"{sp.rows}x{sp.cols} {dt:.2f} s")
        log(f"  oracle {sp.name} {sp.rows}x{sp.cols}: {dt:.2f} s")
        if t_all >= budget_s:
            break
    whole = len(done) == len(specs)
    est = t_all if whole else t_all * total / done_fl
    what = ("the whole set, one step" if whole else
            f"{len(done)} of {len(specs)} matrices within a {budget_s:.0f} s budget, scaled by "
            f"Newton-Schulz flops (x{total / done_fl:.2f}) to the set")
    return {"value": 1.0 / est, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 Muon step (5 iterations) of the workload's matrices: {what} "
                      f"[{'; '.join(done)}]",
            **host}


def run_muon(args, workload_name, groups, norm_mode, sample, dtype="bf16"):
    import torch

    import matrix_aware_optimizers_amd as mao
    log(f"setting up {workload_name}")
    wl = MuonWorkload(groups, dtype=dtype, norm_mode=norm_mode, seed_config=sample[2],
                      ns_dtype=dtype)
    log("warmup")
    for i in range(args.warmup):
        wl.step(i)
    torch.cuda.synchronize()
    # timed region: K steps, no per-launch instrumentation
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    start.record()
    for i in range(args.steps):
        wl.step(args.warmup + i)
        marks[i].record()  # one event between steps: per-step median and p90
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    per_step = sorted([start.elapsed_time(marks[0])] +
                      [marks[i - 1].elapsed_time(marks[i]) for i in range(1, args.steps)])
    # second region of K steps with HIP events around every contraction
    # launch (recorded on the library's stream): the per-kernel split
    mao.timing_collect()
    mao.timing_enable(True)
    start.record()
    for i in range(args.steps):
        wl.step(args.warmup + args.steps + i)
    end.record()
    torch.cuda.synchronize()
    mao.timing_enable(False)
    tim = mao.timing_collect()
    ms_instr = start.elapsed_time(end) / args.steps
    ns_ms = sum(tim[k][0] for k in ("ns_gram", "ns_square", "ns_apply"))
    ns_cnt = sum(tim[k][1] for k in ("ns_gram", "ns_square", "ns_apply"))
    ns_fl = sum(tim[k][2] for k in ("ns_gram", "ns_square", "ns_apply"))
    achieved = ns_fl / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else 0.0
    log(f"{ms:.3f} ms/step; NS launches {ns_cnt}, {ns_ms / max(ns_cnt, 1):.3f} ms avg, "
        f"{achieved:.1f} TFLOP/s")
    per_tag = {k: {"ms_total": round(v[0], 4), "launches": v[1],
                   "tflops": round(v[2] / (v[0] * 1e-3) / 1e12, 2) if v[0] > 0 else 0.0}
               for k, v in tim.items() if v[1] > 0 and k != "elementwise"}
    ew_ms, ew_n, ew_bytes = tim.get("elementwise", (0.0, 0, 0.0))
    ew_gbs = ew_bytes / (ew_ms * 1e-3) / 1e9 if ew_ms > 0 else 0.0
    line = {
        "metric": METRIC,
        "value": 1000.0 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": workload_name,
                   "matrices": [f"{c}x{m}x{n}" for c, m, n in wl.shapes],
                   "ns_steps": 5, "ns_dtype": dtype, "norm_mode": norm_mode,
                   "weights": dtype, "momentum": "fp32"},
        "step_tflops_alg": wl.ns_flops() / (ms * 1e-3) / 1e12,
        "ms_per_step_instrumented": ms_instr,
        "roofline": {"bound": "mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": achieved / (PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS),
                     "traffic": recorded_traffic() if workload_name == "llama8b_layer_muon_bf16" else None,
                     "kernel": "Newton-Schulz contraction (X X^T, A A, B X)",
                     "launches": ns_cnt, "avg_launch_ms": ns_ms / max(ns_cnt, 1),
                     "alg_tflop_per_launch": ns_fl / max(ns_cnt, 1) / 1e12},
        "kernels": per_tag,
        "ms_per_step_median": statistics.median(per_step),
        "ms_per_step_p90": per_step[min(len(per_step) - 1, int(0.9 * len(per_step)))],
        # the memory-bound passes (momentum EMA with its norm, X0 cast, Muon+
        # sums of squares, update): algorithmic bytes / their event time
        "elementwise": {"ms_per_step": ew_ms / args.steps, "launches": ew_n,
                        "bytes_per_step": ew_bytes / args.steps, "achieved_gbs": ew_gbs,
                        "peak_gbs": PEAK_HBM_GBS, "frac": ew_gbs / PEAK_HBM_GBS},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline_muon(groups, sample[2])
    return line


# ---------------------------------------------------------------------------
# SOAP / FOAM workloads
# ---------------------------------------------------------------------------

def _padded_empty(torch, rows, cols, dtype):
    ld = (cols + 7) // 8 * 8
    return torch.empty((rows, ld), dtype=dtype, device="cuda")[:, :cols]


def qr_fused_bytes(n, nb=64):
    """HBM bytes the fused QR panel updates move for one n x n refresh: every
    element of each updated block is read and written once in fp32 (the
    factorisation's next-panel rows and the rest of the trailing rows, columns
    >= the panel; the explicit-Q blocks below and right of each panel)."""
    elems = 0
    panels = -(-n // nb)
    for p in range(1, panels):
        j0 = p * nb
        length = n - j0
        elems += length * length          # factorisation: rows >= j0, columns >= j0
        elems += length * length          # explicit Q: the block at j0
    return 8.0 * elems


def soap_alg_flops(m, n, refresh=True):
    """SYRK m^2 n + n^2 m (half cost), refresh 2(m^3 + n^3) (F Q) + 8/3 (m^3 + n^3)
    (Householder QR with explicit Q), rotations 2 x (2mn(m + n)) forward (G, M)
    and 2mn(m + n) back."""
    f = m * m * n + n * n * m + 6.0 * m * n * (m + n)
    if refresh:
        f += (2.0 + 8.0 / 3.0) * (m ** 3 + n ** 3)
    return f


def foam_alg_flops(m, n, checked=False, refreshed=False):
    """SYRK n^2 m (half cost), rotations 2 x 2mn^2 (G, M) + back 2mn^2; a check
    adds 4 n^3, a refresh 8/3 n^3."""
    f = n * n * m + 6.0 * m * n * n
    if checked:
        f += 4.0 * n ** 3
    if refreshed:
        f += 8.0 / 3.0 * n ** 3
    return f


class SoapLikeWorkload:
    """A set of matrices stepped together by soap_step_many or foam_step_many
    (equal-size QR refreshes batched), with a ring of two gradients per
    matrix."""

    def __init__(self, kind, config, specs, g_dtype, w_dtype, pf=10, tol=0.1, side="input",
                 refresh="qr", back="f32", fwd="f32", prod="f32"):
        import torch

        import matrix_aware_optimizers_amd as mao
        import synth
        self.mao, self.lib, self.kind = mao, mao.load(), kind
        self.items = []
        tg = torch.bfloat16 if g_dtype == "bf16" else torch.float32
        tw = torch.bfloat16 if w_dtype == "bf16" else torch.float32
        if kind == "foam" and refresh == "eigh":
            prod = "f32"  # the eigendecomposition takes fp32 criterion products
        self.prod = prod
        if kind == "soap":
            self.hp = mao.soap_hparams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                                       refresh_every=1, back_rot_dtype=back, fwd_rot=fwd,
                                       refresh_prod=prod)
        else:
            self.hp = mao.foam_hparams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                                       pf=pf, tol=tol, side=side, refresh=refresh,
                                       back_rot_dtype=back, fwd_rot=fwd, refresh_prod=prod)
        for idx, sp in enumerate(specs):
            if idx % 16 == 15:
                log(f"  {idx + 1}/{len(specs)} matrices set up")
            m, n = sp.rows, sp.cols
            W = _padded_empty(torch, m, n, tw)
            W.copy_(torch.from_numpy(synth.init_weight(config, sp)))
            Gs = []
            for k in range(2):
                G = _padded_empty(torch, m, n, tg)
                G.copy_(torch.from_numpy(synth.gradient(config, sp, k + 1)))
                Gs.append(G)
            z = lambda r, c: _padded_empty(torch, r, c, torch.float32).zero_()
            if kind == "soap":
                st = {"M": z(m, n), "V": z(m, n), "L": z(m, m), "R": z(n, n),
                      "QL": z(m, m), "QR": z(n, n)}
                st["QL"].fill_diagonal_(1.0)
                st["QR"].fill_diagonal_(1.0)
                cst = mao.soap_state(st["M"], st["V"], st["L"], st["R"], st["QL"], st["QR"])
            else:
                k = m if side == "output" else n
                st = {"M": z(m, n), "R": z(k, k), "QR": z(k, k),
                      "r": torch.zeros(m, device="cuda"), "c": torch.zeros(n, device="cuda"),
                      "aux": torch.zeros(4, device="cuda")}
                st["QR"].fill_diagonal_(1.0)
                cst = mao.FoamStateC(mao.mat(st["M"]), mao.mat(st["R"]), mao.mat(st["QR"]),
                                     st["r"].data_ptr(), st["c"].data_ptr(), st["aux"].data_ptr())
            self.items.append((sp, W, Gs, st, cst, mao.mat(W), [mao.mat(G) for G in Gs]))
        k = len(self.items)
        self.Ws = (mao.Mat * k)(*[it[5] for it in self.items])
        self.Gs = [(mao.Mat * k)(*[it[6][r] for it in self.items]) for r in range(2)]
        St = mao.SoapStateC if kind == "soap" else mao.FoamStateC
        self.sts = (St * k)(*[it[4] for it in self.items])
        size = (self.lib.soap_step_many_workspace_size if kind == "soap"
                else self.lib.foam_step_many_workspace_size)
        need = size(k, self.Ws, ctypes.byref(self.hp))
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.embedding = None
        torch.cuda.synchronize()

    def add_embedding(self, rows, cols):
        import torch

        import synth
        w = (0.02 * torch.randn(rows, cols, generator=torch.Generator().manual_seed(5))).cuda()
        g = [torch.from_numpy(synth.embedding_gradient(k + 1, rows, cols)).cuda() for k in range(2)]
        self.embedding = (w, g, torch.zeros_like(w), torch.zeros_like(w))

    def step(self, t: int):
        fn = self.lib.soap_step_many if self.kind == "soap" else self.lib.foam_step_many
        rc = fn(len(self.items), self.Ws, self.Gs[t % 2], self.sts, t, ctypes.byref(self.hp),
                ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(), None, self.stream)
        if rc != 0:
            self.mao._check(rc, self.kind + "_step_many")
        if self.embedding is not None:
            w, g, m, v = self.embedding
            rc = self.lib.adamw_step(w.data_ptr(), 0, g[t % 2].data_ptr(), 0, m.data_ptr(),
                                     v.data_ptr(), w.numel(), t, 1e-3, 0.9, 0.95, 1e-8, 0.1, None,
                                     self.stream)
            if rc != 0:
                self.mao._check(rc, "adamw_step")


def run_soaplike(args, workload_name, kind, config, specs, g_dtype, w_dtype, embedding=None,
                 side="input", split_steps=0, refresh="qr", back="f32", fwd="f32", prod="f32"):
    import torch

    import matrix_aware_optimizers_amd as mao
    log(f"setting up {workload_name} ({len(specs)} matrices)")
    wl = SoapLikeWorkload(kind, config, specs, g_dtype, w_dtype, side=side, refresh=refresh,
                          back=back, fwd=fwd, prod=prod)
    if embedding:
        wl.add_embedding(*embedding)
    log("warmup")
    t = 1
    w0 = time.perf_counter()
    for _ in range(args.warmup):
        wl.step(t)
        t += 1
    torch.cuda.synchronize()
    # steps of a second or more: wait for each step and say so, so that a long
    # run keeps printing (the added host wait per step is microseconds)
    slow = (time.perf_counter() - w0) / max(args.warmup, 1) > 1.0
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    def region(steps, tag):
        nonlocal t
        start.record()
        for i in range(steps):
            wl.step(t)
            t += 1
            if slow:
                torch.cuda.synchronize()
                log(f"{tag} step {i + 1}/{steps} done")
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    # timed region without per-launch instrumentation, then a shorter one with
    # HIP events around every contraction launch for the per-kernel split
    ms = region(args.steps, "timed")
    split_steps = max(1, min(args.steps, split_steps if split_steps else args.steps))
    mao.timing_collect()
    mao.timing_enable(True)
    ms_instr = region(split_steps, "instrumented")
    mao.timing_enable(False)
    tim = mao.timing_collect()
    per_tag = {k: {"ms_total": round(v[0], 4), "launches": v[1],
                   "tflops": round(v[2] / (v[0] * 1e-3) / 1e12, 2) if v[0] > 0 else 0.0}
               for k, v in tim.items() if v[1] > 0}
    # roofline of the dominant kernel class: the fused QR panel updates
    # against HBM where they run ungated (SOAP refreshes every step), else
    # the bf16 products (rotations) against the bf16 peak. Launches gated by
    # FOAM's device-side refresh flag are timed apart ("gated").
    if "qr_fused" in tim and tim["qr_fused"][0] > 0:
        fused_ms = tim["qr_fused"][0] / split_steps
        nbytes = 0.0
        for sp in specs:
            if kind == "soap":
                nbytes += qr_fused_bytes(sp.rows) + qr_fused_bytes(sp.cols)
        achieved = nbytes / (fused_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                "kernel": "qr_fused_update_kernel (QR refresh: panel update and next projection, "
                          "8 B per element of each updated block)",
                "alg_bytes_per_step": nbytes, "ms_per_step": fused_ms}
    else:
        t = tim.get("other_bf16", (0.0, 0, 0.0))
        achieved = t[2] / (t[0] * 1e-3) / 1e12 if t[0] > 0 else 0.0
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                "kernel": "gemm_bf16_dl_kernel products on bf16 MFMA (bf16x3 rotations, rotation "
                          "back), executed flops"}
    log(f"{ms:.3f} ms/step; dominant kernel {roof['achieved']:.1f} {roof['unit']}")
    return {
        "metric": METRIC, "value": 1000.0 / ms, "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload_name, "matrices": len(specs), "optimizer": kind,
                   "gradients": g_dtype, "weights": w_dtype, "back_rotation": back,
                   "forward_rotation": fwd, "refresh_products": wl.prod, **({"side": side, "refresh": refresh} if kind == "foam" else {})},
        "roofline": roof,
        "kernels": per_tag,
        "ms_per_step_instrumented": ms_instr,
        "instrumented_steps": split_steps,
    }


def soap8b_summary(args):
    """The 8B layer under SOAP (soap_step_many over the five matrices, refresh
    every step, bf16 W and G, fp32 state, rotation back in bf16, forward
    rotations and power-iteration products as bf16x3 unless --fwd /
    --refresh-prod say f32): steps/s from a timed region without
    instrumentation, and the contraction split from an instrumented step.
    fp32 MFMA work (the QR's updates and projections, and any fp32 rotation
    or product) is given against both the fp32 and the bf16 dense peaks; the
    bf16 products (bf16x3 products counted at the three bf16 products they
    execute, factor SYRKs of the bf16 gradient, rotation back) against the
    bf16 peak."""
    import synth
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup = args.soap8b_steps, 2
    line = run_soaplike(sub, "llama8b_layer_soap", "soap", "c3", synth.specs("c3"), "bf16",
                        "bf16", split_steps=1, back="bf16", fwd=args.fwd,
                        prod=args.refresh_prod)
    k = line["kernels"]
    out = {"workload": "llama8b_layer_soap", "value": line["value"], "unit": "steps/s",
           "ms_per_step": line["ms_per_step"], "steps": sub.steps, "warmup": sub.warmup,
           "back_rotation": "bf16", "forward_rotation": args.fwd,
           "refresh_products": args.refresh_prod}
    out["qr_fused_hbm"] = {k: line["roofline"][k] for k in ("achieved", "unit", "frac")}
    for tag, name in (("other", "rotations_and_products"), ("qr", "qr_updates"),
                      ("qr_proj", "qr_projections"), ("qr_fused", "qr_fused_updates"),
                      ("qr_panel", "qr_panels"), ("other_bf16", "bf16_products")):
        if tag in k:
            tf = k[tag]["tflops"]
            out[name] = {"ms_per_step": k[tag]["ms_total"] / line["instrumented_steps"]}
            if tag == "qr_panel":  # latency-bound factorisations: time only
                continue
            out[name].update({"tflops": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS})
            if tag != "other_bf16":
                out[name]["frac_fp32_peak"] = tf / PEAK_F32_TFLOPS
    return out


def other_configs(args):
    """The MoE expert bank under Muon+ and the GPT-2-760M set under FOAM
    (the pages' other two workloads at full size), each timed on its own for
    --others-steps steps (FOAM: from t = 2, so its criterion and refresh at
    t = 11 fall inside a 10-step region); compact lines next to the default
    one."""
    import gc

    import torch

    import synth
    out = {}
    for name in ("moe", "foam760m"):
        gc.collect()
        torch.cuda.empty_cache()
        sub = argparse.Namespace(**vars(args))
        sub.steps, sub.warmup, sub.no_cpu_baseline = args.others_steps, 1 if name == "foam760m" else 2, True
        if name == "moe":
            line = run_muon(sub, "moe128_expert_bank_muonplus_bf16", moe_groups(), "col_row",
                            (1536, 2048, "c4", 0))
        else:
            line = run_soaplike(sub, "gpt2_760m_foam", "foam", "c5", synth.specs("c5"), "f32", "f32",
                                embedding=(synth.GPT2_VOCAB, synth.GPT2_760M_WIDTH),
                                back=args.back, fwd=args.fwd, prod=args.refresh_prod)
        r = line["roofline"]
        out[name] = {"workload": line["config"]["workload"], "value": line["value"],
                     "unit": line["unit"], "ms_per_step": line["ms_per_step"],
                     "steps": sub.steps, "warmup": sub.warmup,
                     "roofline": {k: r[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                                    "kernel")}}
        if "elementwise" in line:
            out[name]["elementwise"] = line["elementwise"]
    return out


def run_observe(args):
    """The observability reductions over the Llama-8B layer set, each timed on
    its own with events on the library's stream: the update RMS of the five
    fp32 updates (one read), their Newton-Schulz residuals (fp32 SYRK on the
    wide orientation), the rank-1 share of a 4096 x 14336 second moment (30
    power steps) and the Rayleigh quotients of a 4096 x 4096 factor in a
    basis. One pass = all four."""
    import torch

    import matrix_aware_optimizers_amd as mao
    import synth
    specs = synth.specs("c2")
    gen = torch.Generator(device="cuda").manual_seed(7)
    ups = []
    for sp in specs:
        u = _padded_empty(torch, sp.rows, sp.cols, torch.float32)
        u.normal_(generator=gen)
        ups.append(u)
    v = _padded_empty(torch, 4096, 14336, torch.float32)
    v.normal_(generator=gen)
    v.mul_(v)
    f = _padded_empty(torch, 4096, 4096, torch.float32)
    f.normal_(generator=gen)
    f.copy_(f @ f.T / 4096.0)
    q = torch.linalg.qr(torch.randn(4096, 4096, device="cuda", generator=gen))[0].contiguous()
    scales = [math.sqrt(sp.cols / sp.rows) for sp in specs]
    iters = 30
    calls = {
        "update_rms": lambda: [mao.matrix_rms(u) for u in ups],
        "ns_residual": lambda: [mao.ns_residual(u, sc) for u, sc in zip(ups, scales)],
        "rank1_share": lambda: mao.rank1_share(v, iters),
        "rayleigh": lambda: mao.rayleigh(f, q),
    }
    elems = sum(sp.rows * sp.cols for sp in specs)
    work = {
        "update_rms": (4.0 * elems, "GB/s"),
        "ns_residual": (float(sum(min(sp.rows, sp.cols) ** 2 * max(sp.rows, sp.cols)
                                  for sp in specs)), "TFLOP/s"),
        "rank1_share": (4.0 * 4096 * 14336 * (2 * iters + 2), "GB/s"),
        "rayleigh": (2.0 * 4096 ** 3, "TFLOP/s"),
    }
    out, total = {}, 0.0
    for name, fn in calls.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        amount, unit = work[name]
        rate = amount / (ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
        out[name] = {"ms": round(ms, 4), unit: round(rate, 1)}
        total += ms
        log(f"{name}: {ms:.3f} ms, {rate:.1f} {unit}")
    rms = out["update_rms"]["GB/s"]
    return {
        "metric": "observability passes/s on 8B-layer matrix set", "value": 1000.0 / total,
        "unit": "passes/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "llama8b_layer_observability", "matrices": len(specs),
                   "rank1_iters": iters},
        "roofline": {"bound": "hbm", "achieved": rms, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": rms / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "sumsq_partial_kernel (update RMS)"},
        "kernels": out,
    }


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "moe", "c1muon", "c1soap", "soap8b", "foam760m",
                             "foam760m_output", "foam760m_eigh", "soap760m", "observe8b"])
    ap.add_argument("--back", default="bf16", choices=["f32", "bf16"],
                    help="precision of the rotation back of the SOAP / FOAM workloads")
    ap.add_argument("--fwd", default="bf16x3", choices=["f32", "bf16x3"],
                    help="forward rotations of the SOAP / FOAM workloads: fp32 products, or "
                         "three bf16 products over hi/lo splits (fp32-accurate)")
    ap.add_argument("--refresh-prod", default="bf16x3", choices=["f32", "bf16x3"],
                    help="power-iteration products L Q / R Q of SOAP and the criterion products "
                         "of FOAM: fp32, or bf16x3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--soap8b-steps", type=int, default=5,
                    help="timed steps of the 8B layer under SOAP reported beside the default "
                         "workload (0: skip)")
    ap.add_argument("--others-steps", type=int, default=10,
                    help="timed steps of the MoE bank (Muon+) and of GPT-2-760M (FOAM) reported "
                         "beside the default workload (0: skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (a known-size reference "
                         "for profiler byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 counter CSVs of this workload into the "
                         "committed traffic record, then exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic,
                      command="rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -f csv -- python3 "
                              "bench.py --steps 2 --warmup 1 --no-cpu-baseline --soap8b-steps 0 "
                              "--others-steps 0 --calibrate-copy")
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build's step runs whole matrices on one device "
              "and has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")
        del src, dst
    if args.workload == "llama8b":
        line = run_muon(args, "llama8b_layer_muon_bf16", llama8b_groups(), "none",
                        (4096, 4096, "c2", 1))
        if args.soap8b_steps > 0:
            import gc
            gc.collect()
            torch.cuda.empty_cache()
            line["soap8b"] = soap8b_summary(args)
        if args.others_steps > 0:
            line.update(other_configs(args))
    elif args.workload == "moe":
        line = run_muon(args, "moe128_expert_bank_muonplus_bf16", moe_groups(), "col_row",
                        (1536, 2048, "c4", 0))
    elif args.workload == "c1muon":
        import synth
        line = run_muon(args, "single_256x512_muon_f32", [("w", synth.specs("c1"))], "none",
                        (256, 512, "c1", 0), dtype="f32")
    elif args.workload == "c1soap":
        import synth
        line = run_soaplike(args, "single_256x512_soap_f32", "soap", "c1", synth.specs("c1"),
                            "f32", "f32", back=args.back, fwd=args.fwd, prod=args.refresh_prod)
    elif args.workload == "soap8b":
        import synth
        line = run_soaplike(args, "llama8b_layer_soap", "soap", "c3", synth.specs("c3"),
                            "bf16", "bf16", back=args.back, fwd=args.fwd, prod=args.refresh_prod)
    elif args.workload == "foam760m_eigh":
        import synth
        line = run_soaplike(args, "gpt2_760m_foam_eigh_refresh", "foam", "c5", synth.specs("c5"),
                            "f32", "f32", embedding=(synth.GPT2_VOCAB, synth.GPT2_760M_WIDTH),
                            refresh="eigh", back=args.back, fwd=args.fwd, prod=args.refresh_prod)
    elif args.workload == "foam760m":
        import synth
        line = run_soaplike(args, "gpt2_760m_foam", "foam", "c5", synth.specs("c5"), "f32", "f32",
                            embedding=(synth.GPT2_VOCAB, synth.GPT2_760M_WIDTH), back=args.back, fwd=args.fwd, prod=args.refresh_prod)
    elif args.workload == "foam760m_output":
        import synth
        line = run_soaplike(args, "gpt2_760m_foam_output_side", "foam", "c5", synth.specs("c5"),
                            "f32", "f32", embedding=(synth.GPT2_VOCAB, synth.GPT2_760M_WIDTH),
                            side="output", back=args.back, fwd=args.fwd, prod=args.refresh_prod)
    elif args.workload == "observe8b":
        line = run_observe(args)
    else:
        import synth
        line = run_soaplike(args, "gpt2_760m_soap", "soap", "c5", synth.specs("c5"), "f32", "f32",
                            back=args.back, fwd=args.fwd, prod=args.refresh_prod)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
