"""Parity at the benchmark workloads' full sizes, in the launch configurations
the benchmark times (GPU).

* The Llama-8B layer Muon step is one grouped call over all five matrices;
  the O (4096x4096) and QKV (4096x6144) updates are compared with the oracle
  in full.
* The 128-expert MoE bank is one batched Muon+ call over all 384 matrices; six
  sampled matrices are compared in full.
* SOAP on the 8B layer: O and QKV teacher-forced in full at t = 1; the
  14336-sized factors of the gate projection through sampled rows of the
  factor EMAs, sampled columns of the refreshed basis (orthonormality,
  Q^T P upper triangular, non-negative diagonal) and sampled rows of V.
* FOAM on one GPT-2-760M layer at full size, t = 1 (criterion evaluated,
  basis refreshed), teacher-forced.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import bf16_round
from tests.helpers import log, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

LR, WD, MU = 1e-3, 0.1, 0.95
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def test_llama8b_layer_grouped_muon(gpu_lib):
    import torch
    log("llama8b grouped muon (5 matrices, one call)")
    groups, host = [], []
    for sp in synth.specs("c2"):
        w = bf16_round(synth.init_weight("c2", sp))
        g = bf16_round(synth.gradient("c2", sp, 1))
        W, G = to_dev(w[None], "bf16"), to_dev(g[None], "bf16")
        M = torch.zeros(W.shape, dtype=torch.float32, device="cuda")
        groups.append((W, G, M))
        host.append((sp, w, g))
    outs = [torch.empty(W.shape, dtype=torch.float32, device="cuda") for W, _, _ in groups]
    gpu_lib.muon_step_batched(groups, update_out=outs, lr=LR, mu=MU, weight_decay=WD, ns_steps=5,
                              ns_dtype="bf16")
    torch.cuda.synchronize()
    for (sp, w, g), out in zip(host, outs):
        if sp.name not in ("o", "qkv"):
            continue
        _, _, upd = oracle.muon_step(w, g, np.zeros(w.shape), lr=LR, mu=MU, weight_decay=WD,
                                     ns_steps=5)
        e = rel(to_host(out[0]), upd)
        log(f"  {sp.name} {sp.rows}x{sp.cols}: update error {e:.2e}")
        assert e < 2e-2


def test_moe_bank_batched_muon_plus(gpu_lib):
    import torch
    log("moe bank batched muon+ (384 matrices, one call)")
    specs = synth.specs("c4")
    groups, outs = [], []
    sample = {("gate", 0), ("up", 37), ("down", 5), ("gate", 101), ("down", 127), ("up", 64)}
    keep = {}
    for name in ("gate", "up", "down"):
        sps = [s for s in specs if s.name.endswith("." + name)]
        m, n = sps[0].rows, sps[0].cols
        W = torch.empty((len(sps), m, n), dtype=torch.bfloat16, device="cuda")
        G = torch.empty_like(W)
        for b, sp in enumerate(sps):
            w = synth.init_weight("c4", sp)
            g = synth.gradient("c4", sp, 1)
            W[b].copy_(torch.from_numpy(w))
            G[b].copy_(torch.from_numpy(g))
            if (name, b) in sample:
                keep[(name, b)] = (bf16_round(w), bf16_round(g))
        M = torch.zeros((len(sps), m, n), dtype=torch.float32, device="cuda")
        groups.append((W, G, M))
        outs.append(torch.empty((len(sps), m, n), dtype=torch.float32, device="cuda"))
    gpu_lib.muon_step_batched(groups, update_out=outs, lr=LR, mu=MU, weight_decay=WD, ns_steps=5,
                              ns_dtype="bf16", norm_mode="col_row")
    torch.cuda.synchronize()
    gi = {"gate": 0, "up": 1, "down": 2}
    for (name, b), (w, g) in sorted(keep.items()):
        _, _, upd = oracle.muon_step(w, g, np.zeros(w.shape), lr=LR, mu=MU, weight_decay=WD,
                                     ns_steps=5, norm_mode="col_row")
        e = rel(to_host(outs[gi[name]][b]), upd)
        log(f"  expert {b} {name}: update error {e:.2e}")
        assert e < 2e-2


def _soap_dev_state(m, n):
    import torch
    z = lambda r, c: torch.zeros((r, c), dtype=torch.float32, device="cuda")
    return {"M": z(m, n), "V": z(m, n), "L": z(m, m), "R": z(n, n),
            "QL": torch.eye(m, dtype=torch.float32, device="cuda"),
            "QR": torch.eye(n, dtype=torch.float32, device="cuda")}


def _idx(a):
    import torch
    return torch.as_tensor(a, dtype=torch.long, device="cuda")


@pytest.mark.parametrize("name", ["o", "qkv"])
def test_soap_full_size_teacher_forced(gpu_lib, name):
    import torch
    sp = [s for s in synth.specs("c3") if s.name == name][0]
    m, n = sp.rows, sp.cols
    log(f"soap full size {name} {m}x{n}")
    w = bf16_round(synth.init_weight("c3", sp))
    g = bf16_round(synth.gradient("c3", sp, 1))
    W = to_dev(w, "bf16")
    st = _soap_dev_state(m, n)
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    gpu_lib.soap_step(W, to_dev(g, "bf16"), st, 1, update_out=out, **HP)
    torch.cuda.synchronize()
    ql, qr = to_host(st["QL"]), to_host(st["QR"])
    prev = oracle.soap_init(m, n)
    _, ref, upd, info = oracle.soap_step(w, g, prev, 1, refresh_every=0, q_override=(ql, qr), **HP)
    assert rel(to_host(st["L"]), ref.L) < 1e-5 and rel(to_host(st["R"]), ref.R) < 1e-5
    for q, p in ((ql, 0.05 * g.astype(np.float64) @ g.T), (qr, 0.05 * g.T.astype(np.float64) @ g)):
        k = q.shape[0]
        assert np.abs(q.T @ q - np.eye(k)).max() < 1e-4
        rr = q.T @ p
        assert np.linalg.norm(np.tril(rr, -1)) < 1e-4 * np.linalg.norm(p)
    # t = 1: the step is a sign function of G~ where |G~| >> eps; compare where
    # the rotated gradient is not at the roundoff level of a rank-deficient side
    ev = rel(to_host(st["V"]), ref.V)
    log(f"  V error {ev:.2e}")
    assert ev < 1e-4


def test_soap_full_size_gate_properties(gpu_lib):
    import torch
    sp = [s for s in synth.specs("c3") if s.name == "gate"][0]
    m, n = sp.rows, sp.cols
    log(f"soap full size gate {m}x{n} (sampled properties)")
    g = bf16_round(synth.gradient("c3", sp, 1)).astype(np.float64)
    W = to_dev(bf16_round(synth.init_weight("c3", sp)), "bf16")
    st = _soap_dev_state(m, n)
    gpu_lib.soap_step(W, to_dev(g, "bf16"), st, 1, **HP)
    torch.cuda.synchronize()
    r = np.random.default_rng(0)
    rows = np.sort(r.choice(m, 24, replace=False))
    L_rows = to_host(st["L"][_idx(rows)])
    assert rel(L_rows, 0.05 * g[rows] @ g.T) < 1e-5
    cols_r = np.sort(r.choice(n, 24, replace=False))
    R_rows = to_host(st["R"][_idx(cols_r)])
    assert rel(R_rows, 0.05 * g[:, cols_r].T @ g) < 1e-5
    # refreshed left basis: P = L Q_prev = L (Q_prev = I); columns j of Q
    ql = st["QL"]
    js = np.sort(np.concatenate([r.choice(4096, 12, replace=False),
                                 4096 + r.choice(m - 4096, 12, replace=False)]))
    qcols = to_host(ql[:, _idx(js)])
    assert np.abs(qcols.T @ qcols - np.eye(len(js))).max() < 1e-4
    # Q^T P is upper triangular: q_i . p_j = 0 for i > j, p_j = 0.05 G G^T e_j
    pj = 0.05 * g @ g[js].T  # columns j of P
    prod = qcols.T @ pj      # (i in js) x (j in js)
    scale = np.linalg.norm(pj, axis=0).max()
    for a, i in enumerate(js):
        for b, j in enumerate(js):
            if i > j:
                assert abs(prod[a, b]) < 1e-4 * scale, (i, j, prod[a, b])
            if i == j and j < 4096:
                assert prod[a, b] > 0
    # V rows at t = 1: V = 0.05 (Q_L^T G Q_R)^2
    qr = to_host(st["QR"])
    vr = np.sort(r.choice(4096, 8, replace=False))
    gt_rows = (to_host(ql[:, _idx(vr)]).T @ g) @ qr
    assert rel(to_host(st["V"][_idx(vr)]), 0.05 * gt_rows ** 2) < 1e-4


def test_foam_full_size_gpt2_layer(gpu_lib):
    import torch
    specs = [s for s in synth.specs("c5") if s.name.startswith("l0.")]
    for sp in specs:
        m, n = sp.rows, sp.cols
        log(f"foam full size {sp.name} {m}x{n}")
        w = synth.init_weight("c5", sp)
        g = synth.gradient("c5", sp, 1)
        W = to_dev(w)
        st = {"M": to_dev(np.zeros((m, n), np.float32)), "R": to_dev(np.zeros((n, n), np.float32)),
              "QR": to_dev(np.eye(n, dtype=np.float32)),
              "r": torch.zeros(m, device="cuda"), "c": torch.zeros(n, device="cuda"),
              "aux": torch.zeros(4, device="cuda")}
        out = torch.empty((m, n), dtype=torch.float32, device="cuda")
        gpu_lib.foam_step(W, to_dev(g), st, 1, update_out=out, pf=10, tol=0.1, **HP)
        torch.cuda.synchronize()
        aux = to_host(st["aux"])
        prev = oracle.foam_init(m, n)
        _, ref, _, info = oracle.foam_step(w, g, prev, 1, pf=10, tol=0.1, **HP)
        assert aux[3] == 1.0 and abs(aux[0] - info["rho"]) < 1e-4
        assert bool(aux[1]) == info["refreshed"]
        q = to_host(st["QR"])
        assert np.abs(q.T @ q - np.eye(n)).max() < 1e-4
        _, ref2, upd, info2 = oracle.foam_step(w, g, prev, 1, pf=10, tol=0.1, q_override=q,
                                               refresh_override=bool(aux[1]), **HP)
        assert rel(to_host(st["r"]), ref2.r) < 1e-4 and rel(to_host(st["c"]), ref2.c) < 1e-4
        assert abs(aux[2] - info2["tau"]) <= 1e-4 * abs(info2["tau"])
        if n <= m:  # R has full rank at t = 1, the update is determined
            e = rel(to_host(out), upd)
            log(f"  update error {e:.2e}")
            assert e < 1e-4
