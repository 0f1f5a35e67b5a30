"""Mutation sweep of the fp64 oracle against its CPU pins.

Applies one plausible mistake at a time (a dropped or rescaled term, a wrong
sign, index or transposed operand, an off-by-one schedule) to a scratch copy
of the repository and runs tests/test_oracle_pins.py there; every mutant must
make a pin fail. Not collected by pytest (it runs the pin suite once per
mutant, about a minute in all):

    python tests/oracle_mutation_sweep.py [index ...]

Exit status 1 when a mutant survives. The one change of qr_positive's sign
rule for an exactly zero diagonal entry of R is listed as equivalent: either
choice keeps diag(R) >= 0, so both results are correct."""
import os, shutil, subprocess, sys
import tempfile
SRC = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DST = os.path.join(tempfile.gettempdir(), "mao_oracle_mutants", "repo")
M = [
 ("oracle/muon.py", "(1.0 - mu) * g", "(1.0 - mu) * g * 1.01"),
 ("oracle/muon.py", "mu * np.asarray(mom", "0.9 * mu * np.asarray(mom"),
 ("oracle/muon.py", "x / (np.linalg.norm(x) + eps)", "x / (np.linalg.norm(x) + 1e-3)"),
 ("oracle/muon.py", "poly = b * gram + c * (gram @ gram)", "poly = b * gram + c * (gram @ gram.T @ gram)"),
 ("oracle/muon.py", "x = a * x + poly @ x", "x = a * x + x @ x.T @ poly @ x"),
 ("oracle/muon.py", "np.sqrt(rows / cols) * o", "np.sqrt(cols / rows) * o"),
 ("oracle/muon.py", "target = np.linalg.norm(x) / np.sqrt(n)", "target = np.linalg.norm(x) / np.sqrt(m)"),
 ("oracle/muon.py", "return row(col(o))", "return col(row(o))"),
 ("oracle/muon.py", "return col(row(o))", "return row(col(o))"),
 ("oracle/muon.py", "w - lr * (weight_decay * w + upd)", "w - lr * (weight_decay * w - upd)"),
 ("oracle/muon.py", "norms = np.sqrt(np.sum(x * x, axis=1))", "norms = np.sqrt(np.sum(x * x, axis=1)) + 1e-3"),
 ("oracle/soap.py", "s.L = beta2 * s.L + (1.0 - beta2) * (g @ g.T)", "s.L = beta2 * s.L + (1.0 - beta2) * (g @ g.T) * 1.0001"),
 ("oracle/soap.py", "info[\"PL\"] = s.L @ s.QL", "info[\"PL\"] = s.L"),
 ("oracle/soap.py", "info[\"PR\"] = s.R @ s.QR", "info[\"PR\"] = s.R"),
 ("oracle/soap.py", "info[\"PL\"] = s.L @ s.QL", "info[\"PL\"] = s.QL.T @ s.L"),
 ("oracle/soap.py", "g_rot = s.QL.T @ g @ s.QR", "g_rot = s.QL @ g @ s.QR"),
 ("oracle/soap.py", "g_rot = s.QL.T @ g @ s.QR", "g_rot = s.QL.T @ g @ s.QR.T"),
 ("oracle/soap.py", "m_rot = s.QL.T @ s.M @ s.QR", "m_rot = s.QL.T @ s.M @ s.QR.T"),
 ("oracle/soap.py", "m_rot = s.QL.T @ s.M @ s.QR", "m_rot = s.QL @ s.M @ s.QR"),
 ("oracle/soap.py", "(1.0 - beta2) * g_rot * g_rot", "(1.0 - beta2) * m_rot * m_rot"),
 ("oracle/soap.py", "upd = s.QL @ n_rot @ s.QR.T", "upd = s.QL.T @ n_rot @ s.QR"),
 ("oracle/soap.py", "upd = s.QL @ n_rot @ s.QR.T", "upd = s.QL @ n_rot @ s.QR"),
 ("oracle/soap.py", "(m_rot / b1) / (np.sqrt(s.V / b2) + eps)", "(m_rot / b1) / (np.sqrt(s.V / b1) + eps)"),
 ("oracle/soap.py", "(m_rot / b1) / (np.sqrt(s.V / b2) + eps)", "(m_rot) / (np.sqrt(s.V / b2) + eps)"),
 ("oracle/soap.py", "return refresh_every > 0 and (t - 1) % refresh_every == 0", "return refresh_every > 0 and t % refresh_every == 0"),
 ("oracle/soap.py", "s.M = beta1 * s.M + (1.0 - beta1) * g", "s.M = beta1 * s.M + (1.0 - beta1) * g * 1.0001"),
 ("oracle/foam.py", "info[\"P\"] = s.R @ s.QR", "info[\"P\"] = s.R"),
 ("oracle/foam.py", "info[\"P\"] = s.R @ s.QR", "info[\"P\"] = s.QR.T @ s.R"),
 ("oracle/foam.py", "refresh = rho > tol", "refresh = rho >= tol"),
 ("oracle/foam.py", "d = s.QR.T @ s.R @ s.QR", "d = s.R"),
 ("oracle/foam.py", "s.r = beta2 * s.r + (1.0 - beta2) * sq.mean(axis=1)", "s.r = beta2 * s.r + (1.0 - beta2) * sq.sum(axis=1)"),
 ("oracle/foam.py", "s.c = beta2 * s.c + (1.0 - beta2) * sq.mean(axis=0)", "s.c = beta2 * s.c + (1.0 - beta2) * sq.sum(axis=0)"),
 ("oracle/foam.py", "tau = float(np.trace(s.R / b2) / denom)", "tau = float(np.trace(s.R) / denom)"),
 ("oracle/foam.py", "n_rot = (m_rot / b1) / (np.sqrt(v_hat) + eps)", "n_rot = (m_rot) / (np.sqrt(v_hat) + eps)"),
 ("oracle/foam.py", "upd = (s.QR @ n_rot) if out_side else (n_rot @ s.QR.T)", "upd = (s.QR.T @ n_rot) if out_side else (n_rot @ s.QR.T)"),
 ("oracle/foam.py", "upd = (s.QR @ n_rot) if out_side else (n_rot @ s.QR.T)", "upd = (s.QR @ n_rot) if out_side else (n_rot @ s.QR)"),
 ("oracle/foam.py", "m_rot = s.M @ s.QR", "m_rot = s.M @ s.QR.T"),
 ("oracle/foam.py", "m_rot = s.QR.T @ s.M", "m_rot = s.QR @ s.M"),
 ("oracle/foam.py", "return (t - 1) % pf == 0", "return t % pf == 0"),
 ("oracle/foam.py", "s.R = beta2 * s.R + (1.0 - beta2) * ((g @ g.T) if out_side else (g.T @ g))", "s.R = beta2 * s.R + (1.0 - beta2) * ((g @ g.T) if out_side else (g.T @ g)) * 1.001"),
 ("oracle/linalg.py", "order = np.argsort(-w, kind=\"stable\")", "order = np.argsort(w, kind=\"stable\")"),
 ("oracle/foam.py", "info[\"eigenvalues\"], s.QR = eigh_descending(s.R, ref=s.QR)", "info[\"eigenvalues\"], s.QR = eigh_descending(s.R @ s.QR, ref=s.QR)"),
 ("oracle/adamw.py", "(m_new / b1) / (np.sqrt(v_new / b2) + eps)", "(m_new / b1) / (np.sqrt(v_new / b2) + 1e-3)"),
 ("oracle/adamw.py", "w - lr * (weight_decay * w + upd)", "w - lr * (weight_decay * w) - lr * upd * 1.001"),
 ("oracle/linalg.py", "return q * d[None, :], r * d[:, None]", "return q, r"),
 ("oracle/observe.py", "return float(np.sqrt(np.sum(e * e) / a))", "return float(np.sqrt(np.sum(e * e)) / a)"),
 ("oracle/observe.py", "s1 = np.linalg.svd(v, compute_uv=False)[0]", "s1 = np.linalg.svd(v, compute_uv=False)[0] * 1.0001"),
]
only = sys.argv[1:]
survivors = []
for i, (f, old, new) in enumerate(M):
    if only and str(i) not in only:
        continue
    if os.path.exists(DST):
        shutil.rmtree(DST)
    shutil.copytree(SRC, DST, ignore=shutil.ignore_patterns(".git", "_work", "gpurun_out", "_build", "*.so", "__pycache__"))
    p = os.path.join(DST, f)
    s = open(p).read()
    if old not in s:
        print(f"[{i}] PATTERN MISSING {f}: {old}"); continue
    open(p, "w").write(s.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q", "-p", "no:cacheprovider"], cwd=DST, capture_output=True, text=True)
    caught = r.returncode != 0
    print(f"[{i}] {'caught ' if caught else 'SURVIVES'} {f}: {new}", flush=True)
    if not caught:
        survivors.append(i)
print("survivors:", survivors)
sys.exit(1 if survivors else 0)
