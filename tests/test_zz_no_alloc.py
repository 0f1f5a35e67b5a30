"""The allocation-free Muon entry point against muon_step (GPU).

muon_step_noalloc runs muon_step's kernels on the library's static scratch
array instead of a caller workspace, so on the same inputs its outputs must
equal muon_step's bit for bit. Two calls in a row, the second smaller,
check that nothing depends on what the previous call left in the array."""
import numpy as np
import pytest

from tests.helpers import log, to_dev

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, mu=0.95, weight_decay=0.1, ns_steps=5)


def _case(shape, dtype, seed):
    import torch
    m, n = shape
    r = np.random.default_rng(seed)
    w = (0.02 * r.standard_normal((m, n))).astype(np.float32)
    g = r.standard_normal((m, n)).astype(np.float32)
    m0 = (0.1 * r.standard_normal((m, n))).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return to_dev(w).to(tdt), to_dev(g).to(tdt), to_dev(m0)


@pytest.mark.parametrize("ns_dtype,shapes", [
    ("bf16", [(1536, 2048), (300, 520)]),
    ("bf16", [(2048, 1536), (96, 160)]),
    ("f32", [(1616, 1616), (130, 200)]),
])
def test_noalloc_matches_muon_step_twice(gpu_lib, ns_dtype, shapes):
    import torch
    for i, shape in enumerate(shapes):
        log(f"noalloc {ns_dtype} {shape}")
        W1, G, M1 = _case(shape, ns_dtype, 900 + 10 * i + len(ns_dtype))
        W2, M2 = W1.clone(), M1.clone()
        o1 = torch.empty(shape, dtype=torch.float32, device="cuda")
        o2 = torch.empty(shape, dtype=torch.float32, device="cuda")
        gpu_lib.muon_step(W1, G, M1, update_out=o1, ns_dtype=ns_dtype, **HP)
        gpu_lib.muon_step_noalloc(W2, G, M2, update_out=o2, ns_dtype=ns_dtype, **HP)
        torch.cuda.synchronize()
        assert torch.isfinite(o2).all().item()
        assert torch.equal(o1, o2)
        assert torch.equal(W1, W2) and torch.equal(M1, M2)


def test_noalloc_rejects_steps_beyond_the_array(gpu_lib):
    import torch
    W, G, M = _case((2560, 2560), "bf16", 7)
    with pytest.raises(gpu_lib.MaoError) as e:
        gpu_lib.muon_step_noalloc(W, G, M, ns_dtype="bf16", **HP)
    assert e.value.status == 7
