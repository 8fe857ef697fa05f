"""Full-size parity on the named workloads, in the launch configuration the benchmark
times (one fla_linattn_fwd call with the library's automatic schedule).

The oracle runs every head of every workload; the million-token workload records a
sample of ~1% of the output rows (every 97th token and the last one) plus the whole
final state, to bound host memory.
"""
import sys
import time

import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_host
from workloads import WORKLOADS, generate_torch, to_numpy_input

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size_workload(name):
    w = WORKLOADS[name]
    print(f"[workload] {name}: {w}", flush=True)
    t0 = time.time()
    inp = generate_torch(w, "cuda")
    out, fin = fla.fwd(inp["q"], inp["k"], inp["v"], inp["decay"], decay_kind=w.decay,
                       init_state=inp["init"], chunk=w.chunk, phi_elu1=w.phi_elu1,
                       normalize=w.normalize)
    torch.cuda.synchronize()
    print(f"[workload] {name}: gpu done {time.time() - t0:.1f}s", flush=True)
    host = {k: (None if v is None else to_numpy_input(v)) for k, v in inp.items()}
    rows = None
    if w.T > 100000:
        rows = list(range(0, w.T, 97)) + ([w.T - 1] if (w.T - 1) % 97 else [])
    ro, rf = oracle.fwd(host["q"], host["k"], host["v"], host["decay"], w.decay, host["init"],
                        phi_elu1=w.phi_elu1, normalize=w.normalize, rows=rows)
    print(f"[workload] {name}: oracle done {time.time() - t0:.1f}s", flush=True)
    del host
    o = out if rows is None else out[:, :, torch.tensor(rows, device=out.device)]
    o = to_host(o)
    f = to_host(fin)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(f))
    assert torch.isfinite(out.float()).all().item()
    eo, ef = rel_err(o, ro), rel_err(f, rf)
    print(f"[workload] {name}: out rel err {eo:.3e}, final rel err {ef:.3e}", flush=True)
    tol = TOL[w.dtype]
    assert eo <= tol and ef <= tol
