"""The no-allocation forward entry point (fla_linattn_fwd_noalloc) against fla_linattn_fwd,
through the C ABI: two calls in a row (the second smaller, so the shared scratch array
still holds the first call's contents), plus the scratch-size rejection."""
import sys

import numpy as np
import pytest

from parity_util import TOL, rel_err, to_device, to_host
from workloads import Workload, generate

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def both(w, inp, in_place=False):
    """(out, final) of fla_linattn_fwd and of fla_linattn_fwd_noalloc on the same inputs."""
    bf = w.dtype == "bf16"
    q, k, v = (to_device(inp[n], bf16=bf) for n in ("q", "k", "v"))
    dec = to_device(inp["decay"])
    res = []
    for noalloc in (False, True):
        ini = to_device(inp["init"]) if inp["init"] is not None else None
        fin = ini if in_place else None
        out, fin = fla.fwd(q, k, v, dec, decay_kind=w.decay, init_state=ini, final_state=fin,
                           chunk=w.chunk, phi_elu1=w.phi_elu1, normalize=w.normalize,
                           noalloc=noalloc)
        torch.cuda.synchronize()
        res.append((to_host(out), to_host(fin)))
    return res


def test_noalloc_two_calls_match_allocating_entry_point():
    # 1: the segment schedule (2 heads x 2 value slices over 12,800 tokens: 25 segments),
    #    its workspace in the scratch array
    w1 = Workload("noalloc_seg", 1, 2, 12800, 128, 128, 64, "bf16", "gate", False, False,
                  128 ** -0.5, 0.1, seed=71)
    say(f"[noalloc] call 1: {w1}")
    nseg = fla.segments_for(w1.B, w1.H, w1.T, w1.dk, w1.dv, w1.chunk,
                            fla.flags_for(torch.bfloat16, "gate", False, False))
    assert nseg > 1
    (o_a, f_a), (o_n, f_n) = both(w1, generate(w1))
    assert rel_err(o_n, o_a) <= TOL["bf16"] and rel_err(f_n, f_a) <= TOL["bf16"]
    assert np.array_equal(o_n, o_a) and np.array_equal(f_n, f_a)  # same schedule, same bits
    # 2: smaller, in-place resume with the normaliser over two value slices (the private
    #    start-state copy comes from the scratch array, over call 1's contents)
    w2 = Workload("noalloc_inplace", 1, 2, 300, 64, 128, 64, "f32", "gamma", True, True, 1.0,
                  0.1, gamma_exp="1-2^(-5-h)", seed=72)
    say(f"[noalloc] call 2: {w2}")
    (o_a, f_a), (o_n, f_n) = both(w2, generate(w2), in_place=True)
    assert rel_err(o_n, o_a) <= TOL["f32"] and rel_err(f_n, f_a) <= TOL["f32"]
    assert np.array_equal(o_n, o_a) and np.array_equal(f_n, f_a)


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    # an in-place resume with the normaliser needs a private copy of all start states:
    # 64 x 16 x 128 x 129 fp32 = 67.6 MB > 64 MiB
    B, H, dk, dv = 64, 16, 128, 128
    say("[noalloc] scratch rejection")
    q = torch.zeros((B, H, 1, dk), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((B, H, 1, dv), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((B, H, dk, dv + 1), dtype=torch.float32, device="cuda")
    with pytest.raises(fla.FlaError) as e:
        fla.fwd(q, q, v, None, init_state=st, final_state=st, phi_elu1=True, normalize=True,
                noalloc=True)
    assert e.value.status == fla.FLA_ERR_SCRATCH
