"""GPU parity of the chunkwise backward (fla_linattn_bwd through the C ABI) against the
fp64 oracle's back-propagation through the recurrence.

Bar (per gradient tensor, over all batches/heads/tokens/columns): max|g - g_ref| /
max|g_ref| <= 1e-5 for fp32 inputs and <= 1e-2 for bf16 inputs (the forward's bar), for
dq, dk, dv, the decay gradient and the initial state's gradient.  The decay gradient sums
phi(q) dphi(q) - phi(k) dphi(k) over all later tokens, so per-token rounding errors add up
along the sequence; the full-size cases (16384 tokens) check that they stay inside the bar.
"""
import itertools
import time

import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_device, to_host
from workloads import (Workload, generate, generate_grads, generate_grads_torch, generate_torch,
                       to_numpy_input, WORKLOADS)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


def say(msg):
    print(msg, flush=True)


def case(dtype, decay, dk, dv, T, *, B=2, H=2, phi=False, init=True, seed=0):
    w = Workload("bwd", B, H, T, dk, dv, 64, dtype, decay, phi, False,
                 1.0 if dtype == "f32" else dk ** -0.5, 0.1 if init else 0.0,
                 gamma_exp="1-2^(-5-h)", seed=seed)
    return w, generate(w)


def run_gpu_bwd(w, inp, grads, want_dgate=True):
    bf = w.dtype == "bf16"
    q, k, v = (to_device(inp[n], bf16=bf) for n in ("q", "k", "v"))
    dec = to_device(inp["decay"])
    ini = to_device(inp["init"])
    do = to_device(grads["dout"], bf16=bf)
    dfin = to_device(grads["dfinal"])
    dq, dk, dv, dg, di = fla.bwd(q, k, v, do, dec, decay_kind=w.decay, init_state=ini,
                                 dfinal=dfin, want_dgate=want_dgate, phi_elu1=w.phi_elu1)
    torch.cuda.synchronize()
    return {"dq": to_host(dq), "dk": to_host(dk), "dv": to_host(dv), "dgate": to_host(dg),
            "dinit": to_host(di)}


def run_oracle_bwd(w, inp, grads):
    init = inp["init"]
    if init is not None:
        init = init[..., :w.dv]
    return oracle.bwd(inp["q"], inp["k"], inp["v"], grads["dout"], inp["decay"], w.decay, init,
                      grads["dfinal"], phi_elu1=w.phi_elu1)


def tol_for(dtype, name):
    return TOL[dtype]


def check_bwd(w, inp, grads, tag):
    say(f"[bwd] {tag}: {w}")
    got = run_gpu_bwd(w, inp, grads)
    ref = run_oracle_bwd(w, inp, grads)
    names = ["dq", "dk", "dv", "dinit"] + (["dgate"] if w.decay in ("gate", "token") else [])
    errs = {}
    for n in names:
        assert got[n] is not None and np.all(np.isfinite(got[n])), (tag, n)
        errs[n] = rel_err(got[n], ref[n])
    say(f"[bwd] {tag}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= tol_for(w.dtype, n), f"{tag}: {n} rel err {e:.3e} > {tol_for(w.dtype, n)}"
    return errs


COMBOS = list(itertools.product(["f32", "bf16"], ["none", "gamma", "gate", "token"],
                                [False, True]))


@pytest.mark.parametrize("dtype,decay,phi", COMBOS)
def test_bwd_flags(dtype, decay, phi):
    i = COMBOS.index((dtype, decay, phi))
    w, inp = case(dtype, decay, 64, 64, 3 * 64 + 5, phi=phi, seed=300 + i)
    g = generate_grads(w)
    check_bwd(w, inp, g, f"flags {dtype} {decay} phi={phi}")


SHAPES = [("bf16", 128, 128), ("bf16", 128, 64), ("bf16", 64, 128), ("bf16", 256, 128),
          ("bf16", 128, 256), ("bf16", 256, 256), ("f32", 128, 128), ("f32", 64, 128)]


@pytest.mark.parametrize("dtype,dk,dv", SHAPES)
@pytest.mark.parametrize("decay", ["gate", "token", "gamma"])
def test_bwd_shapes(dtype, dk, dv, decay):
    i = SHAPES.index((dtype, dk, dv))
    w, inp = case(dtype, decay, dk, dv, 2 * 64 + 33, B=1, H=2, phi=(i % 2 == 1), seed=400 + i)
    g = generate_grads(w)
    check_bwd(w, inp, g, f"shape {dtype} dk={dk} dv={dv} {decay}")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 128])
def test_bwd_lengths(T):
    w, inp = case("bf16", "gate", 64, 64, T, seed=500 + T)
    g = generate_grads(w)
    check_bwd(w, inp, g, f"T={T}")


def test_bwd_without_init_and_dfinal():
    w, inp = case("f32", "gate", 64, 64, 150, init=False, seed=600)
    g = generate_grads(w, with_dfinal=False)
    check_bwd(w, inp, g, "no init, no dfinal")


def test_bwd_skip_dgate_matches():
    w, inp = case("bf16", "gate", 64, 128, 200, seed=601)
    g = generate_grads(w)
    a = run_gpu_bwd(w, inp, g, want_dgate=True)
    b = run_gpu_bwd(w, inp, g, want_dgate=False)
    assert b["dgate"] is None
    for n in ("dq", "dk", "dv", "dinit"):
        assert np.array_equal(a[n], b[n]), n


def test_bwd_deterministic():
    w, inp = case("bf16", "token", 128, 128, 300, seed=602)
    g = generate_grads(w)
    a = run_gpu_bwd(w, inp, g)
    b = run_gpu_bwd(w, inp, g)
    for n in a:
        if a[n] is not None:
            assert np.array_equal(a[n], b[n]), n


def test_bwd_empty_sequence():
    w, inp = case("f32", "gate", 64, 64, 0, seed=603)
    g = generate_grads(w)
    r = run_gpu_bwd(w, inp, g)
    assert r["dq"].shape == (2, 2, 0, 64)
    assert np.array_equal(r["dinit"], g["dfinal"].astype(np.float64))


def test_bwd_rejects():
    q = torch.zeros((1, 1, 64, 64), device="cuda")
    gam = torch.full((1,), 0.9, device="cuda")
    with pytest.raises(fla.FlaError) as e:
        fla.bwd(q, q, q, q, chunk=48)
    assert e.value.status == fla.FLA_ERR_UNSUPPORTED
    q32 = torch.zeros((1, 1, 64, 32), device="cuda")
    with pytest.raises(fla.FlaError) as e:
        fla.bwd(q32, q32, q32, q32)
    assert e.value.status == fla.FLA_ERR_UNSUPPORTED
    q256 = torch.zeros((1, 1, 64, 256), device="cuda")
    with pytest.raises(fla.FlaError) as e:
        fla.bwd(q256, q256, q256, q256)   # fp32 tiles at 256 exceed the LDS
    assert e.value.status == fla.FLA_ERR_UNSUPPORTED
    lib = fla.load_library()
    p = q.data_ptr()
    g = torch.zeros((1,), device="cuda")
    rc = lib.fla_linattn_bwd(p, p, p, gam.data_ptr(), None, p, None, p, p, p, g.data_ptr(),
                             None, 1, 1, 64, 64, 64, 64, fla.FLA_DECAY_GAMMA, None)
    assert rc == fla.FLA_ERR_INVALID_ARG    # no gamma gradient


@pytest.mark.parametrize("name", ["gla_d128", "token_decay_d128"])
def test_bwd_full_size_all_heads(name):
    """The full-size workload in one backward call; the oracle checks every head, one
    batch row at a time, with the global max-norm error per gradient."""
    w = WORKLOADS[name]
    say(f"[bwd-full] {name}: {w}")
    inp = generate_torch(w, "cuda")
    g = generate_grads_torch(w, "cuda")
    t0 = time.time()
    dq, dk, dv, dg, di = fla.bwd(inp["q"], inp["k"], inp["v"], g["dout"], inp["decay"],
                                 decay_kind=w.decay, init_state=inp["init"], dfinal=g["dfinal"])
    torch.cuda.synchronize()
    say(f"[bwd-full] {name}: gpu done {time.time() - t0:.1f}s")
    got = {"dq": dq, "dk": dk, "dv": dv, "dgate": dg, "dinit": di}
    diff = {n: 0.0 for n in got}
    mag = {n: 0.0 for n in got}
    for b in range(w.B):
        sl = (slice(b, b + 1),)
        host = {n: to_numpy_input(inp[n][sl]) for n in ("q", "k", "v")}
        ref = oracle.bwd(host["q"], host["k"], host["v"], to_numpy_input(g["dout"][sl]),
                         to_numpy_input(inp["decay"][sl]), w.decay, None,
                         to_numpy_input(g["dfinal"][sl]))
        for n, t in got.items():
            x = to_host(t[sl])
            diff[n] = max(diff[n], float(np.max(np.abs(x - ref[n]))))
            mag[n] = max(mag[n], float(np.max(np.abs(ref[n]))))
        say(f"[bwd-full] {name} batch row {b} done {time.time() - t0:.1f}s")
    for n in got:
        e = diff[n] / mag[n]
        say(f"[bwd-full] {name} {n}: {e:.2e} (all heads)")
        assert e <= tol_for(w.dtype, n), (name, n, e)
