"""GPU parity of the backward pass in the token-major layout ([B][T][H][d],
FLA_LAYOUT_BTHD) and over packed variable-length sequences (fla_linattn_bwd_varlen).
Both run the same arithmetic on the same values as the [B][H][T][d] backward (one
sequence at a time), so every gradient must agree bit for bit; packed sequences are also
checked against the fp64 back-propagation oracle.
"""
import itertools

import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_device, to_host
from workloads import Workload, generate, generate_grads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


def say(msg):
    print(msg, flush=True)


def case(dtype, decay, dk, dv, T, *, B=2, H=3, phi=False, seed=0):
    w = Workload("bwd_layout", B, H, T, dk, dv, 64, dtype, decay, phi, False,
                 1.0 if dtype == "f32" else dk ** -0.5, 0.1, gamma_exp="1-2^(-5-h)", seed=seed)
    return w, generate(w), generate_grads(w)


def swap(x):
    """[B,H,T,...] <-> [B,T,H,...] (contiguous)."""
    return None if x is None else np.ascontiguousarray(np.swapaxes(x, 1, 2))


def dev(w, x):
    return to_device(x, bf16=(w.dtype == "bf16"))


def host(t):
    return None if t is None else to_host(t)


def run_bwd(w, inp, gr, layout="bhtd", init=None, dfinal=None):
    tr = swap if layout == "bthd" else (lambda x: x)
    per_token = w.decay in ("gate", "token")
    dec = tr(inp["decay"]) if per_token else inp["decay"]
    init = inp["init"][..., :w.dv] if init is None else init
    dfinal = gr["dfinal"] if dfinal is None else dfinal
    res = fla.bwd(dev(w, tr(inp["q"])), dev(w, tr(inp["k"])), dev(w, tr(inp["v"])),
                  dev(w, tr(gr["dout"])), to_device(dec), decay_kind=w.decay,
                  init_state=to_device(init), dfinal=to_device(dfinal), phi_elu1=w.phi_elu1,
                  layout=layout)
    torch.cuda.synchronize()
    dq, dk, dv, dg, di = (host(t) for t in res)
    if layout == "bthd":
        dq, dk, dv = swap(dq), swap(dk), swap(dv)
        dg = swap(dg) if dg is not None else None
    return dq, dk, dv, dg, di


COMBOS = list(itertools.product(["f32", "bf16"], ["none", "gamma", "gate", "token"]))


@pytest.mark.parametrize("dtype,decay", COMBOS)
def test_bwd_bthd_matches_bhtd(dtype, decay):
    i = COMBOS.index((dtype, decay))
    w, inp, gr = case(dtype, decay, 64, 128, 3 * 64 + 9, phi=(i % 3 == 1), seed=900 + i)
    say(f"[bwd-bthd] {dtype} {decay} phi={w.phi_elu1}")
    g1 = run_bwd(w, inp, gr, "bthd")
    g0 = run_bwd(w, inp, gr, "bhtd")
    for name, a1, a0 in zip(("dq", "dk", "dv", "dgate", "dinit"), g1, g0):
        assert (a1 is None) == (a0 is None), name
        if a1 is not None:
            assert np.array_equal(a1, a0), name


@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (256, 128)])
def test_bwd_bthd_shapes(dk, dv):
    w, inp, gr = case("bf16", "gate", dk, dv, 2 * 64 + 5, seed=920 + dk + dv)
    say(f"[bwd-bthd] dk={dk} dv={dv}")
    g1 = run_bwd(w, inp, gr, "bthd")
    g0 = run_bwd(w, inp, gr, "bhtd")
    for name, a1, a0 in zip(("dq", "dk", "dv", "dgate", "dinit"), g1, g0):
        assert np.array_equal(a1, a0), name


LENGTHS = [0, 1, 63, 64, 65, 200, 7, 129]


@pytest.mark.parametrize("dtype,decay", [("bf16", "gate"), ("f32", "token"), ("bf16", "token"),
                                         ("bf16", "gamma"), ("f32", "none")])
def test_bwd_varlen(dtype, decay):
    i = ["gate", "token", "gamma", "none"].index(decay) + (10 if dtype == "bf16" else 0)
    total = sum(LENGTHS)
    w, inp, gr = case(dtype, decay, 64, 128, total, B=1, H=2, phi=(decay == "token"),
                      seed=940 + i)
    n = len(LENGTHS)
    cu = np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int64)
    rng = np.random.default_rng(941 + i)
    init = (0.1 * rng.standard_normal((n, w.H, w.dk, w.dv))).astype(np.float32)
    dfinal = rng.standard_normal((n, w.H, w.dk, w.dv)).astype(np.float32)
    per_token = decay in ("gate", "token")
    tok = lambda x: np.ascontiguousarray(np.swapaxes(x[0], 0, 1))   # [1,H,T,..] -> [T,H,..]
    say(f"[bwd-varlen] {dtype} {decay} lengths={LENGTHS}")
    res = fla.bwd_varlen(dev(w, tok(inp["q"])), dev(w, tok(inp["k"])), dev(w, tok(inp["v"])),
                         dev(w, tok(gr["dout"])), to_device(cu),
                         to_device(tok(inp["decay"]) if per_token else inp["decay"]),
                         decay_kind=decay, init_state=to_device(init), dfinal=to_device(dfinal),
                         phi_elu1=w.phi_elu1)
    torch.cuda.synchronize()
    dq, dk, dv, dg, di = (host(t) for t in res)
    for s in range(n):
        s0, s1 = int(cu[s]), int(cu[s + 1])
        part = lambda x: x[:, :, s0:s1]
        d = {m: part(inp[m]) for m in ("q", "k", "v")}
        d["decay"] = part(inp["decay"]) if per_token else inp["decay"]
        g = {"dout": part(gr["dout"]), "dfinal": dfinal[s:s + 1]}
        ws = w.with_(T=LENGTHS[s])
        ref = run_bwd(ws, d, g, init=init[s:s + 1], dfinal=dfinal[s:s + 1])
        mine = [np.swapaxes(x[s0:s1], 0, 1)[None] for x in (dq, dk, dv)]
        mine.append(np.swapaxes(dg[s0:s1], 0, 1)[None] if dg is not None else None)
        mine.append(di[s:s + 1])
        for name, a1, a0 in zip(("dq", "dk", "dv", "dgate", "dinit"), mine, ref):
            assert (a1 is None) == (a0 is None), (s, name)
            if a1 is not None:
                assert np.array_equal(a1, a0), (s, name)
        if LENGTHS[s] in (65, 200):
            o = oracle.bwd(d["q"], d["k"], d["v"], g["dout"], d["decay"], decay, init[s:s + 1],
                           dfinal[s:s + 1], phi_elu1=w.phi_elu1)
            for name, a1 in zip(("dq", "dk", "dv", "dgate", "dinit"), mine):
                if a1 is not None:
                    e = rel_err(a1, o[name])
                    say(f"[bwd-varlen] sequence {s} {name}: {e:.2e}")
                    assert e <= TOL[dtype], (s, name, e)


def test_full_size_bwd_bthd_headline_matches_bhtd():
    """The GLA workload's backward at full size in token-major order: bitwise the
    [B][H][T][d] result."""
    from workloads import WORKLOADS, generate_grads_torch, generate_torch
    w = WORKLOADS["gla_d128"]
    say(f"[bwd-bthd-full] {w}")
    inp = generate_torch(w, "cuda")
    gr = generate_grads_torch(w, "cuda")
    r0 = fla.bwd(inp["q"], inp["k"], inp["v"], gr["dout"], inp["decay"], decay_kind="gate",
                 dfinal=gr["dfinal"])
    t = {n: x.transpose(1, 2).contiguous() for n, x in
         (("q", inp["q"]), ("k", inp["k"]), ("v", inp["v"]), ("decay", inp["decay"]),
          ("dout", gr["dout"]))}
    r1 = fla.bwd(t["q"], t["k"], t["v"], t["dout"], t["decay"], decay_kind="gate",
                 dfinal=gr["dfinal"], layout="bthd")
    torch.cuda.synchronize()
    for name, a1, a0 in zip(("dq", "dk", "dv", "dgate"), r1[:4], r0[:4]):
        assert torch.equal(a1.transpose(1, 2), a0), name
    assert torch.equal(r1[4], r0[4])
