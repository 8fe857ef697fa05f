"""GPU parity under strong decays: gates whose products along a chunk underflow fp32.

Any decay in [0, 1] is valid input (textbook chapter 1.6: the gated delta rule's alpha near
0 clears the memory; decay-masked linear attention).  The forward pass hands the (b, h)
units whose chunk products fall below the fused kernel's range to the exact 16-token
kernel; the gated delta rule forms its decay ratios in mantissa-exponent form.  Three
decay sets (workloads.strong_gates: plain sigmoid gates, uniform [0.02, 0.5], isolated
1e-6 and 0 entries), each against the fp64 oracle at the usual bar, through every
schedule and layout.
"""
import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_device, to_host
from workloads import Workload, generate, generate_gdn, strong_gates

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402

SETS = ["sigmoid", "uniform", "isolated"]


def say(msg):
    print(msg, flush=True)


def case(dtype, kind, dk, dv, T, gate_set, *, B=2, H=3, chunk=64, norm=False, init=True,
         seed=0):
    w = Workload("strong", B, H, T, dk, dv, chunk, dtype, kind, norm, norm,
                 1.0 if dtype == "f32" else dk ** -0.5, 0.1 if init else 0.0, seed=seed)
    inp = generate(w)
    inp["decay"] = strong_gates(kind, B, H, T, dk, seed + 17)[gate_set]
    if init and norm:
        inp["init"][..., dv] = np.abs(inp["init"][..., dv])
    return w, inp


def dev(w, x):
    return to_device(x, bf16=(w.dtype == "bf16"))


def check(tag, w, o, f, inp):
    ro, rf = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["decay"], w.decay, inp["init"],
                        phi_elu1=w.phi_elu1, normalize=w.normalize)
    eo, ef = rel_err(o, ro), rel_err(f, rf)
    say(f"[strong] {tag}: out {eo:.2e} final {ef:.2e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(f)), tag
    assert eo <= TOL[w.dtype] and ef <= TOL[w.dtype], (tag, eo, ef)


FWD = [(dt, kind, s) for dt in ("bf16", "f32") for kind in ("gate", "token") for s in SETS]


@pytest.mark.parametrize("dtype,kind,gate_set", FWD)
def test_forward_strong_decay(dtype, kind, gate_set):
    i = FWD.index((dtype, kind, gate_set))
    w, inp = case(dtype, kind, 64, 128, 4 * 64 + 21, gate_set, seed=900 + i)
    say(f"[strong] fwd {dtype} {kind} {gate_set}")
    out, fin = fla.fwd(dev(w, inp["q"]), dev(w, inp["k"]), dev(w, inp["v"]),
                       to_device(inp["decay"]), decay_kind=kind, init_state=to_device(inp["init"]))
    torch.cuda.synchronize()
    check(f"fwd {dtype} {kind} {gate_set}", w, to_host(out), to_host(fin), inp)


@pytest.mark.parametrize("dk,dv,chunk", [(128, 128, 64), (256, 64, 64), (32, 64, 128),
                                         (16, 16, 16), (128, 64, 512)])
@pytest.mark.parametrize("kind", ["gate", "token"])
def test_forward_strong_decay_shapes(dk, dv, chunk, kind):
    w, inp = case("bf16", kind, dk, dv, 3 * 64 + 7, "uniform", B=1, H=2, chunk=chunk,
                  seed=950 + dk + dv + chunk)
    say(f"[strong] shape dk={dk} dv={dv} C={chunk} {kind}")
    out, fin = fla.fwd(dev(w, inp["q"]), dev(w, inp["k"]), dev(w, inp["v"]),
                       to_device(inp["decay"]), decay_kind=kind, init_state=to_device(inp["init"]),
                       chunk=chunk)
    torch.cuda.synchronize()
    check(f"dk={dk} dv={dv} C={chunk} {kind}", w, to_host(out), to_host(fin), inp)


@pytest.mark.parametrize("gate_set", SETS)
def test_forward_strong_decay_normaliser_in_place(gate_set):
    """elu+1 with the normaliser, two value slices, in-place resume (init aliases final):
    the flagged units' start states must survive the fused kernel."""
    w, inp = case("f32", "gate", 64, 128, 5 * 64 + 3, gate_set, norm=True, seed=970)
    say(f"[strong] norm in-place {gate_set}")
    st = to_device(inp["init"]).clone()
    out, fin = fla.fwd(dev(w, inp["q"]), dev(w, inp["k"]), dev(w, inp["v"]),
                       to_device(inp["decay"]), decay_kind="gate", init_state=st, final_state=st,
                       phi_elu1=True, normalize=True)
    torch.cuda.synchronize()
    check(f"norm in-place {gate_set}", w, to_host(out), to_host(st), inp)


@pytest.mark.parametrize("kind", ["gate", "token"])
@pytest.mark.parametrize("gate_set", SETS)
def test_segment_schedule_strong_decay(kind, gate_set):
    """Segments (three launches and a scan), with an in-place resume."""
    w, inp = case("bf16", kind, 128, 128, 40 * 64 + 5, gate_set, B=1, H=2, seed=980)
    say(f"[strong] segments {kind} {gate_set}")
    st = to_device(inp["init"]).clone()
    out, fin = fla.fwd(dev(w, inp["q"]), dev(w, inp["k"]), dev(w, inp["v"]),
                       to_device(inp["decay"]), decay_kind=kind, init_state=st, final_state=st,
                       n_segments=5)
    torch.cuda.synchronize()
    check(f"segments {kind} {gate_set}", w, to_host(out), to_host(st), inp)


@pytest.mark.parametrize("kind", ["gate", "token"])
def test_token_major_and_packed_strong_decay(kind):
    w, inp = case("bf16", kind, 64, 64, 3 * 64 + 11, "isolated", B=2, H=3, seed=990)
    say(f"[strong] token-major {kind}")
    sw = lambda x: None if x is None else np.ascontiguousarray(np.swapaxes(x, 1, 2))
    out, fin = fla.fwd(dev(w, sw(inp["q"])), dev(w, sw(inp["k"])), dev(w, sw(inp["v"])),
                       to_device(sw(inp["decay"])), decay_kind=kind,
                       init_state=to_device(inp["init"]), layout="bthd")
    torch.cuda.synchronize()
    check(f"bthd {kind}", w, np.swapaxes(to_host(out), 1, 2), to_host(fin), inp)
    # packed: three sequences of one batch row's worth of heads (lengths 70, 0, 125)
    lens = [70, 0, 125]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    wv, iv = case("bf16", kind, 64, 64, int(cu[-1]), "uniform", B=1, H=3, seed=991)
    say(f"[strong] packed {kind}")
    pk = lambda x: np.ascontiguousarray(np.swapaxes(x[0], 0, 1))
    init = np.concatenate([iv["init"]] * 3, axis=0)
    out, fin = fla.fwd_varlen(dev(wv, pk(iv["q"])), dev(wv, pk(iv["k"])), dev(wv, pk(iv["v"])),
                              torch.from_numpy(cu).cuda(), to_device(pk(iv["decay"])),
                              decay_kind=kind, init_state=to_device(init))
    torch.cuda.synchronize()
    o, f = to_host(out), to_host(fin)
    for s in range(3):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: None if x is None else np.ascontiguousarray(x[:, :, a:b])
        ro, rf = oracle.fwd(sl(iv["q"]), sl(iv["k"]), sl(iv["v"]), sl(iv["decay"]), kind,
                            iv["init"])
        assert np.all(np.isfinite(o[a:b])) and np.all(np.isfinite(f[s]))
        if b > a:
            assert rel_err(np.swapaxes(o[a:b], 0, 1)[None], ro) <= TOL["bf16"], s
        assert rel_err(f[s:s + 1], rf) <= TOL["bf16"], s


def test_decode_steps_strong_decay():
    w, inp = case("f32", "gate", 64, 64, 40, "isolated", B=1, H=2, seed=995)
    q, k, v = (to_device(inp[n]) for n in ("q", "k", "v"))
    dec = to_device(inp["decay"])
    st = to_device(inp["init"]).clone()
    outs = [fla.step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                     st, dec[:, :, t].contiguous(), decay_kind="gate") for t in range(w.T)]
    torch.cuda.synchronize()
    check("steps", w, np.stack([to_host(x) for x in outs], axis=2), to_host(st), inp)


GDN_CASES = [(dt, s) for dt in ("bf16", "f32") for s in SETS]


@pytest.mark.parametrize("dtype,gate_set", GDN_CASES)
def test_gated_delta_rule_strong_decay(dtype, gate_set):
    i = GDN_CASES.index((dtype, gate_set))
    dk = 128 if dtype == "bf16" else 64
    w = Workload("gdn_strong", 2, 2, 3 * 64 + 29, dk, 64, 64, dtype, "token", False, False,
                 1.0 if dtype == "f32" else dk ** -0.5, 0.1, seed=1100 + i)
    inp = generate_gdn(w)
    inp["alpha"] = strong_gates("token", w.B, w.H, w.T, dk, 1200 + i)[gate_set]
    say(f"[strong] gdn {dtype} {gate_set}")
    bf = dtype == "bf16"
    out, fin = fla.gdn_fwd(to_device(inp["q"], bf16=bf), to_device(inp["k"], bf16=bf),
                           to_device(inp["v"], bf16=bf), to_device(inp["alpha"]),
                           to_device(inp["beta"]), init_state=to_device(inp["init"]))
    torch.cuda.synchronize()
    o, f = to_host(out), to_host(fin)
    ro, rf = oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["init"])
    eo, ef = rel_err(o, ro), rel_err(f, rf)
    say(f"[strong] gdn {dtype} {gate_set}: out {eo:.2e} final {ef:.2e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(f))
    assert eo <= TOL[dtype] and ef <= TOL[dtype], (eo, ef)



@pytest.mark.parametrize("name", ["gla_d128", "token_decay_d128"])
def test_full_size_plain_sigmoid_gates(name):
    """A full-size workload (B8 H16 T16384 d128, bf16) with plain sigmoid(x) decays in place
    of its usual ones: a 64-token chunk then multiplies to about 2^-74 and many units fall
    below the fused kernel's range.  Same call as the benchmark; every output row of every
    head against the oracle."""
    import time

    from workloads import WORKLOADS, generate_torch, to_numpy_input

    w = WORKLOADS[name]
    inp = generate_torch(w, "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 99)
    decay = torch.empty_like(inp["decay"])
    for b in range(w.B):
        x = torch.randn(decay.shape[1:], generator=gen, device="cuda", dtype=torch.float64)
        decay[b] = torch.sigmoid(x).to(torch.float32)
    say(f"[strong-full] {name}: {w}")
    torch.cuda.synchronize()
    t0 = time.time()
    out, fin = fla.fwd(inp["q"], inp["k"], inp["v"], decay, decay_kind=w.decay,
                       init_state=inp["init"], chunk=w.chunk)
    torch.cuda.synchronize()
    say(f"[strong-full] {name}: gpu done {time.time() - t0:.2f}s")
    assert torch.isfinite(out.float()).all().item() and torch.isfinite(fin).all().item()

    def part(t):
        return None if t is None else to_numpy_input(t)

    ro, rf = oracle.fwd(part(inp["q"]), part(inp["k"]), part(inp["v"]), part(decay), w.decay,
                        part(inp["init"]))
    eo, ef = rel_err(to_host(out), ro), rel_err(to_host(fin), rf)
    say(f"[strong-full] {name}: out {eo:.2e} final {ef:.2e} (all rows) {time.time() - t0:.1f}s")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
