"""GPU parity of the token-major layout ([B][T][H][d], FLA_LAYOUT_BTHD) and of packed
variable-length sequences (fla_linattn_fwd_varlen) against the fp64 oracle, and against
the [B][H][T][d] path: the same arithmetic on the same values, so results agree bit for
bit — except for the per-key gate at dk = 128 in bf16 with 64-token tiles, whose
token-major and packed producers scan the gate in two row halves (the chunk's products
associated in another order), where both layouts are held to the oracle's bar and to each
other within LAYOUT_TOL.
"""
import itertools

import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_device, to_host
from workloads import Workload, generate

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


def say(msg):
    print(msg, flush=True)


def case(dtype, decay, dk, dv, T, *, B=2, H=3, chunk=64, phi=False, norm=False, init=True,
         seed=0):
    w = Workload("layout", B, H, T, dk, dv, chunk, dtype, decay, phi, norm,
                 1.0 if dtype == "f32" else dk ** -0.5, 0.1 if init else 0.0,
                 gamma_exp="1-2^(-5-h)", seed=seed)
    return w, generate(w)


def bthd(x):
    """[B,H,T,...] -> [B,T,H,...] (contiguous)."""
    return None if x is None else np.ascontiguousarray(np.swapaxes(x, 1, 2))


# row halves change only the association of the fp32 gate products, so the layouts differ
# by bf16 roundings of single Qt / Kt elements
LAYOUT_TOL = 1e-2


def row_halves(w):
    """Whether the token-major producers of this case scan the gate in row halves."""
    return w.decay == "gate" and w.dtype == "bf16" and w.dk == 128 and w.chunk in (64, 128)


def dev(w, x):
    return to_device(x, bf16=(w.dtype == "bf16"))


def run_bhtd(w, inp, **kw):
    out, fin = fla.fwd(dev(w, inp["q"]), dev(w, inp["k"]), dev(w, inp["v"]),
                       to_device(inp["decay"]), decay_kind=w.decay,
                       init_state=to_device(inp["init"]), chunk=w.chunk, phi_elu1=w.phi_elu1,
                       normalize=w.normalize, **kw)
    torch.cuda.synchronize()
    return to_host(out), to_host(fin)


def run_bthd(w, inp, **kw):
    dec = inp["decay"] if w.decay in ("none", "gamma") else bthd(inp["decay"])
    out, fin = fla.fwd(dev(w, bthd(inp["q"])), dev(w, bthd(inp["k"])), dev(w, bthd(inp["v"])),
                       to_device(dec), decay_kind=w.decay, init_state=to_device(inp["init"]),
                       chunk=w.chunk, phi_elu1=w.phi_elu1, normalize=w.normalize,
                       layout="bthd", **kw)
    torch.cuda.synchronize()
    return np.swapaxes(to_host(out), 1, 2), to_host(fin)


COMBOS = list(itertools.product(["f32", "bf16"], ["none", "gamma", "gate", "token"],
                                [False, True]))


@pytest.mark.parametrize("dtype,decay,norm", COMBOS)
def test_bthd_matches_bhtd_and_oracle(dtype, decay, norm):
    i = COMBOS.index((dtype, decay, norm))
    w, inp = case(dtype, decay, 64, 128, 3 * 64 + 9, phi=norm, norm=norm, seed=700 + i)
    say(f"[bthd] {dtype} {decay} norm={norm}")
    o1, f1 = run_bthd(w, inp)
    o0, f0 = run_bhtd(w, inp)
    assert np.array_equal(o1, o0) and np.array_equal(f1, f0)
    ro, rf = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["decay"], w.decay, inp["init"],
                        phi_elu1=w.phi_elu1, normalize=w.normalize)
    assert rel_err(o1, ro) <= TOL[dtype] and rel_err(f1, rf) <= TOL[dtype]


@pytest.mark.parametrize("dk,dv,chunk", [(128, 128, 64), (256, 64, 32), (32, 256, 128),
                                         (16, 16, 16)])
def test_bthd_shapes(dk, dv, chunk):
    w, inp = case("bf16", "gate", dk, dv, 2 * chunk + 5, chunk=chunk, seed=720 + dk + dv)
    say(f"[bthd] dk={dk} dv={dv} C={chunk}")
    o1, f1 = run_bthd(w, inp)
    o0, f0 = run_bhtd(w, inp)
    if row_halves(w):
        ro, rf = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["decay"], w.decay, inp["init"])
        say(f"  layouts differ by out {rel_err(o1, o0):.2e} final {rel_err(f1, f0):.2e}; "
            f"oracle {rel_err(o1, ro):.2e} / {rel_err(f1, rf):.2e}")
        assert rel_err(o1, ro) <= TOL["bf16"] and rel_err(f1, rf) <= TOL["bf16"]
        assert rel_err(o1, o0) <= LAYOUT_TOL and rel_err(f1, f0) <= LAYOUT_TOL
    else:
        assert np.array_equal(o1, o0) and np.array_equal(f1, f0)


@pytest.mark.parametrize("nseg", [2, 5])
def test_bthd_segments(nseg):
    w, inp = case("bf16", "gamma", 128, 128, 20 * 64 + 3, B=1, H=2, seed=740 + nseg)
    say(f"[bthd] segments={nseg}")
    o1, f1 = run_bthd(w, inp, n_segments=nseg)
    o0, f0 = run_bhtd(w, inp, n_segments=nseg)
    assert np.array_equal(o1, o0) and np.array_equal(f1, f0)


@pytest.mark.parametrize("nseg", [1, 3])
def test_bthd_gate_row_halves(nseg):
    """Token-major per-key gate at dk = 128 in bf16 (the producers' row halves), streaming
    and through the segment schedule (whose end-state pass runs the same hand-off), with a
    ragged last chunk of 17 rows (the second half sees none), against the oracle."""
    w, inp = case("bf16", "gate", 128, 128, 5 * 64 + 17, B=1, H=3, seed=745 + nseg)
    say(f"[bthd] gate dk=128 row halves, segments={nseg}")
    o1, f1 = run_bthd(w, inp, n_segments=nseg)
    ro, rf = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["decay"], w.decay, inp["init"])
    assert rel_err(o1, ro) <= TOL["bf16"] and rel_err(f1, rf) <= TOL["bf16"]


LENGTHS = [0, 1, 63, 64, 65, 200, 7, 129]


def test_varlen_gate_row_halves():
    """Packed sequences with the per-key gate at dk = 128 in bf16 (row-half producers),
    lengths whose last chunk ends in either half or exactly at a half, against the oracle
    per sequence."""
    lengths = [1, 20, 32, 33, 64, 97, 0, 130]
    w, inp = case("bf16", "gate", 128, 128, sum(lengths), B=1, H=2, init=False, seed=766)
    cu, seqs, packed = pack(w, inp, lengths)
    rng = np.random.default_rng(767)
    init = (0.1 * rng.standard_normal((len(lengths), w.H, w.dk, w.dv))).astype(np.float32)
    say(f"[varlen] gate dk=128 row halves lengths={lengths}")
    out, fin = fla.fwd_varlen(dev(w, packed["q"]), dev(w, packed["k"]), dev(w, packed["v"]),
                              to_device(cu), to_device(packed["decay"]), decay_kind="gate",
                              init_state=to_device(init))
    torch.cuda.synchronize()
    out, fin = to_host(out), to_host(fin)
    for s, d in enumerate(seqs):
        ro, rf = oracle.fwd(d["q"], d["k"], d["v"], d["decay"], "gate", init[s:s + 1])
        assert rel_err(fin[s:s + 1], rf) <= TOL["bf16"], s
        if lengths[s]:
            o_s = np.swapaxes(out[cu[s]:cu[s + 1]], 0, 1)[None]
            assert rel_err(o_s, ro) <= TOL["bf16"], s


def pack(w, inp, lengths):
    """Per-sequence BHTD inputs (B=1) from one long draw, packed token-major."""
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    seqs = []
    for s in range(len(lengths)):
        sl = slice(int(cu[s]), int(cu[s + 1]))
        d = {n: inp[n][:, :, sl] for n in ("q", "k", "v")}
        d["decay"] = (inp["decay"] if w.decay in ("none", "gamma")
                      else inp["decay"][:, :, sl])
        seqs.append(d)
    packed = {n: np.ascontiguousarray(np.swapaxes(inp[n][0], 0, 1)) for n in ("q", "k", "v")}
    packed["decay"] = (inp["decay"] if w.decay in ("none", "gamma")
                       else np.ascontiguousarray(np.swapaxes(inp["decay"][0], 0, 1)))
    return cu, seqs, packed


@pytest.mark.parametrize("dtype,decay,norm", [("bf16", "gate", False), ("f32", "token", True),
                                              ("bf16", "gamma", False), ("f32", "none", True)])
def test_varlen(dtype, decay, norm):
    i = ["gate", "token", "gamma", "none"].index(decay)
    total = sum(LENGTHS)
    w, inp = case(dtype, decay, 64, 128, total, B=1, H=2, phi=norm, norm=norm, init=False,
                  seed=760 + i)
    cu, seqs, packed = pack(w, inp, LENGTHS)
    ncol = w.dv + (1 if norm else 0)
    rng = np.random.default_rng(761 + i)
    init = (0.1 * rng.standard_normal((len(LENGTHS), w.H, w.dk, ncol))).astype(np.float32)
    say(f"[varlen] {dtype} {decay} norm={norm} lengths={LENGTHS}")
    out, fin = fla.fwd_varlen(dev(w, packed["q"]), dev(w, packed["k"]), dev(w, packed["v"]),
                              to_device(cu), to_device(packed["decay"]), decay_kind=decay,
                              init_state=to_device(init), phi_elu1=norm, normalize=norm)
    torch.cuda.synchronize()
    out, fin = to_host(out), to_host(fin)
    for s, d in enumerate(seqs):
        o_s = np.swapaxes(out[cu[s]:cu[s + 1]], 0, 1)[None]
        ws = w.with_(T=LENGTHS[s])
        dd = dict(d, init=init[s:s + 1])
        o0, f0 = run_bhtd(ws, dd)
        assert np.array_equal(o_s, o0), s
        assert np.array_equal(fin[s:s + 1], f0), s
        ro, rf = oracle.fwd(d["q"], d["k"], d["v"], d["decay"], decay, init[s:s + 1],
                            phi_elu1=norm, normalize=norm)
        assert rel_err(o_s, ro) <= TOL[dtype] and rel_err(fin[s:s + 1], rf) <= TOL[dtype], s


@pytest.mark.parametrize("n_seqs", [8192, 8193])
def test_varlen_many_sequences(n_seqs):
    """Many short sequences with a few long ones among them: at 8192 sequences the
    longest-first order is ranked by the multi-block ranking kernel, above that the
    sequences run in their given order.  Sampled sequences (all long ones, some empty ones)
    against the oracle; every empty sequence keeps its initial state exactly."""
    rng = np.random.default_rng(790 + n_seqs)
    lengths = rng.integers(0, 4, size=n_seqs)
    long_at = rng.choice(n_seqs, size=4, replace=False)
    lengths[long_at] = [130, 200, 64, 257]
    lengths = [int(x) for x in lengths]
    w, inp = case("f32", "gate", 64, 64, sum(lengths), B=1, H=1, init=False, seed=791)
    cu, seqs, packed = pack(w, inp, lengths)
    init = (0.1 * rng.standard_normal((n_seqs, w.H, w.dk, w.dv))).astype(np.float32)
    say(f"[varlen-many] {n_seqs} sequences, {sum(lengths)} tokens")
    out, fin = fla.fwd_varlen(dev(w, packed["q"]), dev(w, packed["k"]), dev(w, packed["v"]),
                              to_device(cu), to_device(packed["decay"]), decay_kind="gate",
                              init_state=to_device(init))
    torch.cuda.synchronize()
    out, fin = to_host(out), to_host(fin)
    empty = [s for s in range(n_seqs) if lengths[s] == 0]
    assert empty and all(np.array_equal(fin[s], init[s]) for s in empty)
    sample = sorted(set(long_at.tolist()) | set(rng.choice(n_seqs, size=120, replace=False).tolist()))
    for s in sample:
        d = seqs[s]
        ro, rf = oracle.fwd(d["q"], d["k"], d["v"], d["decay"], "gate", init[s:s + 1])
        assert rel_err(fin[s:s + 1], rf) <= TOL["f32"], s
        if lengths[s]:
            o_s = np.swapaxes(out[cu[s]:cu[s + 1]], 0, 1)[None]
            assert rel_err(o_s, ro) <= TOL["f32"], s


def test_varlen_bad_offsets_are_clamped():
    """Offsets outside [0, total] or decreasing are clamped: no fault, sequences of
    length zero keep their initial state."""
    w, inp = case("f32", "none", 64, 64, 100, B=1, H=1, init=False, seed=780)
    cu = np.array([0, 50, 40, 1000, -5], dtype=np.int64)
    _, _, packed = pack(w, inp, [100])
    out, fin = fla.fwd_varlen(dev(w, packed["q"]), dev(w, packed["k"]), dev(w, packed["v"]),
                              to_device(cu))
    torch.cuda.synchronize()
    fin = to_host(fin)
    assert np.all(np.isfinite(fin))
    assert np.all(fin[1] == 0) and np.all(fin[3] == 0)   # [50, 50) and [100, 100)


def test_full_size_bthd_headline_matches_bhtd():
    """The GLA workload at full size in token-major order against the [B][H][T][d] result
    (which the full-size workload test holds to the oracle on every row): within
    LAYOUT_TOL, the token-major producers scanning the gate in row halves."""
    from workloads import WORKLOADS, generate_torch
    w = WORKLOADS["gla_d128"]
    say(f"[bthd-full] {w}")
    inp = generate_torch(w, "cuda")
    o0, f0 = fla.fwd(inp["q"], inp["k"], inp["v"], inp["decay"], decay_kind="gate")
    t = {n: inp[n].transpose(1, 2).contiguous() for n in ("q", "k", "v", "decay")}
    o1, f1 = fla.fwd(t["q"], t["k"], t["v"], t["decay"], decay_kind="gate", layout="bthd")
    torch.cuda.synchronize()
    o1 = o1.transpose(1, 2).float()
    eo = ((o1 - o0.float()).abs().max() / o0.float().abs().max()).item()
    ef = ((f1 - f0).abs().max() / f0.abs().max()).item()
    say(f"  layouts differ by out {eo:.2e} final {ef:.2e}")
    assert eo <= LAYOUT_TOL and ef <= LAYOUT_TOL


def test_full_size_varlen_workload():
    """The packed-sequence workload in the launch configuration bench.py times; the oracle
    checks every sequence (global max-norm error over all of them)."""
    from workloads import generate_torch, to_numpy_input, varlen_workload
    w, lengths = varlen_workload("varlen_gla_d128")
    say(f"[varlen-full] {w.name}: {len(lengths)} sequences, {w.T} tokens")
    cu_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    inp = generate_torch(w, "cuda")
    packed = {k: inp[k][0].transpose(0, 1).contiguous() for k in ("q", "k", "v", "decay")}
    out, fin = fla.fwd_varlen(packed["q"], packed["k"], packed["v"], to_device(cu_h),
                              packed["decay"], decay_kind="gate")
    torch.cuda.synchronize()
    d_o = m_o = d_f = m_f = 0.0
    for s in range(len(lengths)):
        s0, s1 = int(cu_h[s]), int(cu_h[s + 1])
        part = lambda t: to_numpy_input(t[:, :, s0:s1])
        ro, rf = oracle.fwd(part(inp["q"]), part(inp["k"]), part(inp["v"]), part(inp["decay"]),
                            "gate", None)
        o, f = to_host(out[s0:s1].transpose(0, 1)[None]), to_host(fin[s:s + 1])
        d_o, m_o = max(d_o, float(np.max(np.abs(o - ro)))), max(m_o, float(np.max(np.abs(ro))))
        d_f, m_f = max(d_f, float(np.max(np.abs(f - rf)))), max(m_f, float(np.max(np.abs(rf))))
    eo, ef = d_o / m_o, d_f / m_f
    say(f"[varlen-full] all {len(lengths)} sequences: out {eo:.2e} final {ef:.2e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
