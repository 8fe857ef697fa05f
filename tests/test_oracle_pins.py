"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: brute-force masked attention, the
parallel (matrix) form, closed forms, hand-worked cases, and invariants of the
recurrence (textbook chapter 1.6, "linear attention" section and its code listing;
decays as in the FLA RetNet/GLA posts).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import forms
from workloads import as_f64, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
KINDS = ["none", "gamma", "gate", "token"]


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (m if m > 0 else 1.0))


def make_case(rng, B, H, T, dk, dv, kind, *, normalize=False, phi_elu1=False, init=False,
              dtype="f32", gate_lo=0.6):
    q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    if normalize and not phi_elu1:   # keep phi(q).phi(k) > 0 so the denominator is well posed
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    if kind == "gamma":
        decay = rng.uniform(gate_lo, 1.0, H).astype(np.float32)
    elif kind == "gate":
        decay = rng.uniform(gate_lo, 1.0, (B, H, T, dk)).astype(np.float32)
    elif kind == "token":
        decay = rng.uniform(gate_lo, 1.0, (B, H, T)).astype(np.float32)
    else:
        decay = None
    ncol = dv + (1 if normalize else 0)
    h0 = None
    if init:
        h0 = rng.standard_normal((B, H, dk, ncol)).astype(np.float32)
        if normalize:
            h0[..., dv] = np.abs(h0[..., dv])
    if dtype == "bf16":
        q, k, v = (f32_to_bf16_bits(x) for x in (q, k, v))
    return dict(q=q, k=k, v=v, decay=decay, init=h0)


def f64(case, name, dtype):
    return as_f64(case[name], dtype)


COMBOS = list(itertools.product(KINDS, [False, True], [False, True], [False, True],
                                ["f32", "bf16"]))


@pytest.mark.parametrize("kind,phi_elu1,normalize,init,dtype", COMBOS)
def test_P1_recurrence_equals_brute_force(kind, phi_elu1, normalize, init, dtype):
    """P1: recurrent oracle == O(T^2) masked attention with explicit decay products."""
    rng = np.random.default_rng(COMBOS.index((kind, phi_elu1, normalize, init, dtype)))
    B, H, T, dk, dv = 1, 2, 7, 3, 2
    c = make_case(rng, B, H, T, dk, dv, kind, normalize=normalize, phi_elu1=phi_elu1,
                  init=init, dtype=dtype)
    out, fin = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], kind, c["init"],
                          phi_elu1=phi_elu1, normalize=normalize)
    ref = forms.brute_force(f64(c, "q", dtype), f64(c, "k", dtype), f64(c, "v", dtype),
                            c["decay"], kind, c["init"], phi_elu1=phi_elu1,
                            normalize=normalize)
    assert rel_err(out, ref) <= 1e-12
    fref = forms.final_state_closed_form(f64(c, "k", dtype), f64(c, "v", dtype), c["decay"],
                                         kind, c["init"], phi_elu1=phi_elu1,
                                         normalize=normalize)
    assert rel_err(fin, fref) <= 1e-12


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("normalize", [False, True])
def test_P2_recurrence_equals_parallel_form(kind, normalize):
    """P2: recurrent == parallel (masked matrix) form, dk != dv, with an initial state."""
    rng = np.random.default_rng(7 + KINDS.index(kind) + 10 * normalize)
    B, H, T, dk, dv = 2, 2, 24, 5, 3
    c = make_case(rng, B, H, T, dk, dv, kind, normalize=normalize, phi_elu1=True,
                  init=True, gate_lo=0.8)
    out, _ = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], kind, c["init"], phi_elu1=True,
                        normalize=normalize)
    ref = forms.parallel(c["q"], c["k"], c["v"], c["decay"], kind, c["init"], phi_elu1=True,
                         normalize=normalize)
    assert rel_err(out, ref) <= 1e-12


def test_P2_page_self_check_shape():
    """The chapter's own check: parallel == recurrent at T=50, d=16, elu+1, normalised,
    atol 1e-5 (the page prints only True)."""
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((1, 1, 50, 16)).astype(np.float32) for _ in range(3))
    out, _ = oracle.fwd(q, k, v, phi_elu1=True, normalize=True, want_final=False)
    ref = forms.parallel(q, k, v, phi_elu1=True, normalize=True)
    assert np.allclose(out, ref, atol=1e-5)
    assert rel_err(out, ref) <= 1e-12


@pytest.mark.parametrize("normalize", [False, True])
def test_P3_unit_decay_is_plain_linear_attention(normalize):
    """P3: gamma == 1 and alpha == 1 reproduce the undecayed (Katharopoulos) path bitwise."""
    rng = np.random.default_rng(3)
    B, H, T, dk, dv = 2, 3, 40, 8, 6
    c = make_case(rng, B, H, T, dk, dv, "none", normalize=normalize, phi_elu1=True,
                  init=True)
    base = oracle.fwd(c["q"], c["k"], c["v"], None, "none", c["init"], phi_elu1=True,
                      normalize=normalize)
    ones_g = np.ones(H, np.float32)
    ones_a = np.ones((B, H, T, dk), np.float32)
    ones_t = np.ones((B, H, T), np.float32)
    for dec, kind in ((ones_g, "gamma"), (ones_a, "gate"), (ones_t, "token")):
        o, f = oracle.fwd(c["q"], c["k"], c["v"], dec, kind, c["init"], phi_elu1=True,
                          normalize=normalize)
        assert np.array_equal(o, base[0]) and np.array_equal(f, base[1])


def test_P4_broadcast_gate_equals_gamma():
    """P4: alpha_t[c] = gamma_h for all t, c gives the gamma path bitwise (and the
    per-token scalar gate likewise)."""
    rng = np.random.default_rng(4)
    B, H, T, dk, dv = 2, 3, 33, 8, 5
    c = make_case(rng, B, H, T, dk, dv, "gamma", init=True)
    g = c["decay"]
    a = np.broadcast_to(g[None, :, None, None], (B, H, T, dk)).astype(np.float32)
    tk = np.broadcast_to(g[None, :, None], (B, H, T)).astype(np.float32)
    ref = oracle.fwd(c["q"], c["k"], c["v"], g, "gamma", c["init"])
    for dec, kind in ((a, "gate"), (tk, "token")):
        o, f = oracle.fwd(c["q"], c["k"], c["v"], dec, kind, c["init"])
        assert np.array_equal(o, ref[0]) and np.array_equal(f, ref[1])


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("phi_elu1", [False, True])
def test_P5i_normalised_constant_values(kind, phi_elu1):
    """P5(i): with the normaliser, zero init and v_t = c for all t, o_t = c exactly in
    real arithmetic (numerator = c * denominator)."""
    rng = np.random.default_rng(51)
    B, H, T, dk, dv = 1, 2, 30, 4, 3
    c = make_case(rng, B, H, T, dk, dv, kind, normalize=True, phi_elu1=phi_elu1)
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25], np.float32), (B, H, T, dv)).copy()
    out, _ = oracle.fwd(c["q"], c["k"], v, c["decay"], kind, None, phi_elu1=phi_elu1,
                        normalize=True)
    assert np.max(np.abs(out - v)) <= 1e-12


@pytest.mark.parametrize("gamma", [1.0, 0.5, 0.96875, 0.999])
def test_P5ii_scalar_geometric_series(gamma):
    """P5(ii): dk=dv=1, q=k=v=1, identity phi, decay gamma, init s0:
    o_t = (1 - gamma^{t+1}) / (1 - gamma) + gamma^{t+1} s0  (t + 1 + s0 when gamma = 1)."""
    T, s0 = 200, 0.75
    ones = np.ones((1, 1, T, 1), np.float32)
    init = np.full((1, 1, 1, 1), s0, np.float32)
    out, fin = oracle.fwd(ones, ones, ones, np.array([gamma], np.float32), "gamma", init)
    t = np.arange(T, dtype=np.float64)
    g = float(np.float32(gamma))
    if g == 1.0:
        ref = t + 1 + s0
    else:
        ref = (1 - g ** (t + 1)) / (1 - g) + g ** (t + 1) * s0
    assert rel_err(out[0, 0, :, 0], ref) <= 1e-12
    assert abs(fin[0, 0, 0, 0] - ref[-1]) <= 1e-12 * abs(ref[-1])


@pytest.mark.parametrize("kind", KINDS)
def test_P5iii_single_token(kind):
    """P5(iii): T = 1: o_0 = (phi(k_0).phi(q_0)) v_0 + (g_0 (.) h0)^T phi(q_0); with the
    normaliser and zero init o_0 = v_0."""
    rng = np.random.default_rng(53)
    B, H, dk, dv = 2, 2, 6, 4
    c = make_case(rng, B, H, 1, dk, dv, kind, phi_elu1=True, init=True)
    out, _ = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], kind, c["init"], phi_elu1=True)
    qb = forms.phi(c["q"][:, :, 0], True)
    kb = forms.phi(c["k"][:, :, 0], True)
    g = forms.gates(c["decay"], kind, B, H, 1, dk)[:, :, 0]
    h0 = c["init"].astype(np.float64)
    ref = (np.sum(qb * kb, -1)[..., None] * c["v"][:, :, 0]
           + np.einsum("bhc,bhce->bhe", qb * g, h0))
    assert rel_err(out[:, :, 0], ref) <= 1e-13
    c2 = make_case(rng, B, H, 1, dk, dv, kind, phi_elu1=True, normalize=True)
    out2, _ = oracle.fwd(c2["q"], c2["k"], c2["v"], c2["decay"], kind, None, phi_elu1=True,
                         normalize=True)
    assert np.max(np.abs(out2[:, :, 0] - c2["v"][:, :, 0])) <= 1e-12


def test_golden_hand_worked():
    """Hand-worked tiny cases (arithmetic written out in the fixture)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        T, dk, dv = cs["T"], cs["dk"], cs["dv"]
        q = np.array(cs["q"], np.float32).reshape(1, 1, T, dk)
        k = np.array(cs["k"], np.float32).reshape(1, 1, T, dk)
        v = np.array(cs["v"], np.float32).reshape(1, 1, T, dv)
        dec = None if cs["decay"] is None else np.array(cs["decay"], np.float32)
        if cs["decay_kind"] == "gate":
            dec = dec.reshape(1, 1, T, dk)
        ncol = dv + (1 if cs["normalize"] else 0)
        init = None if cs["init"] is None else np.array(cs["init"], np.float32).reshape(1, 1, dk, ncol)
        out, fin = oracle.fwd(q, k, v, dec, cs["decay_kind"], init, phi_elu1=cs["phi_elu1"],
                              normalize=cs["normalize"])
        assert np.allclose(out[0, 0], np.array(cs["out"]), rtol=0, atol=1e-14), cs["name"]
        assert np.allclose(fin[0, 0], np.array(cs["final"]), rtol=0, atol=1e-14), cs["name"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("normalize", [False, True])
def test_P6_split_resume_is_bitwise(kind, normalize):
    """P6: running T1 tokens, then T2 tokens from the final state, equals one run."""
    rng = np.random.default_rng(6)
    B, H, T, dk, dv = 2, 2, 50, 7, 5
    c = make_case(rng, B, H, T, dk, dv, kind, normalize=normalize, phi_elu1=True, init=True)
    full_o, full_f = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], kind, c["init"],
                                phi_elu1=True, normalize=normalize)
    T1 = 19

    def part(x, sl):
        return None if x is None else np.ascontiguousarray(x[:, :, sl])

    dec1 = c["decay"] if kind in ("none", "gamma") else part(c["decay"], slice(0, T1))
    dec2 = c["decay"] if kind in ("none", "gamma") else part(c["decay"], slice(T1, T))
    o1, f1 = oracle.fwd(part(c["q"], slice(0, T1)), part(c["k"], slice(0, T1)),
                        part(c["v"], slice(0, T1)), dec1, kind, c["init"], phi_elu1=True,
                        normalize=normalize)
    o2, f2 = oracle.fwd(part(c["q"], slice(T1, T)), part(c["k"], slice(T1, T)),
                        part(c["v"], slice(T1, T)), dec2, kind, f1, phi_elu1=True,
                        normalize=normalize)
    assert np.array_equal(np.concatenate([o1, o2], axis=2), full_o)
    assert np.array_equal(f2, full_f)


@pytest.mark.parametrize("kind", KINDS)
def test_P7_chained_steps_equal_forward(kind):
    """P7: T single-token decode steps reproduce the forward pass bitwise."""
    rng = np.random.default_rng(7)
    B, H, T, dk, dv = 2, 2, 12, 6, 4
    c = make_case(rng, B, H, T, dk, dv, kind, normalize=True, phi_elu1=True, init=True)
    fo, ff = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], kind, c["init"], phi_elu1=True,
                        normalize=True)
    state = c["init"].astype(np.float64)
    for t in range(T):
        if kind == "gate":
            d = c["decay"][:, :, t]
        elif kind == "token":
            d = c["decay"][:, :, t]
        else:
            d = c["decay"]
        o = oracle.step(c["q"][:, :, t], c["k"][:, :, t], c["v"][:, :, t], state, d, kind,
                        phi_elu1=True, normalize=True)
        assert np.array_equal(o, fo[:, :, t])
    assert np.array_equal(state, ff)


@pytest.mark.parametrize("kind", KINDS)
def test_P8_linearity_without_normaliser(kind):
    """P8: o(2v) = 2 o(v) bitwise; o(v, h0) = o(v, 0) + o(0, h0)."""
    rng = np.random.default_rng(8)
    B, H, T, dk, dv = 1, 3, 40, 6, 5
    c = make_case(rng, B, H, T, dk, dv, kind, init=True)
    o1, f1 = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], kind, None)
    o2, f2 = oracle.fwd(c["q"], c["k"], 2 * c["v"], c["decay"], kind, None)
    assert np.array_equal(o2, 2 * o1) and np.array_equal(f2, 2 * f1)
    oa, fa = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], kind, c["init"])
    ob, fb = oracle.fwd(c["q"], c["k"], np.zeros_like(c["v"]), c["decay"], kind, c["init"])
    assert rel_err(oa, o1 + ob) <= 1e-12 and rel_err(fa, f1 + fb) <= 1e-12


@pytest.mark.parametrize("C", [1, 2, 3, 16, 64])
@pytest.mark.parametrize("kind", KINDS)
def test_P9_chunk_algebra_matches_oracle(C, kind):
    """P9: the chunk algebra the kernels use (fp64 model) equals the recurrence, including
    a ragged last chunk."""
    from chunk_model import chunked
    rng = np.random.default_rng(9 + C)
    B, H, T, dk, dv = 1, 2, 70, 6, 4
    for normalize in (False, True):
        c = make_case(rng, B, H, T, dk, dv, kind, normalize=normalize, phi_elu1=True,
                      init=True, gate_lo=0.7)
        o, f = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], kind, c["init"], phi_elu1=True,
                          normalize=normalize)
        mo, mf = chunked(c["q"], c["k"], c["v"], c["decay"], kind, c["init"], chunk=C,
                         phi_elu1=True, normalize=normalize)
        assert rel_err(mo, o) <= 1e-12 and rel_err(mf, f) <= 1e-12


def test_sampled_rows_match_full_output():
    rng = np.random.default_rng(10)
    c = make_case(rng, 2, 2, 64, 8, 8, "gate", init=True)
    full, _ = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], "gate", c["init"])
    rows = [0, 5, 31, 63]
    part, _ = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], "gate", c["init"], rows=rows)
    assert np.array_equal(part, full[:, :, rows])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(11)
    c = make_case(rng, 2, 3, 80, 16, 40, "gate", normalize=True, phi_elu1=True, init=True)
    a = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], "gate", c["init"], phi_elu1=True,
                   normalize=True, nthreads=1)
    b = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], "gate", c["init"], phi_elu1=True,
                   normalize=True, nthreads=8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_sequence_returns_init():
    rng = np.random.default_rng(12)
    c = make_case(rng, 1, 2, 0, 4, 3, "gamma", init=True)
    out, fin = oracle.fwd(c["q"], c["k"], c["v"], c["decay"], "gamma", c["init"])
    assert out.shape == (1, 2, 0, 3)
    assert np.array_equal(fin, c["init"].astype(np.float64))


# ---------------------------------------------------------------------------------------
# Strong decays: the exact 16-token path and the gated delta rule's decay ratios

def _strong_gates(kind, B, H, T, dk, seed):
    from workloads import strong_gates
    return strong_gates(kind, B, H, T, dk, seed)


@pytest.mark.parametrize("kind", ["gate", "token"])
@pytest.mark.parametrize("norm", [False, True])
def test_exact16_path_matches_oracle_under_strong_decay(kind, norm):
    """The exact 16-token algorithm (running products only) equals the recurrence for
    gates whose chunk products underflow fp32, with ragged tails and an initial state."""
    from chunk_model import exact16
    B, H, T, dk, dv = 1, 2, 53, 8, 6
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    ncol = dv + (1 if norm else 0)
    init = (0.1 * rng.standard_normal((B, H, dk, ncol))).astype(np.float32)
    if norm:
        init[..., dv] = np.abs(init[..., dv])
    for name, dec in _strong_gates(kind, B, H, T, dk, 9).items():
        ro, rf = oracle.fwd(q, k, v, dec, kind, init, phi_elu1=norm, normalize=norm)
        mo, mf = exact16(q, k, v, dec, kind, init, phi_elu1=norm, normalize=norm)
        assert np.allclose(mo, ro, rtol=1e-11, atol=1e-11 * np.max(np.abs(ro))), name
        assert np.allclose(mf, rf, rtol=1e-11, atol=1e-11 * np.max(np.abs(rf))), name


def test_strong_gate_sets_leave_the_factorised_range():
    """The sets used for the GPU's strong-decay tests do cross the fused kernel's limit
    (a chunk product below 2^-100) on some units and not on others, so both paths run;
    the headline's gates never do."""
    from chunk_model import unsafe_units
    B, H, T, dk = 2, 4, 640, 64
    for kind in ("gate", "token"):
        sets = _strong_gates(kind, B, H, T, dk, 3)
        assert unsafe_units(sets["uniform"], kind, B, H, T, dk, 64).all()
        assert unsafe_units(sets["isolated"], kind, B, H, T, dk, 64).any()
    from workloads import generate, small
    w = small("gla_d128", B=2, H=2, T=4096)
    inp = generate(w)
    assert not unsafe_units(inp["decay"], "gate", 2, 2, 4096, 128, 64).any()


def test_gdn_decay_ratio_in_mantissa_exponent_form():
    """g_t / g_j formed as ldexp(m_t / m_j, e_t - e_j) from the scanned (m, e) pairs equals
    the product of the decays over tokens j+1..t (fp32 rounding, or both below 2^-126),
    also when the plain product g underflows to zero and when a decay is exactly 0."""
    from chunk_model import ext_decay_ratio
    rng = np.random.default_rng(11)
    cases = [rng.uniform(0.02, 0.5, 64), rng.uniform(1e-6, 1e-3, 64),
             np.where(rng.random(64) < 0.1, 0.0, rng.uniform(0.5, 1.0, 64)),
             np.full(64, 0.999), np.ones(64)]
    for a in cases:
        a = a.astype(np.float32).astype(np.float64)
        r = ext_decay_ratio(a)
        for t in range(64):
            for j in range(t + 1):
                exact = float(np.prod(a[j + 1:t + 1]))
                if exact >= 2.0 ** -126:
                    assert abs(r[t, j] - exact) <= 64 * 2.0 ** -23 * exact, (t, j, r[t, j], exact)
                else:
                    assert r[t, j] <= 2.0 ** -126


# ---------------------------------------------------------------------------------------
# The layer's input side: projections + feature map before the recurrence

def test_fp64_inputs_equal_fp32_inputs_bitwise():
    """fp64 inputs (the projection leg's own values) run the same arithmetic as fp32
    inputs that hold the same numbers."""
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((1, 2, 37, 8)).astype(np.float32) for _ in range(3))
    dec = rng.uniform(0.5, 1.0, (1, 2, 37, 8)).astype(np.float32)
    a = oracle.fwd(q, k, v, dec, "gate", None, phi_elu1=True, normalize=True)
    b = oracle.fwd(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), dec, "gate",
                   None, phi_elu1=True, normalize=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("kind", ["none", "gate", "token"])
def test_projection_leg_with_identity_weights_is_the_plain_path(kind):
    """W = identity (hidden = H*d): head h of token t takes x[b, t, h*d : h*d + d], the
    token-major layout; the projection leg then equals fwd() on x rearranged by head, for
    the decay laid out token-major.  Pins the head / column mapping and the transposes."""
    from workloads import f32_to_bf16_bits
    B, T, H, d = 2, 29, 3, 4
    rng = np.random.default_rng(23)
    x = f32_to_bf16_bits(rng.standard_normal((B, T, H * d)).astype(np.float32))
    eye = f32_to_bf16_bits(np.eye(H * d, dtype=np.float32))
    dec = None
    if kind == "gate":
        dec = rng.uniform(0.5, 1.0, (B, T, H, d)).astype(np.float32)
    elif kind == "token":
        dec = rng.uniform(0.5, 1.0, (B, T, H)).astype(np.float32)
    out, fin = oracle.fwd_proj(x, eye, eye, eye, H, dec, kind, phi_elu1=True, normalize=True)
    heads = np.ascontiguousarray(x.reshape(B, T, H, d).transpose(0, 2, 1, 3))
    dh = None if dec is None else np.ascontiguousarray(np.swapaxes(dec, 1, 2))
    ro, rf = oracle.fwd(heads, heads, heads, dh, kind, None, phi_elu1=True, normalize=True)
    assert np.array_equal(out, ro.transpose(0, 2, 1, 3)) and np.array_equal(fin, rf)


def test_projection_leg_mixes_hidden_features():
    """The projections contract the hidden features: permuting them in x and in the rows of
    every W leaves the result unchanged (a transposed W, or a contraction over the wrong
    axis, would not), and scaling W_v scales the output (no normaliser; v carries no
    feature map)."""
    B, T, H, d, D = 1, 17, 2, 4, 8
    rng = np.random.default_rng(29)
    x = rng.standard_normal((B, T, D)).astype(np.float32)
    wq, wk, wv = (rng.standard_normal((D, H * d)).astype(np.float32) for _ in range(3))
    o1, f1 = oracle.fwd_proj(x, wq, wk, wv, H, phi_elu1=True)
    perm = rng.permutation(D)
    xp = np.ascontiguousarray(x[:, :, perm])
    o2, f2 = oracle.fwd_proj(xp, *(np.ascontiguousarray(w[perm]) for w in (wq, wk, wv)), H,
                             phi_elu1=True)
    assert np.allclose(o2, o1, rtol=1e-12, atol=1e-12 * np.max(np.abs(o1)))
    assert np.allclose(f2, f1, rtol=1e-12, atol=1e-12 * np.max(np.abs(f1)))
    o3, _ = oracle.fwd_proj(x, wq, wk, (2.0 * wv).astype(np.float32), H, phi_elu1=True)
    assert np.allclose(o3, 2.0 * o1, rtol=1e-13, atol=1e-13 * np.max(np.abs(o1)))
    assert not np.allclose(oracle.fwd_proj(x, wq, wk, np.ascontiguousarray(wv[::-1]), H,
                                           phi_elu1=True)[0], o1)
