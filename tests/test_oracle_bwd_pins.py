"""Pins of the oracle's backward pass (CPU only).

The gradients come from back-propagation through the recurrence (oracle.bwd).  They are
checked against things that do not share its arithmetic:
  * central finite differences of the forward oracle (itself pinned in
    test_oracle_pins.py) on tiny inputs, for every input, every decay kind, both feature
    maps, with an initial state and an upstream gradient on the final state;
  * the closed-form gradients of plain causal linear attention O = tril(Q K^T) V
    (matrix calculus: dV = tril(QK^T)^T dO, dQ = tril(dO V^T) K, dK = tril(dO V^T)^T Q),
    the chunk-free parallel form of the textbook chapter 1.6 "linear attention" section;
  * linearity in the upstream gradient.
"""
import numpy as np
import pytest

import oracle

KINDS = ["none", "gamma", "gate", "token"]


def make(rng, B, H, T, dk, dv, kind, elu):
    q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    do = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    dec = None
    if kind == "gamma":
        dec = rng.uniform(0.5, 0.99, H).astype(np.float32)
    elif kind == "gate":
        dec = rng.uniform(0.5, 0.99, (B, H, T, dk)).astype(np.float32)
    elif kind == "token":
        dec = rng.uniform(0.5, 0.99, (B, H, T)).astype(np.float32)
    init = rng.standard_normal((B, H, dk, dv))
    dfin = rng.standard_normal((B, H, dk, dv))
    return dict(q=q, k=k, v=v, do=do, dec=dec, init=init, dfin=dfin)


def loss(c, kind, elu, **over):
    x = dict(c, **over)
    o, f = oracle.fwd(x["q"], x["k"], x["v"], x["dec"], kind, x["init"], phi_elu1=elu)
    return float(np.sum(o * x["do"].astype(np.float64)) + np.sum(f * x["dfin"]))


def fd_grad(c, name, kind, elu, h=2.0 ** -9):
    """Central differences, element by element; fp32 inputs are perturbed in fp32 and the
    actual (rounded) step is used as the denominator."""
    x = c[name]
    g = np.zeros(x.shape)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] = x[idx] + x.dtype.type(h)
        xm[idx] = x[idx] - x.dtype.type(h)
        step = float(xp[idx]) - float(xm[idx])
        g[idx] = (loss(c, kind, elu, **{name: xp}) - loss(c, kind, elu, **{name: xm})) / step
    return g


@pytest.mark.parametrize("elu", [False, True])
@pytest.mark.parametrize("kind", KINDS)
def test_bwd_matches_finite_differences(kind, elu):
    rng = np.random.default_rng(100 + KINDS.index(kind) + 10 * elu)
    c = make(rng, 1, 2, 5, 3, 2, kind, elu)
    r = oracle.bwd(c["q"], c["k"], c["v"], c["do"], c["dec"], kind, c["init"], c["dfin"],
                   phi_elu1=elu)
    checks = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("init", "dinit")]
    if kind != "none":
        checks.append(("dec", "dgate"))
    for name, gname in checks:
        # gamma enters every step (the loss is a degree-T polynomial in it): a smaller step
        # keeps the central difference's O(h^2) error below the tolerance
        g = fd_grad(c, name, kind, elu, h=2.0 ** -14 if name == "dec" else 2.0 ** -9)
        ref = r[gname]
        scale = max(1.0, float(np.max(np.abs(g))))
        assert np.max(np.abs(ref - g)) <= 2e-6 * scale, (kind, elu, gname)


def test_bwd_closed_form_plain():
    rng = np.random.default_rng(7)
    B, H, T, dk, dv = 2, 2, 9, 4, 3
    Q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    K = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    V = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    dO = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    r = oracle.bwd(Q, K, V, dO)
    q, k, v, do = (x.astype(np.float64) for x in (Q, K, V, dO))
    A = np.tril(q @ np.swapaxes(k, -1, -2))
    M = np.tril(do @ np.swapaxes(v, -1, -2))
    np.testing.assert_allclose(r["dv"], np.swapaxes(A, -1, -2) @ do, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dq"], M @ k, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dk"], np.swapaxes(M, -1, -2) @ q, rtol=1e-12, atol=1e-12)
    # no initial state: its gradient is still the reverse state at t = 0, sum_t q_t do_t^T
    np.testing.assert_allclose(r["dinit"], np.swapaxes(q, -1, -2) @ do, rtol=1e-12,
                               atol=1e-12)


def test_bwd_linear_in_upstream_gradient():
    rng = np.random.default_rng(8)
    c = make(rng, 1, 2, 12, 4, 5, "gate", True)
    # upstream gradients on a 2^-10 grid, so that their fp32 sum is exact
    c["do"] = (np.round(c["do"] * 1024) / 1024).astype(np.float32)
    do2 = (np.round(rng.standard_normal(c["do"].shape) * 1024) / 1024).astype(np.float32)
    r1 = oracle.bwd(c["q"], c["k"], c["v"], c["do"], c["dec"], "gate", c["init"], None,
                    phi_elu1=True)
    r2 = oracle.bwd(c["q"], c["k"], c["v"], do2, c["dec"], "gate", c["init"], None,
                    phi_elu1=True)
    r3 = oracle.bwd(c["q"], c["k"], c["v"], c["do"] + do2, c["dec"], "gate", c["init"],
                    None, phi_elu1=True)
    for n in ("dq", "dk", "dv", "dgate", "dinit"):
        np.testing.assert_allclose(r3[n], r1[n] + r2[n], rtol=1e-11, atol=1e-11)


def test_bwd_thread_count_independent():
    rng = np.random.default_rng(9)
    c = make(rng, 2, 2, 40, 8, 40, "gate", False)
    a = oracle.bwd(c["q"], c["k"], c["v"], c["do"], c["dec"], "gate", c["init"], c["dfin"],
                   nthreads=1)
    b = oracle.bwd(c["q"], c["k"], c["v"], c["do"], c["dec"], "gate", c["init"], c["dfin"],
                   nthreads=3)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_bwd_empty_sequence():
    q = np.zeros((1, 1, 0, 4), np.float32)
    v = np.zeros((1, 1, 0, 3), np.float32)
    dfin = np.arange(12, dtype=np.float64).reshape(1, 1, 4, 3)
    r = oracle.bwd(q, q, v, v, None, "none", None, dfin)
    assert r["dq"].shape == (1, 1, 0, 4)
    assert np.array_equal(r["dinit"], dfin)
