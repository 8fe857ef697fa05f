"""Pins of the oracle's gated delta rule (CPU only).

The recurrence (oracle.gdn_fwd, C) follows the textbook chapter 1.6 section "gated delta
rule".  It is checked against:
  * exact recall, the pages' own property: writing one (key, value) pair repeatedly with
    beta = 1, alpha = 1 leaves S k^ = v (linear attention would read back a multiple), and
    any step with beta_t = alpha_t = 1 leaves S_t k^_t = v_t whatever the history;
  * mutually orthogonal keys from a zero state: S_{t-1} k^_t = 0, so the rule is decayed
    linear attention with keys k^_t and values beta_t v_t (the pinned linear-attention
    oracle with a per-token decay);
  * beta = 0: pure decay of the initial state, o_t = (prod_{s<=t} alpha_s) S_0 q_t;
  * an independent chunked (UT-transform) form in numpy, for several chunk sizes.
"""
import numpy as np
import pytest

import oracle
from oracle import forms


def rnd(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def test_exact_recall_repeated_write():
    rng = np.random.default_rng(1)
    d = 16
    key = rnd(rng, 1, 1, 1, d)
    khat = key / np.linalg.norm(key.astype(np.float64))
    val = rnd(rng, 1, 1, 1, d)
    T = 3
    k = np.repeat(key, T, axis=2)
    v = np.repeat(val, T, axis=2)
    q = np.repeat(khat.astype(np.float32), T, axis=2)
    one = np.ones((1, 1, T), np.float32)
    o, fin = oracle.gdn_fwd(q, k, v, one, one)
    # o_t = S_t q with q = k^ (rounded to fp32): recall of v after every write, not t * v
    qk = q[0, 0, 0].astype(np.float64) @ khat[0, 0, 0].astype(np.float64)
    for t in range(T):
        np.testing.assert_allclose(o[0, 0, t], val[0, 0, 0] * qk, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(fin[0, 0].T @ khat[0, 0, 0].astype(np.float64),
                               val[0, 0, 0].astype(np.float64), rtol=1e-12, atol=1e-12)


def test_full_write_step_stores_value():
    rng = np.random.default_rng(2)
    B, H, T, dk, dv = 1, 2, 9, 8, 5
    q, k, v = rnd(rng, B, H, T, dk), rnd(rng, B, H, T, dk), rnd(rng, B, H, T, dv)
    al = rng.uniform(0.5, 1.0, (B, H, T)).astype(np.float32)
    be = rng.uniform(0.1, 1.0, (B, H, T)).astype(np.float32)
    init = rng.standard_normal((B, H, dk, dv))
    t = 6
    al[:, :, t] = 1.0
    be[:, :, t] = 1.0
    _, fin_t = oracle.gdn_fwd(q[:, :, :t + 1], k[:, :, :t + 1], v[:, :, :t + 1],
                              al[:, :, :t + 1], be[:, :, :t + 1], init)
    kh = k[:, :, t].astype(np.float64)
    kh /= np.linalg.norm(kh, axis=-1, keepdims=True)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(fin_t[b, h].T @ kh[b, h], v[b, h, t], rtol=1e-10,
                                       atol=1e-10)


def test_orthogonal_keys_reduce_to_decayed_linear_attention():
    rng = np.random.default_rng(3)
    B, H, dk, dv = 2, 2, 12, 7
    T = dk
    perm = rng.permutation(dk)
    k = np.zeros((B, H, T, dk), np.float32)
    for t in range(T):
        k[:, :, t, perm[t]] = rng.uniform(0.5, 2.0)          # normalised to e_perm[t]
    q, v = rnd(rng, B, H, T, dk), rnd(rng, B, H, T, dv)
    al = rng.uniform(0.6, 1.0, (B, H, T)).astype(np.float32)
    be = rng.uniform(0.1, 1.0, (B, H, T)).astype(np.float32)
    o, fin = oracle.gdn_fwd(q, k, v, al, be)
    khat = (k != 0).astype(np.float32)
    # values beta_t v_t (exact in fp64) through the pinned parallel form of decayed
    # linear attention
    vb = be[..., None].astype(np.float64) * v.astype(np.float64)
    po = forms.parallel(q, khat, vb, al, "token")
    np.testing.assert_allclose(o, po, rtol=1e-10, atol=1e-10)
    # beta = 1: the recurrent linear-attention oracle itself, outputs and final state
    ro, rf = oracle.fwd(q, khat, v, al, "token")
    o1, f1 = oracle.gdn_fwd(q, k, v, al, np.ones_like(be))
    np.testing.assert_allclose(o1, ro, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(f1, rf, rtol=1e-10, atol=1e-10)


def test_zero_beta_is_pure_decay():
    rng = np.random.default_rng(4)
    B, H, T, dk, dv = 1, 3, 11, 6, 4
    q, k, v = rnd(rng, B, H, T, dk), rnd(rng, B, H, T, dk), rnd(rng, B, H, T, dv)
    al = rng.uniform(0.5, 1.0, (B, H, T)).astype(np.float32)
    init = rng.standard_normal((B, H, dk, dv))
    o, fin = oracle.gdn_fwd(q, k, v, al, np.zeros((B, H, T), np.float32), init)
    p = np.cumprod(al.astype(np.float64), axis=-1)
    ref = p[..., None] * np.einsum("bhtc,bhce->bhte", q.astype(np.float64), init)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin, p[..., -1][..., None, None] * init, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_matches_chunked_form(chunk):
    rng = np.random.default_rng(5 + chunk)
    B, H, T, dk, dv = 2, 2, 70, 16, 12
    q, k, v = rnd(rng, B, H, T, dk), rnd(rng, B, H, T, dk), rnd(rng, B, H, T, dv)
    al = rng.uniform(0.8, 1.0, (B, H, T)).astype(np.float32)
    be = rng.uniform(0.0, 1.0, (B, H, T)).astype(np.float32)
    init = 0.1 * rng.standard_normal((B, H, dk, dv))
    o, fin = oracle.gdn_fwd(q, k, v, al, be, init)
    co, cf = forms.gdn_chunked(q, k, v, al, be, init, chunk=chunk)
    np.testing.assert_allclose(o, co, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(fin, cf, rtol=1e-9, atol=1e-9)


def test_bf16_inputs_widen_exactly():
    from workloads import bf16_bits_to_f32, f32_to_bf16_bits
    rng = np.random.default_rng(6)
    B, H, T, dk, dv = 1, 1, 20, 8, 8
    q, k, v = (f32_to_bf16_bits(rnd(rng, B, H, T, d)) for d in (dk, dk, dv))
    al = rng.uniform(0.8, 1.0, (B, H, T)).astype(np.float32)
    be = rng.uniform(0.0, 1.0, (B, H, T)).astype(np.float32)
    o, f = oracle.gdn_fwd(q, k, v, al, be)
    o2, f2 = oracle.gdn_fwd(*(bf16_bits_to_f32(x) for x in (q, k, v)), al, be)
    assert np.array_equal(o, o2) and np.array_equal(f, f2)
