"""fp64 numpy model of the chunk algebra the HIP kernels implement (test helper).

Per (b, h) and chunk n of length L (tokens t = nC + i), with b_i[c] = prod_{s<=i} g_s[c]
the inclusive product of the decays inside the chunk (e^{lambda_i}):
    Qt = phi(Q) * b,  Kt = phi(K) / b,  Kh = phi(K) * b_{L-1} / b
    A  = tril(Qt Kt^T)                      (intra-chunk, causal)
    O  = A V + Qt H_n,   den = A 1 + Qt z_n  (output; H_n = state before the chunk)
    H_{n+1} = diag(b_{L-1}) H_n + Kh^T V,   z_{n+1} = b_{L-1} z_n + Kh^T 1
It unrolls the recurrence S_t = G_t (.) S_{t-1} + v_t phi(k_t)^T over one chunk
(textbook chapter 1.6 "linear attention"; decay as in the FLA RetNet/GLA posts; the
chapter's Mamba-2 remark: decay-masked linear attention trained in chunks).  The tests
check it against the token-by-token oracle; it shares no code with either side.
"""
from __future__ import annotations

import numpy as np

from oracle.forms import gates, phi  # plain helpers (feature map, decay broadcast)


def chunked(q, k, v, decay=None, kind="none", init=None, *, chunk=64, phi_elu1=False,
            normalize=False):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = v.shape[3]
    g = gates(decay, kind, B, H, T, dk)
    qb, kb = phi(q, phi_elu1), phi(k, phi_elu1)
    ncol = dv + (1 if normalize else 0)
    out = np.zeros((B, H, T, dv))
    final = np.zeros((B, H, dk, ncol))
    for b in range(B):
        for h in range(H):
            Hs = np.zeros((dk, ncol)) if init is None else np.array(init[b, h], dtype=np.float64)
            for t0 in range(0, T, chunk):
                L = min(chunk, T - t0)
                sl = slice(t0, t0 + L)
                bcum = np.cumprod(g[b, h, sl], axis=0)          # [L, dk]
                Qt = qb[b, h, sl] * bcum
                Kt = kb[b, h, sl] / bcum
                Kh = kb[b, h, sl] * (bcum[-1] / bcum)
                A = np.tril(Qt @ Kt.T)
                Vx = v[b, h, sl]
                if normalize:
                    Vx = np.concatenate([Vx, np.ones((L, 1))], axis=1)
                O = A @ Vx + Qt @ Hs
                out[b, h, sl] = O[:, :dv] / O[:, dv:] if normalize else O[:, :dv]
                Hs = bcum[-1][:, None] * Hs + Kh.T @ Vx
            final[b, h] = Hs
    return out, final


SAFE_DECAY = 2.0 ** -100   # the fused kernel's smallest chunk decay product (per key)


def unsafe_units(decay, kind, B, H, T, dk, chunk):
    """[B, H] booleans: units where some chunk's product of the decays (per key) falls
    below SAFE_DECAY, i.e. the ones the fused kernel hands to the exact 16-token path."""
    g = gates(decay, kind, B, H, T, dk).astype(np.float32)
    out = np.zeros((B, H), dtype=bool)
    for t0 in range(0, T, chunk):
        p = np.prod(g[:, :, t0:t0 + chunk].astype(np.float64), axis=2)   # [B, H, dk]
        out |= np.any(p < SAFE_DECAY, axis=2)
    return out


def exact16(q, k, v, decay=None, kind="none", init=None, *, phi_elu1=False, normalize=False):
    """The exact 16-token path (exact_fwd.hpp) in fp64: per chunk of 16 tokens,
        A_ij = sum_c phi(q_ic) phi(k_jc) P_c(j+1..i)  with a running product per key
               (j = i, i-1, .., 0; P multiplied by the decay of row j after row j is used),
        O    = A V + (phi(Q) P(0..i)) H,   H <- diag(P(0..15)) H + (phi(K) P(j+1..15))^T V,
    every product formed by multiplying decays in (0, 1] only (no division)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = v.shape[3]
    g = gates(decay, kind, B, H, T, dk)
    qb, kb = phi(q, phi_elu1), phi(k, phi_elu1)
    ncol = dv + (1 if normalize else 0)
    out = np.zeros((B, H, T, dv))
    final = np.zeros((B, H, dk, ncol))
    R = 16
    for b in range(B):
        for h in range(H):
            Hs = np.zeros((dk, ncol)) if init is None else np.array(init[b, h], dtype=np.float64)
            for t0 in range(0, T, R):
                L = min(R, T - t0)
                sl = slice(t0, t0 + L)
                Q, Kr, G = qb[b, h, sl], kb[b, h, sl], g[b, h, sl]
                Vx = v[b, h, sl]
                if normalize:
                    Vx = np.concatenate([Vx, np.ones((L, 1))], axis=1)
                A = np.zeros((L, L))
                for i in range(L):
                    run = np.ones(dk)
                    for j in range(i, -1, -1):
                        A[i, j] = np.sum(Q[i] * Kr[j] * run)
                        run = run * G[j]
                pre = np.ones(dk)
                Qt = np.zeros_like(Q)
                for i in range(L):
                    pre = pre * G[i]
                    Qt[i] = Q[i] * pre
                suf = np.ones(dk)
                Kh = np.zeros_like(Kr)
                for j in range(L - 1, -1, -1):
                    Kh[j] = Kr[j] * suf
                    suf = suf * G[j]
                O = A @ Vx + Qt @ Hs
                out[b, h, sl] = O[:, :dv] / O[:, dv:] if normalize else O[:, :dv]
                Hs = pre[:, None] * Hs + Kh.T @ Vx
            final[b, h] = Hs
    return out, final


def ext_decay_ratio(alpha):
    """g_t / g_j (t >= j) of one chunk's per-token decays as the gated delta rule kernels
    form it, emulated in fp32: the inclusive product g = m 2^e is scanned with m renormalised
    to [0.5, 1) by frexp after every product (Hillis-Steele over 64 lanes, as the wave does),
    then ratio = ldexp(m_t * (1 / m_j), e_t - e_j).  alpha = 0 enters as m = 0.5,
    e = -65536.  Returns a [C, C] fp64 array (upper triangle 0)."""
    a = np.asarray(alpha, dtype=np.float32)
    C = a.shape[0]
    m, e = np.frexp(a)
    m = m.astype(np.float32)
    e = e.astype(np.int64)
    zero = ~(a > 0)
    m[zero], e[zero] = np.float32(0.5), -65536
    d = 1
    while d < C:
        om, oe = m.copy(), e.copy()
        for lane in range(C - 1, d - 1, -1):
            mm, k = np.frexp(np.float32(m[lane] * om[lane - d]))
            m[lane], e[lane] = np.float32(mm), e[lane] + oe[lane - d] + k
        d *= 2
    mi = (np.float32(1.0) / m).astype(np.float32)
    r = np.zeros((C, C))
    for t in range(C):
        for j in range(t + 1):
            x = np.float32(m[t] * mi[j])
            r[t, j] = float(np.ldexp(x, int(max(e[t] - e[j], -2000))))   # fp32 result
    return r
