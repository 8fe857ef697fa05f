"""Two independent fp64 restatements of causal linear attention, used only to pin the
recurrent oracle (TEST INFRASTRUCTURE ONLY; tiny inputs; numpy).

* ``brute_force`` — masked O(T^2) attention written from the definition:
  o_t = [sum_{j<=t} w_tj v_j + (P(0,t) (.) phi(q_t))^T h0]
        / [sum_{j<=t} w_tj + (P(0,t) (.) phi(q_t))^T z0],
  w_tj = sum_c phi(q_t)_c phi(k_j)_c P_c(j+1, t),  P_c(a, t) = prod_{s=a..t} g_s[c].
  This is the similarity form of the textbook chapter 1.6 "linear attention" section
  (sim(q,k) = phi(q)^T phi(k)) times the product of the decays between key and query.
  Products and sums are explicit Python loops.

* ``parallel`` — the training-style parallel form of the same chapter's code listing,
  A = tril(phi(Q) phi(K)^T), O = A V / A 1, extended to decays by the whole-sequence
  factorisation A_tj = (phi(q_t) e^{G_t}) . (phi(k_j) e^{-G_j}) with G the inclusive
  cumulative sum of ln g (valid only for short sequences: e^{-G} grows without bound).
"""
from __future__ import annotations

import numpy as np


def phi(x: np.ndarray, elu1: bool) -> np.ndarray:
    if not elu1:
        return np.array(x, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def gates(decay, kind: str, B: int, H: int, T: int, dk: int) -> np.ndarray:
    """Per-token, per-key decay g[b,h,t,c] in fp64."""
    if kind == "none":
        return np.ones((B, H, T, dk))
    d = np.asarray(decay, dtype=np.float64)
    if kind == "gamma":
        return np.broadcast_to(d[None, :, None, None], (B, H, T, dk)).copy()
    if kind == "gate":
        return d.reshape(B, H, T, dk).copy()
    if kind == "token":
        return np.broadcast_to(d.reshape(B, H, T)[..., None], (B, H, T, dk)).copy()
    raise ValueError(kind)


def brute_force(q, k, v, decay=None, kind="none", init=None, *, phi_elu1=False,
                normalize=False):
    """O(T^2 dk) masked attention with explicit decay products.  All inputs fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = v.shape[3]
    g = gates(decay, kind, B, H, T, dk)
    qb, kb = phi(q, phi_elu1), phi(k, phi_elu1)
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            h0 = None if init is None else np.asarray(init, dtype=np.float64)[b, h]
            for t in range(T):
                num = np.zeros(dv)
                den = 0.0
                for j in range(t + 1):
                    w = 0.0
                    for c in range(dk):
                        p = 1.0
                        for s in range(j + 1, t + 1):
                            p *= g[b, h, s, c]
                        w += qb[b, h, t, c] * kb[b, h, j, c] * p
                    num += w * v[b, h, j]
                    den += w
                if h0 is not None:
                    for c in range(dk):
                        p = 1.0
                        for s in range(0, t + 1):
                            p *= g[b, h, s, c]
                        num += qb[b, h, t, c] * p * h0[c, :dv]
                        if normalize:
                            den += qb[b, h, t, c] * p * h0[c, dv]
                out[b, h, t] = num / den if normalize else num
    return out


def final_state_closed_form(k, v, decay=None, kind="none", init=None, *, phi_elu1=False,
                            normalize=False):
    """h_T = sum_j diag(P(j+1, T-1)) phi(k_j) v_j^T + diag(P(0, T-1)) h0, with the z column
    (v replaced by 1) appended when normalising."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, dk = k.shape
    dv = v.shape[3]
    g = gates(decay, kind, B, H, T, dk)
    kb = phi(k, phi_elu1)
    ncol = dv + (1 if normalize else 0)
    res = np.zeros((B, H, dk, ncol))
    for b in range(B):
        for h in range(H):
            for j in range(T):
                p = np.prod(g[b, h, j + 1:T], axis=0) if j + 1 < T else np.ones(dk)
                res[b, h, :, :dv] += (p * kb[b, h, j])[:, None] * v[b, h, j][None, :]
                if normalize:
                    res[b, h, :, dv] += p * kb[b, h, j]
            if init is not None:
                p0 = np.prod(g[b, h, :T], axis=0) if T > 0 else np.ones(dk)
                res[b, h] += p0[:, None] * np.asarray(init, dtype=np.float64)[b, h]
    return res


def parallel(q, k, v, decay=None, kind="none", init=None, *, phi_elu1=False,
             normalize=False):
    """Masked matrix form with the whole-sequence factorisation of the decay."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = v.shape[3]
    g = gates(decay, kind, B, H, T, dk)
    G = np.cumsum(np.log(g), axis=2)          # inclusive: G_t = sum_{s<=t} ln g_s
    Qd = phi(q, phi_elu1) * np.exp(G)         # phi(q_t) e^{G_t}
    Kd = phi(k, phi_elu1) * np.exp(-G)        # phi(k_j) e^{-G_j}
    A = np.tril(Qd @ np.swapaxes(Kd, -1, -2))  # [B,H,T,T], A_tj for j <= t
    num = A @ v
    den = A.sum(-1)
    if init is not None:
        h0 = np.asarray(init, dtype=np.float64)
        num = num + Qd @ h0[..., :dv]
        if normalize:
            den = den + (Qd @ h0[..., dv:]).squeeze(-1)
    return num / den[..., None] if normalize else num


def gdn_chunked(q, k, v, alpha, beta, init=None, *, chunk=16):
    """Gated delta rule in chunk form (an independent restatement used to pin the recurrent
    oracle).  Writing the update as h_t = alpha_t h_{t-1} + k^_t u_t^T (h = S^T) with the
    pseudo-value u_t = beta_t (v_t - alpha_t h_{t-1}^T k^_t), the u of one chunk solve the
    unit lower-triangular system (I + A) U = diag(beta) V - diag(beta g) K^ H with
    A_tj = beta_t (g_t / g_j) k^_t . k^_j (j < t) and g the cumulative product of alpha in
    the chunk; then O = diag(g) Q H + (M (.) Q K^^T) U with M_tj = g_t / g_j (j <= t), and
    H <- g_L H + (diag(g_L / g) K^)^T U.  fp64, numpy solve."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    al = np.asarray(alpha, dtype=np.float64)
    be = np.asarray(beta, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = v.shape[3]
    out = np.zeros((B, H, T, dv))
    fin = np.zeros((B, H, dk, dv))
    nrm = np.maximum(np.sqrt(np.sum(k * k, axis=-1, keepdims=True)), 1e-12)
    kh = k / nrm
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if init is None else np.array(init[b, h], dtype=np.float64)
            for t0 in range(0, T, chunk):
                sl = slice(t0, min(T, t0 + chunk))
                Q, K, V = q[b, h, sl], kh[b, h, sl], v[b, h, sl]
                a, bt = al[b, h, sl], be[b, h, sl]
                L = Q.shape[0]
                g = np.cumprod(a)
                ratio = g[:, None] / g[None, :]
                A = np.tril(bt[:, None] * ratio * (K @ K.T), -1)
                rhs_v = bt[:, None] * V
                rhs_k = (bt * g)[:, None] * K
                Tm = np.linalg.solve(np.eye(L) + A, np.eye(L))
                U = Tm @ rhs_v - (Tm @ rhs_k) @ S
                M = np.tril(ratio)
                out[b, h, sl] = g[:, None] * (Q @ S) + (M * (Q @ K.T)) @ U
                S = g[-1] * S + ((g[-1] / g)[:, None] * K).T @ U
            fin[b, h] = S
    return out, fin
