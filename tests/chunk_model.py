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
