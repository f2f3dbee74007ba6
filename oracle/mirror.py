"""fp64 chunkwise form of the KDA recurrence -- TEST INFRASTRUCTURE.

Not the oracle: the oracle is the token loop in kda_oracle.c.  This mirror
exists to pin that the chunkwise algebra (the WY / UT form used by chunked
prefill kernels) reproduces the token loop for every chunk size, which is the
"outputs do not depend on the chunk size" invariant.

Within a chunk of n rows, with G the inclusive cumulative sum of the log-decay
g over the chunk's rows (per key channel), Gam_r = exp(G_r) and the normalised
q, k:

    A[r,i] = beta_r * sum_d k[r,d] k[i,d] exp(G[r,d] - G[i,d])     (i < r)
    P[r,i] =          sum_d q[r,d] k[i,d] exp(G[r,d] - G[i,d])     (i <= r)
    T      = (I + A)^-1
    W      = T Diag(beta) (K * Gam)          U~ = T Diag(beta) V
    U      = U~ - W S
    O      = (Q * Gam) S + P U
    S'     = Diag(exp(G_last)) S + (K * exp(G_last - G))^T U

Derivation: unrolling S_r = Diag(Gam_r) S + sum_{i<=r} Diag(Gam_r / Gam_i) k_i u_i^T
inside the chunk and substituting into u_r = beta_r (v_r - (Diag(alpha_r) S_{r-1})^T k_r)
gives (I + A) U = Diag(beta) V - Diag(beta) (K * Gam) S.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def _norm_rows(x, scale=1.0):
    return x * (scale / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS))


def chunk_terms(q, k, g, beta, scale=1.0, qk_l2norm=1):
    """Per-chunk factors for one chunk (rows of one sequence, one head)."""
    if qk_l2norm:
        Q = _norm_rows(q, scale)
        K = _norm_rows(k)
    else:
        Q, K = q * scale, k
    n = K.shape[0]
    G = np.cumsum(g, axis=0)
    diff = G[:, None, :] - G[None, :, :]                     # [r, i, d]
    lower_incl = np.tril(np.ones((n, n), dtype=bool))
    lower_strict = np.tril(np.ones((n, n), dtype=bool), -1)
    E = np.exp(np.where(lower_incl[:, :, None], diff, -np.inf))
    KK = np.einsum("rd,id,rid->ri", K, K, E)
    A = np.where(lower_strict, beta[:, None] * KK, 0.0)
    P = np.where(lower_incl, np.einsum("rd,id,rid->ri", Q, K, E), 0.0)
    T = np.linalg.inv(np.eye(n) + A)
    Gam = np.exp(G)
    W = T @ (beta[:, None] * K * Gam)
    Kbar = K * np.exp(G[-1][None, :] - G)
    gamma = np.exp(G[-1])
    return dict(T=T, W=W, P=P, Qbar=Q * Gam, Kbar=Kbar, gamma=gamma)


def chunked_unit(q, k, v, g, beta, S0, C, scale=1.0, qk_l2norm=1):
    """One (sequence, head): q,k,g [L,dk], v [L,dv], beta [L], S0 [dk,dv].
    Returns (o [L,dv], S_final)."""
    L = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        f = chunk_terms(q[sl], k[sl], g[sl], beta[sl], scale, qk_l2norm)
        Ut = f["T"] @ (beta[sl][:, None] * v[sl])
        U = Ut - f["W"] @ S
        o[sl] = f["Qbar"] @ S + f["P"] @ U
        S = f["gamma"][:, None] * S + f["Kbar"].T @ U
    return o, S


def chunked_prefill(q, k, v, g, beta, cu_seqlens, S0, C, scale=1.0, qk_l2norm=1):
    """Chunkwise fp64 prefill over all (sequence, head) units; same shapes as
    oracle.prefill."""
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu_seqlens) - 1
    o = np.zeros((T, H, dv))
    Sf = np.zeros((N, H, dk, dv))
    for n in range(N):
        a, b = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        for h in range(H):
            s0 = np.zeros((dk, dv)) if S0 is None else S0[n, h]
            o[a:b, h], Sf[n, h] = chunked_unit(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h],
                                               beta[a:b, h], s0, C, scale, qk_l2norm)
    return o, Sf
