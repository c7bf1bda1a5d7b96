"""Chunk-parallel (WY) form of KDA in fp64 numpy.

TEST INFRASTRUCTURE ONLY (same rules as ``oracle.py``).  This is a second,
independent CPU implementation that exists to pin the chunk algebra the GPU
path is built on against the token-by-token recurrence.  It does not call the
recurrence, and the HIP path does not call it.

The pages describe the prefill as a chunked computation (the prhub report on
SGLang PR #32890, sections "实现拆解" and "关键源码片段": 64-row chunks,
16-row sub-blocks, a strictly lower A_kk with a lower-triangular inverse and a
recompute of w and u, then a per-chunk state kernel) but print no formulas.
The formulas below are derived from the recurrence.  For one head and one
chunk of C rows starting from state S0 (d_k x d_v):

    Gam_r = sum_{s<=r} g_s                      (inclusive, per key channel)
    A_kk[r, s] = beta_r sum_c k_r[c] k_s[c] exp(Gam_r[c] - Gam_s[c])   s < r
    A_qk[r, s] =        sum_c q_r[c] k_s[c] exp(Gam_r[c] - Gam_s[c])   s <= r
    Tm = (I + A_kk)^{-1}
    w  = Tm diag(beta) (K * exp(Gam))           u = Tm diag(beta) V
    U  = u - w S0                               (U_r = beta_r (v_r - S'_r^T k_r))
    O  = scale ((Q * exp(Gam)) S0 + A_qk U)
    S  = Diag(exp(Gam_C)) S0 + (K * exp(Gam_C - Gam))^T U

With C = 1 this is the recurrence itself; for larger C it reorders the same
sums.
"""
from __future__ import annotations

import numpy as np


def chunk_seq_head(q, k, v, g, beta, s0, chunk=64, scale=1.0):
    """One (sequence, head): q, k, g [T, d_k]; v [T, d_v]; beta [T];
    s0 [d_k, d_v] (math orientation).  Returns (o [T, d_v], S [d_k, d_v])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    S = np.array(s0, dtype=np.float64, copy=True)
    T = q.shape[0]
    o = np.zeros((T, v.shape[1]), dtype=np.float64)
    for c0 in range(0, T, chunk):
        r = slice(c0, min(c0 + chunk, T))
        qc, kc, vc, gc, bc = q[r], k[r], v[r], g[r], beta[r]
        C = qc.shape[0]
        gam = np.cumsum(gc, axis=0)
        # pairwise decays exp(Gam_r - Gam_s), [C, C, d_k]
        dec = np.exp(gam[:, None, :] - gam[None, :, :])
        lower_strict = np.tril(np.ones((C, C)), -1)
        lower_incl = np.tril(np.ones((C, C)), 0)
        akk = bc[:, None] * np.einsum("rc,sc,rsc->rs", kc, kc, dec) * lower_strict
        aqk = np.einsum("rc,sc,rsc->rs", qc, kc, dec) * lower_incl
        tm = np.linalg.inv(np.eye(C) + akk)
        w = tm @ (bc[:, None] * kc * np.exp(gam))
        u = tm @ (bc[:, None] * vc)
        U = u - w @ S
        o[r] = scale * ((qc * np.exp(gam)) @ S + aqk @ U)
        S = np.exp(gam[-1])[:, None] * S + (kc * np.exp(gam[-1][None, :] - gam)).T @ U
    return o, S


def chunk_prefill(q, k, v, g, beta, cu_seqlens, s0=None, chunk=64, scale=1.0):
    """Packed sequences, all heads.  s0: [N, H, d_v, d_k] or None.
    Returns (o [T, H, d_v], s_final [N, H, d_v, d_k])."""
    q = np.asarray(q)
    T, H, dk = q.shape
    dv = np.shape(v)[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    o = np.zeros((T, H, dv), dtype=np.float64)
    s_fin = np.zeros((N, H, dv, dk), dtype=np.float64)
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            st = np.zeros((dk, dv)) if s0 is None else np.asarray(s0[n, h], dtype=np.float64).T
            on, sn = chunk_seq_head(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h], beta[a:b, h],
                                    st, chunk=chunk, scale=scale)
            o[a:b, h] = on
            s_fin[n, h] = sn.T
    return o, s_fin
