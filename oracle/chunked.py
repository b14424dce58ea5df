"""Brute-force float64 chunked (WY / UT) form of the gated delta rule.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It pins the token
recurrence and the chunk algebra the HIP kernels use: run with chunk sizes 16
and 64 it must agree with ``oracle.recurrence`` to ~1e-12 (pin P7).

The pages name a WY-form chunk (TensorRT-LLM PR #19960, KDA MTP verify item)
and 64-token chunks (the v64 of the cudnn-frontend Hopper kernel's name, PR #1056)
but print no chunk equations.  The form below is derived from the recurrence.
Unrolling S_t = D_t S_{t-1} + k_t u_t^T inside one chunk (rows 0..L-1, start
state S0, Gamma_i = sum_{s<=i} g_s the in-chunk inclusive cumulative sum of the
log decays, a vector over key channels):

    A_ij = beta_i * sum_c k_ic k_jc exp(Gamma_ic - Gamma_jc)     (j < i, else 0)
    P_ij =          sum_c q_ic k_jc exp(Gamma_ic - Gamma_jc)     (j <= i, else 0)
    Kt = K o exp(Gamma),  Qt = Q o exp(Gamma),  Kh = K o exp(Gamma_L - Gamma)
    (I + A) U = diag(beta) (V - Kt S0)
    O   = Qt S0 + P U
    S_L = Diag(exp Gamma_L) S0 + Kh^T U

Every exp here is of a non-positive number (pairwise differences only for
j <= i), so nothing overflows at any gate; the linear solve uses numpy.linalg.
No blocking, factorisation or reordering beyond these definitions.
"""
from __future__ import annotations

import numpy as np

from . import _packed


def chunk_step(Q, K, V, G, beta, S0):
    """One chunk: Q, K, G [L, DK], V [L, DV], beta [L], S0 [DK, DV] -> (O, S_L)."""
    L = Q.shape[0]
    Gam = np.cumsum(G, axis=0)                               # inclusive in-chunk cumsum
    A = np.zeros((L, L))
    P = np.zeros((L, L))
    for i in range(L):
        for j in range(i + 1):
            dec = np.exp(Gam[i] - Gam[j])                    # exp(Gamma_i - Gamma_j), <= 1
            if j < i:
                A[i, j] = beta[i] * np.dot(K[i] * K[j], dec)
            P[i, j] = np.dot(Q[i] * K[j], dec)
    Kt = K * np.exp(Gam)
    Qt = Q * np.exp(Gam)
    Kh = K * np.exp(Gam[L - 1] - Gam)
    U = np.linalg.solve(np.eye(L) + A, beta[:, None] * (V - Kt @ S0))
    O = Qt @ S0 + P @ U
    S = np.exp(Gam[L - 1])[:, None] * S0 + Kh.T @ U
    return O, S


def chunked(q, k, v, g, beta, initial_state=None, cu_seqlens=None, chunk=64):
    """Chunked form over every (sequence, head); chunks start at each sequence
    start and the last chunk of a sequence is shorter.  Returns (o, final_state)
    in packed layout, like ``oracle.recurrence``."""
    q, k, v, g, beta, s0, cu = _packed(q, k, v, g, beta, initial_state, cu_seqlens)
    T, H, DK = q.shape
    DV = v.shape[-1]
    N = len(cu) - 1
    o = np.zeros((T, H, DV))
    sT = np.zeros((N, H, DK, DV))
    for n in range(N):
        for h in range(H):
            S = np.zeros((DK, DV)) if s0 is None else s0[n, h].copy()
            for c0 in range(cu[n], cu[n + 1], chunk):
                c1 = min(c0 + chunk, cu[n + 1])
                O, S = chunk_step(q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], g[c0:c1, h],
                                  beta[c0:c1, h], S)
                o[c0:c1, h] = O
            sT[n, h] = S
    return o, sT
