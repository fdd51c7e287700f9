"""Chunkwise (WY / UT-transform) form of the KLA recurrence in fp64 numpy.

Test-only model used to pin the oracle against an independent formulation:
the KLA summary page ("Resumo Tecnico: Atencao Linear Kaczmarz (KLA)",
section "Implementacao") states that KLA keeps Gated DeltaNet's
chunk-parallel algorithm and changes only the diagonal coefficient matrix
B = Diag(beta_1..beta_C) inside the chunk solver.  Written out for one
chunk of n tokens with chunk-start state S (dk x dv):

  g_r = sum_{i<=r} log alpha_i,  gamma_r = exp(g_r),
  Gam_rs = exp(g_r - g_s) for r >= s, else 0
  L   = strictly-lower( Diag(beta) (K K^T o Gam) )
  T   = (I + L)^{-1} Diag(beta)
  U   = T V,   W = T Diag(gamma) K,   Delta = U - W S
  O   = Diag(gamma) Q S + lower(Q K^T o Gam) Delta
  S'  = gamma_n S + K^T Diag(gamma_n / gamma) Delta

It shares no code with the oracle or the HIP library.
"""
import numpy as np
from scipy.linalg import solve_triangular


def chunked_seq(q, k, v, alpha, eta, eps, C, S0):
    """One (sequence, head): q,k [L,dk], v [L,dv], alpha,eta [L]."""
    L = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        K, Q, V = k[sl], q[sl], v[sl]
        n = K.shape[0]
        g = np.cumsum(np.log(alpha[sl]))
        gam = np.exp(g)
        beta = eta[sl] / (np.sum(K * K, axis=1) + eps)
        tri = np.tril(np.ones((n, n)))
        Gam = np.exp(np.minimum(g[:, None] - g[None, :], 0.0)) * tri
        Lm = np.tril(beta[:, None] * (K @ K.T) * Gam, -1)
        T = solve_triangular(np.eye(n) + Lm, np.diag(beta), lower=True)
        U = T @ V
        W = T @ (gam[:, None] * K)
        Delta = U - W @ S
        M = (Q @ K.T) * Gam
        o[sl] = gam[:, None] * (Q @ S) + M @ Delta
        S = gam[-1] * S + K.T @ ((gam[-1] / gam)[:, None] * Delta)
    return o, S


def chunked(q, k, v, alpha, eta, cu_seqlens, eps, C, initial_state=None):
    """Packed layout: q,k [tok,H,dk], v [tok,H,dv], alpha/eta [tok,H]."""
    tok, H, dk = q.shape
    dv = v.shape[2]
    n = len(cu_seqlens) - 1
    o = np.zeros((tok, H, dv))
    fin = np.zeros((n, H, dk, dv))
    for s in range(n):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        for h in range(H):
            S0 = np.zeros((dk, dv)) if initial_state is None else initial_state[s, h]
            o[a:b, h], fin[s, h] = chunked_seq(q[a:b, h], k[a:b, h], v[a:b, h],
                                               alpha[a:b, h], eta[a:b, h], eps, C, S0)
    return o, fin
