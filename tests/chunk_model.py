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


# ---------------------------------------------------------------------------
# Per-channel decay (Kimi Delta Attention's gate, survey page section
# "Metodologia e Estrutura"): S~ = Diag(a_t) S.  With G_t the cumulative
# log-decay vector inside the chunk (one entry per key channel) the chunk
# form keeps its shape; every decay factor becomes a per-channel one:
#
#   Ahat_ts = sum_i k_t[i] k_s[i] exp(G_t[i] - G_s[i])   (t > s)
#   M_ts    = sum_i q_t[i] k_s[i] exp(G_t[i] - G_s[i])   (t >= s)
#   R       = V - (K o exp(G)) S,      Delta = (I + StrictLower(Diag(beta) Ahat))^{-1} Diag(beta) R
#   O       = (Q o exp(G)) S + M Delta
#   S'      = Diag(exp(G_n)) S + (K o exp(G_n - G))^T Delta
#
# factored=True forms Ahat and M the way the GPU kernel does, from operands
# decayed relative to the start of each block of `blk` rows (so every
# factor is at most 1, except the within-block growth exp(ref - G_s)):
#   E_t = exp(G_t - ref_b(t)),  F_s = exp(ref_b(s) - G_s),
#   P_bc = exp(ref_b - ref_c),  ref_b = G just before block b,
#   Ahat_ts = sum_i (k_t E_t)[i] P_b(t)b(s)[i] (k_s F_s)[i].

def chunked_ch_seq(q, k, v, alpha, eta, eps, C, S0, factored=False, blk=16):
    """One (sequence, head): q,k [L,dk], v [L,dv], alpha [L,dk], eta [L]."""
    L = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        K, Q, V = k[sl], q[sl], v[sl]
        n = K.shape[0]
        G = np.cumsum(np.log(alpha[sl]), axis=0)          # [n, dk]
        beta = eta[sl] / (np.sum(K * K, axis=1) + eps)
        if factored:
            ref = np.zeros_like(G)
            for t in range(n):
                b0 = (t // blk) * blk
                ref[t] = G[b0 - 1] if b0 > 0 else 0.0
            E, F = np.exp(G - ref), np.exp(ref - G)
            KE, KF, QE = K * E, K * F, Q * E
            Ah = np.zeros((n, n))
            M = np.zeros((n, n))
            for t in range(n):
                for s in range(t + 1):
                    P = np.exp(ref[t] - ref[s])
                    if s < t:
                        Ah[t, s] = np.sum(KE[t] * P * KF[s])
                    M[t, s] = np.sum(QE[t] * P * KF[s])
        else:
            D = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))  # [n, n, dk]
            Ah = np.tril(np.einsum("ti,si,tsi->ts", K, K, D), -1)
            M = np.tril(np.einsum("ti,si,tsi->ts", Q, K, D))
        gam = np.exp(G)
        Lm = np.tril(beta[:, None] * Ah, -1)
        R = V - (K * gam) @ S
        Delta = solve_triangular(np.eye(n) + Lm, beta[:, None] * R, lower=True)
        o[sl] = (Q * gam) @ S + M @ Delta
        S = gam[-1][:, None] * S + (K * np.exp(G[-1] - G)).T @ Delta
    return o, S


def chunked_ch(q, k, v, alpha, eta, cu_seqlens, eps, C, initial_state=None, factored=False):
    """Packed layout: q,k [tok,H,dk], v [tok,H,dv], alpha [tok,H,dk], eta [tok,H]."""
    tok, H, dk = q.shape
    dv = v.shape[2]
    n = len(cu_seqlens) - 1
    o = np.zeros((tok, H, dv))
    fin = np.zeros((n, H, dk, dv))
    for s in range(n):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        for h in range(H):
            S0 = np.zeros((dk, dv)) if initial_state is None else initial_state[s, h]
            o[a:b, h], fin[s, h] = chunked_ch_seq(q[a:b, h], k[a:b, h], v[a:b, h], alpha[a:b, h],
                                                  eta[a:b, h], eps, C, S0, factored)
    return o, fin
