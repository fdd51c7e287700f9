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
    """One (sequence, head): q,k [L,dk], v [L,dv], alpha [L,dk], eta [L].

    factored: False for the direct exponent differences; True for factors
    referenced per block of `blk` rows (E = 2^{G - ref_b}, F = 1/E, P per
    block pair); "mid" for factors referenced per channel to the chunk's
    midpoint decay r = G_n / 2 (E' = 2^{G - r}, F' = 1/E'), with Q S and K S
    on the state scaled by 2^r and the update 2^r (2^r S + (K F')^T Delta),
    the operands of the bf16-input kernel."""
    L = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        K, Q, V = k[sl], q[sl], v[sl]
        n = K.shape[0]
        G = np.cumsum(np.log(alpha[sl]), axis=0)          # [n, dk]
        beta = eta[sl] / (np.sum(K * K, axis=1) + eps)
        if factored == "mid":
            r = 0.5 * G[-1]                                   # [dk]
            E, F = np.exp(G - r), np.exp(r - G)
            KE, KF, QE = K * E, K * F, Q * E
            Ah = np.tril(KE @ KF.T, -1)
            M = np.tril(QE @ KF.T)
            Sr = np.exp(r)[:, None] * S
            Lm = np.tril(beta[:, None] * Ah, -1)
            R = V - KE @ Sr
            Delta = solve_triangular(np.eye(n) + Lm, beta[:, None] * R, lower=True)
            o[sl] = QE @ Sr + M @ Delta
            S = np.exp(r)[:, None] * (Sr + KF.T @ Delta)
            continue
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


# ---------------------------------------------------------------------------
# Chunk form of the backward (gradient of o and of the final state).
#
# The gradient of the state after token t, G_t (with the read's q_t d_o_t^T
# added), obeys the reverse of the forward recurrence:
#   G_t = dS_t + q_t d_o_t^T,   u_t = G_t^T k_t,
#   dS_{t-1} = alpha_t (G_t - beta_t k_t u_t^T).
# Inside a chunk of n tokens, with Gamma_ts = gamma_t / gamma_s (t >= s) and
# Gend the gradient of the state after the chunk:
#   (I + StrictLower(Gam o K K^T) B) E = V - Diag(gamma) K S          (residuals)
#   (I + StrictUpper(Gam^T o K K^T) B) U = Diag(gamma_n/gamma) K Gend
#                                          + Upper(Gam^T o K Q^T) dO
#   O   = Diag(gamma) Q S + Lower(Gam o Q K^T) B E
#   dv  = B U,   dbeta_t = u_t . e_t
#   G e = Diag(gamma_n/gamma) E Gend^T + Upper(Gam^T o E dO^T) Q
#         - StrictUpper(Gam^T o E U^T) B K                  (rows G_t e_t)
#   S u = Diag(gamma) U S^T + Lower(Gam o U E^T) B K          (rows S_t u_t)
#   dq  = Diag(gamma) dO S^T + Lower(Gam o dO E^T) B K
#   dk  = B (G e - S u) + Diag(dbeta o (beta^2 - 2 beta/(|k|^2+eps))) K
#         (the direct step drops the second beta term)
#   dS_start = gamma_n Gend + Q^T Diag(gamma) dO - K^T Diag(gamma beta) U
# with B = Diag(beta).  The decay gradient uses
#   alpha_t dalpha_t = <G_t, S_t> - beta_t u_t . v_t   and
#   <G_t, S_t> = alpha_{t+1} dalpha_{t+1} + d_o_t . o_t,
# so c_t = alpha_t dalpha_t is a reverse running sum inside the chunk that
# starts from <Gend, S_end> at the chunk's end.
# Every quantity is linear in the columns of the state (dv), so the model
# can run on column slices and add the slices' contributions.
# ---------------------------------------------------------------------------

def chunked_bwd_seq(q, k, v, alpha, eta, eps, C, S0, d_o, d_fin, beta_direct=False,
                    dv_slices=1):
    """One (sequence, head) in fp64: returns dq, dk, dv, dalpha, deta, dS0."""
    L, dk = q.shape
    dv = v.shape[1]
    alpha = np.ones(L) if alpha is None else alpha
    kk = np.sum(k * k, axis=1)
    beta_all = eta if beta_direct else eta / (kk + eps)
    # forward pass: chunk-start states and the final state
    starts = []
    S = np.array(S0, dtype=np.float64, copy=True)
    chunks = [(c0, min(c0 + C, L)) for c0 in range(0, L, C)]
    ops = []
    for a, b in chunks:
        K, Q, V = k[a:b], q[a:b], v[a:b]
        n = b - a
        g = np.cumsum(np.log(alpha[a:b]))
        gam = np.exp(g)
        Gam = np.tril(np.exp(np.minimum(g[:, None] - g[None, :], 0.0)))
        beta = beta_all[a:b]
        E = solve_triangular(np.eye(n) + np.tril(Gam * (K @ K.T), -1) * beta[None, :],
                             V - gam[:, None] * (K @ S), lower=True)
        starts.append(S.copy())
        ops.append((gam, Gam, beta, E))
        S = gam[-1] * S + K.T @ ((beta * gam[-1] / gam)[:, None] * E)
    S_L = S
    dq = np.zeros((L, dk))
    dkp = np.zeros((L, dk))
    dvv = np.zeros((L, dv))
    dbeta = np.zeros(L)
    c = np.zeros(L)
    dS0 = np.zeros((dk, dv))
    for cols in np.array_split(np.arange(dv), dv_slices):
        Gend = np.array(d_fin[:, cols], dtype=np.float64, copy=True)
        cend = float(np.sum(Gend * S_L[:, cols]))
        for (a, b), Sc, (gam, Gam, beta, E) in reversed(list(zip(chunks, starts, ops))):
            K, Q, V, dO = k[a:b], q[a:b], v[a:b][:, cols], d_o[a:b][:, cols]
            Sc, E = Sc[:, cols], E[:, cols]
            n = b - a
            B = beta
            O = gam[:, None] * (Q @ Sc) + (Gam * (Q @ K.T) * B[None, :]) @ E
            U = solve_triangular(np.eye(n) + np.triu(Gam.T * (K @ K.T), 1) * B[None, :],
                                 (gam[-1] / gam)[:, None] * (K @ Gend) + (Gam.T * (K @ Q.T)) @ dO,
                                 lower=False)
            dvv[a:b, cols] = B[:, None] * U
            dbeta[a:b] += np.sum(U * E, axis=1)
            terms = np.sum(dO * O, axis=1) - B * np.sum(U * V, axis=1)
            c[a:b] += cend + np.cumsum(terms[::-1])[::-1]
            Ge = ((gam[-1] / gam)[:, None] * (E @ Gend.T) + (Gam.T * (E @ dO.T)) @ Q
                  - (np.triu(Gam.T * (E @ U.T), 1) * B[None, :]) @ K)
            Su = gam[:, None] * (U @ Sc.T) + (Gam * (U @ E.T) * B[None, :]) @ K
            dq[a:b] += gam[:, None] * (dO @ Sc.T) + (Gam * (dO @ E.T) * B[None, :]) @ K
            dkp[a:b] += B[:, None] * (Ge - Su)
            Gend = gam[-1] * Gend + Q.T @ (gam[:, None] * dO) - K.T @ ((gam * B)[:, None] * U)
            cend = float(np.sum(Gend * Sc))
        dS0[:, cols] = Gend
    if beta_direct:
        dkk = dkp + (dbeta * beta_all ** 2)[:, None] * k
        deta = dbeta
    else:
        dkk = dkp + (dbeta * (beta_all ** 2 - 2 * beta_all / (kk + eps)))[:, None] * k
        deta = dbeta / (kk + eps)
    return dq, dkk, dvv, c / alpha, deta, dS0


def chunked_bwd(q, k, v, alpha, eta, d_o, cu_seqlens, eps, C, initial_state=None, d_final=None,
                beta_direct=False, dv_slices=1):
    """Packed layout as `chunked`; returns a dict like the oracle's bwd."""
    tok, H, dk = q.shape
    dv = v.shape[2]
    n = len(cu_seqlens) - 1
    out = {"dq": np.zeros((tok, H, dk)), "dk": np.zeros((tok, H, dk)),
           "dv": np.zeros((tok, H, dv)), "dalpha": np.zeros((tok, H)),
           "deta": np.zeros((tok, H)), "dS0": np.zeros((n, H, dk, dv))}
    for s in range(n):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        for h in range(H):
            S0 = np.zeros((dk, dv)) if initial_state is None else initial_state[s, h]
            dF = np.zeros((dk, dv)) if d_final is None else d_final[s, h]
            r = chunked_bwd_seq(q[a:b, h], k[a:b, h], v[a:b, h],
                                None if alpha is None else alpha[a:b, h], eta[a:b, h], eps, C,
                                S0, d_o[a:b, h], dF, beta_direct, dv_slices)
            for key, val in zip(("dq", "dk", "dv", "dalpha", "deta"), r[:5]):
                out[key][a:b, h] = val
            out["dS0"][s, h] = r[5]
    if alpha is None:
        out["dalpha"] = None
    return out
