"""Pins of the fp64 oracle against facts the KLA pages and the mathematics fix.

Each pin takes the reference under test as two callables,
  fwd(q, k, v, alpha, eta, cu_seqlens=None, eps=..., initial_state=None,
      beta_mode="kaczmarz") -> (o, final_state)
  decode(q, k, v, alpha, eta, state, eps=..., beta_mode="kaczmarz")
      -> (o, new_state)
(alpha may be None: no decay; beta_mode "direct": beta = eta)
so the same checks can run against deliberately broken builds of the
reference (tests/test_oracle_mutants.py) and must fail there.

Sources: the KLA technical summary ("Resumo Tecnico: Atencao Linear
Kaczmarz (KLA)", gist.science/pt/paper/2605.08587): the constrained write
and its projection solution (section "Derivacao Teorica"), the relaxed
coefficient and the update (section "A Regra de Atualizacao KLA"), the
three properties of the unrelaxed step (section "Propriedades Chave") and
the drop-in relation to Gated DeltaNet (section "Implementacao").  The
linear-attention survey page (gist.science/pt/paper/2607.07953, section
"Metodologia e Estrutura" and "Notacao Unificada") gives DeltaNet and Gated
DeltaNet; the KLA summary's introduction gives Gated DeltaNet's learned
scalar step that KLA replaces (the "direct" step-size mode).  The survey
page's Kimi Delta Attention (section "Metodologia e Estrutura") decays each
feature channel at its own rate: with channel_decay=True alpha holds one
decay per key channel and S~ = Diag(a_t) S (the pin_channel_* checks).
The curvature-conditioned read ("Don't Read Everything: A Curvature-
Conditioned Query for Linear Attention", sections "Derivacao Teorica" and
"O Mecanismo") cleans the query with the keys' covariance (pin_ccq_*).
"""
import json
import os

import numpy as np

from chunk_model import chunked, chunked_bwd, chunked_ch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-12


def rel(x, y):
    """Normwise max relative error max|x-y| / max|y|."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.max(np.abs(y))
    return float(np.max(np.abs(x - y)) / (den if den > 0 else 1.0))


def _rand_seq(rng, L, H, dk, dv, amin=0.3):
    q = rng.standard_normal((L, H, dk))
    k = rng.standard_normal((L, H, dk)) * np.exp(rng.standard_normal((L, H, 1)))
    v = rng.standard_normal((L, H, dv))
    alpha = rng.uniform(amin, 1.0, (L, H))
    eta = rng.uniform(0.05, 1.0, (L, H))
    return q, k, v, alpha, eta


def pin_worked_example(fwd, decode):
    """Hand-worked two-token example (tests/golden/kla_worked_2x2.json)."""
    with open(os.path.join(GOLDEN, "kla_worked_2x2.json")) as f:
        g = json.load(f)
    o, S = fwd(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
               np.array(g["alpha"]), np.array(g["eta"]), cu_seqlens=[0, 2],
               eps=g["eps"], initial_state=np.array(g["initial_state"]))
    assert np.allclose(o, np.array(g["expected_o"]), rtol=0, atol=1e-14), o
    assert np.allclose(S, np.array(g["expected_final_state"]), rtol=0, atol=1e-14), S


def pin_orthogonal_projection(fwd, decode):
    """eta=1, eps=0: every write satisfies the constraint S_t^T k_t = v_t
    (projection onto the constraint set).  Reading with q_t = k_t therefore
    returns v_t exactly, for any decay and any start state."""
    rng = np.random.default_rng(1)
    L, H, dk, dv = 40, 3, 8, 5
    _, k, v, alpha, _ = _rand_seq(rng, L, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, _ = fwd(k, k, v, alpha, np.ones((L, H)), eps=0.0, initial_state=S0)
    assert rel(o, v) < TIGHT, rel(o, v)


def pin_min_norm_bruteforce(fwd, decode):
    """Each write is the minimum-Frobenius-norm change that meets S^T k = v,
    scaled by the relaxation eta |k|^2/(|k|^2+eps).  Solved here directly as
    a least-norm problem on vec(S) with the Kronecker constraint
    (I_dv kron k^T) vec(S) = v, token by token, with numpy's lstsq."""
    rng = np.random.default_rng(2)
    L, dk, dv, eps = 7, 4, 3, 0.3
    q, k, v, alpha, eta = _rand_seq(rng, L, 1, dk, dv)
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, S_fin = fwd(q, k, v, alpha, eta, eps=eps, initial_state=S0)
    S = S0[0, 0].copy()
    for t in range(L):
        kt, vt = k[t, 0], v[t, 0]
        St = alpha[t, 0] * S
        # vec(S) stacks columns: vec(S)[j*dk + i] = S[i, j]; (S^T k)_j = sum_i S[i,j] k_i
        Cmat = np.kron(np.eye(dv), kt[None, :])
        r = vt - Cmat @ St.reshape(-1, order="F")
        x = np.linalg.lstsq(Cmat, r, rcond=None)[0]
        kk = float(kt @ kt)
        S = St + (eta[t, 0] * kk / (kk + eps)) * x.reshape(dk, dv, order="F")
        assert rel(o[t, 0], S.T @ q[t, 0]) < 1e-11
    assert rel(S_fin[0, 0], S) < 1e-11


def pin_exact_line_search(fwd, decode):
    """eta=1, eps=0: along the write direction k e^T, the step is the exact
    minimiser of the per-token loss l(b) = 1/2 |(S~ + b k e^T)^T k - v|^2,
    found here by a numerical scalar minimiser, and the loss at it is 0."""
    from scipy.optimize import minimize_scalar
    rng = np.random.default_rng(3)
    dk, dv = 6, 4
    for trial in range(5):
        k = rng.standard_normal((1, 1, dk)) * np.exp(rng.standard_normal())
        v = rng.standard_normal((1, 1, dv))
        a = np.array([[rng.uniform(0.2, 1.0)]])
        S0 = rng.standard_normal((1, 1, dk, dv))
        _, S1 = fwd(k, k, v, a, np.ones((1, 1)), eps=0.0, initial_state=S0)
        St = a[0, 0] * S0[0, 0]
        kt, vt = k[0, 0], v[0, 0]
        D = S1[0, 0] - St                         # the write the reference made
        resid = lambda S: 0.5 * float(np.sum((S.T @ kt - vt) ** 2))
        # D must be a multiple of a rank-one k e^T: project onto k to get e-direction
        e_dir = kt @ D                            # = b |k|^2 e, any b
        ke = np.outer(kt, e_dir)
        b_ref = float(np.sum(D * ke) / np.sum(ke * ke))
        assert rel(D, b_ref * ke) < 1e-12         # rank-one along k
        res = minimize_scalar(lambda b: resid(St + b * ke), bracket=(0.0, 2.0 * abs(b_ref) + 1.0),
                              tol=1e-14)
        assert abs(res.x - b_ref) <= 1e-6 * abs(b_ref), (res.x, b_ref)
        assert resid(S1[0, 0]) < 1e-20 * max(1.0, float(vt @ vt))


def pin_normalised_gradient(fwd, decode):
    """The write equals S~ - eta/(|k|^2+eps) grad l(S~) with
    l(S) = 1/2 |S^T k - v|^2; the gradient is taken by central differences
    (exact for this quadratic up to rounding)."""
    rng = np.random.default_rng(4)
    dk, dv = 5, 4
    for trial in range(4):
        eps = [0.0, 1e-3, 0.5, 2.0][trial]
        k = rng.standard_normal((1, 1, dk)) * np.exp(rng.standard_normal())
        v = rng.standard_normal((1, 1, dv))
        a = np.array([[rng.uniform(0.2, 1.0)]])
        et = np.array([[rng.uniform(0.1, 1.0)]])
        S0 = rng.standard_normal((1, 1, dk, dv))
        _, S1 = fwd(k, k, v, a, et, eps=eps, initial_state=S0)
        St = a[0, 0] * S0[0, 0]
        kt, vt = k[0, 0], v[0, 0]
        loss = lambda S: 0.5 * float(np.sum((S.T @ kt - vt) ** 2))
        G = np.zeros_like(St)
        h = 1e-3
        for i in range(dk):
            for j in range(dv):
                E = np.zeros_like(St)
                E[i, j] = h
                G[i, j] = (loss(St + E) - loss(St - E)) / (2 * h)
        step = et[0, 0] / (float(kt @ kt) + eps)
        assert rel(S1[0, 0], St - step * G) < 1e-9, rel(S1[0, 0], St - step * G)


def pin_exact_recall(fwd, decode):
    """No decay, eta=1, eps=0 and orthonormal keys: after n <= dk writes the
    state returns every stored value, S^T k_j = v_j for all j (each later
    write leaves earlier orthogonal constraints intact)."""
    rng = np.random.default_rng(5)
    dk, dv = 8, 6
    for n in (1, 5, 8):
        Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        K = Qm[:, :n].T.reshape(n, 1, dk)
        V = rng.standard_normal((n, 1, dv))
        S0 = rng.standard_normal((1, 1, dk, dv))
        _, S = fwd(K, K, V, np.ones((n, 1)), np.ones((n, 1)), eps=0.0, initial_state=S0)
        assert rel(K[:, 0] @ S[0, 0], V[:, 0]) < 1e-12


def pin_eta_zero(fwd, decode):
    """eta = 0: no write; the state only decays, so
    o_t = (prod_{i<=t} alpha_i) S0^T q_t."""
    rng = np.random.default_rng(6)
    L, H, dk, dv = 30, 2, 5, 7
    q, k, v, alpha, _ = _rand_seq(rng, L, H, dk, dv, amin=0.8)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = fwd(q, k, v, alpha, np.zeros((L, H)), eps=1e-6, initial_state=S0)
    decay = np.cumprod(alpha, axis=0)
    exp_o = np.einsum("th,hij,thi->thj", decay, S0[0], q)
    assert rel(o, exp_o) < TIGHT
    assert rel(S[0], decay[-1][:, None, None] * S0[0]) < TIGHT


def pin_scalar_case(fwd, decode):
    """dk = dv = 1, eta = 1, eps = 0: the write solves s k = v, so
    s_t = v_t / k_t and o_t = q_t v_t / k_t, whatever the decay."""
    rng = np.random.default_rng(7)
    L = 25
    q = rng.standard_normal((L, 1, 1))
    k = rng.uniform(0.5, 2.0, (L, 1, 1)) * rng.choice([-1, 1], (L, 1, 1))
    v = rng.standard_normal((L, 1, 1))
    o, S = fwd(q, k, v, rng.uniform(0.3, 1, (L, 1)), np.ones((L, 1)), eps=0.0,
               initial_state=rng.standard_normal((1, 1, 1, 1)))
    assert rel(o, q * v / k) < TIGHT
    assert abs(S[0, 0, 0, 0] - v[-1, 0, 0] / k[-1, 0, 0]) < 1e-12


def pin_gated_deltanet_form(fwd, decode):
    """Unit-norm keys: KLA is Gated DeltaNet's product form
    S_t = alpha_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T with
    b_t = eta_t/(1+eps); with alpha = 1 it is DeltaNet."""
    rng = np.random.default_rng(8)
    L, dk, dv, eps = 20, 6, 4, 0.25
    q, k, v, alpha, eta = _rand_seq(rng, L, 1, dk, dv)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    for a in (alpha, np.ones_like(alpha)):
        S0 = rng.standard_normal((dk, dv))
        o, S_fin = fwd(q, k, v, a, eta, eps=eps, initial_state=S0[None, None])
        S = S0.copy()
        for t in range(L):
            kt = k[t, 0]
            b = eta[t, 0] / (1.0 + eps)
            S = a[t, 0] * (np.eye(dk) - b * np.outer(kt, kt)) @ S + b * np.outer(kt, v[t, 0])
            assert rel(o[t, 0], S.T @ q[t, 0]) < 1e-11
        assert rel(S_fin[0, 0], S) < 1e-11


def pin_chunk_form(fwd, decode):
    """The chunkwise WY/UT form with B = Diag(beta) gives the same result
    for every chunk size, including ragged last chunks."""
    rng = np.random.default_rng(9)
    H, dk, dv = 2, 6, 5
    cu = np.array([0, 1, 17, 80, 143])
    L = int(cu[-1])
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    S0 = rng.standard_normal((len(cu) - 1, H, dk, dv))
    o, S = fwd(q, k, v, alpha, eta, cu_seqlens=cu, eps=1e-3, initial_state=S0)
    for C in (1, 7, 16, 64):
        oc, Sc = chunked(q, k, v, alpha, eta, cu, 1e-3, C, S0)
        assert rel(o, oc) < 1e-11 and rel(S, Sc) < 1e-11, (C, rel(o, oc), rel(S, Sc))


def pin_packed_and_resume(fwd, decode):
    """Packed sequences equal separate runs, and splitting one sequence in two
    with the first part's final state as the second part's start state
    equals one run."""
    rng = np.random.default_rng(10)
    H, dk, dv = 2, 4, 3
    cu = np.array([0, 9, 9, 30, 41])   # includes an empty sequence
    L = int(cu[-1])
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    S0 = rng.standard_normal((4, H, dk, dv))
    o, S = fwd(q, k, v, alpha, eta, cu_seqlens=cu, eps=1e-6, initial_state=S0)
    for s in range(4):
        a, b = cu[s], cu[s + 1]
        oi, Si = fwd(q[a:b], k[a:b], v[a:b], alpha[a:b], eta[a:b], cu_seqlens=[0, b - a],
                     eps=1e-6, initial_state=S0[s:s + 1])
        assert rel(o[a:b], oi) < TIGHT if b > a else True
        assert rel(S[s], Si[0]) < TIGHT
    # resume: [0,13) then [13,30) of sequence 2
    a, m, b = 9, 13, 30
    o1, S1 = fwd(q[a:m], k[a:m], v[a:m], alpha[a:m], eta[a:m], cu_seqlens=[0, m - a],
                 eps=1e-6, initial_state=S0[2:3])
    o2, S2 = fwd(q[m:b], k[m:b], v[m:b], alpha[m:b], eta[m:b], cu_seqlens=[0, b - m],
                 eps=1e-6, initial_state=S1)
    assert rel(np.concatenate([o1, o2]), o[a:b]) < TIGHT
    assert rel(S2[0], S[2]) < TIGHT
    # an empty sequence returns its start state unchanged
    assert np.array_equal(S[1], S0[1])


def pin_decode_is_one_token(fwd, decode):
    """A decode step on the state after a prefill equals the prefill that is
    one token longer (its last output and final state)."""
    rng = np.random.default_rng(11)
    L, H, dk, dv = 12, 3, 5, 4
    q, k, v, alpha, eta = _rand_seq(rng, L + 1, H, dk, dv)
    _, S = fwd(q[:L], k[:L], v[:L], alpha[:L], eta[:L], eps=1e-4)
    od, Sd = decode(q[L:], k[L:], v[L:], alpha[L:], eta[L:], S, eps=1e-4)
    o_all, S_all = fwd(q, k, v, alpha, eta, eps=1e-4)
    assert rel(od[0], o_all[L]) < TIGHT
    assert rel(Sd, S_all) < TIGHT


def pin_zero_key(fwd, decode):
    """A zero key with eps > 0 writes nothing: the token only decays the
    state, and the read is alpha S^T q."""
    rng = np.random.default_rng(12)
    dk, dv = 4, 3
    S0 = rng.standard_normal((1, 1, dk, dv))
    q = rng.standard_normal((1, 1, dk))
    o, S = fwd(q, np.zeros((1, 1, dk)), rng.standard_normal((1, 1, dv)), np.array([[0.7]]),
               np.array([[0.9]]), eps=1e-6, initial_state=S0)
    assert np.array_equal(S[0, 0], 0.7 * S0[0, 0])
    assert rel(o[0, 0], 0.7 * S0[0, 0].T @ q[0, 0]) < TIGHT


def _gdn_product_form(q, k, v, alpha, b, S0):
    """Gated DeltaNet written as a product of maps, per head:
    S_t = alpha_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T, o_t = S_t^T q_t."""
    L, H, dk = k.shape
    S = S0.copy()
    o = np.zeros(v.shape)
    for t in range(L):
        for h in range(H):
            kt = k[t, h]
            a = 1.0 if alpha is None else alpha[t, h]
            S[h] = a * (np.eye(dk) - b[t, h] * np.outer(kt, kt)) @ S[h] + b[t, h] * np.outer(kt, v[t, h])
            o[t, h] = S[h].T @ q[t, h]
    return o, S


def pin_direct_step_product_form(fwd, decode):
    """Step size given directly (beta = eta, Gated DeltaNet's learned scalar):
    the recurrence equals Gated DeltaNet's product form with b_t = eta_t for
    keys of any norm, and with no decay gate it is DeltaNet.  The decode step
    in the same mode equals one more token."""
    rng = np.random.default_rng(13)
    L, H, dk, dv = 17, 2, 6, 4
    q, k, v, alpha, _ = _rand_seq(rng, L + 1, H, dk, dv)
    k = k * 0.3  # keep |b| |k|^2 moderate so the product form stays well conditioned
    eta = rng.uniform(0.05, 1.0, (L + 1, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    for a in (alpha, None):
        aa = None if a is None else a[:L]
        o, S = fwd(q[:L], k[:L], v[:L], aa, eta[:L], eps=0.5, initial_state=S0,
                   beta_mode="direct")
        eo, eS = _gdn_product_form(q[:L], k[:L], v[:L], aa, eta[:L], S0[0])
        assert rel(o, eo) < 1e-11 and rel(S[0], eS) < 1e-11
        ad = None if a is None else a[L:]
        od, Sd = decode(q[L:], k[L:], v[L:], ad, eta[L:], S, eps=0.5, beta_mode="direct")
        eo1, eS1 = _gdn_product_form(q[L:], k[L:], v[L:], ad, eta[L:], eS)
        assert rel(od[0], eo1[0]) < 1e-11 and rel(Sd[0], eS1) < 1e-11


def pin_no_alpha_is_unit_decay(fwd, decode):
    """Leaving out the decay gate is alpha_t = 1 exactly, in both step-size
    modes, for prefill and decode."""
    rng = np.random.default_rng(14)
    L, H, dk, dv = 21, 2, 5, 3
    q, k, v, _, eta = _rand_seq(rng, L, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    ones = np.ones((L, H))
    for mode in ("kaczmarz", "direct"):
        o1, S1 = fwd(q, k, v, None, eta, eps=1e-3, initial_state=S0, beta_mode=mode)
        o2, S2 = fwd(q, k, v, ones, eta, eps=1e-3, initial_state=S0, beta_mode=mode)
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
        d1 = decode(q[:1], k[:1], v[:1], None, eta[:1], S0, eps=1e-3, beta_mode=mode)
        d2 = decode(q[:1], k[:1], v[:1], ones[:1], eta[:1], S0, eps=1e-3, beta_mode=mode)
        assert np.array_equal(d1[0], d2[0]) and np.array_equal(d1[1], d2[1])
    # and it is not the same as a decaying run
    o3, _ = fwd(q, k, v, 0.5 * ones, eta, eps=1e-3, initial_state=S0)
    assert rel(o3, o1) > 1e-3


def pin_direct_equals_kaczmarz_on_unit_keys(fwd, decode):
    """With unit-norm keys and eps = 0 the Kaczmarz step eta / |k|^2 is eta,
    so the two step-size modes agree; with other norms they differ."""
    rng = np.random.default_rng(15)
    L, H, dk, dv = 19, 2, 7, 5
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    ku = k / np.linalg.norm(k, axis=-1, keepdims=True)
    a = fwd(q, ku, v, alpha, eta, eps=0.0, beta_mode="kaczmarz")
    b = fwd(q, ku, v, alpha, eta, eps=0.0, beta_mode="direct")
    assert rel(a[0], b[0]) < 1e-12 and rel(a[1], b[1]) < 1e-12
    c = fwd(q, 2.0 * ku, v, alpha, eta, eps=0.0, beta_mode="direct")
    d = fwd(q, 2.0 * ku, v, alpha, eta, eps=0.0, beta_mode="kaczmarz")
    assert rel(c[0], d[0]) > 1e-3


def pin_deltanet_exact_recall(fwd, decode):
    """DeltaNet (no decay) with beta = 1 and orthonormal keys stores every
    pair exactly: S^T k_j = v_j for all j after n <= dk writes."""
    rng = np.random.default_rng(16)
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:, :n].T.reshape(n, 1, dk)
    V = rng.standard_normal((n, 1, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, S = fwd(K, K, V, None, np.ones((n, 1)), eps=0.3, initial_state=S0, beta_mode="direct")
    assert rel(K[:, 0] @ S[0, 0], V[:, 0]) < 1e-12


def pin_segment_map_is_affine(fwd, decode):
    """The end state of a stretch of tokens is affine in its start state,
    S_end = A S_start + B: B is the end state from a zero start and A the end
    state from the start I with v = 0 (the columns of the state evolve
    independently, each driven by its own column of v).  Composing two
    stretches composes the maps.  This is what the split-sequence prefill
    runs on (chunk form of the KLA summary, section "Implementacao")."""
    rng = np.random.default_rng(17)
    L, H, dk, dv = 23, 2, 5, 4
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    eye = np.broadcast_to(np.eye(dk), (1, H, dk, dk)).copy()
    X = rng.standard_normal((1, H, dk, dv))
    for mode, kk in (("kaczmarz", k), ("direct", k / np.linalg.norm(k, axis=-1, keepdims=True))):
        _, B = fwd(q, kk, v, alpha, eta, eps=1e-3, beta_mode=mode)
        _, A = fwd(q, kk, np.zeros((L, H, dk)), alpha, eta, eps=1e-3, initial_state=eye,
                   beta_mode=mode)
        _, SX = fwd(q, kk, v, alpha, eta, eps=1e-3, initial_state=X, beta_mode=mode)
        assert rel(SX[0], A[0] @ X[0] + B[0]) < 1e-12
        # two stretches: the maps compose
        m = 9
        _, B1 = fwd(q[:m], kk[:m], v[:m], alpha[:m], eta[:m], eps=1e-3, beta_mode=mode)
        _, A1 = fwd(q[:m], kk[:m], np.zeros((m, H, dk)), alpha[:m], eta[:m], eps=1e-3,
                    initial_state=eye, beta_mode=mode)
        _, B2 = fwd(q[m:], kk[m:], v[m:], alpha[m:], eta[m:], eps=1e-3, beta_mode=mode)
        _, A2 = fwd(q[m:], kk[m:], np.zeros((L - m, H, dk)), alpha[m:], eta[m:], eps=1e-3,
                    initial_state=eye, beta_mode=mode)
        assert rel(A2[0] @ (A1[0] @ X[0] + B1[0]) + B2[0], SX[0]) < 1e-12
        assert rel(A2[0] @ A1[0], A[0]) < 1e-12



# ---- per-channel decay (Kimi Delta Attention's gate) ------------------------

def _rand_ch(rng, L, H, dk, amin=0.3):
    return rng.uniform(amin, 1.0, (L, H, dk))


def pin_channel_uniform_is_scalar(fwd, decode):
    """A per-channel decay with the same rate in every channel is the
    scalar decay (prefill and decode, both step modes)."""
    rng = np.random.default_rng(31)
    L, H, dk, dv = 21, 2, 5, 4
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    ach = np.repeat(alpha[..., None], dk, axis=-1)
    S0 = rng.standard_normal((1, H, dk, dv))
    for mode in ("kaczmarz", "direct"):
        o1, S1 = fwd(q, k, v, ach, eta, eps=1e-3, initial_state=S0, beta_mode=mode,
                     channel_decay=True)
        o2, S2 = fwd(q, k, v, alpha, eta, eps=1e-3, initial_state=S0, beta_mode=mode)
        assert rel(o1, o2) < TIGHT and rel(S1, S2) < TIGHT
        Sd0 = np.repeat(S0, 3, axis=0)                         # 3 sequences x H heads
        od1, Sd1 = decode(q[:3], k[:3], v[:3], ach[:3], eta[:3], Sd0, eps=1e-3, beta_mode=mode,
                          channel_decay=True)
        od2, Sd2 = decode(q[:3], k[:3], v[:3], alpha[:3], eta[:3], Sd0, eps=1e-3, beta_mode=mode)
        assert rel(od1, od2) < TIGHT and rel(Sd1, Sd2) < TIGHT


def pin_channel_eta_zero(fwd, decode):
    """eta = 0: no write; row i of the state (key channel i) decays by the
    product of that channel's rates, so o_t = (Diag(prod_{s<=t} a_s) S0)^T q_t."""
    rng = np.random.default_rng(32)
    L, H, dk, dv = 17, 2, 6, 4
    q, k, v, _, _ = _rand_seq(rng, L, H, dk, dv)
    a = _rand_ch(rng, L, H, dk, amin=0.7)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = fwd(q, k, v, a, np.zeros((L, H)), eps=1e-6, initial_state=S0, channel_decay=True)
    decay = np.cumprod(a, axis=0)                              # [L, H, dk]
    exp_o = np.einsum("thi,hij,thi->thj", decay, S0[0], q)
    assert rel(o, exp_o) < TIGHT
    assert rel(S[0], decay[-1][:, :, None] * S0[0]) < TIGHT


def pin_channel_orthogonal_projection(fwd, decode):
    """eta = 1, eps = 0: whatever the decay, each write meets S_t^T k_t = v_t,
    so reading with q_t = k_t returns v_t."""
    rng = np.random.default_rng(33)
    L, H, dk, dv = 30, 2, 7, 5
    _, k, v, _, _ = _rand_seq(rng, L, H, dk, dv)
    a = _rand_ch(rng, L, H, dk)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, _ = fwd(k, k, v, a, np.ones((L, H)), eps=0.0, initial_state=S0, channel_decay=True)
    assert rel(o, v) < TIGHT, rel(o, v)


def pin_channel_min_norm_bruteforce(fwd, decode):
    """Each write is the least-norm change of the channel-decayed state
    Diag(a_t) S_{t-1} that meets S^T k = v (relaxed by eta |k|^2/(|k|^2+eps)),
    solved with lstsq on the Kronecker constraint."""
    rng = np.random.default_rng(34)
    L, dk, dv, eps = 6, 4, 3, 0.2
    q, k, v, _, eta = _rand_seq(rng, L, 1, dk, dv)
    a = _rand_ch(rng, L, 1, dk)
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, S_fin = fwd(q, k, v, a, eta, eps=eps, initial_state=S0, channel_decay=True)
    S = S0[0, 0].copy()
    for t in range(L):
        kt, vt = k[t, 0], v[t, 0]
        St = a[t, 0][:, None] * S
        Cmat = np.kron(np.eye(dv), kt[None, :])
        r = vt - Cmat @ St.reshape(-1, order="F")
        x = np.linalg.lstsq(Cmat, r, rcond=None)[0]
        kk = float(kt @ kt)
        S = St + (eta[t, 0] * kk / (kk + eps)) * x.reshape(dk, dv, order="F")
        assert rel(o[t, 0], S.T @ q[t, 0]) < 1e-11
    assert rel(S_fin[0, 0], S) < 1e-11


def pin_channel_untouched_channel(fwd, decode):
    """A key channel that no key and no query ever uses only decays: its row
    of the final state is (prod_t a_t[c]) S0[c], and the outputs do not
    depend on that channel's rates."""
    rng = np.random.default_rng(35)
    L, H, dk, dv, c = 19, 2, 5, 5, 2
    q, k, v, _, eta = _rand_seq(rng, L, H, dk, dv)
    q[:, :, c] = 0.0
    k[:, :, c] = 0.0
    a = _rand_ch(rng, L, H, dk)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = fwd(q, k, v, a, eta, eps=1e-3, initial_state=S0, channel_decay=True)
    assert rel(S[0, :, c], np.prod(a[:, :, c], axis=0)[:, None] * S0[0, :, c]) < TIGHT
    a2 = a.copy()
    a2[:, :, c] = rng.uniform(0.3, 1.0, (L, H))
    o2, S2 = fwd(q, k, v, a2, eta, eps=1e-3, initial_state=S0, channel_decay=True)
    assert rel(o2, o) < TIGHT
    others = [i for i in range(dk) if i != c]
    assert rel(S2[0][:, others], S[0][:, others]) < TIGHT


def pin_channel_chunk_form(fwd, decode):
    """The chunk form with per-channel decay factors (direct; factored per
    block of 16 rows as the fp32-input GPU kernel forms it; and referenced to
    the chunk's midpoint decay as the bf16-input kernel forms it) gives the
    sequential result for every chunk size, ragged last chunks included."""
    rng = np.random.default_rng(36)
    H, dk, dv = 2, 6, 5
    cu = np.array([0, 1, 17, 80, 143])
    L = int(cu[-1])
    q, k, v, _, eta = _rand_seq(rng, L, H, dk, dv)
    a = _rand_ch(rng, L, H, dk, amin=0.5)
    S0 = rng.standard_normal((len(cu) - 1, H, dk, dv))
    o, S = fwd(q, k, v, a, eta, cu_seqlens=cu, eps=1e-3, initial_state=S0, channel_decay=True)
    for C in (1, 7, 16, 64):
        for fac in (False, True, "mid"):
            oc, Sc = chunked_ch(q, k, v, a, eta, cu, 1e-3, C, S0, factored=fac)
            assert rel(o, oc) < 1e-10 and rel(S, Sc) < 1e-10, (C, fac, rel(o, oc), rel(S, Sc))


def pin_channel_decode_is_one_token(fwd, decode):
    """A per-channel decode step after a prefill equals the prefill that is
    one token longer."""
    rng = np.random.default_rng(37)
    L, H, dk, dv = 11, 3, 6, 4
    q, k, v, _, eta = _rand_seq(rng, L + 1, H, dk, dv)
    a = _rand_ch(rng, L + 1, H, dk)
    _, S = fwd(q[:L], k[:L], v[:L], a[:L], eta[:L], eps=1e-4, channel_decay=True)
    od, Sd = decode(q[L:], k[L:], v[L:], a[L:], eta[L:], S, eps=1e-4, channel_decay=True)
    o_all, S_all = fwd(q, k, v, a, eta, eps=1e-4, channel_decay=True)
    assert rel(od[0], o_all[L]) < TIGHT
    assert rel(Sd, S_all) < TIGHT


# ---- curvature-conditioned read ---------------------------------------------

def _ccq(fwd):
    """The oracle's fwd_ccq / decode_step_ccq bound to the build under test."""
    import functools
    import oracle
    lp = getattr(fwd, "keywords", {}).get("lib_path")
    return (functools.partial(oracle.fwd_ccq, lib_path=lp),
            functools.partial(oracle.decode_step_ccq, lib_path=lp))


def _clean_queries_numpy(q, k, lam, covariance):
    """q_clean_t = q_t - lambda_t Sigma_t q_t per head, Sigma_t from `covariance`
    applied to the keys k[0..t] of that head."""
    L, H, dk = q.shape
    out = np.empty_like(q)
    for h in range(H):
        for t in range(L):
            Sig = covariance(k[:t + 1, h])
            out[t, h] = q[t, h] - lam[t, h] * Sig @ q[t, h]
    return out


def pin_ccq_numpy_covariance(fwd, decode):
    """The read uses q - lambda Sigma_t q with Sigma_t the uniformly weighted
    covariance of the keys k_1..k_t (numpy.cov with bias=True); the state
    recurrence is the plain one, so the CCQ output equals the plain oracle
    fed those cleaned queries."""
    fwd_ccq, _ = _ccq(fwd)
    rng = np.random.default_rng(41)
    L, H, dk, dv = 23, 2, 5, 4
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    lam = rng.uniform(0.0, 1.0, (L, H))
    cov = lambda K: np.cov(K.T, bias=True).reshape(dk, dk) if K.shape[0] > 1 else np.zeros((dk, dk))
    qc = _clean_queries_numpy(q, k, lam, cov)
    S0 = rng.standard_normal((1, H, dk, dv))
    for mode in ("kaczmarz", "direct"):
        o, S, _ = fwd_ccq(q, k, v, alpha, eta, lam, eps=1e-3, initial_state=S0, beta_mode=mode)
        o2, S2 = fwd(qc, k, v, alpha, eta, eps=1e-3, initial_state=S0, beta_mode=mode)
        assert rel(o, o2) < 1e-12 and rel(S, S2) < TIGHT


def pin_ccq_logsumexp_hessian(fwd, decode):
    """Sigma_t is the Hessian at q = 0 of log sum_{j<=t} exp(k_j^T q), the
    softmax normaliser the read stands in for; here by central differences
    of scipy's logsumexp."""
    from scipy.special import logsumexp
    fwd_ccq, _ = _ccq(fwd)
    rng = np.random.default_rng(42)
    L, H, dk, dv = 9, 1, 3, 2
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    lam = rng.uniform(0.2, 1.0, (L, H))
    hstep = 1e-3

    def hessian(K):
        f = lambda x: logsumexp(K @ x)
        Hm = np.zeros((dk, dk))
        E = np.eye(dk) * hstep
        for a in range(dk):
            for b in range(dk):
                Hm[a, b] = (f(E[a] + E[b]) - f(E[a] - E[b]) - f(-E[a] + E[b]) + f(-E[a] - E[b])) / (4 * hstep * hstep)
        return Hm

    qc = _clean_queries_numpy(q, k, lam, hessian)
    o, _, _ = fwd_ccq(q, k, v, alpha, eta, lam, eps=1e-3)
    o2, _ = fwd(qc, k, v, alpha, eta, eps=1e-3)
    assert rel(o, o2) < 1e-5, rel(o, o2)


def pin_ccq_lambda_zero_and_state(fwd, decode):
    """lambda = 0 reads with the raw query (the plain recurrence); for any
    lambda the state is the plain one (only the read changes)."""
    fwd_ccq, _ = _ccq(fwd)
    rng = np.random.default_rng(43)
    L, H, dk, dv = 17, 2, 4, 3
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    o0, S0 = fwd(q, k, v, alpha, eta, eps=1e-4)
    o, S, _ = fwd_ccq(q, k, v, alpha, eta, np.zeros((L, H)), eps=1e-4)
    assert rel(o, o0) < TIGHT and rel(S, S0) < TIGHT
    o1, S1, _ = fwd_ccq(q, k, v, alpha, eta, rng.uniform(0, 1, (L, H)), eps=1e-4)
    assert rel(S1, S0) < TIGHT and rel(o1, o0) > 1e-3


def pin_ccq_constant_keys(fwd, decode):
    """Every key the same: the covariance is zero and the read is the raw
    query's, whatever lambda."""
    fwd_ccq, _ = _ccq(fwd)
    rng = np.random.default_rng(44)
    L, H, dk, dv = 12, 1, 4, 3
    q, _, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    k = np.broadcast_to(rng.standard_normal((1, H, dk)), (L, H, dk)).copy()
    o, _, c = fwd_ccq(q, k, v, alpha, eta, rng.uniform(0.5, 1, (L, H)), eps=1e-4)
    o0, _ = fwd(q, k, v, alpha, eta, eps=1e-4)
    assert rel(o, o0) < 1e-12
    assert c[0, 0, dk * dk + dk] == L


def pin_ccq_resume_and_decode(fwd, decode):
    """Carrying the running sums (and the state): two prefills equal one,
    and a decode step after a prefill equals the prefill one token longer."""
    fwd_ccq, dec_ccq = _ccq(fwd)
    rng = np.random.default_rng(45)
    L, H, dk, dv, m = 26, 2, 4, 3, 11
    q, k, v, alpha, eta = _rand_seq(rng, L + 1, H, dk, dv)
    lam = rng.uniform(0, 1, (L + 1, H))
    o_all, S_all, c_all = fwd_ccq(q[:L], k[:L], v[:L], alpha[:L], eta[:L], lam[:L], eps=1e-4)
    o1, S1, c1 = fwd_ccq(q[:m], k[:m], v[:m], alpha[:m], eta[:m], lam[:m], eps=1e-4)
    o2, S2, c2 = fwd_ccq(q[m:L], k[m:L], v[m:L], alpha[m:L], eta[m:L], lam[m:L], eps=1e-4,
                         initial_state=S1, ccq_state=c1)
    assert rel(np.concatenate([o1, o2]), o_all) < TIGHT
    assert rel(S2, S_all) < TIGHT and rel(c2, c_all) < TIGHT
    od, Sd, cd = dec_ccq(q[L:][0][None], k[L:][0][None], v[L:][0][None], alpha[L:][0][None],
                         eta[L:][0][None], lam[L:][0][None], S_all, c_all, eps=1e-4)
    o_l, S_l, c_l = fwd_ccq(q, k, v, alpha, eta, lam, eps=1e-4)
    assert rel(od[0], o_l[L]) < TIGHT and rel(Sd, S_l) < TIGHT and rel(cd, c_l) < TIGHT


# ---- backward (gradient of the prefill) -------------------------------------

def _bwd(fwd):
    """The oracle's bwd bound to the build under test."""
    import functools
    import oracle
    lp = getattr(fwd, "keywords", {}).get("lib_path")
    return functools.partial(oracle.bwd, lib_path=lp)


def _fd_check(fwd, bwd, q, k, v, alpha, eta, S0, d_o, d_fin, cu, eps, beta_mode, tol):
    """Every gradient the reverse sweep returns equals the central finite
    difference of L = sum(d_o * o) + sum(d_fin * S_final), with o and
    S_final from the forward reference (pinned on its own above)."""
    def loss(q, k, v, alpha, eta, S0):
        o, S = fwd(q, k, v, alpha, eta, cu_seqlens=cu, eps=eps, initial_state=S0,
                   beta_mode=beta_mode)
        return float(np.sum(o * d_o) + np.sum(S * d_fin))

    g = bwd(q, k, v, alpha, eta, d_o, cu_seqlens=cu, eps=eps, initial_state=S0, d_final=d_fin,
            beta_mode=beta_mode)
    args = {"q": q, "k": k, "v": v, "alpha": alpha, "eta": eta, "S0": S0}
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "eta": "deta", "S0": "dS0"}
    for name, x in list(args.items()):
        if x is None:
            assert g[names[name]] is None
            continue
        fd = np.zeros_like(x)
        h = 1e-6
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xp[idx] += h
            xm = x.copy()
            xm[idx] -= h
            fd[idx] = (loss(**dict(args, **{name: xp})) - loss(**dict(args, **{name: xm}))) / (2 * h)
        assert rel(g[names[name]], fd) < tol, (name, rel(g[names[name]], fd))


def pin_bwd_finite_differences(fwd, decode):
    """The gradient of the prefill with respect to q, k, v, alpha, eta and the
    initial state equals central finite differences of the forward
    reference, over two packed sequences and an empty one, with a gradient
    arriving both through o and through the final state."""
    rng = np.random.default_rng(50)
    lens = [5, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    L, H, dk, dv = int(cu[-1]), 2, 3, 2
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    S0 = rng.standard_normal((3, H, dk, dv))
    d_o = rng.standard_normal((L, H, dv))
    d_fin = rng.standard_normal((3, H, dk, dv))
    _fd_check(fwd, _bwd(fwd), q, k, v, alpha, eta, S0, d_o, d_fin, cu, 1e-3, "kaczmarz", 1e-7)


def pin_bwd_finite_differences_direct(fwd, decode):
    """The same check for the direct step (beta = eta) without a decay gate
    (DeltaNet), and for the direct step with decay (Gated DeltaNet)."""
    rng = np.random.default_rng(51)
    L, H, dk, dv = 6, 1, 3, 3
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True) * 0.8  # a contraction for beta <= 1
    S0 = rng.standard_normal((1, H, dk, dv))
    d_o = rng.standard_normal((L, H, dv))
    d_fin = rng.standard_normal((1, H, dk, dv))
    cu = np.array([0, L])
    _fd_check(fwd, _bwd(fwd), q, k, v, None, eta, S0, d_o, d_fin, cu, 1e-3, "direct", 1e-7)
    _fd_check(fwd, _bwd(fwd), q, k, v, alpha, eta, S0, d_o, d_fin, cu, 1e-3, "direct", 1e-7)


def pin_bwd_eta_zero_closed_form(fwd, decode):
    """eta = 0: no write, o_t = g_t S0^T q_t and S_L = g_L S0 with
    g_t = alpha_1 ... alpha_t.  The gradients then have closed forms:
    dq_t = g_t S0 d_o_t;  dv = dk = 0;
    dS0 = sum_t g_t q_t d_o_t^T + g_L d_fin;
    dalpha_t = (1/alpha_t) (sum_{r>=t} g_r q_r^T S0 d_o_r + g_L <d_fin, S0>);
    deta_t = k_t^T G_t e_t / (|k_t|^2 + eps) with e_t = v_t - g_t S0^T k_t and
    G_t = sum_{r>=t} (g_r/g_t) q_r d_o_r^T + (g_L/g_t) d_fin."""
    bwd = _bwd(fwd)
    rng = np.random.default_rng(52)
    L, H, dk, dv, eps = 7, 2, 4, 3, 1e-3
    q, k, v, alpha, _ = _rand_seq(rng, L, H, dk, dv)
    eta = np.zeros((L, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    d_o = rng.standard_normal((L, H, dv))
    d_fin = rng.standard_normal((1, H, dk, dv))
    g = bwd(q, k, v, alpha, eta, d_o, eps=eps, initial_state=S0, d_final=d_fin)
    assert np.max(np.abs(g["dv"])) == 0.0 and np.max(np.abs(g["dk"])) == 0.0
    for h in range(H):
        S, F = S0[0, h], d_fin[0, h]
        gam = np.cumprod(alpha[:, h])
        dq = np.stack([gam[t] * S @ d_o[t, h] for t in range(L)])
        assert rel(g["dq"][:, h], dq) < TIGHT
        dS0 = sum(gam[t] * np.outer(q[t, h], d_o[t, h]) for t in range(L)) + gam[-1] * F
        assert rel(g["dS0"][0, h], dS0) < TIGHT
        read = np.array([gam[r] * q[r, h] @ S @ d_o[r, h] for r in range(L)])
        fin = gam[-1] * np.sum(F * S)
        da = np.array([(read[t:].sum() + fin) / alpha[t, h] for t in range(L)])
        assert rel(g["dalpha"][:, h], da) < TIGHT
        de = np.zeros(L)
        for t in range(L):
            G = sum((gam[r] / gam[t]) * np.outer(q[r, h], d_o[r, h]) for r in range(t, L))
            G = G + (gam[-1] / gam[t]) * F
            e = v[t, h] - gam[t] * S.T @ k[t, h]
            de[t] = k[t, h] @ G @ e / (k[t, h] @ k[t, h] + eps)
        assert rel(g["deta"][:, h], de) < TIGHT


def pin_bwd_linear_in_upstream(fwd, decode):
    """The gradient is linear in (d_o, d_fin): the gradients for d_o alone and
    for d_fin alone add up to the gradients for both."""
    bwd = _bwd(fwd)
    rng = np.random.default_rng(53)
    L, H, dk, dv = 9, 2, 3, 4
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    d_o = rng.standard_normal((L, H, dv))
    d_fin = rng.standard_normal((1, H, dk, dv))
    both = bwd(q, k, v, alpha, eta, d_o, initial_state=S0, d_final=d_fin)
    a = bwd(q, k, v, alpha, eta, d_o, initial_state=S0)
    b = bwd(q, k, v, alpha, eta, np.zeros_like(d_o), initial_state=S0, d_final=d_fin)
    for key in ("dq", "dk", "dv", "dalpha", "deta", "dS0"):
        assert rel(a[key] + b[key], both[key]) < TIGHT, key



def pin_bwd_chunk_form(fwd, decode):
    """The chunk form of the backward (tests/chunk_model.py: adjoint
    triangular solve, W and Z planes, reverse running sum for the decay,
    also split into column slices of the state) gives the reverse sweep's
    gradients for C in {1, 7, 16, 64}, ragged and empty sequences, both step
    modes, with and without decay."""
    bwd = _bwd(fwd)
    rng = np.random.default_rng(54)
    lens = [37, 0, 70, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    L, H, dk, dv = int(cu[-1]), 2, 5, 6
    q, k, v, alpha, eta = _rand_seq(rng, L, H, dk, dv)
    S0 = rng.standard_normal((4, H, dk, dv))
    d_o = rng.standard_normal((L, H, dv))
    d_fin = rng.standard_normal((4, H, dk, dv))
    for mode in ("kaczmarz", "direct"):
        for a in (alpha, None):
            ref = bwd(q, k, v, a, eta, d_o, cu_seqlens=cu, eps=1e-3, initial_state=S0,
                      d_final=d_fin, beta_mode=mode)
            for C, sl in ((1, 1), (7, 3), (16, 1), (64, 3)):
                m = chunked_bwd(q, k, v, a, eta, d_o, cu, 1e-3, C, S0, d_fin,
                                beta_direct=mode == "direct", dv_slices=sl)
                for key in ref:
                    if ref[key] is None:
                        assert m[key] is None
                    else:
                        assert rel(m[key], ref[key]) < 1e-11, (mode, a is None, C, key)

ALL_PINS = [pin_worked_example, pin_orthogonal_projection, pin_min_norm_bruteforce,
            pin_exact_line_search, pin_normalised_gradient, pin_exact_recall, pin_eta_zero,
            pin_scalar_case, pin_gated_deltanet_form, pin_chunk_form, pin_packed_and_resume,
            pin_decode_is_one_token, pin_zero_key, pin_direct_step_product_form,
            pin_no_alpha_is_unit_decay, pin_direct_equals_kaczmarz_on_unit_keys,
            pin_deltanet_exact_recall, pin_segment_map_is_affine,
            pin_channel_uniform_is_scalar, pin_channel_eta_zero,
            pin_channel_orthogonal_projection, pin_channel_min_norm_bruteforce,
            pin_channel_untouched_channel, pin_channel_chunk_form,
            pin_channel_decode_is_one_token,
            pin_ccq_numpy_covariance, pin_ccq_logsumexp_hessian, pin_ccq_lambda_zero_and_state,
            pin_ccq_constant_keys, pin_ccq_resume_and_decode,
            pin_bwd_finite_differences, pin_bwd_finite_differences_direct,
            pin_bwd_eta_zero_closed_form, pin_bwd_linear_in_upstream, pin_bwd_chunk_form]
