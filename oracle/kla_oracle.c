/*
 * kla_oracle.c -- fp64 reference for the Kaczmarz Linear Attention (KLA)
 * recurrence.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark call it; the library under
 * delta_rule_linear_amd/ never does.  It shares no code with the HIP path.
 *
 * Source: "Resumo Tecnico: Atencao Linear Kaczmarz (KLA)"
 * (gist.science/pt/paper/2605.08587), sections "Derivacao Teorica" and
 * "A Regra de Atualizacao KLA".  Per head, with state S in R^{dk x dv}:
 *
 *   beta_t  = eta_t / (k_t^T k_t + eps)          (relaxed Kaczmarz step)
 *   S~      = alpha_t S_{t-1}                     (decayed previous state)
 *   e_t     = v_t - S~^T k_t                      (residual)
 *   S_t     = S~ + beta_t k_t e_t^T               (rank-one write)
 *   o_t     = S_t^T q_t                           (read of the written state)
 *
 * The page fixes the first four lines.  The decay alpha_t is the scalar
 * gate that the page keeps from Gated DeltaNet (section "Implementacao";
 * the linear-attention survey page, gist.science/pt/paper/2607.07953,
 * section "Metodologia e Estrutura", describes it as a decay applied to
 * the memory before the residual).  The read o_t = S_t^T q_t uses the
 * state after the write; the pages never print the read, so this is a
 * stated reading.
 *
 * Gate variants (the *_ex entry points): with beta_direct the step is
 * beta_t = eta_t itself, the learned scalar of Gated DeltaNet that KLA
 * replaces (KLA summary, introduction); alpha == NULL means alpha_t = 1,
 * no decay, which with the direct step is DeltaNet (survey page, section
 * "Notacao Unificada").  Everything else is the same recurrence.
 *
 * Per-channel decay (the *_ch entry points): the survey page's Kimi Delta
 * Attention (section "Metodologia e Estrutura") replaces the scalar decay by
 * a vector with one rate per feature channel.  The state's rows are the key
 * channels, so the decay becomes S~ = Diag(a_t) S_{t-1}: row i of the state
 * is scaled by a_t[i].  The residual, the step and the write are KLA's.
 *
 * Curvature-conditioned query (the *_ccq entry points; "Don't Read
 * Everything: A Curvature-Conditioned Query for Linear Attention", sections
 * "Derivacao Teorica" and "O Mecanismo"): only the read changes.  With
 * Sigma_t the covariance of the keys seen so far, weighted uniformly (the
 * Hessian of log sum_{j<=t} exp(k_j^T q) at q = 0),
 *   Sigma_t = (1/n) sum_{j<=t} k_j k_j^T - mu_t mu_t^T,  mu_t = (1/n) sum_{j<=t} k_j,
 *   q_clean = q_t - lambda_t Sigma_t q_t,   o_t = S_t^T q_clean,
 * where n counts the keys j <= t.  The running sums (sum k k^T, sum k, n)
 * are the extra state per head; a sequence may start from given sums.
 *
 * Backward (kla_oracle_bwd_ex): the gradient of the prefill's outputs (o and
 * the final state) with respect to q, k, v, alpha, eta and the initial
 * state, by the reverse sweep of the same token loop (each forward line's
 * adjoint, in reverse order; see the function).
 *
 * This is the plain definition, token by token, in double precision,
 * with no blocking or chunking: the chunkwise algorithm of the GPU path
 * reaches the same result up to rounding.  Inputs arrive as doubles that
 * hold the exact values the GPU reads (bf16 and fp32 convert to fp64
 * exactly).
 *
 * Layouts (all row-major, contiguous):
 *   q, k      [total_tok][H][dk]
 *   v, o      [total_tok][H][dv]
 *   alpha,eta [total_tok][H]        (per-channel alpha: [total_tok][H][dk])
 *   state     [n_seqs][H][dk][dv]
 *   cu_seqlens[n_seqs+1], cu_seqlens[0] = 0, non-decreasing.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One KLA write followed by the read, on one (sequence, head) state. */
static void kla_token(double *S, double *e, const double *q, const double *k,
                      const double *v, double alpha, double eta, double eps,
                      int beta_direct, int dk, int dv, double *o)
{
    double kk = 0.0;
    for (int i = 0; i < dk; ++i) kk += k[i] * k[i];
    const double beta = beta_direct ? eta : eta / (kk + eps);

    /* S~ = alpha S */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha;

    /* e = v - S~^T k */
    for (int j = 0; j < dv; ++j) e[j] = v[j];
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) e[j] -= S[(size_t)i * dv + j] * k[i];

    /* S = S~ + beta k e^T */
    for (int i = 0; i < dk; ++i) {
        const double bk = beta * k[i];
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bk * e[j];
    }

    /* o = S^T q */
    if (o) {
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) o[j] += S[(size_t)i * dv + j] * q[i];
    }
}

/* The same token with the decay per key channel: S~ = Diag(a) S. */
static void kla_token_ch(double *S, double *e, const double *q, const double *k,
                         const double *v, const double *a, double eta, double eps,
                         int beta_direct, int dk, int dv, double *o)
{
    double kk = 0.0;
    for (int i = 0; i < dk; ++i) kk += k[i] * k[i];
    const double beta = beta_direct ? eta : eta / (kk + eps);

    /* S~ = Diag(a) S: row i (key channel i) decays by a[i] */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a[i];

    /* e = v - S~^T k */
    for (int j = 0; j < dv; ++j) e[j] = v[j];
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) e[j] -= S[(size_t)i * dv + j] * k[i];

    /* S = S~ + beta k e^T */
    for (int i = 0; i < dk; ++i) {
        const double bk = beta * k[i];
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bk * e[j];
    }

    /* o = S^T q */
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) o[j] += S[(size_t)i * dv + j] * q[i];
}

int kla_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Prefill over packed sequences.  The state starts at initial_state[s] (or
 * zero when initial_state is NULL) at the first token of each sequence and
 * the final state of each sequence goes to final_state (when not NULL).
 * alpha may be NULL (alpha_t = 1).  beta_direct selects beta_t = eta_t.
 * Returns 0, or -1 on a malformed argument.
 */
int kla_oracle_fwd_ex(const double *q, const double *k, const double *v,
                      const double *alpha, const double *eta,
                      const int64_t *cu_seqlens, int n_seqs, int H, int dk, int dv,
                      double eps, int beta_direct, const double *initial_state, double *o,
                      double *final_state)
{
    if (!q || !k || !v || !eta || !cu_seqlens || !o) return -1;
    if (n_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    for (int s = 0; s < n_seqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    if (cu_seqlens[0] != 0) return -1;

    const size_t sdim = (size_t)dk * dv;
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < n_seqs; ++s) {
        for (int h = 0; h < H; ++h) {
            double *S = (double *)malloc(sizeof(double) * (sdim + dv));
            if (!S) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            double *e = S + sdim;
            const size_t sh = (size_t)s * H + h;
            if (initial_state)
                memcpy(S, initial_state + sh * sdim, sizeof(double) * sdim);
            else
                memset(S, 0, sizeof(double) * sdim);
            for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
                const size_t th = (size_t)t * H + h;
                kla_token(S, e, q + th * dk, k + th * dk, v + th * dv,
                          alpha ? alpha[th] : 1.0, eta[th], eps, beta_direct, dk, dv,
                          o + th * dv);
            }
            if (final_state) memcpy(final_state + sh * sdim, S, sizeof(double) * sdim);
            free(S);
        }
    }
    return failed ? -1 : 0;
}

/* The KLA step (beta_t = eta_t / (|k_t|^2 + eps)). */
int kla_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *alpha, const double *eta,
                   const int64_t *cu_seqlens, int n_seqs, int H, int dk, int dv,
                   double eps, const double *initial_state, double *o,
                   double *final_state)
{
    return kla_oracle_fwd_ex(q, k, v, alpha, eta, cu_seqlens, n_seqs, H, dk, dv, eps, 0,
                             initial_state, o, final_state);
}

/*
 * One decode step: every (sequence, head) state advances by one token in
 * place and o receives the read of the new state.
 *   q, k [n_seqs][H][dk], v, o [n_seqs][H][dv], alpha, eta [n_seqs][H]
 * alpha may be NULL (alpha = 1); beta_direct selects beta = eta.
 */
int kla_oracle_decode_step_ex(const double *q, const double *k, const double *v,
                              const double *alpha, const double *eta, double *state,
                              int n_seqs, int H, int dk, int dv, double eps, int beta_direct,
                              double *o)
{
    if (!q || !k || !v || !eta || !state || !o) return -1;
    if (n_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    const size_t sdim = (size_t)dk * dv;
    int failed = 0;
#pragma omp parallel for schedule(static)
    for (int64_t sh = 0; sh < (int64_t)n_seqs * H; ++sh) {
        double *e = (double *)malloc(sizeof(double) * dv);
        if (!e) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        kla_token(state + sh * sdim, e, q + sh * dk, k + sh * dk, v + sh * dv,
                  alpha ? alpha[sh] : 1.0, eta[sh], eps, beta_direct, dk, dv, o + sh * dv);
        free(e);
    }
    return failed ? -1 : 0;
}

/* The KLA step (beta = eta / (|k|^2 + eps)). */
int kla_oracle_decode_step(const double *q, const double *k, const double *v,
                           const double *alpha, const double *eta, double *state,
                           int n_seqs, int H, int dk, int dv, double eps, double *o)
{
    return kla_oracle_decode_step_ex(q, k, v, alpha, eta, state, n_seqs, H, dk, dv, eps, 0, o);
}

/*
 * Prefill with the per-channel decay: alpha [total_tok][H][dk], required.
 * Everything else as kla_oracle_fwd_ex.
 */
int kla_oracle_fwd_ch(const double *q, const double *k, const double *v,
                      const double *alpha, const double *eta,
                      const int64_t *cu_seqlens, int n_seqs, int H, int dk, int dv,
                      double eps, int beta_direct, const double *initial_state, double *o,
                      double *final_state)
{
    if (!q || !k || !v || !alpha || !eta || !cu_seqlens || !o) return -1;
    if (n_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    for (int s = 0; s < n_seqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    if (cu_seqlens[0] != 0) return -1;

    const size_t sdim = (size_t)dk * dv;
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < n_seqs; ++s) {
        for (int h = 0; h < H; ++h) {
            double *S = (double *)malloc(sizeof(double) * (sdim + dv));
            if (!S) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            double *e = S + sdim;
            const size_t sh = (size_t)s * H + h;
            if (initial_state)
                memcpy(S, initial_state + sh * sdim, sizeof(double) * sdim);
            else
                memset(S, 0, sizeof(double) * sdim);
            for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
                const size_t th = (size_t)t * H + h;
                kla_token_ch(S, e, q + th * dk, k + th * dk, v + th * dv, alpha + th * dk,
                             eta[th], eps, beta_direct, dk, dv, o + th * dv);
            }
            if (final_state) memcpy(final_state + sh * sdim, S, sizeof(double) * sdim);
            free(S);
        }
    }
    return failed ? -1 : 0;
}

/* One decode step with the per-channel decay: alpha [n_seqs][H][dk]. */
int kla_oracle_decode_step_ch(const double *q, const double *k, const double *v,
                              const double *alpha, const double *eta, double *state,
                              int n_seqs, int H, int dk, int dv, double eps, int beta_direct,
                              double *o)
{
    if (!q || !k || !v || !alpha || !eta || !state || !o) return -1;
    if (n_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    const size_t sdim = (size_t)dk * dv;
    int failed = 0;
#pragma omp parallel for schedule(static)
    for (int64_t sh = 0; sh < (int64_t)n_seqs * H; ++sh) {
        double *e = (double *)malloc(sizeof(double) * dv);
        if (!e) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        kla_token_ch(state + sh * sdim, e, q + sh * dk, k + sh * dk, v + sh * dv,
                     alpha + sh * dk, eta[sh], eps, beta_direct, dk, dv, o + sh * dv);
        free(e);
    }
    return failed ? -1 : 0;
}

/*
 * Curvature-conditioned read.  The extra state per (sequence, head) is the
 * running sums in one record of CCQ_STRIDE(dk) doubles:
 *   [0, dk*dk)        P = sum k k^T (row-major)
 *   [dk*dk, dk*dk+dk) m = sum k
 *   [dk*dk+dk]        n, the number of keys
 */
#define CCQ_STRIDE(dk) ((size_t)(dk) * (dk) + (dk) + 4)

/* Sums += k; qc = q - lambda Sigma q with Sigma from the updated sums. */
static void ccq_clean(double *P, double *m, double *n, const double *q, const double *k,
                      double lambda, int dk, double *qc)
{
    *n += 1.0;
    for (int i = 0; i < dk; ++i) {
        m[i] += k[i];
        for (int c = 0; c < dk; ++c) P[(size_t)i * dk + c] += k[i] * k[c];
    }
    const double inv = 1.0 / *n;
    double mq = 0.0;
    for (int c = 0; c < dk; ++c) mq += m[c] * q[c];
    for (int i = 0; i < dk; ++i) {
        double pq = 0.0;
        for (int c = 0; c < dk; ++c) pq += P[(size_t)i * dk + c] * q[c];
        const double sq = pq * inv - (m[i] * inv) * (mq * inv);  /* (Sigma q)_i */
        qc[i] = q[i] - lambda * sq;
    }
}

/*
 * Prefill with the curvature-conditioned read: lambda [total_tok][H];
 * ccq_in / ccq_out [n_seqs][H][CCQ_STRIDE(dk)] (NULL: start from zero sums /
 * do not write).  Everything else as kla_oracle_fwd_ex.
 */
int kla_oracle_fwd_ccq(const double *q, const double *k, const double *v,
                       const double *alpha, const double *eta, const double *lambda,
                       const int64_t *cu_seqlens, int n_seqs, int H, int dk, int dv,
                       double eps, int beta_direct, const double *initial_state,
                       const double *ccq_in, double *o, double *final_state, double *ccq_out)
{
    if (!q || !k || !v || !eta || !lambda || !cu_seqlens || !o) return -1;
    if (n_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    for (int s = 0; s < n_seqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    if (cu_seqlens[0] != 0) return -1;

    const size_t sdim = (size_t)dk * dv, cst = CCQ_STRIDE(dk);
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < n_seqs; ++s) {
        for (int h = 0; h < H; ++h) {
            double *S = (double *)malloc(sizeof(double) * (sdim + dv + cst + dk));
            if (!S) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            double *e = S + sdim, *cs = e + dv, *qc = cs + cst;
            const size_t sh = (size_t)s * H + h;
            if (initial_state)
                memcpy(S, initial_state + sh * sdim, sizeof(double) * sdim);
            else
                memset(S, 0, sizeof(double) * sdim);
            if (ccq_in)
                memcpy(cs, ccq_in + sh * cst, sizeof(double) * cst);
            else
                memset(cs, 0, sizeof(double) * cst);
            double *P = cs, *m = cs + (size_t)dk * dk, *n = m + dk;
            for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
                const size_t th = (size_t)t * H + h;
                ccq_clean(P, m, n, q + th * dk, k + th * dk, lambda[th], dk, qc);
                kla_token(S, e, qc, k + th * dk, v + th * dv, alpha ? alpha[th] : 1.0, eta[th],
                          eps, beta_direct, dk, dv, o + th * dv);
            }
            if (final_state) memcpy(final_state + sh * sdim, S, sizeof(double) * sdim);
            if (ccq_out) memcpy(ccq_out + sh * cst, cs, sizeof(double) * cst);
            free(S);
        }
    }
    return failed ? -1 : 0;
}

/* One decode step with the curvature-conditioned read; ccq_state
 * [n_seqs][H][CCQ_STRIDE(dk)] is updated in place with the new key. */
int kla_oracle_decode_step_ccq(const double *q, const double *k, const double *v,
                               const double *alpha, const double *eta, const double *lambda,
                               double *state, double *ccq_state, int n_seqs, int H, int dk,
                               int dv, double eps, int beta_direct, double *o)
{
    if (!q || !k || !v || !eta || !lambda || !state || !ccq_state || !o) return -1;
    if (n_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    const size_t sdim = (size_t)dk * dv, cst = CCQ_STRIDE(dk);
    int failed = 0;
#pragma omp parallel for schedule(static)
    for (int64_t sh = 0; sh < (int64_t)n_seqs * H; ++sh) {
        double *e = (double *)malloc(sizeof(double) * (dv + dk));
        if (!e) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *qc = e + dv, *cs = ccq_state + sh * cst;
        ccq_clean(cs, cs + (size_t)dk * dk, cs + (size_t)dk * dk + dk, q + sh * dk, k + sh * dk,
                  lambda[sh], dk, qc);
        kla_token(state + sh * sdim, e, qc, k + sh * dk, v + sh * dv, alpha ? alpha[sh] : 1.0,
                  eta[sh], eps, beta_direct, dk, dv, o + sh * dv);
        free(e);
    }
    return failed ? -1 : 0;
}

/*
 * Backward (reverse-mode gradient) of the prefill.
 *
 * The pages keep Gated DeltaNet's training algorithm and change only the
 * step size (KLA summary, section "Implementacao"), so the gradient is
 * the derivative of the same recurrence.  Given the loss's gradients with
 * respect to every output o_t (d_o) and to each sequence's final state
 * (d_final, or none), this returns the gradients of the loss with respect
 * to q, k, v, alpha, eta and the initial state.
 *
 * It is the plain reverse sweep: the forward pass runs token by token and
 * keeps every state; then, from the last token back, the adjoint of each of
 * the five forward lines is applied in reverse order, with dS the gradient
 * of the state just after the token's write:
 *   (5) o = S^T q          dS += q d_o^T            dq  = S d_o
 *   (4) S = S~ + b k e^T   dS~ = dS                 db  = k^T dS e
 *                          dk  = b dS e             de  = b dS^T k
 *   (3) e = v - S~^T k     dv  = de                 dS~ -= k de^T
 *                          dk -= S~ de
 *   (2) S~ = alpha S_prev  dalpha = <dS~, S_prev>   dS_prev = alpha dS~
 *   (1) b = eta / (k.k + eps)
 *                          deta = db / (k.k + eps)
 *                          dk  -= 2 eta db / (k.k + eps)^2 k
 * (with beta_direct: b = eta, deta = db and no k term).  After the first
 * token of a sequence dS is the gradient of its initial state.
 *
 * Layouts as the forward; d_alpha may be NULL when alpha is NULL (no decay
 * gate), d_final and d_initial may be NULL.
 */
int kla_oracle_bwd_ex(const double *q, const double *k, const double *v, const double *alpha,
                      const double *eta, const int64_t *cu_seqlens, int n_seqs, int H, int dk,
                      int dv, double eps, int beta_direct, const double *initial_state,
                      const double *d_o, const double *d_final, double *dq, double *dk_out,
                      double *dv_out, double *d_alpha, double *d_eta, double *d_initial)
{
    if (!q || !k || !v || !eta || !cu_seqlens || !d_o || !dq || !dk_out || !dv_out || !d_eta)
        return -1;
    if (alpha && !d_alpha) return -1;
    if (n_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    for (int s = 0; s < n_seqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    if (cu_seqlens[0] != 0) return -1;

    const size_t sdim = (size_t)dk * dv;
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < n_seqs; ++s) {
        for (int h = 0; h < H; ++h) {
            const int64_t t0 = cu_seqlens[s], L = cu_seqlens[s + 1] - t0;
            const size_t sh = (size_t)s * H + h;
            /* states S_0 .. S_L (the state after each token), the gradient
             * dS, the decayed state S~ and the vectors e, de */
            double *St = (double *)malloc(sizeof(double) * ((size_t)(L + 1) * sdim + 2 * sdim +
                                                            2 * (size_t)dv));
            if (!St) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            double *dS = St + (size_t)(L + 1) * sdim, *Sd = dS + sdim;
            double *e = Sd + sdim, *de = e + dv;

            /* forward, keeping every state */
            if (initial_state)
                memcpy(St, initial_state + sh * sdim, sizeof(double) * sdim);
            else
                memset(St, 0, sizeof(double) * sdim);
            for (int64_t t = 0; t < L; ++t) {
                const size_t th = (size_t)(t0 + t) * H + h;
                double *S = St + (size_t)(t + 1) * sdim;
                memcpy(S, St + (size_t)t * sdim, sizeof(double) * sdim);
                kla_token(S, e, q + th * dk, k + th * dk, v + th * dv, alpha ? alpha[th] : 1.0,
                          eta[th], eps, beta_direct, dk, dv, NULL);
            }

            /* reverse sweep */
            if (d_final)
                memcpy(dS, d_final + sh * sdim, sizeof(double) * sdim);
            else
                memset(dS, 0, sizeof(double) * sdim);
            for (int64_t t = L - 1; t >= 0; --t) {
                const size_t th = (size_t)(t0 + t) * H + h;
                const double *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv;
                const double *gt = d_o + th * dv;
                const double *S = St + (size_t)(t + 1) * sdim, *Sp = St + (size_t)t * sdim;
                const double a = alpha ? alpha[th] : 1.0;
                double *gq = dq + th * dk, *gk = dk_out + th * dk, *gv = dv_out + th * dv;

                double kk = 0.0;
                for (int i = 0; i < dk; ++i) kk += kt[i] * kt[i];
                const double b = beta_direct ? eta[th] : eta[th] / (kk + eps);
                /* recompute S~ and e of this token */
                for (size_t x = 0; x < sdim; ++x) Sd[x] = a * Sp[x];
                for (int j = 0; j < dv; ++j) e[j] = vt[j];
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) e[j] -= Sd[(size_t)i * dv + j] * kt[i];

                /* (5) */
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        dS[(size_t)i * dv + j] += qt[i] * gt[j];
                        acc += S[(size_t)i * dv + j] * gt[j];
                    }
                    gq[i] = acc;
                }
                /* (4) */
                double db = 0.0;
                for (int j = 0; j < dv; ++j) de[j] = 0.0;
                for (int i = 0; i < dk; ++i) {
                    double dse = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        dse += dS[(size_t)i * dv + j] * e[j];
                        de[j] += dS[(size_t)i * dv + j] * kt[i];
                    }
                    db += kt[i] * dse;
                    gk[i] = b * dse;
                }
                for (int j = 0; j < dv; ++j) de[j] *= b;
                /* (3) */
                for (int j = 0; j < dv; ++j) gv[j] = de[j];
                for (int i = 0; i < dk; ++i) {
                    double sde = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        sde += Sd[(size_t)i * dv + j] * de[j];
                        dS[(size_t)i * dv + j] -= kt[i] * de[j];
                    }
                    gk[i] -= sde;
                }
                /* (2) */
                double da = 0.0;
                for (size_t x = 0; x < sdim; ++x) {
                    da += dS[x] * Sp[x];
                    dS[x] *= a;
                }
                if (d_alpha) d_alpha[th] = alpha ? da : 0.0;
                /* (1) */
                if (beta_direct) {
                    d_eta[th] = db;
                } else {
                    d_eta[th] = db / (kk + eps);
                    const double c = 2.0 * eta[th] * db / ((kk + eps) * (kk + eps));
                    for (int i = 0; i < dk; ++i) gk[i] -= c * kt[i];
                }
            }
            if (d_initial) memcpy(d_initial + sh * sdim, dS, sizeof(double) * sdim);
            free(St);
        }
    }
    return failed ? -1 : 0;
}
