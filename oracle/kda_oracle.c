/*
 * kda_oracle.c - plain, slow, fp64 CPU oracle for the Kimi Delta Attention
 * (KDA) operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP path.
 *
 * What it computes (Kimi Linear review notes, research-notes-dl6.pages.dev,
 * section "Method / from Linear Attention to KDA", the KDA recurrence and
 * its read-then-write reading): for every sequence n and head h,
 * independently, starting from S_0 = h0[n,h] (zeros if absent),
 *
 *     alpha_t = exp(g_t)                      (per key channel)
 *     S~      = Diag(alpha_t) S_{t-1}         (decay first ...)
 *     S_t     = S~ + beta_t k_t (v_t - S~^T k_t)^T   (... then the delta write)
 *     o_t     = scale * S_t^T q_t             (read after this token's write)
 *
 * and the final state S_T.  The same page's code-verification table states
 * that the public naive recurrence multiplies by exp(g) first and then writes
 * beta k (v - k^T S); this is that order.  `scale` is 1 in the pages' formula.
 *
 * Two optional input transforms, which the kernels can fuse (the pages'
 * parameterization table has the Q/K L2 normalization done inside the KDA
 * kernel, and their test list names a fused gate), are applied per token
 * before the recurrence:
 *  - qk_l2norm: q_t and k_t are divided by sqrt(sum_i x_i^2 + eps) over the
 *    key channels, eps = 1e-6 (the pages give no eps; this is the reading);
 *  - gate_logits: g holds logits z and the log-gate is
 *    g_t = -gate_scale * softplus(z_t), softplus(z) = log(1 + exp(z)), the
 *    form of the synthetic gate recipe.
 * With scalar_gate, g holds one value per token and head ([T_total, H]) that
 * applies to every key channel: Gated DeltaNet's scalar forget gate, which
 * the pages name as the special case KDA generalises.
 *
 * Arithmetic is fp64 throughout; inputs arrive as float32 arrays holding the
 * exact values the GPU receives (bf16 values are exactly representable in
 * float32) and are widened to double before use.
 *
 * Layout: tokens are packed along one axis; q, k, g are [T_total, H, dk],
 * v is [T_total, H, dv], beta is [T_total, H], sequence n owns tokens
 * [cu[n], cu[n+1]).  Only the heads listed in `heads` (nh of them) are
 * computed; outputs are [T_total, nh, dv] and [N, nh, dk, dv], in that order
 * of heads.  h0, when given, is a double array [N, H, dk, dv] (all heads), so
 * that a state can be chained from one call to the next without rounding.
 *
 * Parallelism: OpenMP over the independent (sequence, head) pairs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_L2_EPS 1e-6

/* log(1 + exp(z)) without overflow: for z > 0 it is z + log(1 + exp(-z)) */
static double softplus(double z) { return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z)); }

/* x <- x / sqrt(sum x^2 + eps) */
static void l2_normalise(double *x, int64_t n)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i)
        ss += x[i] * x[i];
    const double inv = 1.0 / sqrt(ss + KDA_ORACLE_L2_EPS);
    for (int64_t i = 0; i < n; ++i)
        x[i] *= inv;
}

int kda_oracle_forward(int64_t n_seqs, const int64_t *cu, int64_t H, int64_t dk,
                       int64_t dv, const float *q, const float *k, const float *v,
                       const float *g, const float *beta, const double *h0,
                       double scale, const int32_t *heads, int64_t nh, double *o,
                       double *hT, int nthreads, int qk_l2norm, int gate_logits,
                       double gate_scale, int scalar_gate)
{
    if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || nh <= 0)
        return 1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n])
            return 2;
    for (int64_t j = 0; j < nh; ++j)
        if (heads[j] < 0 || heads[j] >= H)
            return 3;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t units = n_seqs * nh;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        int64_t n = u / nh, hj = u % nh, h = heads[hj];
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *kv = (double *)malloc(sizeof(double) * (size_t)(dk + dk + dv + dv));
        if (!S || !kv) {
            free(S);
            free(kv);
#pragma omp atomic write
            err = 4;
            continue;
        }
        double *kt = kv, *qt = kv + dk, *vt = kv + 2 * dk, *p = kv + 2 * dk + dv;
        /* S_0 */
        for (int64_t i = 0; i < dk * dv; ++i)
            S[i] = h0 ? h0[((n * H + h) * dk) * dv + i] : 0.0;
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t base_k = (t * H + h) * dk, base_v = (t * H + h) * dv;
            for (int64_t i = 0; i < dk; ++i) {
                kt[i] = (double)k[base_k + i];
                qt[i] = (double)q[base_k + i];
            }
            if (qk_l2norm) {
                l2_normalise(kt, dk);
                l2_normalise(qt, dk);
            }
            for (int64_t j = 0; j < dv; ++j)
                vt[j] = (double)v[base_v + j];
            const double b = (double)beta[t * H + h];
            /* S~ = Diag(exp(g_t)) S_{t-1} */
            for (int64_t i = 0; i < dk; ++i) {
                const double graw = scalar_gate ? (double)g[t * H + h] : (double)g[base_k + i];
                const double gi = gate_logits ? -gate_scale * softplus(graw) : graw;
                const double a = exp(gi);
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] *= a;
            }
            /* p = S~^T k_t */
            for (int64_t j = 0; j < dv; ++j)
                p[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    p[j] += S[i * dv + j] * kt[i];
            /* S_t = S~ + beta k (v - p)^T */
            for (int64_t i = 0; i < dk; ++i) {
                const double bk = b * kt[i];
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] += bk * (vt[j] - p[j]);
            }
            /* o_t = scale * S_t^T q_t */
            double *ot = o + (t * nh + hj) * dv;
            for (int64_t j = 0; j < dv; ++j)
                ot[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    ot[j] += S[i * dv + j] * qt[i];
            for (int64_t j = 0; j < dv; ++j)
                ot[j] *= scale;
        }
        if (hT)
            memcpy(hT + ((n * nh + hj) * dk) * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S);
        free(kv);
    }
    return err;
}

/*
 * General diagonal-plus-low-rank (DPLR) recurrence, the family KDA belongs to
 * (Kimi Linear review notes, section "Chunkwise Algorithm": KDA is a DPLR
 * transition with D = Diag(alpha_t), a_t = beta_t k_t, b_t = k_t .* alpha_t;
 * the jxzklqfsx.com article's efficiency section compares the two kernels).
 * The pages' own formula for the general form is lost in extraction; the
 * plainest reading, which the KDA case must reproduce, is
 *
 *     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,
 *     o_t = scale * S_t^T q_t,        alpha_t = exp(g_t),
 *
 * with a_t, b_t free vectors of dk channels.  Per token the oracle forms
 * x = b_t^T S_{t-1} from the state before the decay, then
 * S_t = Diag(alpha_t) S_{t-1} - a_t x + k_t v_t^T.  Layout as in
 * kda_oracle_forward (a, b like k); all heads; fp64.
 */
int kda_oracle_dplr_forward(int64_t n_seqs, const int64_t *cu, int64_t H, int64_t dk,
                            int64_t dv, const float *q, const float *k, const float *v,
                            const float *g, const float *a, const float *b, const double *h0,
                            double scale, double *o, double *hT, int nthreads)
{
    if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return 1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n])
            return 2;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_seqs * H; ++u) {
        int64_t n = u / H, h = u % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *x = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !x) {
            free(S);
            free(x);
#pragma omp atomic write
            err = 4;
            continue;
        }
        for (int64_t i = 0; i < dk * dv; ++i)
            S[i] = h0 ? h0[(n * H + h) * dk * dv + i] : 0.0;
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t bk = (t * H + h) * dk, bv = (t * H + h) * dv;
            /* x = b^T S_{t-1} */
            for (int64_t j = 0; j < dv; ++j)
                x[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    x[j] += (double)b[bk + i] * S[i * dv + j];
            /* S_t = Diag(alpha) S_{t-1} - a x^T + k v^T */
            for (int64_t i = 0; i < dk; ++i) {
                const double al = exp((double)g[bk + i]), ai = (double)a[bk + i], ki = (double)k[bk + i];
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = al * S[i * dv + j] - ai * x[j] + ki * (double)v[bv + j];
            }
            /* o_t = scale S_t^T q_t */
            double *ot = o + (t * H + h) * dv;
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i)
                    acc += S[i * dv + j] * (double)q[bk + i];
                ot[j] = scale * acc;
            }
        }
        if (hT)
            memcpy(hT + (n * H + h) * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S);
        free(x);
    }
    return err;
}

int kda_oracle_version(void) { return 3; }

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Gradients of the recurrence above (no input transforms) by reverse-mode
 * differentiation, step by step backwards through each token:
 *
 *   forward:  S~ = Diag(alpha) S_{t-1};  p = S~^T k;  u = v - p;
 *             S_t = S~ + beta k u^T;  o_t = scale S_t^T q
 *   backward, with dS the gradient of the loss with respect to S_t
 *   (dS = d final_state at t = T, 0 if absent):
 *             dS  += scale q do^T;       dq = scale S_t do
 *             du   = beta dS^T k;        dk = beta dS u;   dbeta = k^T dS u
 *             dv   = du;                 dp = -du
 *             dS~  = dS + k dp^T;        dk += S~ dp
 *             dg   = rowsum(S~ . dS~)    (d alpha_i times alpha_i)
 *             dS   = Diag(alpha) dS~     (the gradient for S_{t-1})
 *   and d initial_state = dS after the first token.
 *
 * Every state S_0 .. S_T of a (sequence, head) is kept, so memory is
 * (T_n + 1) dk dv doubles per pair in flight.  Outputs are double arrays with
 * the inputs' layouts: dq, dk, dg [T_total, H, dk], dv [T_total, H, dv],
 * dbeta [T_total, H], dh0 [N, H, dk, dv].  All heads are computed.
 *
 * With scalar_gate, g is [T_total, H] (one gate per token and head for every
 * key channel, Gated DeltaNet's gate) and so is dg: the gate's gradient is the
 * sum over channels of the per-channel dg above.
 *
 * With the input transforms of kda_oracle_forward (qk_l2norm: x^ = x / r,
 * r = sqrt(sum x^2 + eps); gate_logits: log-gate = -gate_scale softplus(z))
 * the recurrence runs on the transformed values and the gradients are carried
 * back through the transforms by the chain rule:
 *   dx = (dx^ - x^ (x^ . dx^)) / r           for q and k,
 *   dz = dloggate * (-gate_scale * sigmoid(z)),
 * so dq, dk and dg are gradients with respect to the raw q, k and g.
 */
int kda_oracle_backward(int64_t n_seqs, const int64_t *cu, int64_t H, int64_t dk,
                        int64_t dv, const float *q, const float *k, const float *v,
                        const float *g, const float *beta, const double *h0,
                        double scale, const float *d_o, const double *dhT,
                        double *dq, double *dkk, double *dvv, double *dg,
                        double *dbeta, double *dh0, int nthreads, int scalar_gate,
                        int qk_l2norm, int gate_logits, double gate_scale)
{
    if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return 1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n])
            return 2;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t units = n_seqs * H, sz = dk * dv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uix = 0; uix < units; ++uix) {
        const int64_t n = uix / H, h = uix % H, T0 = cu[n], Tn = cu[n + 1] - cu[n];
        double *S = (double *)malloc(sizeof(double) * (size_t)((Tn + 1) * sz));
        double *w = (double *)malloc(sizeof(double) * (size_t)(3 * sz + 4 * dk + 4 * dv));
        if (!S || !w) {
            free(S);
            free(w);
#pragma omp atomic write
            err = 4;
            continue;
        }
        double *dS = w, *St = w + sz, *dSt = w + 2 * sz;
        double *kt = w + 3 * sz, *qt = kt + dk, *al = qt + dk, *tmp = al + dk;
        double *vt = tmp + dk, *u = vt + dv, *dov = u + dv, *du = dov + dv;
        /* forward, keeping every state */
        for (int64_t i = 0; i < sz; ++i)
            S[i] = h0 ? h0[(n * H + h) * sz + i] : 0.0;
        for (int64_t t = 0; t < Tn; ++t) {
            const int64_t bk = ((T0 + t) * H + h) * dk, bv = ((T0 + t) * H + h) * dv;
            const double *Sp = S + t * sz;
            double *Sn = S + (t + 1) * sz;
            const double b = (double)beta[(T0 + t) * H + h];
            for (int64_t j = 0; j < dv; ++j)
                u[j] = (double)v[bv + j];
            for (int64_t i = 0; i < dk; ++i)
                kt[i] = (double)k[bk + i];
            if (qk_l2norm)
                l2_normalise(kt, dk);
            for (int64_t i = 0; i < dk; ++i) {
                const double graw = (double)g[scalar_gate ? (T0 + t) * H + h : bk + i];
                const double a = exp(gate_logits ? -gate_scale * softplus(graw) : graw);
                for (int64_t j = 0; j < dv; ++j) {
                    Sn[i * dv + j] = a * Sp[i * dv + j];
                    u[j] -= Sn[i * dv + j] * kt[i];
                }
            }
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    Sn[i * dv + j] += b * kt[i] * u[j];
        }
        /* backward */
        for (int64_t i = 0; i < sz; ++i)
            dS[i] = dhT ? dhT[(n * H + h) * sz + i] : 0.0;
        for (int64_t t = Tn - 1; t >= 0; --t) {
            const int64_t tt = T0 + t, bk = (tt * H + h) * dk, bv = (tt * H + h) * dv;
            const double *Sp = S + t * sz, *Sn = S + (t + 1) * sz;
            const double b = (double)beta[tt * H + h];
            double rk = 1.0, rq = 1.0;  /* the norms' r, for the chain rule */
            for (int64_t i = 0; i < dk; ++i) {
                kt[i] = (double)k[bk + i];
                qt[i] = (double)q[bk + i];
                const double graw = (double)g[scalar_gate ? tt * H + h : bk + i];
                al[i] = exp(gate_logits ? -gate_scale * softplus(graw) : graw);
            }
            if (qk_l2norm) {
                double sk = 0.0, sq = 0.0;
                for (int64_t i = 0; i < dk; ++i) {
                    sk += kt[i] * kt[i];
                    sq += qt[i] * qt[i];
                }
                rk = sqrt(sk + 1e-6);
                rq = sqrt(sq + 1e-6);
                for (int64_t i = 0; i < dk; ++i) {
                    kt[i] /= rk;
                    qt[i] /= rq;
                }
            }
            for (int64_t j = 0; j < dv; ++j) {
                vt[j] = (double)v[bv + j];
                dov[j] = (double)d_o[bv + j];
            }
            /* S~ = Diag(alpha) S_{t-1} and u = v - S~^T k, recomputed */
            for (int64_t j = 0; j < dv; ++j)
                u[j] = vt[j];
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) {
                    St[i * dv + j] = al[i] * Sp[i * dv + j];
                    u[j] -= St[i * dv + j] * kt[i];
                }
            /* o_t = scale S_t^T q */
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    dS[i * dv + j] += scale * qt[i] * dov[j];
                    acc += Sn[i * dv + j] * dov[j];
                }
                dq[bk + i] = scale * acc;
            }
            /* S_t = S~ + beta k u^T */
            double db = 0.0;
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i)
                    acc += kt[i] * dS[i * dv + j];
                du[j] = b * acc;
                db += acc * u[j];
            }
            dbeta[tt * H + h] = db;
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j)
                    acc += dS[i * dv + j] * u[j];
                tmp[i] = b * acc;
            }
            /* u = v - p, p = S~^T k */
            for (int64_t j = 0; j < dv; ++j)
                dvv[bv + j] = du[j];
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    dSt[i * dv + j] = dS[i * dv + j] - kt[i] * du[j];
                    acc -= St[i * dv + j] * du[j];
                }
                dkk[bk + i] = tmp[i] + acc;
            }
            /* S~ = Diag(alpha) S_{t-1} */
            double dgs = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    acc += St[i * dv + j] * dSt[i * dv + j];
                    dS[i * dv + j] = al[i] * dSt[i * dv + j];
                }
                if (gate_logits) {  /* d/dz of -gate_scale softplus(z) is -gate_scale sigmoid(z) */
                    const double z = (double)g[scalar_gate ? tt * H + h : bk + i];
                    acc *= -gate_scale / (1.0 + exp(-z));
                }
                if (scalar_gate)
                    dgs += acc;
                else
                    dg[bk + i] = acc;
            }
            if (scalar_gate)
                dg[tt * H + h] = dgs;
            if (qk_l2norm) {  /* dx = (dx^ - x^ (x^ . dx^)) / r */
                double pq = 0.0, pk = 0.0;
                for (int64_t i = 0; i < dk; ++i) {
                    pq += qt[i] * dq[bk + i];
                    pk += kt[i] * dkk[bk + i];
                }
                for (int64_t i = 0; i < dk; ++i) {
                    dq[bk + i] = (dq[bk + i] - qt[i] * pq) / rq;
                    dkk[bk + i] = (dkk[bk + i] - kt[i] * pk) / rk;
                }
            }
        }
        memcpy(dh0 + (n * H + h) * sz, dS, sizeof(double) * (size_t)sz);
        free(S);
        free(w);
    }
    return err;
}
