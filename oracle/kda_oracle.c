/*
 * kda_oracle.c -- plain fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg load this library.  The GPU path never calls
 * it, links it or shares code with it.  It is deliberately slow and literal:
 * one token at a time, in double precision, in the order the recurrence is
 * written.
 *
 * Sources (the web pages describe KDA in words only; they print no formula):
 *  - "TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and training
 *    practice" (jinguxun.com news 11080097), section "Kimi K3.1 Pro model
 *    structure": KDA accumulates history through a gated matrix-state
 *    recurrence whose state reads/writes replace access to all past K/V.
 *  - same page, section "KDA pre/post-processing fusion": the sequence is
 *    processed as intra-chunk work plus inter-chunk state passing; Q/K
 *    normalisation, the beta transform and the gating belong to the forward;
 *    the backward reuses the saved normalisation statistics and states and
 *    joins state-gradient propagation with the Q/K gradients.
 *  - same page, section "Kimi K3.1 Pro Ascend training adaptation": packed
 *    sequences carry document boundaries.
 *
 * Reading taken for the recurrence (the gated delta rule), per head, with a
 * dk x dv state S and S_0 = the document's initial state (or 0):
 *     qh = q / sqrt(sum q^2 + eps),  kh = k / sqrt(sum k^2 + eps)
 *     beta = 1 / (1 + exp(-b)),      alpha = exp(g)   (per key channel)
 *     S'  = Diag(alpha_t) S_{t-1}
 *     S_t = (I - beta_t kh_t kh_t^T) S' + beta_t kh_t v_t^T
 *         = S' + kh_t u_t^T,   u_t = beta_t (v_t - S'^T kh_t)
 *     o_t = S_t^T qh_t
 * The state restarts at every document boundary (cu_seqlens).
 *
 * Layouts (all row-major, contiguous):
 *   q, k, g : [T, H, dk]     v, o : [T, H, dv]     b : [T, H]
 *   states  : [num_seqs, H, dk, dv]     cu : [num_seqs + 1] int64
 * Every input is double; the caller upcasts bf16/fp32 values exactly.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t T;
    int N, H, dk, dv;
    const int64_t* cu;
    /* raw inputs (mode 0) or prepared inputs (mode 1) */
    const double *q, *k, *v, *g, *b;
    const double* s0;
    double eps;
    int prepared; /* 1: q,k are already unit, g holds alpha, b holds beta */
    double *o, *s_final;
    /* backward */
    const double *dO, *dS_final;
    double *dq, *dk_out, *dv_out, *dg, *db, *dS0;
    /* work distribution */
    int ncolblk;        /* forward only: split value columns into this many blocks */
    int64_t next_item;  /* shared counter */
    pthread_mutex_t lock;
    int failed;
} job_t;

/* Per-token preparation: normalised q and k, per-channel alpha, scalar beta.
 * "Q/K normalisation, beta transform and gating" of the forward.  Also returns
 * the two norms, which the backward needs. */
static void prep_token(const job_t* J, int64_t t, int h, double* qh, double* kh, double* al,
                       double* beta, double* nq, double* nk) {
    const int dk = J->dk;
    const double* qr = J->q + (t * J->H + h) * (int64_t)dk;
    const double* kr = J->k + (t * J->H + h) * (int64_t)dk;
    const double* gr = J->g + (t * J->H + h) * (int64_t)dk;
    double bb = J->b[t * J->H + h];
    if (J->prepared) {
        for (int i = 0; i < dk; ++i) { qh[i] = qr[i]; kh[i] = kr[i]; al[i] = gr[i]; }
        *beta = bb;
        *nq = 1.0;
        *nk = 1.0;
        return;
    }
    double sq = 0.0, sk = 0.0;
    for (int i = 0; i < dk; ++i) { sq += qr[i] * qr[i]; sk += kr[i] * kr[i]; }
    double a = sqrt(sq + J->eps), c = sqrt(sk + J->eps);
    for (int i = 0; i < dk; ++i) {
        qh[i] = qr[i] / a;
        kh[i] = kr[i] / c;
        al[i] = exp(gr[i]);
    }
    *beta = 1.0 / (1.0 + exp(-bb));
    *nq = a;
    *nk = c;
}

/* One recurrence step on columns [0, nc) of a state whose rows have stride ld.
 * Writes S' (decayed state) into Sp when Sp != NULL, p and u when non-NULL. */
static void step(int dk, int nc, int ld, double* S, const double* kh, const double* al, double beta,
                 const double* v, double* p, double* u) {
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nc; ++j) S[i * ld + j] *= al[i];
    for (int j = 0; j < nc; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += S[i * ld + j] * kh[i];
        p[j] = s;
        u[j] = beta * (v[j] - s);
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nc; ++j) S[i * ld + j] += kh[i] * u[j];
}

static int64_t take_item(job_t* J) {
    pthread_mutex_lock(&J->lock);
    int64_t it = J->next_item++;
    pthread_mutex_unlock(&J->lock);
    return it;
}

/* ---------------------------------------------------------------- forward */
static void* fwd_worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int dk = J->dk, dv = J->dv, H = J->H;
    const int nb = J->ncolblk;
    const int cw = (dv + nb - 1) / nb;
    double* S = (double*)malloc(sizeof(double) * dk * cw);
    double* qh = (double*)malloc(sizeof(double) * dk * 3);
    double* pu = (double*)malloc(sizeof(double) * cw * 2);
    if (!S || !qh || !pu) {
        J->failed = 1;
        free(S); free(qh); free(pu);
        return NULL;
    }
    double *kh = qh + dk, *al = qh + 2 * dk, *p = pu, *u = pu + cw;
    for (;;) {
        int64_t it = take_item(J);
        if (it >= (int64_t)J->N * H * nb) break;
        const int blk = (int)(it % nb);
        const int h = (int)((it / nb) % H);
        const int n = (int)(it / ((int64_t)nb * H));
        const int j0 = blk * cw;
        const int nc = (j0 + cw <= dv) ? cw : dv - j0;
        if (nc <= 0) continue;
        const int64_t sbase = ((int64_t)n * H + h) * dk * dv;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < nc; ++j)
                S[i * cw + j] = J->s0 ? J->s0[sbase + (int64_t)i * dv + j0 + j] : 0.0;
        for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
            double beta, nq, nk;
            prep_token(J, t, h, qh, kh, al, &beta, &nq, &nk);
            const double* vr = J->v + (t * H + h) * (int64_t)dv + j0;
            step(dk, nc, cw, S, kh, al, beta, vr, p, u);
            double* orow = J->o + (t * H + h) * (int64_t)dv + j0;
            for (int j = 0; j < nc; ++j) {
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += S[i * cw + j] * qh[i];
                orow[j] = s;
            }
        }
        if (J->s_final)
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < nc; ++j) J->s_final[sbase + (int64_t)i * dv + j0 + j] = S[i * cw + j];
    }
    free(S); free(qh); free(pu);
    return NULL;
}

static int run_threads(job_t* J, void* (*fn)(void*), int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    pthread_mutex_init(&J->lock, NULL);
    J->next_item = 0;
    J->failed = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[started], NULL, fn, J) != 0) break;
        ++started;
    }
    fn(J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J->lock);
    return J->failed ? -2 : 0;
}

static int check_common(int64_t T, int N, const int64_t* cu, int H, int dk, int dv) {
    if (T < 0 || N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu) return -1;
    if (cu[0] != 0 || cu[N] != T) return -1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    return 0;
}

static int fwd_common(job_t* J, int nthreads) {
    if (check_common(J->T, J->N, J->cu, J->H, J->dk, J->dv)) return -1;
    if (!J->q || !J->k || !J->v || !J->g || !J->b || !J->o) return -1;
    /* Split value columns when there are fewer chains than threads; the value
     * columns of S never mix, so each block runs the same recurrence. */
    int64_t chains = (int64_t)J->N * J->H;
    int nb = 1;
    while (chains * nb < nthreads && nb * 2 <= J->dv && (J->dv / (nb * 2)) >= 8) nb *= 2;
    J->ncolblk = nb;
    return run_threads(J, fwd_worker, nthreads);
}

/* Forward from raw inputs: q, k raw; g = log-decay; b = beta logit. */
int kda_oracle_fwd(int64_t T, int N, const int64_t* cu, int H, int dk, int dv, const double* q,
                   const double* k, const double* v, const double* g, const double* b,
                   const double* s0, double eps, double* o, double* s_final, int nthreads) {
    job_t J;
    memset(&J, 0, sizeof J);
    J.T = T; J.N = N; J.cu = cu; J.H = H; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.g = g; J.b = b; J.s0 = s0; J.eps = eps;
    J.o = o; J.s_final = s_final; J.prepared = 0;
    return fwd_common(&J, nthreads);
}

/* Forward from prepared inputs: qh, kh used as given, alpha [T,H,dk] and
 * beta [T,H] given directly (no norm, exp or sigmoid).  Used to pin the
 * recurrence on special cases (beta = 0, alpha = 1, exact unit keys). */
int kda_oracle_fwd_core(int64_t T, int N, const int64_t* cu, int H, int dk, int dv,
                        const double* qh, const double* kh, const double* v, const double* alpha,
                        const double* beta, const double* s0, double* o, double* s_final,
                        int nthreads) {
    job_t J;
    memset(&J, 0, sizeof J);
    J.T = T; J.N = N; J.cu = cu; J.H = H; J.dk = dk; J.dv = dv;
    J.q = qh; J.k = kh; J.v = v; J.g = alpha; J.b = beta; J.s0 = s0;
    J.o = o; J.s_final = s_final; J.prepared = 1;
    return fwd_common(&J, nthreads);
}

/* --------------------------------------------------------------- backward
 * Reverse-mode differentiation of the forward above, token by token.  With
 * R = dL/dS_t accumulated from the future and do_t given:
 *     dqh_t = S_t do_t ;          R += qh_t do_t^T
 *     du = R^T kh_t ;             dkh_t = R u_t
 *     dbeta_t = du . (v_t - p_t); dv_t = beta_t du;   dp = -beta_t du
 *     R' = R + kh_t dp^T ;        dkh_t += S'_t dp
 *     dalpha_t[i] = sum_j R'[i,j] S_{t-1}[i,j] ;  dg_t = alpha_t * dalpha_t
 *     R = Diag(alpha_t) R'
 * then through the normalisation and the sigmoid (the saved norms are reused):
 *     dq = (dqh - qh (qh . dqh)) / n_q,  dk likewise,  db = dbeta sigma(b) sigma(-b)
 * d(initial state) = R after the first token.  States are checkpointed every
 * SEG tokens and each segment is recomputed during the reverse sweep. */
#define SEG 64

static void* bwd_worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int dk = J->dk, dv = J->dv, H = J->H;
    const int64_t sz = (int64_t)dk * dv;
    double* vecs = (double*)malloc(sizeof(double) * (dk * 7 + dv * 6));
    double* R = (double*)malloc(sizeof(double) * sz * 3);
    double* segS = (double*)malloc(sizeof(double) * sz * (SEG + 1));
    if (!vecs || !R || !segS) {
        J->failed = 1;
        free(vecs); free(R); free(segS);
        return NULL;
    }
    double *Sp = R + sz, *St = R + 2 * sz;
    double *qh = vecs, *kh = vecs + dk, *al = vecs + 2 * dk, *dqh = vecs + 3 * dk,
           *dkh = vecs + 4 * dk, *dal = vecs + 5 * dk, *tmpk = vecs + 6 * dk;
    double *p = vecs + 7 * dk, *u = p + dv, *du = p + 2 * dv, *dp = p + 3 * dv, *tmpv = p + 4 * dv;
    (void)tmpv;
    for (;;) {
        int64_t it = take_item(J);
        if (it >= (int64_t)J->N * H) break;
        const int h = (int)(it % H), n = (int)(it / H);
        const int64_t t0 = J->cu[n], t1 = J->cu[n + 1], len = t1 - t0;
        const int64_t nseg = (len + SEG - 1) / SEG;
        const int64_t sbase = ((int64_t)n * H + h) * sz;
        double* ck = (double*)malloc(sizeof(double) * sz * (nseg + 1));
        if (!ck) { J->failed = 1; break; }
        /* forward sweep: checkpoint the state entering each segment */
        for (int64_t e = 0; e < sz; ++e) ck[e] = J->s0 ? J->s0[sbase + e] : 0.0;
        for (int64_t sg = 0; sg < nseg; ++sg) {
            double* S = ck + (sg + 1) * sz;
            memcpy(S, ck + sg * sz, sizeof(double) * sz);
            for (int64_t t = t0 + sg * SEG; t < t0 + (sg + 1) * SEG && t < t1; ++t) {
                double beta, nq, nk;
                prep_token(J, t, h, qh, kh, al, &beta, &nq, &nk);
                step(dk, dv, dv, S, kh, al, beta, J->v + (t * H + h) * (int64_t)dv, p, u);
            }
        }
        /* reverse sweep */
        for (int64_t e = 0; e < sz; ++e) R[e] = J->dS_final ? J->dS_final[sbase + e] : 0.0;
        for (int64_t sg = nseg - 1; sg >= 0; --sg) {
            const int64_t ta = t0 + sg * SEG;
            const int64_t tb = (ta + SEG < t1) ? ta + SEG : t1;
            /* segS[i] = state before token ta + i */
            memcpy(segS, ck + sg * sz, sizeof(double) * sz);
            for (int64_t t = ta; t < tb; ++t) {
                double beta, nq, nk;
                double* nxt = segS + (t - ta + 1) * sz;
                memcpy(nxt, segS + (t - ta) * sz, sizeof(double) * sz);
                prep_token(J, t, h, qh, kh, al, &beta, &nq, &nk);
                step(dk, dv, dv, nxt, kh, al, beta, J->v + (t * H + h) * (int64_t)dv, p, u);
            }
            for (int64_t t = tb - 1; t >= ta; --t) {
                double beta, nq, nk;
                prep_token(J, t, h, qh, kh, al, &beta, &nq, &nk);
                const double* Sprev = segS + (t - ta) * sz;
                const double* vr = J->v + (t * H + h) * (int64_t)dv;
                const double* dor = J->dO + (t * H + h) * (int64_t)dv;
                /* recompute S', p, u, S_t from the saved S_{t-1} */
                memcpy(St, Sprev, sizeof(double) * sz);
                step(dk, dv, dv, St, kh, al, beta, vr, p, u);
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) Sp[i * dv + j] = al[i] * Sprev[i * dv + j];
                /* output o_t = S_t^T qh */
                for (int i = 0; i < dk; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j) s += St[i * dv + j] * dor[j];
                    dqh[i] = s;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) R[i * dv + j] += qh[i] * dor[j];
                /* S_t = S' + kh u^T */
                for (int j = 0; j < dv; ++j) {
                    double s = 0.0;
                    for (int i = 0; i < dk; ++i) s += R[i * dv + j] * kh[i];
                    du[j] = s;
                }
                for (int i = 0; i < dk; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j) s += R[i * dv + j] * u[j];
                    dkh[i] = s;
                }
                /* u = beta (v - p) */
                double dbeta = 0.0;
                for (int j = 0; j < dv; ++j) dbeta += du[j] * (vr[j] - p[j]);
                double* dvr = J->dv_out + (t * H + h) * (int64_t)dv;
                for (int j = 0; j < dv; ++j) {
                    dvr[j] = beta * du[j];
                    dp[j] = -beta * du[j];
                }
                /* p = S'^T kh */
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) R[i * dv + j] += kh[i] * dp[j];
                for (int i = 0; i < dk; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j) s += Sp[i * dv + j] * dp[j];
                    dkh[i] += s;
                }
                /* S' = Diag(alpha) S_{t-1} */
                for (int i = 0; i < dk; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j) s += R[i * dv + j] * Sprev[i * dv + j];
                    dal[i] = s;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) R[i * dv + j] *= al[i];
                /* through the prep: alpha = exp(g), beta = sigmoid(b), norms */
                double* dgr = J->dg + (t * H + h) * (int64_t)dk;
                double* dqr = J->dq + (t * H + h) * (int64_t)dk;
                double* dkr = J->dk_out + (t * H + h) * (int64_t)dk;
                double aq = 0.0, ak = 0.0;
                for (int i = 0; i < dk; ++i) { aq += qh[i] * dqh[i]; ak += kh[i] * dkh[i]; }
                for (int i = 0; i < dk; ++i) {
                    if (J->prepared) {
                        dgr[i] = dal[i];
                        dqr[i] = dqh[i];
                        dkr[i] = dkh[i];
                    } else {
                        dgr[i] = al[i] * dal[i];
                        dqr[i] = (dqh[i] - qh[i] * aq) / nq;
                        dkr[i] = (dkh[i] - kh[i] * ak) / nk;
                    }
                }
                if (J->prepared) {
                    J->db[t * H + h] = dbeta;
                } else {
                    /* sigma'(b) = sigma(b) sigma(-b) = e / (1 + e)^2, e = exp(-|b|): the
                     * form beta (1 - beta) keeps only ~3 digits of 1 - beta at |b| = 30 */
                    const double e = exp(-fabs(J->b[t * H + h]));
                    J->db[t * H + h] = dbeta * (e / ((1.0 + e) * (1.0 + e)));
                }
                (void)tmpk;
            }
        }
        if (J->dS0)
            for (int64_t e = 0; e < sz; ++e) J->dS0[sbase + e] = R[e];
        free(ck);
    }
    free(vecs); free(R); free(segS);
    return NULL;
}

/* Backward of kda_oracle_fwd.  dO: [T,H,dv]; dS_final: [N,H,dk,dv] or NULL.
 * Outputs dq, dk: [T,H,dk]; dv: [T,H,dv]; dg: [T,H,dk]; db: [T,H];
 * dS0: [N,H,dk,dv] (may be NULL). */
int kda_oracle_bwd(int64_t T, int N, const int64_t* cu, int H, int dk, int dv, const double* q,
                   const double* k, const double* v, const double* g, const double* b,
                   const double* s0, double eps, const double* dO, const double* dS_final,
                   double* dq, double* dk_out, double* dv_out, double* dg, double* db,
                   double* dS0, int nthreads) {
    if (check_common(T, N, cu, H, dk, dv)) return -1;
    if (!q || !k || !v || !g || !b || !dO || !dq || !dk_out || !dv_out || !dg || !db) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.T = T; J.N = N; J.cu = cu; J.H = H; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.g = g; J.b = b; J.s0 = s0; J.eps = eps; J.prepared = 0;
    J.dO = dO; J.dS_final = dS_final;
    J.dq = dq; J.dk_out = dk_out; J.dv_out = dv_out; J.dg = dg; J.db = db; J.dS0 = dS0;
    return run_threads(&J, bwd_worker, nthreads);
}

/* Backward of kda_oracle_fwd_core: gradients with respect to the prepared
 * inputs (qh, kh, alpha, beta) directly. */
int kda_oracle_bwd_core(int64_t T, int N, const int64_t* cu, int H, int dk, int dv,
                        const double* qh, const double* kh, const double* v, const double* alpha,
                        const double* beta, const double* s0, const double* dO,
                        const double* dS_final, double* dqh, double* dkh, double* dv_out,
                        double* dalpha, double* dbeta, double* dS0, int nthreads) {
    if (check_common(T, N, cu, H, dk, dv)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.T = T; J.N = N; J.cu = cu; J.H = H; J.dk = dk; J.dv = dv;
    J.q = qh; J.k = kh; J.v = v; J.g = alpha; J.b = beta; J.s0 = s0; J.prepared = 1;
    J.dO = dO; J.dS_final = dS_final;
    J.dq = dqh; J.dk_out = dkh; J.dv_out = dv_out; J.dg = dalpha; J.db = dbeta; J.dS0 = dS0;
    return run_threads(&J, bwd_worker, nthreads);
}
