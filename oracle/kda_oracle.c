/*
 * kda_oracle.c -- fp64 CPU oracle for the Kimi Delta Attention (KDA) operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library,
 * its headers, its Python binding) includes, links or calls this file.  Only
 * the tests, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or constant with the GPU path.
 *
 * What it computes, and where that comes from:
 *
 *  - Gate ("Architecture Deep Dive: Kimi K3...", section 3.2, equation 1;
 *    "Kimi K3 Deep Dive...", "The Design: Putting a Lower Bound on Log-Decay"
 *    and its illustrative code): the per-channel log-decay of token t is
 *        g_t = g_min * sigmoid(theta_t),  g_min = -5,
 *    so g_t lies in [-5, 0] and the per-step decay factor is exp(g_t).
 *
 *  - Chunk-local cumulative log-decay (same page, "The Problem: The
 *    Diagonal-Block Dilemma"): the decay from position i to j inside a chunk
 *    is the product of the per-step factors, i.e. exp of the sum of g over
 *    (i, j].  With 16-token chunks the inclusive prefix sum of g restarted
 *    at every chunk start is the quantity whose exponent the chunked method
 *    scales by; it is reported by the gate helper.
 *
 *  - The recurrence ("Kimi K3" explainer, "Across the sequence": a gated
 *    delta-rule linear attention; each token reads a fixed-size state,
 *    forgets part of it channel-wise and writes into it).  Per head, with
 *    state S of shape [d_k, d_v] and for every token t in order:
 *        S   <- Diag(exp(g_t)) S                       (channel-wise forget)
 *        u_t  = beta_t * (v_t - S^T k_t)                (delta-rule read)
 *        S   <- S + k_t u_t^T                           (write)
 *        o_t  = S^T q_t                                 (output read)
 *    The decode step is this body for one token with S updated in place.
 *
 *  - Unbounded gate, for the ablation of the bound ("Kimi K3 Deep Dive...",
 *    "The Design: Putting a Lower Bound on Log-Decay", which names the
 *    conventional log-decay it replaces as the negative softplus of the gate
 *    input; "Architecture Deep Dive: Kimi K3...", section 3.1):
 *        g_t = -softplus(theta_t) = -ln(1 + e^{theta_t}),
 *    with range (-inf, 0).  It enters the same recurrence below.
 *
 *  - Gradients (the backward pass a training step needs; the pages' gain is
 *    training throughput, "Architecture Deep Dive: Kimi K3...", section 3.2).
 *    For the scalar L = sum_t <do_t, o_t> + <dS_T, S_T>, the derivatives of L
 *    with respect to q, k, v, g, beta and S0 follow by the chain rule through
 *    the four steps of the recurrence below, taken in reverse token order
 *    (P_t = Diag(exp(g_t)) S_{t-1} is the decayed state):
 *        dS += q_t do_t^T;  dq_t = S_t do_t
 *        du  = dS^T k_t;    dk_t = dS u_t;          dP = dS
 *        dv_t = beta_t du;  dbeta_t = du . (v_t - P_t^T k_t)
 *        dP -= beta_t k_t du^T;  dk_t -= beta_t P_t du
 *        dg_t[i] = sum_j dP[i][j] P_t[i][j];  dS = Diag(exp(g_t)) dP
 *    and dS0 is the dS left after the first token.  Through the gate,
 *    dtheta = dg * (-5) sigmoid(theta) (1 - sigmoid(theta)).
 *
 *  - Output gate ("Kimi K3" explainer, "Across the sequence": the output of
 *    each attention layer is scaled per channel and per token by a learned,
 *    input-dependent sigmoid gate before it rejoins the residual stream).
 *    Read as o'_t[j] = o_t[j] * sigmoid(z_t[j]), where z (the gate's
 *    pre-activation, same shape as o) is an input.  The gate acts on the
 *    output only; the state recurrence above does not see it.
 *
 * Plain loops in double precision, no blocking or reordering beyond the
 * definition.  Threads only split independent (batch, head) sequences.
 * Column j of S evolves independently of the other columns (every operation
 * above acts on columns separately), so an optional column list restricts
 * the computation to those columns of o and S_T; with no list every column
 * is computed.
 *
 * Layouts (row-major, all double):
 *   q, k  [B, T, H, dk]     v  [B, T, H, dv]      g (or theta) [B, T, H, dk]
 *   beta  [B, T, H]         S0 [B, H, dk, dv]
 *   o     [B, T, H, nc]     S_T [B, H, dk, nc]    (nc = ncols, or dv)
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_G_MIN (-5.0)
#define ORACLE_CHUNK 16

/* sigmoid written from its definition 1 / (1 + e^{-x}). */
static double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* g = g_min * sigmoid(theta), elementwise over n values. */
void kda_oracle_gate(long n, const double* theta, double* g) {
    for (long i = 0; i < n; ++i) g[i] = ORACLE_G_MIN * oracle_sigmoid(theta[i]);
}

/* g = -softplus(theta) = -ln(1 + e^theta), elementwise over n values.  Written
 * as max(theta, 0) + ln(1 + e^{-|theta|}), which is the same quantity and stays
 * finite for every finite theta. */
void kda_oracle_gate_softplus(long n, const double* theta, double* g) {
    for (long i = 0; i < n; ++i) {
        const double x = theta[i];
        g[i] = -((x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))));
    }
}

/* Output gate: out = o * sigmoid(z), elementwise over n values (out may be o). */
void kda_oracle_output_gate(long n, const double* o, const double* z, double* out) {
    for (long i = 0; i < n; ++i) out[i] = o[i] * oracle_sigmoid(z[i]);
}

/* Inclusive prefix sum of g along T, restarted at every 16-token chunk start
 * (positions 0, 16, 32, ...).  g and gcum are [B, T, H, dk]. */
void kda_oracle_gate_cumsum(int B, int T, int H, int dk, const double* g, double* gcum) {
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < dk; ++c) {
                double run = 0.0;
                for (int t = 0; t < T; ++t) {
                    size_t idx = (((size_t)b * T + t) * H + h) * dk + c;
                    if (t % ORACLE_CHUNK == 0) run = 0.0;
                    run += g[idx];
                    gcum[idx] = run;
                }
            }
}

typedef struct {
    int B, T, H, dk, dv, nc;
    const double *q, *k, *v, *g, *beta, *S0;
    const int* cols;
    double *o, *S_T;
    int tid, nthreads;
    int status;
} job_t;

/* One (batch, head) sequence, token by token. */
static int run_sequence(const job_t* J, int b, int h) {
    const int T = J->T, H = J->H, dk = J->dk, dv = J->dv, nc = J->nc;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * nc);
    double* u = (double*)malloc(sizeof(double) * (size_t)nc);
    if (!S || !u) { free(S); free(u); return 1; }

    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nc; ++j) {
            int col = J->cols ? J->cols[j] : j;
            S[(size_t)i * nc + j] =
                J->S0 ? J->S0[(((size_t)b * H + h) * dk + i) * dv + col] : 0.0;
        }

    for (int t = 0; t < T; ++t) {
        const size_t row = ((size_t)b * T + t) * H + h;
        const double* qt = J->q + row * dk;
        const double* kt = J->k + row * dk;
        const double* vt = J->v + row * dv;
        const double* gt = J->g + row * dk;
        const double bt = J->beta[row];

        /* forget: S <- Diag(exp(g_t)) S  (row i of S is channel i of d_k) */
        for (int i = 0; i < dk; ++i) {
            const double a = exp(gt[i]);
            for (int j = 0; j < nc; ++j) S[(size_t)i * nc + j] *= a;
        }
        /* read: u = beta * (v - S^T k) */
        for (int j = 0; j < nc; ++j) {
            double r = 0.0;
            for (int i = 0; i < dk; ++i) r += S[(size_t)i * nc + j] * kt[i];
            const int col = J->cols ? J->cols[j] : j;
            u[j] = bt * (vt[col] - r);
        }
        /* write: S <- S + k u^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < nc; ++j) S[(size_t)i * nc + j] += kt[i] * u[j];
        /* output: o_t = S^T q */
        double* ot = J->o + row * nc;
        for (int j = 0; j < nc; ++j) {
            double r = 0.0;
            for (int i = 0; i < dk; ++i) r += S[(size_t)i * nc + j] * qt[i];
            ot[j] = r;
        }
    }

    if (J->S_T)
        memcpy(J->S_T + ((size_t)b * H + h) * dk * nc, S, sizeof(double) * (size_t)dk * nc);
    free(S);
    free(u);
    return 0;
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int n = J->B * J->H;
    for (int s = J->tid; s < n; s += J->nthreads)
        if (run_sequence(J, s / J->H, s % J->H)) J->status = 1;
    return NULL;
}

/* Token-by-token recurrence with the log-decay g given directly.
 * cols: NULL for all d_v columns, else ncols indices into [0, dv).
 * S0 and S_T may be NULL.  Returns 0 on success, nonzero on bad arguments
 * or allocation failure. */
int kda_oracle_recurrence(int B, int T, int H, int dk, int dv,
                          const double* q, const double* k, const double* v,
                          const double* g, const double* beta, const double* S0,
                          const int* cols, int ncols, double* o, double* S_T,
                          int nthreads) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return 2;
    if (!q || !k || !v || !g || !beta || !o) return 2;
    const int nc = cols ? ncols : dv;
    if (nc <= 0) return 2;
    if (cols)
        for (int j = 0; j < nc; ++j)
            if (cols[j] < 0 || cols[j] >= dv) return 2;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B * H) nthreads = B * H > 0 ? B * H : 1;

    job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 1; }
    for (int i = 0; i < nthreads; ++i) {
        job_t J = {B, T, H, dk, dv, nc, q, k, v, g, beta, S0, cols, o, S_T, i, nthreads, 0};
        jobs[i] = J;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &jobs[i]);
    worker(&jobs[0]);
    int status = jobs[0].status;
    for (int i = 1; i < nthreads; ++i) {
        pthread_join(th[i], NULL);
        status |= jobs[i].status;
    }
    free(jobs);
    free(th);
    return status;
}

/* Chunked-prefill result: the gate applied to theta, then the recurrence.
 * (Chunking is an evaluation order; the result is the recurrence's.) */
int kda_oracle_chunk_fwd(int B, int T, int H, int dk, int dv,
                         const double* q, const double* k, const double* v,
                         const double* theta, const double* beta, const double* S0,
                         const int* cols, int ncols, double* o, double* S_T,
                         int nthreads) {
    const size_t n = (size_t)B * T * H * dk;
    double* g = (double*)malloc(sizeof(double) * (n ? n : 1));
    if (!g) return 1;
    kda_oracle_gate((long)n, theta, g);
    int st = kda_oracle_recurrence(B, T, H, dk, dv, q, k, v, g, beta, S0, cols, ncols,
                                   o, S_T, nthreads);
    free(g);
    return st;
}

/* One decode step: the recurrence body for a single token per (batch, head),
 * S [B, H, dk, dv] updated in place, o [B, H, dv]. */
int kda_oracle_decode_step(int B, int H, int dk, int dv,
                           const double* q, const double* k, const double* v,
                           const double* theta, const double* beta, double* S,
                           double* o, int nthreads) {
    const size_t n = (size_t)B * H * dk;
    double* g = (double*)malloc(sizeof(double) * (n ? n : 1));
    double* S_new = (double*)malloc(sizeof(double) * ((size_t)B * H * dk * dv + 1));
    if (!g || !S_new) { free(g); free(S_new); return 1; }
    kda_oracle_gate((long)n, theta, g);
    /* [B, H, d] with T = 1 is the [B, T, H, d] layout with T = 1. */
    int st = kda_oracle_recurrence(B, 1, H, dk, dv, q, k, v, g, beta, S, NULL, 0, o, S_new,
                                   nthreads);
    if (st == 0) memcpy(S, S_new, sizeof(double) * (size_t)B * H * dk * dv);
    free(g);
    free(S_new);
    return st;
}

/* Backward of the recurrence for one (batch, head) sequence; every state S_t is
 * kept from a forward sweep (T*dk*dv doubles).  Layouts as the forward; do
 * [B,T,H,dv], dS_T [B,H,dk,dv] or NULL (zero); outputs dq, dk [B,T,H,dk], dv
 * [B,T,H,dv], dg [B,T,H,dk], dbeta [B,T,H], dS0 [B,H,dk,dv] (may be NULL). */
int kda_oracle_backward(int B, int T, int H, int dk, int dv,
                        const double* q, const double* k, const double* v,
                        const double* g, const double* beta, const double* S0,
                        const double* dout, const double* dS_T,
                        double* dq, double* dkk, double* dvv, double* dg, double* dbeta,
                        double* dS0) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return 2;
    if (!q || !k || !v || !g || !beta || !dout || !dq || !dkk || !dvv || !dg || !dbeta) return 2;
    const size_t SS = (size_t)dk * dv;
    double* St = (double*)malloc(sizeof(double) * SS * (size_t)(T + 1));   /* S_0 .. S_T */
    double* U = (double*)malloc(sizeof(double) * (size_t)dv * (size_t)(T > 0 ? T : 1));
    double* R = (double*)malloc(sizeof(double) * (size_t)dv * (size_t)(T > 0 ? T : 1));   /* P_t^T k_t */
    double* dS = (double*)malloc(sizeof(double) * SS);
    double* dP = (double*)malloc(sizeof(double) * SS);
    double* P = (double*)malloc(sizeof(double) * SS);
    double* du = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!St || !U || !R || !dS || !dP || !P || !du) {
        free(St); free(U); free(R); free(dS); free(dP); free(P); free(du);
        return 1;
    }
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const size_t sh = ((size_t)b * H + h) * SS;
            /* forward sweep, keeping S_t, u_t and P_t^T k_t */
            for (size_t x = 0; x < SS; ++x) St[x] = S0 ? S0[sh + x] : 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t row = ((size_t)b * T + t) * H + h;
                const double *kt = k + row * dk, *vt = v + row * dv, *gt = g + row * dk;
                const double* Sp = St + SS * t;
                double* Sn = St + SS * (t + 1);
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) P[(size_t)i * dv + j] = exp(gt[i]) * Sp[(size_t)i * dv + j];
                for (int j = 0; j < dv; ++j) {
                    double r = 0.0;
                    for (int i = 0; i < dk; ++i) r += P[(size_t)i * dv + j] * kt[i];
                    R[(size_t)t * dv + j] = r;
                    U[(size_t)t * dv + j] = beta[row] * (vt[j] - r);
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        Sn[(size_t)i * dv + j] = P[(size_t)i * dv + j] + kt[i] * U[(size_t)t * dv + j];
            }
            /* reverse sweep */
            for (size_t x = 0; x < SS; ++x) dS[x] = dS_T ? dS_T[sh + x] : 0.0;
            for (int t = T - 1; t >= 0; --t) {
                const size_t row = ((size_t)b * T + t) * H + h;
                const double *qt = q + row * dk, *kt = k + row * dk, *vt = v + row * dv, *gt = g + row * dk;
                const double* dot = dout + row * dv;
                const double* Sn = St + SS * (t + 1);
                const double* Sp = St + SS * t;
                const double* ut = U + (size_t)t * dv;
                const double* rt = R + (size_t)t * dv;
                const double bt = beta[row];
                /* o_t = S_t^T q_t */
                for (int i = 0; i < dk; ++i) {
                    double a = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        dS[(size_t)i * dv + j] += qt[i] * dot[j];
                        a += Sn[(size_t)i * dv + j] * dot[j];
                    }
                    dq[row * dk + i] = a;
                }
                /* S_t = P_t + k_t u_t^T */
                for (int j = 0; j < dv; ++j) {
                    double a = 0.0;
                    for (int i = 0; i < dk; ++i) a += dS[(size_t)i * dv + j] * kt[i];
                    du[j] = a;
                }
                for (int i = 0; i < dk; ++i) {
                    double a = 0.0;
                    for (int j = 0; j < dv; ++j) a += dS[(size_t)i * dv + j] * ut[j];
                    dkk[row * dk + i] = a;
                }
                /* u_t = beta_t (v_t - P_t^T k_t) */
                double db = 0.0;
                for (int j = 0; j < dv; ++j) {
                    dvv[row * dv + j] = bt * du[j];
                    db += du[j] * (vt[j] - rt[j]);
                }
                dbeta[row] = db;
                for (int i = 0; i < dk; ++i) {
                    const double e = exp(gt[i]);
                    double a = 0.0, dgi = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        const double Pij = e * Sp[(size_t)i * dv + j];
                        const double dPij = dS[(size_t)i * dv + j] - bt * kt[i] * du[j];
                        a += Pij * du[j];
                        dgi += dPij * Pij;
                        dP[(size_t)i * dv + j] = dPij;
                    }
                    dkk[row * dk + i] -= bt * a;
                    /* P_t = Diag(exp(g_t)) S_{t-1} */
                    dg[row * dk + i] = dgi;
                    for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] = e * dP[(size_t)i * dv + j];
                }
            }
            if (dS0) memcpy(dS0 + sh, dS, sizeof(double) * SS);
        }
    free(St); free(U); free(R); free(dS); free(dP); free(P); free(du);
    return 0;
}

/* Through the gate g = g_min * sigmoid(theta): dtheta = dg * g_min sigmoid (1 - sigmoid). */
void kda_oracle_gate_backward(long n, const double* theta, const double* dg, double* dtheta) {
    for (long i = 0; i < n; ++i) {
        const double s = oracle_sigmoid(theta[i]);
        dtheta[i] = dg[i] * ORACLE_G_MIN * s * (1.0 - s);
    }
}
