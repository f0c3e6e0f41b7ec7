/*
 * KDA oracle: a plain, slow, sequential fp64 CPU implementation of the
 * Kimi Delta Attention recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP kernels behind include/kda.h) never calls it, shares no code with
 * it, and must fail loudly rather than fall back to it.
 *
 * What it computes (fp64 throughout; inputs are float32 arrays that the
 * caller filled with the exact upcast of the bytes the GPU path reads):
 *
 *   For every sequence n (tokens cu[n] <= t < cu[n+1], in order) and head h,
 *   starting from S = initial_state[n,h] (or 0):
 *     qb = scale * q_t / sqrt(sum q_t^2 + eps),  kb = k_t / sqrt(sum k_t^2 + eps)
 *     S  = Diag(exp g_t) S                 (retention alpha = exp g, per key channel)
 *     vh = S^T kb                          (predict from the existing memory)
 *     S  = S + beta_t kb (v_t - vh)^T      (write only the difference)
 *     o_t = S^T qb                         (read from the updated state)
 *
 * This is S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 * o_t = S_t^T q_t.  Sources: "From KV Cache to Depth Attention: The Bottlenecks
 * Kimi K3 Had to Break", Technical Details, Kimi Delta Attention bullet (predict
 * from memory, write the difference; alpha = retention, beta = update strength,
 * per-channel timescales); "Kimi K3: The Manos, The Mythos, The Legendos",
 * bullets (linear attention -> delta rule -> forget gate -> diagonal gate;
 * L2-normalised queries/keys).  Readings taken where the pages are silent
 * (decay before the prediction, output after the write, beta per token-head,
 * g on the key axis, eps inside the square root, scale on q after the norm)
 * are listed in the repository's design notes.
 *
 * State layout: S[i][j], i = key channel (d_k rows), j = value channel (d_v
 * columns, fastest).  Token-major inputs: q,k,g [T][H][d_k], v [T][H][d_v],
 * beta [T][H]; out [T][H][d_v]; states [N][H][d_k][d_v].
 *
 * kda_oracle_chunked() is a second formulation of the same function: the
 * chunk-wise WY form of the delta rule with a diagonal gate (within a chunk,
 * the unit lower-triangular system (I + A) u = Diag(beta)(V - Khat S0) and
 * its explicit inverse).  It exists so the test suite can check the chunk
 * algebra against the recurrence in fp64; it uses plain loops, explicit
 * exponentials of log-decay differences and no blocking.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -lpthread -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n_seqs, n_heads, dk, dv;
    const int64_t *cu;
    const float *q, *k, *v, *g, *beta, *s0;
    double scale, eps;
    int l2norm;
    int64_t chunk; /* 0: token recurrence; >0: chunk form with this size */
    double *out, *s_final;
    double *state_io; /* decode mode: fp64 state [N][H][dk][dv] updated in place */
    /* work distribution */
    int64_t next_unit;
    pthread_mutex_t lock;
    int failed;
} job_t;

/* Load one token-head vector (float32 -> double, exact) and optionally
 * L2-normalise it as x / sqrt(sum x^2 + eps), then multiply by mul. */
static void load_vec(double *dst, const float *src, int64_t d, int l2norm,
                     double eps, double mul) {
    for (int64_t i = 0; i < d; ++i) dst[i] = (double)src[i];
    if (l2norm) {
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i) ss += dst[i] * dst[i];
        double inv = 1.0 / sqrt(ss + eps);
        for (int64_t i = 0; i < d; ++i) dst[i] *= inv;
    }
    for (int64_t i = 0; i < d; ++i) dst[i] *= mul;
}

/* One token of the recurrence on the fp64 state S[dk][dv]. */
static void token_step(double *S, int64_t dk, int64_t dv, const double *qb,
                       const double *kb, const float *v, const float *g,
                       double beta, double *vh, double *o) {
    /* retention: row i of S is scaled by alpha_i = exp(g_i) */
    for (int64_t i = 0; i < dk; ++i) {
        double a = exp((double)g[i]);
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    /* prediction from the decayed memory: vh = S^T kb */
    for (int64_t j = 0; j < dv; ++j) vh[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) vh[j] += S[i * dv + j] * kb[i];
    /* delta write: S += beta kb (v - vh)^T, stored in vh as the delta */
    for (int64_t j = 0; j < dv; ++j) vh[j] = beta * ((double)v[j] - vh[j]);
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += kb[i] * vh[j];
    /* read-out from the updated state: o = S^T qb */
    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) o[j] += S[i * dv + j] * qb[i];
}

static void run_unit_recurrence(job_t *J, int64_t n, int64_t h, double *S,
                                double *qb, double *kb, double *vh, double *o) {
    const int64_t H = J->n_heads, dk = J->dk, dv = J->dv;
    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const int64_t th = t * H + h;
        load_vec(qb, J->q + th * dk, dk, J->l2norm, J->eps, J->scale);
        load_vec(kb, J->k + th * dk, dk, J->l2norm, J->eps, 1.0);
        token_step(S, dk, dv, qb, kb, J->v + th * dv, J->g + th * dk,
                   (double)J->beta[th], vh, o);
        for (int64_t j = 0; j < dv; ++j) J->out[th * dv + j] = o[j];
    }
}

/* Chunk form for one sequence-head, chunk size C (any C >= 1).
 * Per chunk starting from state S0 with L <= C tokens, gamma_r = sum_{s<=r} g_s:
 *   khat_r = kb_r * exp(gamma_r),  qhat_r = qb_r * exp(gamma_r)
 *   A[s][j] = beta_s * sum_c kb_s[c] kb_j[c] exp(gamma_s[c]-gamma_j[c])   (j < s)
 *   T = (I + A)^{-1}  (forward substitution, explicit inverse)
 *   W = T Diag(beta) Khat,  U = T Diag(beta) V,  u = U - W S0
 *   O_r = qhat_r^T S0 + sum_{j<=r} (sum_c qb_r[c] kb_j[c] exp(gamma_r[c]-gamma_j[c])) u_j
 *   S_L = Diag(exp gamma_L) S0 + sum_j (kb_j * exp(gamma_L - gamma_j)) u_j^T        */
typedef struct {
    double *qb, *kb, *gam, *A, *T, *W, *U, *u, *S0;
} chunk_buf_t;

static int chunk_buf_alloc(chunk_buf_t *b, int64_t C, int64_t dk, int64_t dv) {
    b->qb = malloc(sizeof(double) * C * dk);
    b->kb = malloc(sizeof(double) * C * dk);
    b->gam = malloc(sizeof(double) * C * dk);
    b->A = malloc(sizeof(double) * C * C);
    b->T = malloc(sizeof(double) * C * C);
    b->W = malloc(sizeof(double) * C * dk);
    b->U = malloc(sizeof(double) * C * dv);
    b->u = malloc(sizeof(double) * C * dv);
    b->S0 = malloc(sizeof(double) * dk * dv);
    return b->qb && b->kb && b->gam && b->A && b->T && b->W && b->U && b->u && b->S0;
}

static void chunk_buf_free(chunk_buf_t *b) {
    free(b->qb); free(b->kb); free(b->gam); free(b->A); free(b->T);
    free(b->W); free(b->U); free(b->u); free(b->S0);
}

static void run_unit_chunked(job_t *J, int64_t n, int64_t h, double *S,
                             chunk_buf_t *b) {
    const int64_t H = J->n_heads, dk = J->dk, dv = J->dv, C = J->chunk;
    for (int64_t t0 = J->cu[n]; t0 < J->cu[n + 1]; t0 += C) {
        int64_t L = J->cu[n + 1] - t0;
        if (L > C) L = C;
        memcpy(b->S0, S, sizeof(double) * dk * dv);
        for (int64_t r = 0; r < L; ++r) {
            const int64_t th = (t0 + r) * H + h;
            load_vec(b->qb + r * dk, J->q + th * dk, dk, J->l2norm, J->eps, J->scale);
            load_vec(b->kb + r * dk, J->k + th * dk, dk, J->l2norm, J->eps, 1.0);
            for (int64_t c = 0; c < dk; ++c)
                b->gam[r * dk + c] = (r ? b->gam[(r - 1) * dk + c] : 0.0) +
                                     (double)J->g[th * dk + c];
        }
        /* A (strictly lower), scaled by beta of the row */
        for (int64_t s = 0; s < L; ++s) {
            double bs = (double)J->beta[(t0 + s) * H + h];
            for (int64_t j = 0; j < L; ++j) {
                double a = 0.0;
                if (j < s)
                    for (int64_t c = 0; c < dk; ++c)
                        a += b->kb[s * dk + c] * b->kb[j * dk + c] *
                             exp(b->gam[s * dk + c] - b->gam[j * dk + c]);
                b->A[s * L + j] = bs * a;
            }
        }
        /* T = (I + A)^{-1}: row s of T = e_s - sum_{j<s} A[s][j] T[j] */
        for (int64_t s = 0; s < L; ++s)
            for (int64_t c = 0; c < L; ++c) {
                double x = (s == c) ? 1.0 : 0.0;
                for (int64_t j = 0; j < s; ++j) x -= b->A[s * L + j] * b->T[j * L + c];
                b->T[s * L + c] = x;
            }
        /* W = T Diag(beta) Khat, U = T Diag(beta) V */
        for (int64_t r = 0; r < L; ++r) {
            for (int64_t c = 0; c < dk; ++c) {
                double w = 0.0;
                for (int64_t s = 0; s < L; ++s) {
                    const int64_t th = (t0 + s) * H + h;
                    w += b->T[r * L + s] * (double)J->beta[th] * b->kb[s * dk + c] *
                         exp(b->gam[s * dk + c]);
                }
                b->W[r * dk + c] = w;
            }
            for (int64_t j = 0; j < dv; ++j) {
                double x = 0.0;
                for (int64_t s = 0; s < L; ++s) {
                    const int64_t th = (t0 + s) * H + h;
                    x += b->T[r * L + s] * (double)J->beta[th] * (double)J->v[th * dv + j];
                }
                b->U[r * dv + j] = x;
            }
        }
        /* u = U - W S0 */
        for (int64_t r = 0; r < L; ++r)
            for (int64_t j = 0; j < dv; ++j) {
                double x = b->U[r * dv + j];
                for (int64_t c = 0; c < dk; ++c) x -= b->W[r * dk + c] * b->S0[c * dv + j];
                b->u[r * dv + j] = x;
            }
        /* outputs */
        for (int64_t r = 0; r < L; ++r) {
            const int64_t th = (t0 + r) * H + h;
            for (int64_t j = 0; j < dv; ++j) {
                double o = 0.0;
                for (int64_t c = 0; c < dk; ++c)
                    o += b->qb[r * dk + c] * exp(b->gam[r * dk + c]) * b->S0[c * dv + j];
                for (int64_t s = 0; s <= r; ++s) {
                    double m = 0.0;
                    for (int64_t c = 0; c < dk; ++c)
                        m += b->qb[r * dk + c] * b->kb[s * dk + c] *
                             exp(b->gam[r * dk + c] - b->gam[s * dk + c]);
                    o += m * b->u[s * dv + j];
                }
                J->out[th * dv + j] = o;
            }
        }
        /* state at the chunk end */
        for (int64_t c = 0; c < dk; ++c) {
            double gl = b->gam[(L - 1) * dk + c];
            for (int64_t j = 0; j < dv; ++j) {
                double x = exp(gl) * b->S0[c * dv + j];
                for (int64_t s = 0; s < L; ++s)
                    x += b->kb[s * dk + c] * exp(gl - b->gam[s * dk + c]) * b->u[s * dv + j];
                S[c * dv + j] = x;
            }
        }
    }
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    const int64_t dk = J->dk, dv = J->dv, H = J->n_heads;
    double *S = malloc(sizeof(double) * dk * dv);
    double *qb = malloc(sizeof(double) * dk);
    double *kb = malloc(sizeof(double) * dk);
    double *vh = malloc(sizeof(double) * dv);
    double *o = malloc(sizeof(double) * dv);
    chunk_buf_t cb = {0};
    int ok = S && qb && kb && vh && o;
    if (J->chunk > 0) ok = ok && chunk_buf_alloc(&cb, J->chunk, dk, dv);
    if (!ok) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
    }
    for (;;) {
        if (!ok) break;
        pthread_mutex_lock(&J->lock);
        int64_t unit = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (unit >= J->n_seqs * H) break;
        const int64_t n = unit / H, h = unit % H;
        const int64_t so = (n * H + h) * dk * dv;
        if (J->state_io) {
            /* decode: sequence n holds exactly one token, token index n */
            double *Sd = J->state_io + so;
            const int64_t th = n * H + h;
            load_vec(qb, J->q + th * dk, dk, J->l2norm, J->eps, J->scale);
            load_vec(kb, J->k + th * dk, dk, J->l2norm, J->eps, 1.0);
            token_step(Sd, dk, dv, qb, kb, J->v + th * dv, J->g + th * dk,
                       (double)J->beta[th], vh, o);
            for (int64_t j = 0; j < dv; ++j) J->out[th * dv + j] = o[j];
            continue;
        }
        for (int64_t e = 0; e < dk * dv; ++e)
            S[e] = J->s0 ? (double)J->s0[so + e] : 0.0;
        if (J->chunk > 0)
            run_unit_chunked(J, n, h, S, &cb);
        else
            run_unit_recurrence(J, n, h, S, qb, kb, vh, o);
        if (J->s_final) memcpy(J->s_final + so, S, sizeof(double) * dk * dv);
    }
    if (J->chunk > 0 && ok) chunk_buf_free(&cb);
    free(S); free(qb); free(kb); free(vh); free(o);
    return NULL;
}

static int run_job(job_t *J, int n_threads) {
    const int64_t units = J->n_seqs * J->n_heads;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > units) n_threads = (int)(units > 0 ? units : 1);
    J->next_unit = 0;
    J->failed = 0;
    pthread_mutex_init(&J->lock, NULL);
    pthread_t *th = malloc(sizeof(pthread_t) * n_threads);
    if (!th) return 2;
    int started = 0;
    for (int i = 0; i < n_threads; ++i)
        if (pthread_create(&th[i], NULL, worker, J) == 0) ++started;
    if (started == 0) worker(J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J->lock);
    return J->failed ? 2 : 0;
}

static int check_common(int64_t n_seqs, const int64_t *cu, int64_t H, int64_t dk,
                        int64_t dv) {
    if (n_seqs < 0 || H < 1 || dk < 1 || dv < 1 || !cu) return 1;
    if (cu[0] != 0) return 1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n]) return 1;
    return 0;
}

/* Prefill over packed sequences with the token-by-token recurrence.
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure. */
int kda_oracle_prefill(int64_t n_seqs, const int64_t *cu_seqlens, int64_t n_heads,
                       int64_t dk, int64_t dv, const float *q, const float *k,
                       const float *v, const float *g, const float *beta,
                       const float *initial_state, double scale, double eps,
                       int l2norm, double *out, double *final_state, int n_threads) {
    if (check_common(n_seqs, cu_seqlens, n_heads, dk, dv)) return 1;
    if (!q || !k || !v || !g || !beta || !out) return 1;
    job_t J = {.n_seqs = n_seqs, .n_heads = n_heads, .dk = dk, .dv = dv,
               .cu = cu_seqlens, .q = q, .k = k, .v = v, .g = g, .beta = beta,
               .s0 = initial_state, .scale = scale, .eps = eps, .l2norm = l2norm,
               .chunk = 0, .out = out, .s_final = final_state, .state_io = NULL};
    return run_job(&J, n_threads);
}

/* Same function through the chunk form (chunk >= 1). */
int kda_oracle_chunked(int64_t n_seqs, const int64_t *cu_seqlens, int64_t n_heads,
                       int64_t dk, int64_t dv, const float *q, const float *k,
                       const float *v, const float *g, const float *beta,
                       const float *initial_state, double scale, double eps,
                       int l2norm, int64_t chunk, double *out, double *final_state,
                       int n_threads) {
    if (check_common(n_seqs, cu_seqlens, n_heads, dk, dv) || chunk < 1) return 1;
    if (!q || !k || !v || !g || !beta || !out) return 1;
    job_t J = {.n_seqs = n_seqs, .n_heads = n_heads, .dk = dk, .dv = dv,
               .cu = cu_seqlens, .q = q, .k = k, .v = v, .g = g, .beta = beta,
               .s0 = initial_state, .scale = scale, .eps = eps, .l2norm = l2norm,
               .chunk = chunk, .out = out, .s_final = final_state, .state_io = NULL};
    return run_job(&J, n_threads);
}

/* One decode step: one token per sequence, fp64 state [N][H][dk][dv] updated
 * in place.  Inputs q,k,g [N][H][dk], v [N][H][dv], beta [N][H]; out [N][H][dv]. */
int kda_oracle_decode_step(int64_t n_seqs, int64_t n_heads, int64_t dk, int64_t dv,
                           const float *q, const float *k, const float *v,
                           const float *g, const float *beta, double *state,
                           double scale, double eps, int l2norm, double *out,
                           int n_threads) {
    if (n_seqs < 0 || n_heads < 1 || dk < 1 || dv < 1) return 1;
    if (!q || !k || !v || !g || !beta || !state || !out) return 1;
    job_t J = {.n_seqs = n_seqs, .n_heads = n_heads, .dk = dk, .dv = dv,
               .cu = NULL, .q = q, .k = k, .v = v, .g = g, .beta = beta,
               .s0 = NULL, .scale = scale, .eps = eps, .l2norm = l2norm,
               .chunk = 0, .out = out, .s_final = NULL, .state_io = state};
    return run_job(&J, n_threads);
}
