/*
 * ssm_oracle.c -- plain, slow, fp64 CPU reference of the selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only through
 * the seeded inputs.
 *
 * Every value is evaluated in double precision with libm exp/log1p, compiled
 * without fast-math.  Inputs arrive already decoded to double (after the
 * rounding to the I/O dtype that the GPU path also sees).
 *
 * Sources (web pages on the Mamba selective scan):
 *   [P1] "Mamba hardware-aware operator fusion and selective-scan
 *        parallelisation for long meeting sequences" (ufo.work, first article)
 *   [P2] "From FlashAttention to Mamba: inference optimisation" (kj168168)
 *   [P5] SSM engineering essay (discosf.com)
 *
 * What is computed, per batch row b and channel d, independently:
 *   delta_t = softplus(delta_raw + bias[d]) if the flag is set, else the sum
 *                                  -- [P5] §1.3 (input-dependent step size,
 *                                     through softplus); [P1] §2.1 (dt_proj
 *                                     then softplus); bias added before it.
 *   dA      = exp(delta_t * A[d,n])                   -- [P1] §1.1, [P2] §三.1
 *   dBu     = delta_t * B[b,n,t] * u[b,d,t]           -- [P1] §1.1 (B-bar =
 *                                     Delta*B, applied to the input x_t);
 *             or, with zero-order hold, (exp(delta_t A) - 1) / A * B u
 *                                  -- [P5] §1.2 (B-bar of the ZOH rule)
 *   h_t[n]  = dA * h_{t-1}[n] + dBu,  h_{-1} = 0      -- [P1] §1.1, [P5] §1.2
 *   y_t     = sum_n C[b,n,t] h_t[n] + D[d] u[b,d,t]   -- [P1] §1.1 (y = C h),
 *                                     [P5] §1.1 (skip term D x)
 *   y_t    *= z / (1 + exp(-z))   when a gate z is given (silu gate)
 *   last_state[b,d,n] = h_{L-1}[n]
 * Single-token update ([P1] §4.1, persistent state, h_new = A h_old + B x):
 *   state[b,d,n] <- exp(delta A[d,n]) state + delta B[b,n] u[b,d]
 *   y[b,d]        = (sum_n C[b,n] state[b,d,n] + D[d] u[b,d]) * silu(z)
 *
 * Layouts (row-major, last index fastest):
 *   u, delta, z, y: (batch, d_inner, L)   B, C: (batch, N, L)
 *   A: (d_inner, N)   D, delta_bias: (d_inner)   states: (batch, d_inner, N)
 *
 * The second entry point, oracle_scan_chunked, reaches the same result by
 * the chunked route of [P1] §3.1: each chunk's transfer operator
 * (A_chunk, B_chunk) with h_end = A_chunk h_start + B_chunk, an exclusive
 * combine of the operators across chunks (left fold, or a balanced tree of
 * the associative composition), then a re-run of every chunk from its
 * h_start.  It exists only so that tests can check that chunking is an exact
 * re-association of the sequential loop.
 *
 * Parity pins: see the header of oracle/__init__.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ scalar steps */

/* softplus(x) = log(1 + e^x), written as max(x,0) + log1p(e^{-|x|}) so that
 * it neither overflows for large x nor loses digits for very negative x. */
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Factor of B u in the state update.  Euler (the default): dt.  Zero-order
 * hold -- the input held constant over the step -- (SSM engineering essay,
 * §1.2: B_bar = (dt A)^-1 (exp(dt A) - 1) dt B): (exp(dt A) - 1) / A, whose
 * limit at A = 0 is dt. */
static double input_coeff(double dt, double A, int zoh) {
    if (!zoh) return dt;
    return A != 0.0 ? expm1(dt * A) / A : dt;
}

/* Derivatives of that factor, for the backward pass.  Euler: d/ddt = 1,
 * d/dA = 0.  Zero-order hold, c = (exp(dt A) - 1) / A: dc/ddt = exp(dt A);
 * dc/dA = (dt A exp(dt A) - (exp(dt A) - 1)) / A^2 = dt^2 psi(dt A) with
 * psi(x) = (x e^x - e^x + 1) / x^2 = sum_{m >= 2} (m - 1) x^(m-2) / m!
 * (the power series of x e^x - e^x + 1 divided by x^2), summed term by term
 * for |x| < 1 and taken in closed form otherwise. */
static double zoh_psi(double x) {
    if (fabs(x) >= 1.0) return (x * exp(x) - expm1(x)) / (x * x);
    double s = 0.0, fact = 2.0, xp = 1.0;   /* m! and x^(m-2) for m = 2 */
    for (int m = 2; m < 30; ++m) {
        s += (double)(m - 1) * xp / fact;
        xp *= x;
        fact *= (double)(m + 1);
    }
    return s;
}

static double input_coeff_ddt(double dt, double A, int zoh) {
    return zoh ? exp(dt * A) : 1.0;
}

static double input_coeff_dA(double dt, double A, int zoh) {
    return zoh ? dt * dt * zoh_psi(dt * A) : 0.0;
}

/* ------------------------------------------------------------ arguments */

typedef struct {
    int64_t batch, d_inner, d_state, seqlen;
    const double *u, *delta, *A, *B, *C, *D, *z, *delta_bias, *h0;
    int softplus_flag;
    double *y, *last_state;
    int zoh;            /* zero-order-hold input term instead of Euler */
    int64_t chunk;      /* chunked path only */
    int tree;           /* chunked path only: 1 = balanced tree, 0 = left fold */
} scan_args;

typedef struct {
    const scan_args *a;
    int worker, n_workers;
    int chunked;
    int status;
} worker_args;

static double step_size(const scan_args *a, int64_t d, double raw) {
    double x = raw + (a->delta_bias ? a->delta_bias[d] : 0.0);
    return a->softplus_flag ? softplus(x) : x;
}

/* Run tokens [t0, t1) of row (b, d) starting from state h (updated in
 * place).  Writes y for those tokens when y_row is not NULL. */
static void run_tokens(const scan_args *a, int64_t b, int64_t d, int64_t t0, int64_t t1,
                       double *h, double *y_row) {
    const int64_t N = a->d_state, L = a->seqlen;
    const int64_t row = (b * a->d_inner + d) * L;
    for (int64_t t = t0; t < t1; ++t) {
        const double u = a->u[row + t];
        const double dt = step_size(a, d, a->delta[row + t]);
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double dA = exp(dt * a->A[d * N + n]);
            const double dBu = input_coeff(dt, a->A[d * N + n], a->zoh) *
                               a->B[(b * N + n) * L + t] * u;
            h[n] = dA * h[n] + dBu;
            acc += a->C[(b * N + n) * L + t] * h[n];
        }
        if (!y_row) continue;
        if (a->D) acc += a->D[d] * u;
        if (a->z) acc *= silu(a->z[row + t]);
        y_row[t] = acc;
    }
}

static void init_state(const scan_args *a, int64_t b, int64_t d, double *h) {
    const int64_t N = a->d_state;
    for (int64_t n = 0; n < N; ++n)
        h[n] = a->h0 ? a->h0[(b * a->d_inner + d) * N + n] : 0.0;
}

static void store_state(const scan_args *a, int64_t b, int64_t d, const double *h) {
    if (!a->last_state) return;
    const int64_t N = a->d_state;
    memcpy(a->last_state + (b * a->d_inner + d) * N, h, (size_t)N * sizeof(double));
}

/* ------------------------------------------------------------ sequential */

static int scan_row_sequential(const scan_args *a, int64_t b, int64_t d, double *h) {
    init_state(a, b, d, h);
    run_tokens(a, b, d, 0, a->seqlen, h, a->y + (b * a->d_inner + d) * a->seqlen);
    store_state(a, b, d, h);
    return 0;
}

/* ------------------------------------------------------------ chunked */

/* Transfer operator of a token range: h_end = op.a (elementwise) h_start + op.b.
 * compose(first, second) applies `first`, then `second`:
 *   (a2, b2) o (a1, b1) = (a1 a2, a2 b1 + b2)                                */
static void compose(const double *a1, const double *b1, const double *a2, const double *b2,
                    double *ao, double *bo, int64_t N) {
    for (int64_t n = 0; n < N; ++n) {
        const double a = a1[n] * a2[n];
        const double bb = a2[n] * b1[n] + b2[n];
        ao[n] = a;
        bo[n] = bb;
    }
}

static int scan_row_chunked(const scan_args *a, int64_t b, int64_t d, double *h) {
    const int64_t N = a->d_state, L = a->seqlen, K = a->chunk;
    const int64_t nc = (L + K - 1) / K;
    int64_t P = 1;
    while (P < nc) P <<= 1;
    /* opa/opb: per-chunk operators, padded to a power of two with identity. */
    double *opa = malloc(sizeof(double) * (size_t)(P * N));
    double *opb = malloc(sizeof(double) * (size_t)(P * N));
    double *ta = malloc(sizeof(double) * (size_t)N);
    double *tb = malloc(sizeof(double) * (size_t)N);
    if (!opa || !opb || !ta || !tb) {
        free(opa); free(opb); free(ta); free(tb);
        return -1;
    }
    const int64_t row = (b * a->d_inner + d) * L;

    /* 1. Local scan of each chunk from a zero state: B_chunk is the state it
     *    ends in, A_chunk is the product of its decays. */
    for (int64_t k = 0; k < P; ++k) {
        double *ka = opa + k * N, *kb = opb + k * N;
        for (int64_t n = 0; n < N; ++n) { ka[n] = 1.0; kb[n] = 0.0; }
        if (k >= nc) continue;
        const int64_t t1 = (k + 1) * K < L ? (k + 1) * K : L;
        for (int64_t t = k * K; t < t1; ++t) {
            const double u = a->u[row + t];
            const double dt = step_size(a, d, a->delta[row + t]);
            for (int64_t n = 0; n < N; ++n) {
                const double dA = exp(dt * a->A[d * N + n]);
                ka[n] *= dA;
                kb[n] = dA * kb[n] + input_coeff(dt, a->A[d * N + n], a->zoh) *
                                         a->B[(b * N + n) * L + t] * u;
            }
        }
    }

    /* 2. Exclusive prefix of the operators: slot k receives the composition
     *    of chunks 0..k-1 (identity for chunk 0). */
    if (a->tree) {
        /* Balanced tree: up-sweep builds subtree totals, down-sweep hands
         * every left subtree the prefix of its parent and every right subtree
         * that prefix followed by its left sibling's total. */
        for (int64_t s = 1; s < P; s <<= 1)
            for (int64_t i = 0; i + 2 * s - 1 < P; i += 2 * s) {
                const int64_t l = i + s - 1, r = i + 2 * s - 1;
                compose(opa + l * N, opb + l * N, opa + r * N, opb + r * N,
                        opa + r * N, opb + r * N, N);
            }
        for (int64_t n = 0; n < N; ++n) { opa[(P - 1) * N + n] = 1.0; opb[(P - 1) * N + n] = 0.0; }
        for (int64_t s = P >> 1; s >= 1; s >>= 1)
            for (int64_t i = 0; i + 2 * s - 1 < P; i += 2 * s) {
                const int64_t l = i + s - 1, r = i + 2 * s - 1;
                memcpy(ta, opa + l * N, sizeof(double) * (size_t)N);
                memcpy(tb, opb + l * N, sizeof(double) * (size_t)N);
                memcpy(opa + l * N, opa + r * N, sizeof(double) * (size_t)N);
                memcpy(opb + l * N, opb + r * N, sizeof(double) * (size_t)N);
                compose(opa + r * N, opb + r * N, ta, tb, opa + r * N, opb + r * N, N);
            }
    } else {
        /* Left fold. */
        double *ra = ta, *rb = tb;
        for (int64_t n = 0; n < N; ++n) { ra[n] = 1.0; rb[n] = 0.0; }
        for (int64_t k = 0; k < nc; ++k) {
            double *ka = opa + k * N, *kb = opb + k * N;
            for (int64_t n = 0; n < N; ++n) {
                const double na = ra[n] * ka[n];
                const double nb = ka[n] * rb[n] + kb[n];
                ka[n] = ra[n]; kb[n] = rb[n];   /* exclusive prefix */
                ra[n] = na; rb[n] = nb;
            }
        }
    }

    /* 3. Broadcast h_start = prefix applied to the initial state and re-run
     *    every chunk from it, producing y. */
    double *y_row = a->y + row;
    init_state(a, b, d, ta);   /* ta now holds the initial state */
    for (int64_t k = 0; k < nc; ++k) {
        for (int64_t n = 0; n < N; ++n) h[n] = opa[k * N + n] * ta[n] + opb[k * N + n];
        const int64_t t1 = (k + 1) * K < L ? (k + 1) * K : L;
        run_tokens(a, b, d, k * K, t1, h, y_row);
    }
    store_state(a, b, d, h);
    free(opa); free(opb); free(ta); free(tb);
    return 0;
}

/* ------------------------------------------------------------ threading */

static void *worker_main(void *p) {
    worker_args *w = (worker_args *)p;
    const scan_args *a = w->a;
    double *h = malloc(sizeof(double) * (size_t)(a->d_state > 0 ? a->d_state : 1));
    if (!h) { w->status = -1; return NULL; }
    const int64_t rows = a->batch * a->d_inner;
    for (int64_t r = w->worker; r < rows; r += w->n_workers) {
        const int64_t b = r / a->d_inner, d = r % a->d_inner;
        const int s = w->chunked ? scan_row_chunked(a, b, d, h) : scan_row_sequential(a, b, d, h);
        if (s) { w->status = s; break; }
    }
    free(h);
    return NULL;
}

static int run_rows(const scan_args *a, int chunked, int n_threads) {
    const int64_t rows = a->batch * a->d_inner;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > rows) n_threads = (int)(rows > 0 ? rows : 1);
    pthread_t *tid = malloc(sizeof(pthread_t) * (size_t)n_threads);
    worker_args *wa = malloc(sizeof(worker_args) * (size_t)n_threads);
    if (!tid || !wa) { free(tid); free(wa); return -1; }
    int started = 0, status = 0;
    for (int i = 0; i < n_threads; ++i) {
        wa[i] = (worker_args){a, i, n_threads, chunked, 0};
        if (i == 0) continue;
        if (pthread_create(&tid[i], NULL, worker_main, &wa[i]) != 0) { status = -1; break; }
        started = i;
    }
    if (status == 0) {
        worker_main(&wa[0]);
    }
    for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
    for (int i = 0; i < n_threads && status == 0; ++i) status = wa[i].status;
    free(tid); free(wa);
    return status;
}

static int check_dims(int64_t batch, int64_t d_inner, int64_t d_state, int64_t seqlen) {
    return batch >= 0 && d_inner >= 0 && d_state >= 1 && seqlen >= 0;
}

/* ------------------------------------------------------------ backward */

/* Gradients of the loss  sum_t dy_t y_t + sum_n dlast_n h_{L-1,n}  (dy and
 * dlast are the upstream gradients of y and last_state) with respect to every
 * input of the Euler scan, by reverse-mode differentiation of the recurrence
 * written out by hand -- the backward step the ufo.work article, §2.2, pairs
 * with the fused forward (recompute the states, then walk back).  For one
 * row (b, d), with x_t = delta_raw_t + bias, dt_t = softplus(x_t) (or x_t),
 * a_t = exp(dt_t A), c_t the input factor (dt_t, or (a_t - 1) / A with
 * zero-order hold) with derivatives c' (by dt) and c^A (by A),
 * o_t = C_t . h_t + D u_t and g_t = silu(z_t) (or 1), walking
 * t = L-1 .. 0 with G = dlast:
 *   do_t   = dy_t g_t                      dz_t  = dy_t o_t silu'(z_t)
 *   dh_t   = G + do_t C_t                  dC_t += do_t h_t,  dB_t += c_t u_t dh_t
 *   da_t   = dh_t h_{t-1}   (h_{-1} = h0)  du_t  = do_t D + sum_n dh_t B_t c_t
 *   ddt_t  = sum_n (da_t A a_t + dh_t B_t u_t c'_t)
 *   dA    += da_t a_t dt_t + dh_t B_t u_t c^A_t          dD += do_t u_t
 *   G      = dh_t a_t                      ddelta_t = ddt_t softplus'(x_t)
 *   dbias += ddelta_t;    finally dh0 = G.
 * (Euler: c = dt, c' = 1, c^A = 0.)
 * dB and dC sum over the channels of a batch row, dA, dD and dbias over the
 * batch rows (and tokens): per-thread partial buffers added in a fixed order. */
typedef struct {
    const scan_args *a;
    const double *dy, *dlast;
    double *du, *ddelta, *dz, *dh0;
    double *dA_rows, *dD_rows, *dbias_rows;   /* (batch, d_inner, N) / (batch, d_inner) */
    double *dB_part, *dC_part;                /* per worker: (batch, N, L) */
    int worker, n_workers, status;
} bwd_worker;

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static void *bwd_main(void *p) {
    bwd_worker *w = (bwd_worker *)p;
    const scan_args *a = w->a;
    const int64_t N = a->d_state, L = a->seqlen, Dn = a->d_inner;
    double *hs = malloc(sizeof(double) * (size_t)((L + 1) * N));   /* h_{-1} .. h_{L-1} */
    double *G = malloc(sizeof(double) * (size_t)N);
    double *dh = malloc(sizeof(double) * (size_t)N);
    double *dBp = w->dB_part + (size_t)w->worker * (size_t)(a->batch * N * L);
    double *dCp = w->dC_part + (size_t)w->worker * (size_t)(a->batch * N * L);
    if (!hs || !G || !dh) { free(hs); free(G); free(dh); w->status = -1; return NULL; }
    for (int64_t r = w->worker; r < a->batch * Dn; r += w->n_workers) {
        const int64_t b = r / Dn, d = r % Dn;
        const int64_t row = (b * Dn + d) * L;
        /* forward, keeping every state */
        for (int64_t n = 0; n < N; ++n) hs[n] = a->h0 ? a->h0[(b * Dn + d) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double dt = step_size(a, d, a->delta[row + t]), u = a->u[row + t];
            for (int64_t n = 0; n < N; ++n)
                hs[(t + 1) * N + n] = exp(dt * a->A[d * N + n]) * hs[t * N + n] +
                                      input_coeff(dt, a->A[d * N + n], a->zoh) *
                                          a->B[(b * N + n) * L + t] * u;
        }
        /* backward */
        for (int64_t n = 0; n < N; ++n) G[n] = w->dlast ? w->dlast[(b * Dn + d) * N + n] : 0.0;
        double dD_acc = 0.0, dbias_acc = 0.0;
        double *dA_row = w->dA_rows + (b * Dn + d) * N;
        for (int64_t n = 0; n < N; ++n) dA_row[n] = 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            const double x = a->delta[row + t] + (a->delta_bias ? a->delta_bias[d] : 0.0);
            const double dt = a->softplus_flag ? softplus(x) : x;
            const double u = a->u[row + t];
            const double *ht = hs + (t + 1) * N, *hp = hs + t * N;
            double o = 0.0;
            for (int64_t n = 0; n < N; ++n) o += a->C[(b * N + n) * L + t] * ht[n];
            if (a->D) o += a->D[d] * u;
            double g = 1.0;
            if (a->z) {
                const double zt = a->z[row + t], sg = sigmoid(zt);
                g = zt * sg;
                w->dz[row + t] = w->dy[row + t] * o * sg * (1.0 + zt * (1.0 - sg));
            }
            const double dO = w->dy[row + t] * g;
            dD_acc += dO * u;
            double dux = 0.0, ddt = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double Bn = a->B[(b * N + n) * L + t], Cn = a->C[(b * N + n) * L + t];
                const double An = a->A[d * N + n], at = exp(dt * An);
                const double c = input_coeff(dt, An, a->zoh);
                dh[n] = G[n] + dO * Cn;
                dCp[(b * N + n) * L + t] += dO * ht[n];
                dBp[(b * N + n) * L + t] += c * u * dh[n];
                dux += dh[n] * Bn * c;
                const double da = dh[n] * hp[n];
                ddt += da * An * at + dh[n] * Bn * u * input_coeff_ddt(dt, An, a->zoh);
                dA_row[n] += da * at * dt + dh[n] * Bn * u * input_coeff_dA(dt, An, a->zoh);
                G[n] = dh[n] * at;
            }
            w->du[row + t] = dO * (a->D ? a->D[d] : 0.0) + dux;
            const double dx = a->softplus_flag ? ddt * sigmoid(x) : ddt;
            w->ddelta[row + t] = dx;
            dbias_acc += dx;
        }
        for (int64_t n = 0; n < N; ++n) w->dh0[(b * Dn + d) * N + n] = G[n];
        w->dD_rows[b * Dn + d] = dD_acc;
        w->dbias_rows[b * Dn + d] = dbias_acc;
    }
    free(hs); free(G); free(dh);
    return NULL;
}

int oracle_scan_bwd(int64_t batch, int64_t d_inner, int64_t d_state, int64_t seqlen,
                    const double *u, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *delta_bias,
                    int softplus_flag, const double *initial_state, const double *dy,
                    const double *dlast, double *du, double *ddelta, double *dA, double *dB,
                    double *dC, double *dD, double *dz, double *ddelta_bias, double *dh0,
                    int n_threads, int zoh) {
    if (!check_dims(batch, d_inner, d_state, seqlen)) return -1;
    if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC || !dD ||
        !ddelta_bias || !dh0 || (z && !dz))
        return -1;
    const int64_t N = d_state, L = seqlen, rows = batch * d_inner;
    scan_args a = {batch, d_inner, d_state, seqlen, u, delta, A, B, C, D, z, delta_bias,
                   initial_state, softplus_flag, NULL, NULL, zoh != 0, 0, 0};
    if (n_threads < 1) n_threads = 1;
    if (n_threads > rows) n_threads = (int)(rows > 0 ? rows : 1);
    const size_t part = (size_t)(batch * N * L);
    double *dBp = calloc((size_t)n_threads * part + 1, sizeof(double));
    double *dCp = calloc((size_t)n_threads * part + 1, sizeof(double));
    double *dA_rows = calloc((size_t)(rows * N) + 1, sizeof(double));
    double *dD_rows = calloc((size_t)rows + 1, sizeof(double));
    double *db_rows = calloc((size_t)rows + 1, sizeof(double));
    pthread_t *tid = malloc(sizeof(pthread_t) * (size_t)n_threads);
    bwd_worker *wk = malloc(sizeof(bwd_worker) * (size_t)n_threads);
    int status = 0;
    if (!dBp || !dCp || !dA_rows || !dD_rows || !db_rows || !tid || !wk) status = -1;
    int started = 0;
    for (int i = 0; i < n_threads && status == 0; ++i) {
        wk[i] = (bwd_worker){&a, dy, dlast, du, ddelta, dz, dh0, dA_rows, dD_rows, db_rows,
                             dBp, dCp, i, n_threads, 0};
        if (i == 0) continue;
        if (pthread_create(&tid[i], NULL, bwd_main, &wk[i]) != 0) { status = -1; break; }
        started = i;
    }
    if (status == 0) bwd_main(&wk[0]);
    for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
    for (int i = 0; i < n_threads && status == 0; ++i) status = wk[i].status;
    if (status == 0) {
        /* fixed-order reductions */
        for (size_t k = 0; k < part; ++k) {
            double sb = 0.0, sc = 0.0;
            for (int i = 0; i < n_threads; ++i) { sb += dBp[(size_t)i * part + k]; sc += dCp[(size_t)i * part + k]; }
            dB[k] = sb; dC[k] = sc;
        }
        for (int64_t d = 0; d < d_inner; ++d) {
            double sD = 0.0, sb = 0.0;
            for (int64_t b = 0; b < batch; ++b) { sD += dD_rows[b * d_inner + d]; sb += db_rows[b * d_inner + d]; }
            dD[d] = sD; ddelta_bias[d] = sb;
            for (int64_t n = 0; n < N; ++n) {
                double s = 0.0;
                for (int64_t b = 0; b < batch; ++b) s += dA_rows[(b * d_inner + d) * N + n];
                dA[d * N + n] = s;
            }
        }
    }
    free(dBp); free(dCp); free(dA_rows); free(dD_rows); free(db_rows); free(tid); free(wk);
    return status;
}

/* ------------------------------------------------------------ exports */

int oracle_scan_fwd(int64_t batch, int64_t d_inner, int64_t d_state, int64_t seqlen,
                    const double *u, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *delta_bias,
                    int softplus_flag, const double *initial_state, double *y,
                    double *last_state, int zoh, int n_threads) {
    if (!check_dims(batch, d_inner, d_state, seqlen)) return -1;
    if (batch * d_inner == 0) return 0;
    if (!u || !delta || !A || !B || !C || !y) return -1;
    scan_args a = {batch, d_inner, d_state, seqlen, u, delta, A, B, C, D, z, delta_bias,
                   initial_state, softplus_flag, y, last_state, zoh, 0, 0};
    return run_rows(&a, 0, n_threads);
}

int oracle_scan_chunked(int64_t batch, int64_t d_inner, int64_t d_state, int64_t seqlen,
                        const double *u, const double *delta, const double *A, const double *B,
                        const double *C, const double *D, const double *z,
                        const double *delta_bias, int softplus_flag,
                        const double *initial_state, double *y, double *last_state,
                        int zoh, int64_t chunk, int tree_combine, int n_threads) {
    if (!check_dims(batch, d_inner, d_state, seqlen) || chunk < 1) return -1;
    if (batch * d_inner == 0) return 0;
    if (!u || !delta || !A || !B || !C || !y) return -1;
    scan_args a = {batch, d_inner, d_state, seqlen, u, delta, A, B, C, D, z, delta_bias,
                   initial_state, softplus_flag, y, last_state, zoh, chunk,
                   tree_combine ? 1 : 0};
    return run_rows(&a, 1, n_threads);
}

int oracle_state_update(int64_t batch, int64_t d_inner, int64_t d_state, double *state,
                        const double *u, const double *delta, const double *A, const double *B,
                        const double *C, const double *D, const double *z, double *y, int zoh) {
    if (batch < 0 || d_inner < 0 || d_state < 1) return -1;
    if (batch * d_inner == 0) return 0;
    if (!state || !u || !delta || !A || !B || !C || !y) return -1;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < d_inner; ++d) {
            const int64_t i = b * d_inner + d;
            const double dt = delta[i], x = u[i];
            double *s = state + i * d_state;
            double acc = 0.0;
            for (int64_t n = 0; n < d_state; ++n) {
                const double An = A[d * d_state + n];
                s[n] = exp(dt * An) * s[n] + input_coeff(dt, An, zoh) * B[b * d_state + n] * x;
                acc += C[b * d_state + n] * s[n];
            }
            if (D) acc += D[d] * x;
            if (z) acc *= silu(z[i]);
            y[i] = acc;
        }
    return 0;
}
