/*
 * CPU oracle for the Mamba-2 SSD chunked scan: TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library.  The product path (the HIP library) never calls it, and
 * the two share no code, headers or constants.
 *
 * What it computes (plain definitions, fp64, single-threaded, no blocking):
 *
 *   forward   h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t
 *             y_t = C_t . h_t + D_h * x_t            (h_{-1} = initial state)
 *   backward  the reverse-mode recurrence of that forward (the adjoint G_t of
 *             h_t runs backwards in time), giving d_x, d_dt, d_B, d_C, d_D,
 *             d_A and d_initial_state.
 *   moments   m2 = sum_t h_t^T h_t, m1 = sum_t sum_p h_t[p,:] over the valid
 *             tokens, and their reverse-mode gradient.
 *   PR        the participation ratio (tr S)^2 / ||S||_F^2 of S = m2 / count
 *             (optionally centred), the raw trace tr(m2) / count, and the PR's
 *             gradient with respect to m2 and m1.
 *   y_diag    the gamma-weighted same-step correction of the Mamba-3 SSD
 *             (per token and head: gamma * (C B^T) V over the mimo axis) and its
 *             reverse-mode gradient.
 *   quat scan the quaternion cumulative product cum[t] = q_t (x) cum[t-1] of the
 *             Mamba-3 rotation and its exact reverse-mode gradient.
 *
 * The chunked SSD of the burn-mamba "combined_backward.rs" page (kernels K1-K5
 * and the recompute backward) is a re-association of exactly this recurrence:
 * its K1 inclusive cumsum of dt*A makes exp(cumA[t]) the product of the
 * per-token decays, K3/K4 carry h across chunk ends and K5's BLUE and ORANGE
 * terms are C_t . h_t split into the carried-in and the in-chunk parts.  The
 * oracle therefore evaluates the recurrence token by token and never chunks.
 *
 * The moments follow the burn-mamba "state_moments.rs" page (StateMoments:
 * m2 is the Gram sum pooling the per_head_dim rows, m1 the row sum, count =
 * valid tokens * per_head_dim), and their gradient the per-token cotangent of
 * the "moments/backward" module page (Gradient math, first bullet) with no
 * rotation: d_h_t += mask_t * (h_t (d_m2 + d_m2^T) + 1_p (outer) d_m1).
 *
 * Layouts (row-major, the pages' tensor naming):
 *   x, dy, y, d_x      [batch, nchunks, chunk_len, nheads, headdim]
 *   B, C, d_B, d_C     [batch, nchunks, chunk_len, nheads, dstate]
 *   dt, d_dt           [batch, nheads, nchunks, chunk_len]
 *   A, D, d_A, d_D     [nheads]
 *   init, final, d_*   [batch, nheads, headdim, dstate]
 *   m2 / m1            [batch, nheads, dstate, dstate] / [batch, nheads, dstate]
 * With seq = nchunks * chunk_len and t = chunk * chunk_len + position, the
 * token (b, t, h) of x sits at ((b * seq + t) * nheads + h) * headdim and its
 * dt at (b * nheads + h) * seq + t.
 *
 * Every entry point returns 0 on success, -1 on a bad argument (null pointer
 * or non-positive size; nchunks == 0 is allowed and means an empty sequence)
 * and -2 when memory for the backward's checkpoints cannot be had.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t batch, nchunks, chunk_len, nheads, headdim, dstate;
} oracle_dims;

static int dims_ok(const oracle_dims* d) {
    if (!d) return 0;
    if (d->batch < 0 || d->nchunks < 0 || d->chunk_len <= 0 || d->nheads <= 0 ||
        d->headdim <= 0 || d->dstate <= 0)
        return 0;
    return 1;
}

/* offsets of token t of (b, h) */
static int64_t off_tok(const oracle_dims* d, int64_t b, int64_t t, int64_t h, int64_t width) {
    int64_t seq = d->nchunks * d->chunk_len;
    return ((b * seq + t) * d->nheads + h) * width;
}
static int64_t off_dt(const oracle_dims* d, int64_t b, int64_t h, int64_t t) {
    int64_t seq = d->nchunks * d->chunk_len;
    return (b * d->nheads + h) * seq + t;
}

/* h <- a*h + dt * x (outer) B   (one token of the recurrence) */
static void state_step(double* H, int64_t P, int64_t R, double a, double dtv,
                       const double* xt, const double* Bt) {
    for (int64_t p = 0; p < P; ++p) {
        double s = dtv * xt[p];
        double* row = H + p * R;
        for (int64_t r = 0; r < R; ++r) row[r] = a * row[r] + s * Bt[r];
    }
}

/* ---------------------------------------------------------------- forward */
int oracle_ssd_fwd(const oracle_dims* d, const double* x, const double* dt,
                   const double* A, const double* B, const double* C,
                   const double* D, const double* init, double* y,
                   double* final_state) {
    if (!dims_ok(d) || !x || !dt || !A || !B || !C || !D || !y) return -1;
    const int64_t P = d->headdim, R = d->dstate, Hn = d->nheads;
    const int64_t seq = d->nchunks * d->chunk_len;
    double* H = (double*)malloc(sizeof(double) * P * R);
    if (!H) return -2;
    for (int64_t b = 0; b < d->batch; ++b) {
        for (int64_t h = 0; h < Hn; ++h) {
            const int64_t so = (b * Hn + h) * P * R;
            for (int64_t i = 0; i < P * R; ++i) H[i] = init ? init[so + i] : 0.0;
            for (int64_t t = 0; t < seq; ++t) {
                const double dtv = dt[off_dt(d, b, h, t)];
                const double a = exp(dtv * A[h]);
                const double* xt = x + off_tok(d, b, t, h, P);
                const double* Bt = B + off_tok(d, b, t, h, R);
                const double* Ct = C + off_tok(d, b, t, h, R);
                double* yt = y + off_tok(d, b, t, h, P);
                state_step(H, P, R, a, dtv, xt, Bt);
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t r = 0; r < R; ++r) acc += H[p * R + r] * Ct[r];
                    yt[p] = acc + D[h] * xt[p];
                }
            }
            if (final_state)
                memcpy(final_state + so, H, sizeof(double) * P * R);
        }
    }
    free(H);
    return 0;
}

/*
 * Shared reverse sweep for the SSD backward (mode 0) and the moments backward
 * (mode 1).  For one (b, h) slice it replays the forward in segments of `seg`
 * tokens from stored checkpoints (the state before each segment) and walks each
 * segment backwards with the adjoint G of the current state h_t:
 *
 *   inject   mode 0: G += dy_t (outer) C_t
 *            mode 1: G += mask_t * (h_t S + 1 (outer) d_m1),  S = d_m2 + d_m2^T
 *   d_C_t    = h_t^T dy_t                          (mode 0 only)
 *   d_D     += dy_t . x_t                          (mode 0 only)
 *   d_x_t    = D dy_t + dt_t G B_t                 (D dy_t only in mode 0)
 *   d_B_t    = dt_t G^T x_t
 *   q        = a_t <G, h_{t-1}>,  a_t = exp(dt_t A)
 *   d_dt_t   = <G, x_t (outer) B_t> + A q
 *   d_A     += dt_t q
 *   G       <- a_t G                               (now the adjoint of h_{t-1})
 *
 * After t = 0, G is the gradient of the initial state.
 */
typedef struct {
    int mode;
    const double* dy;   /* mode 0 */
    const double* C;    /* mode 0 */
    const double* D;    /* mode 0 */
    const double* S;    /* mode 1: [R,R] symmetric d_m2 + d_m2^T of this slice */
    const double* dm1;  /* mode 1: [R] or NULL */
    int64_t valid;      /* mode 1: tokens t < valid carry moments */
} sweep_ctx;

static int reverse_sweep(const oracle_dims* d, int64_t b, int64_t h, const sweep_ctx* c,
                         const double* x, const double* dt, const double* A,
                         const double* B, const double* init, const double* G0,
                         double* d_x, double* d_dt, double* d_A_acc, double* d_B,
                         double* d_C, double* d_D_acc, double* d_init, int64_t seg) {
    const int64_t P = d->headdim, R = d->dstate, PR = P * R;
    const int64_t seq = d->nchunks * d->chunk_len;
    const int64_t so = (b * d->nheads + h) * PR;
    const double Ah = A[h];
    if (seg <= 0) seg = 256;
    const int64_t nseg = seq > 0 ? (seq + seg - 1) / seg : 0;
    double* ck = (double*)malloc(sizeof(double) * PR * (nseg > 0 ? nseg : 1));
    double* buf = (double*)malloc(sizeof(double) * PR * (seg + 1));
    double* G = (double*)malloc(sizeof(double) * PR);
    double* tmp = (double*)malloc(sizeof(double) * PR);
    if (!ck || !buf || !G || !tmp) {
        free(ck); free(buf); free(G); free(tmp);
        return -2;
    }
    /* forward pass: checkpoint the state before every segment */
    for (int64_t i = 0; i < PR; ++i) tmp[i] = init ? init[so + i] : 0.0;
    for (int64_t t = 0; t < seq; ++t) {
        if (t % seg == 0) memcpy(ck + (t / seg) * PR, tmp, sizeof(double) * PR);
        const double dtv = dt[off_dt(d, b, h, t)];
        state_step(tmp, P, R, exp(dtv * Ah), dtv, x + off_tok(d, b, t, h, P),
                   B + off_tok(d, b, t, h, R));
    }
    for (int64_t i = 0; i < PR; ++i) G[i] = G0 ? G0[so + i] : 0.0;

    for (int64_t sg = nseg - 1; sg >= 0; --sg) {
        const int64_t t0 = sg * seg;
        const int64_t t1 = (t0 + seg < seq) ? t0 + seg : seq;
        /* replay the segment: buf[k] = state before token t0 + k */
        memcpy(buf, ck + sg * PR, sizeof(double) * PR);
        for (int64_t t = t0; t < t1; ++t) {
            double* nx = buf + (t - t0 + 1) * PR;
            memcpy(nx, buf + (t - t0) * PR, sizeof(double) * PR);
            const double dtv = dt[off_dt(d, b, h, t)];
            state_step(nx, P, R, exp(dtv * Ah), dtv, x + off_tok(d, b, t, h, P),
                       B + off_tok(d, b, t, h, R));
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double* Ht = buf + (t - t0 + 1) * PR;
            const double* Hp = buf + (t - t0) * PR;
            const double dtv = dt[off_dt(d, b, h, t)];
            const double a = exp(dtv * Ah);
            const double* xt = x + off_tok(d, b, t, h, P);
            const double* Bt = B + off_tok(d, b, t, h, R);
            double* dxt = d_x + off_tok(d, b, t, h, P);
            double* dBt = d_B + off_tok(d, b, t, h, R);

            if (c->mode == 0) {
                const double* dyt = c->dy + off_tok(d, b, t, h, P);
                const double* Ct = c->C + off_tok(d, b, t, h, R);
                double* dCt = d_C + off_tok(d, b, t, h, R);
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t r = 0; r < R; ++r) G[p * R + r] += dyt[p] * Ct[r];
                for (int64_t r = 0; r < R; ++r) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) acc += dyt[p] * Ht[p * R + r];
                    dCt[r] = acc;
                }
                double dd = 0.0;
                for (int64_t p = 0; p < P; ++p) dd += dyt[p] * xt[p];
                *d_D_acc += dd;
                for (int64_t p = 0; p < P; ++p) dxt[p] = c->D[h] * dyt[p];
            } else {
                if (t < c->valid) {
                    for (int64_t p = 0; p < P; ++p) {
                        const double* hrow = Ht + p * R;
                        for (int64_t r = 0; r < R; ++r) {
                            double acc = c->dm1 ? c->dm1[r] : 0.0;
                            for (int64_t k = 0; k < R; ++k) acc += hrow[k] * c->S[k * R + r];
                            G[p * R + r] += acc;
                        }
                    }
                }
                for (int64_t p = 0; p < P; ++p) dxt[p] = 0.0;
            }
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t r = 0; r < R; ++r) acc += G[p * R + r] * Bt[r];
                dxt[p] += dtv * acc;
            }
            for (int64_t r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int64_t p = 0; p < P; ++p) acc += G[p * R + r] * xt[p];
                dBt[r] = dtv * acc;
            }
            double gh = 0.0, gw = 0.0;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t r = 0; r < R; ++r) {
                    gh += G[p * R + r] * Hp[p * R + r];
                    gw += G[p * R + r] * xt[p] * Bt[r];
                }
            const double q = a * gh;
            d_dt[off_dt(d, b, h, t)] = gw + Ah * q;
            *d_A_acc += dtv * q;
            for (int64_t i = 0; i < PR; ++i) G[i] *= a;
        }
    }
    if (d_init) memcpy(d_init + so, G, sizeof(double) * PR);
    free(ck); free(buf); free(G); free(tmp);
    return 0;
}

/* --------------------------------------------------------------- backward */
int oracle_ssd_bwd(const oracle_dims* d, const double* dy, const double* d_final,
                   const double* x, const double* dt, const double* A,
                   const double* B, const double* C, const double* D,
                   const double* init, double* d_x, double* d_dt, double* d_A,
                   double* d_B, double* d_C, double* d_D, double* d_init,
                   int64_t seg) {
    if (!dims_ok(d) || !dy || !x || !dt || !A || !B || !C || !D || !d_x || !d_dt ||
        !d_A || !d_B || !d_C || !d_D)
        return -1;
    sweep_ctx c;
    memset(&c, 0, sizeof c);
    c.mode = 0;
    c.dy = dy;
    c.C = C;
    c.D = D;
    for (int64_t h = 0; h < d->nheads; ++h) { d_A[h] = 0.0; d_D[h] = 0.0; }
    for (int64_t h = 0; h < d->nheads; ++h) {
        for (int64_t b = 0; b < d->batch; ++b) {
            int rc = reverse_sweep(d, b, h, &c, x, dt, A, B, init, d_final, d_x, d_dt,
                                   &d_A[h], d_B, d_C, &d_D[h], d_init, seg);
            if (rc) return rc;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- moments */
int oracle_state_moments(const oracle_dims* d, const double* x, const double* dt,
                         const double* A, const double* B, const double* init,
                         const int64_t* valid_len, double* m2, double* m1,
                         int64_t* count) {
    if (!dims_ok(d) || !x || !dt || !A || !B || !m2 || !m1 || !count) return -1;
    const int64_t P = d->headdim, R = d->dstate, Hn = d->nheads;
    const int64_t seq = d->nchunks * d->chunk_len;
    double* H = (double*)malloc(sizeof(double) * P * R);
    if (!H) return -2;
    for (int64_t b = 0; b < d->batch; ++b) {
        int64_t v = valid_len ? valid_len[b] : seq;
        if (v < 0 || v > seq) { free(H); return -1; }
        count[b] = v * P;
        for (int64_t h = 0; h < Hn; ++h) {
            const int64_t so = (b * Hn + h) * P * R;
            double* M2 = m2 + (b * Hn + h) * R * R;
            double* M1 = m1 + (b * Hn + h) * R;
            for (int64_t i = 0; i < R * R; ++i) M2[i] = 0.0;
            for (int64_t i = 0; i < R; ++i) M1[i] = 0.0;
            for (int64_t i = 0; i < P * R; ++i) H[i] = init ? init[so + i] : 0.0;
            for (int64_t t = 0; t < v; ++t) {
                const double dtv = dt[off_dt(d, b, h, t)];
                state_step(H, P, R, exp(dtv * A[h]), dtv, x + off_tok(d, b, t, h, P),
                           B + off_tok(d, b, t, h, R));
                for (int64_t p = 0; p < P; ++p) {
                    const double* row = H + p * R;
                    for (int64_t r1 = 0; r1 < R; ++r1) {
                        M1[r1] += row[r1];
                        for (int64_t r2 = 0; r2 < R; ++r2) M2[r1 * R + r2] += row[r1] * row[r2];
                    }
                }
            }
        }
    }
    free(H);
    return 0;
}

int oracle_state_moments_bwd(const oracle_dims* d, const double* d_m2,
                             const double* d_m1, const double* x, const double* dt,
                             const double* A, const double* B, const double* init,
                             const int64_t* valid_len, double* d_x, double* d_dt,
                             double* d_A, double* d_B, double* d_init, int64_t seg) {
    if (!dims_ok(d) || !d_m2 || !x || !dt || !A || !B || !d_x || !d_dt || !d_A || !d_B)
        return -1;
    const int64_t R = d->dstate, Hn = d->nheads;
    const int64_t seq = d->nchunks * d->chunk_len;
    double* S = (double*)malloc(sizeof(double) * R * R);
    if (!S) return -2;
    for (int64_t h = 0; h < Hn; ++h) d_A[h] = 0.0;
    for (int64_t h = 0; h < Hn; ++h) {
        for (int64_t b = 0; b < d->batch; ++b) {
            const double* dm2 = d_m2 + (b * Hn + h) * R * R;
            for (int64_t i = 0; i < R; ++i)
                for (int64_t j = 0; j < R; ++j) S[i * R + j] = dm2[i * R + j] + dm2[j * R + i];
            sweep_ctx c;
            memset(&c, 0, sizeof c);
            c.mode = 1;
            c.S = S;
            c.dm1 = d_m1 ? d_m1 + (b * Hn + h) * R : NULL;
            c.valid = valid_len ? valid_len[b] : seq;
            if (c.valid < 0 || c.valid > seq) { free(S); return -1; }
            double unused = 0.0;
            int rc = reverse_sweep(d, b, h, &c, x, dt, A, B, init, NULL, d_x, d_dt, &d_A[h],
                                   d_B, NULL, &unused, d_init, seg);
            if (rc) { free(S); return rc; }
        }
    }
    free(S);
    return 0;
}

/* ------------------------------------------------------- participation ratio
 * StateMoments::pr of the burn-mamba "state_moments.rs" page, per (batch, head):
 *   Sigma     = m2 / count            (centred: minus mu mu^T, mu = m1 / count)
 *   s         = max(tr Sigma, min_positive)          (held fixed for the gradient)
 *   Sigma_hat = Sigma / s
 *   PR        = tr(Sigma_hat)^2 / max(||Sigma_hat||_F^2, div_eps)
 * and StateMoments::trace = tr(m2) / count.  The floors are the page's fp32 ones:
 * min_positive = 2^-126 (fp32's smallest normal) and div_eps = 1e-12 (the value
 * the page's trace() documentation gives for PR's denominator clamp).  count is
 * per batch row here; every count must be positive (the page asserts samples). */
#define PR_MIN_POSITIVE 1.1754943508222875e-38
#define PR_DIV_EPS 1e-12

static void pr_sigma(int64_t R, const double* M2, const double* M1, double n, int center,
                     double* S, double* mu) {
    for (int64_t i = 0; i < R; ++i) mu[i] = (center && M1) ? M1[i] / n : 0.0;
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < R; ++j) S[i * R + j] = M2[i * R + j] / n - mu[i] * mu[j];
}

int oracle_moments_pr(int64_t batch, int64_t nheads, int64_t R, const double* m2,
                      const double* m1, const int64_t* count, int center, double* pr,
                      double* trace) {
    if (batch < 0 || nheads <= 0 || R <= 0 || !m2 || !count || !pr || (center && !m1)) return -1;
    double* S = (double*)malloc(sizeof(double) * (R * R + R));
    if (!S) return -2;
    double* mu = S + R * R;
    for (int64_t b = 0; b < batch; ++b) {
        if (count[b] <= 0) { free(S); return -1; }
        const double n = (double)count[b];
        for (int64_t h = 0; h < nheads; ++h) {
            const int64_t o = b * nheads + h;
            pr_sigma(R, m2 + o * R * R, m1 ? m1 + o * R : NULL, n, center, S, mu);
            double tr = 0.0, trm2 = 0.0;
            for (int64_t i = 0; i < R; ++i) {
                tr += S[i * R + i];
                trm2 += m2[o * R * R + i * R + i];
            }
            const double s = tr > PR_MIN_POSITIVE ? tr : PR_MIN_POSITIVE;
            double tr1 = 0.0, tr2 = 0.0;
            for (int64_t i = 0; i < R; ++i) tr1 += S[i * R + i] / s;
            for (int64_t k = 0; k < R * R; ++k) tr2 += (S[k] / s) * (S[k] / s);
            if (tr2 < PR_DIV_EPS) tr2 = PR_DIV_EPS;
            pr[o] = tr1 * tr1 / tr2;
            if (trace) trace[o] = trm2 / n;
        }
    }
    free(S);
    return 0;
}

/* Gradient of sum_{b,h} d_pr * PR with the normaliser s held fixed (the page
 * detaches it): with G_hat = dPR/dSigma_hat = 2 tr1/tr2 I - 2 tr1^2/tr2^2 Sigma_hat
 * (the second term only while ||Sigma_hat||^2 exceeds div_eps, where the clamp
 * is inactive), dPR/dSigma = G_hat / s, d_m2 = dPR/dSigma / count and, centred,
 * d_m1 = -(G + G^T) mu / count with G = dPR/dSigma; uncentred d_m1 = 0. */
int oracle_moments_pr_bwd(int64_t batch, int64_t nheads, int64_t R, const double* d_pr,
                          const double* m2, const double* m1, const int64_t* count, int center,
                          double* d_m2, double* d_m1) {
    if (batch < 0 || nheads <= 0 || R <= 0 || !d_pr || !m2 || !count || !d_m2 ||
        (center && !m1))
        return -1;
    double* S = (double*)malloc(sizeof(double) * (2 * R * R + R));
    if (!S) return -2;
    double* G = S + R * R;
    double* mu = G + R * R;
    for (int64_t b = 0; b < batch; ++b) {
        if (count[b] <= 0) { free(S); return -1; }
        const double n = (double)count[b];
        for (int64_t h = 0; h < nheads; ++h) {
            const int64_t o = b * nheads + h;
            pr_sigma(R, m2 + o * R * R, m1 ? m1 + o * R : NULL, n, center, S, mu);
            double tr = 0.0;
            for (int64_t i = 0; i < R; ++i) tr += S[i * R + i];
            const double s = tr > PR_MIN_POSITIVE ? tr : PR_MIN_POSITIVE;
            double tr1 = 0.0, tr2 = 0.0;
            for (int64_t i = 0; i < R; ++i) tr1 += S[i * R + i] / s;
            for (int64_t k = 0; k < R * R; ++k) tr2 += (S[k] / s) * (S[k] / s);
            const int live = tr2 > PR_DIV_EPS;
            if (!live) tr2 = PR_DIV_EPS;
            for (int64_t i = 0; i < R; ++i)
                for (int64_t j = 0; j < R; ++j) {
                    double gh = (i == j) ? 2.0 * tr1 / tr2 : 0.0;
                    if (live) gh -= 2.0 * tr1 * tr1 / (tr2 * tr2) * (S[i * R + j] / s);
                    G[i * R + j] = d_pr[o] * gh / s;
                }
            for (int64_t k = 0; k < R * R; ++k) d_m2[o * R * R + k] = G[k] / n;
            if (d_m1)
                for (int64_t i = 0; i < R; ++i) {
                    double acc = 0.0;
                    if (center)
                        for (int64_t j = 0; j < R; ++j) acc -= (G[i * R + j] + G[j * R + i]) * mu[j];
                    d_m1[o * R + i] = acc / n;
                }
        }
    }
    free(S);
    return 0;
}

/* ------------------------------------------------------ same-step correction
 * The gamma-weighted same-step term of the burn-mamba page
 * "mamba3/single_ssd/ssd/serial_recalculated/diag.rs" (module doc and the
 * general MIMO path), for every token t (the [b, n, l] axes flattened) and head h:
 *   qk[mo][mi]   = sum_r C[t,mo,h,r] B[t,mi,h,r]
 *   y[t,mo,h,p]  = gamma[t,h] sum_mi qk[mo][mi] V[t,mi,h,p]
 * Layouts: V, y [T, M, H, P]; B, C [T, M, H, R]; gamma [T, H]. */
static int64_t dg_off(int64_t t, int64_t m, int64_t h, int64_t M, int64_t H, int64_t W) {
    return ((t * M + m) * H + h) * W;
}

int oracle_diag_fwd(int64_t T, int64_t M, int64_t H, int64_t P, int64_t R, const double* V,
                    const double* B, const double* C, const double* gamma, double* y) {
    if (T < 0 || M <= 0 || H <= 0 || P <= 0 || R <= 0) return -1;
    if (T > 0 && (!V || !B || !C || !gamma || !y)) return -1;
    double* qk = (double*)malloc(sizeof(double) * M * M);
    if (!qk) return -2;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t mo = 0; mo < M; ++mo)
                for (int64_t mi = 0; mi < M; ++mi) {
                    double acc = 0.0;
                    for (int64_t r = 0; r < R; ++r)
                        acc += C[dg_off(t, mo, h, M, H, R) + r] * B[dg_off(t, mi, h, M, H, R) + r];
                    qk[mo * M + mi] = acc;
                }
            const double g = gamma[t * H + h];
            for (int64_t mo = 0; mo < M; ++mo)
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t mi = 0; mi < M; ++mi) acc += qk[mo * M + mi] * V[dg_off(t, mi, h, M, H, P) + p];
                    y[dg_off(t, mo, h, M, H, P) + p] = g * acc;
                }
        }
    free(qk);
    return 0;
}

/* Reverse mode of that definition, in the page's order (general MIMO backward):
 *   yu = qk V (unweighted), d_gamma = sum dy o yu, dyu = gamma dy,
 *   d_qk = dyu V^T, d_V = qk^T dyu, d_C = d_qk B, d_B = d_qk^T C. */
int oracle_diag_bwd(int64_t T, int64_t M, int64_t H, int64_t P, int64_t R, const double* dy,
                    const double* V, const double* B, const double* C, const double* gamma,
                    double* d_v, double* d_b, double* d_c, double* d_gamma) {
    if (T < 0 || M <= 0 || H <= 0 || P <= 0 || R <= 0) return -1;
    if (T > 0 && (!dy || !V || !B || !C || !gamma || !d_v || !d_b || !d_c || !d_gamma)) return -1;
    double* qk = (double*)malloc(sizeof(double) * 2 * M * M);
    if (!qk) return -2;
    double* dqk = qk + M * M;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            const double g = gamma[t * H + h];
            for (int64_t mo = 0; mo < M; ++mo)
                for (int64_t mi = 0; mi < M; ++mi) {
                    double acc = 0.0;
                    for (int64_t r = 0; r < R; ++r)
                        acc += C[dg_off(t, mo, h, M, H, R) + r] * B[dg_off(t, mi, h, M, H, R) + r];
                    qk[mo * M + mi] = acc;
                }
            double dg = 0.0;
            for (int64_t mo = 0; mo < M; ++mo)
                for (int64_t p = 0; p < P; ++p) {
                    double yu = 0.0;
                    for (int64_t mi = 0; mi < M; ++mi) yu += qk[mo * M + mi] * V[dg_off(t, mi, h, M, H, P) + p];
                    dg += dy[dg_off(t, mo, h, M, H, P) + p] * yu;
                }
            d_gamma[t * H + h] = dg;
            for (int64_t mo = 0; mo < M; ++mo)
                for (int64_t mi = 0; mi < M; ++mi) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p)
                        acc += g * dy[dg_off(t, mo, h, M, H, P) + p] * V[dg_off(t, mi, h, M, H, P) + p];
                    dqk[mo * M + mi] = acc;
                }
            for (int64_t mi = 0; mi < M; ++mi)
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t mo = 0; mo < M; ++mo)
                        acc += qk[mo * M + mi] * g * dy[dg_off(t, mo, h, M, H, P) + p];
                    d_v[dg_off(t, mi, h, M, H, P) + p] = acc;
                }
            for (int64_t mo = 0; mo < M; ++mo)
                for (int64_t r = 0; r < R; ++r) {
                    double acc = 0.0;
                    for (int64_t mi = 0; mi < M; ++mi) acc += dqk[mo * M + mi] * B[dg_off(t, mi, h, M, H, R) + r];
                    d_c[dg_off(t, mo, h, M, H, R) + r] = acc;
                }
            for (int64_t mi = 0; mi < M; ++mi)
                for (int64_t r = 0; r < R; ++r) {
                    double acc = 0.0;
                    for (int64_t mo = 0; mo < M; ++mo) acc += dqk[mo * M + mi] * C[dg_off(t, mo, h, M, H, R) + r];
                    d_b[dg_off(t, mi, h, M, H, R) + r] = acc;
                }
        }
    free(qk);
    return 0;
}

/* --------------------------------------------- quaternion cumulative product
 * The scan of the burn-mamba page "mamba3/quat_scan/backward.rs" (Gradient
 * math): for every lane (b, h, j), cum[t] = q_t (x) cum[t-1], cum[-1] = init,
 * with the Hamilton product of quaternions stored as (w, x, y, z).
 * Layouts: q, cum, d_cum, d_q [B, S, H, J, 4]; init, d_init [B, H, J, 4]
 * (init NULL = the identity quaternion). */
static void qmul(const double* a, const double* b, double* o) {
    const double w = a[0] * b[0] - a[1] * b[1] - a[2] * b[2] - a[3] * b[3];
    const double x = a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2];
    const double y = a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1];
    const double z = a[0] * b[3] + a[1] * b[2] - a[2] * b[1] + a[3] * b[0];
    o[0] = w;
    o[1] = x;
    o[2] = y;
    o[3] = z;
}

static void qconj(const double* a, double* o) {
    o[0] = a[0];
    o[1] = -a[1];
    o[2] = -a[2];
    o[3] = -a[3];
}

int oracle_quat_scan(int64_t B, int64_t S, int64_t H, int64_t J, const double* q,
                     const double* init, double* cum) {
    if (B < 0 || S < 0 || H <= 0 || J <= 0) return -1;
    if (B > 0 && S > 0 && (!q || !cum)) return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t j = 0; j < J; ++j) {
                double c[4] = {1.0, 0.0, 0.0, 0.0};
                if (init)
                    for (int e = 0; e < 4; ++e) c[e] = init[((b * H + h) * J + j) * 4 + e];
                for (int64_t t = 0; t < S; ++t) {
                    const int64_t o = (((b * S + t) * H + h) * J + j) * 4;
                    double n[4];
                    qmul(q + o, c, n);
                    for (int e = 0; e < 4; ++e) cum[o + e] = c[e] = n[e];
                }
            }
    return 0;
}

/* Reverse mode of that scan, exact for all quaternions: with o = a (x) b and a
 * cotangent g of o, the real inner product gives grad_a = g (x) conj(b) and
 * grad_b = conj(a) (x) g (the page's per-factor VJPs).  The total cotangent G_t
 * of cum[t] is d_cum[t] plus what cum[t+1] hands back:
 *   G_t = d_cum[t] + conj(q_{t+1}) (x) G_{t+1},  d_q[t] = G_t (x) conj(cum[t-1]),
 *   d_init = conj(q_0) (x) G_0. */
int oracle_quat_scan_bwd(int64_t B, int64_t S, int64_t H, int64_t J, const double* q,
                         const double* init, const double* d_cum, double* d_q, double* d_init) {
    if (B < 0 || S < 0 || H <= 0 || J <= 0) return -1;
    if (B > 0 && S > 0 && (!q || !d_cum || !d_q)) return -1;
    double* cum = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1) * 4);
    if (!cum) return -2;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t j = 0; j < J; ++j) {
                double c0[4] = {1.0, 0.0, 0.0, 0.0};
                if (init)
                    for (int e = 0; e < 4; ++e) c0[e] = init[((b * H + h) * J + j) * 4 + e];
                double c[4] = {c0[0], c0[1], c0[2], c0[3]};
                for (int64_t t = 0; t < S; ++t) {  /* forward again: cum[t] of this lane */
                    double n[4];
                    qmul(q + (((b * S + t) * H + h) * J + j) * 4, c, n);
                    for (int e = 0; e < 4; ++e) cum[t * 4 + e] = c[e] = n[e];
                }
                double G[4] = {0.0, 0.0, 0.0, 0.0};
                for (int64_t t = S - 1; t >= 0; --t) {
                    const int64_t o = (((b * S + t) * H + h) * J + j) * 4;
                    for (int e = 0; e < 4; ++e) G[e] += d_cum[o + e];
                    const double* prev = t > 0 ? cum + (t - 1) * 4 : c0;
                    double pc[4], qc[4], n[4];
                    qconj(prev, pc);
                    qmul(G, pc, d_q + o);
                    qconj(q + o, qc);
                    qmul(qc, G, n);
                    for (int e = 0; e < 4; ++e) G[e] = n[e];
                }
                if (d_init)
                    for (int e = 0; e < 4; ++e) d_init[((b * H + h) * J + j) * 4 + e] = G[e];
            }
    free(cum);
    return 0;
}
