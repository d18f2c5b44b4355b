/*
 * s6_oracle.c -- plain fp64 CPU reference of the selective scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or constant with the HIP library and must never
 * be reached from the product path.
 *
 * What it computes (source: "Mamba 状态空间模型原理与 Transformer 对比",
 * kb.agiseed.tech, the one page that states the mathematics):
 *   - section 2.1, eq. (2): zero-order-hold discretisation
 *       Abar = exp(dt*A),  Bbar = (dt*A)^-1 (exp(dt*A) - I) * dt*B.
 *     A is diagonal per channel (Figure 1: every channel is an independent
 *     SSM with an N-dimensional latent), so per state n this is
 *       Abar_n = exp(dt*A_n),  Bbar_n = expm1(dt*A_n)/(dt*A_n) * dt * B_n,
 *     and in the limit dt*A_n -> 0 the factor expm1(x)/x tends to 1.
 *   - eq. (3a)/(3b): h_t = Abar_t h_{t-1} + Bbar_t x_t,  y_t = C_t h_t
 *     (the readout uses the state after the update at t).
 *   - section 3.2: B and C are per-token projections of width N shared by
 *     all channels, dt is per token per channel, made positive by softplus.
 *   - Figure 3 caption: the SSM branch is gated multiplicatively by SiLU.
 * Readings where the page is silent (all listed in the design notes):
 *   - the per-channel dt bias is added before the softplus;
 *   - a skip term Dskip[d]*x_t is added to y_t before the gate;
 *   - out = (y + Dskip*x) * z * sigmoid(z) when a gate z is given;
 *   - the initial state is zero unless h0 is given.
 * Arithmetic: IEEE fp64 with C99 libm exp/expm1/log1p, in the plain order of
 * the equations; softplus in the overflow-free form max(v,0)+log1p(e^-|v|).
 *
 * Layouts (row-major, last index fastest):
 *   u, delta, z, out : (batch, L, D)     B, C : (batch, L, N)
 *   A : (D, N)     delta_bias, Dskip : (D)     h0, last_state : (batch, D, N)
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus_exact(double v) {
    /* log(1 + e^v) without overflow */
    return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));
}

static double silu(double z) {
    return z / (1.0 + exp(-z));
}

/* One token of one channel: eq. (2) then eq. (3a) then eq. (3b).
 * h has N entries and is updated in place; returns y before skip and gate. */
static double s6_token(int64_t N, double dt, double x, const double* A_row,
                       const double* B_tok, const double* C_tok, double* h) {
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double a = dt * A_row[n];                         /* dt*A_n             */
        double abar = exp(a);                             /* eq. (2), Abar      */
        double phi = (a == 0.0) ? 1.0 : expm1(a) / a;      /* (e^a - 1)/a        */
        double bbar = phi * dt * B_tok[n];                 /* eq. (2), Bbar      */
        h[n] = abar * h[n] + bbar * x;                     /* eq. (3a)           */
        y += C_tok[n] * h[n];                              /* eq. (3b)           */
    }
    return y;
}

static double token_dt(double raw, const double* bias, int64_t d, int softplus_flag) {
    double v = raw + (bias ? bias[d] : 0.0);
    return softplus_flag ? softplus_exact(v) : v;
}

static double finish(double y, double x, const double* Dskip, int64_t d, const double* zp) {
    if (Dskip) y += Dskip[d] * x;
    if (zp) y *= silu(*zp);
    return y;
}

/* Full-sequence forward scan.  Returns 0, or 1 on a bad argument. */
int s6_oracle_scan(int64_t batch, int64_t L, int64_t D, int64_t N,
                   const double* u, const double* delta, const double* delta_bias,
                   const double* A, const double* B, const double* C,
                   const double* Dskip, const double* z, int softplus_flag,
                   const double* h0, double* out, double* last_state, int nthreads) {
    if (batch < 0 || L < 0 || D < 0 || N <= 0 || !A || !out) return 1;
    if (L > 0 && (!u || !delta || !B || !C)) return 1;
    if (nthreads <= 0) nthreads = 1;
    int64_t units = batch * D;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (int64_t unit = 0; unit < units; ++unit) {
        int64_t b = unit / D, d = unit % D;
        double* h = (double*)malloc((size_t)N * sizeof(double));
        if (!h) { bad |= 1; continue; }
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            int64_t i = (b * L + t) * D + d;
            double dt = token_dt(delta[i], delta_bias, d, softplus_flag);
            double x = u[i];
            double y = s6_token(N, dt, x, A + d * N, B + (b * L + t) * N, C + (b * L + t) * N, h);
            out[i] = finish(y, x, Dskip, d, z ? z + i : NULL);
        }
        if (last_state)
            for (int64_t n = 0; n < N; ++n) last_state[(b * D + d) * N + n] = h[n];
        free(h);
    }
    return bad ? 2 : 0;
}

/* One decode step: every (batch, channel) advances by one token in place.
 * u, delta, z, out : (batch, D)   B, C : (batch, N)   state : (batch, D, N). */
int s6_oracle_step(int64_t batch, int64_t D, int64_t N, double* state,
                   const double* u, const double* delta, const double* delta_bias,
                   const double* A, const double* B, const double* C,
                   const double* Dskip, const double* z, int softplus_flag,
                   double* out, int nthreads) {
    if (batch < 0 || D < 0 || N <= 0 || !state || !A || !out) return 1;
    if (nthreads <= 0) nthreads = 1;
    int64_t units = batch * D;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t unit = 0; unit < units; ++unit) {
        int64_t b = unit / D, d = unit % D;
        double dt = token_dt(delta[unit], delta_bias, d, softplus_flag);
        double x = u[unit];
        double y = s6_token(N, dt, x, A + d * N, B + b * N, C + b * N, state + unit * N);
        out[unit] = finish(y, x, Dskip, d, z ? z + unit : NULL);
    }
    return 0;
}

int s6_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Backward of s6_oracle_scan: gradients of the scalar
 *     sum(dout * out) + sum(dlast * last_state)
 * with respect to every input, by differentiating the forward definition
 * above step by step (the backward pass itself is not on the page; it is
 * the derivative of eq. (2), (3a), (3b), the softplus front end and the SiLU
 * gate).  For one channel, with x = dt*A_n, a = e^x, beta = (a - 1)/A_n:
 *     d a / d dt    = A_n a            d a / d A_n    = dt a
 *     d beta / d dt = a                d beta / d A_n = dt^2 psi(x),
 *     psi(x) = (x e^x - e^x + 1) / x^2  (psi(0) = 1/2)
 * and the state gradient runs backwards: g_{t-1} = a_t g_t + dy_{t-1} C_{t-1}.
 * The forward states are recomputed and kept per channel (plain, slow).
 * Outputs (all overwritten; nullable ones are skipped when NULL):
 *   du, ddelta, dz (nullable) : (batch, L, D)
 *   dB, dC : (batch, L, N)      dA : (D, N)
 *   dDskip, dbias (nullable) : (D)      dh0 (nullable) : (batch, D, N)
 * dlast (nullable) is the gradient arriving at last_state.
 * ------------------------------------------------------------------------ */
static double psi_fn(double x) {
    if (fabs(x) < 1e-3) /* series of (x e^x - e^x + 1)/x^2 */
        return 0.5 + x * (1.0 / 3.0 + x * (1.0 / 8.0 + x * (1.0 / 30.0 + x * (1.0 / 144.0))));
    return (x * exp(x) - expm1(x)) / (x * x);
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

int s6_oracle_scan_bwd(int64_t batch, int64_t L, int64_t D, int64_t N,
                       const double* u, const double* delta, const double* delta_bias,
                       const double* A, const double* B, const double* C,
                       const double* Dskip, const double* z, int softplus_flag,
                       const double* h0, const double* dout, const double* dlast,
                       double* du, double* ddelta, double* dA, double* dB, double* dC,
                       double* dDskip, double* dz, double* dbias, double* dh0, int nthreads) {
    if (batch < 0 || L < 0 || D < 0 || N <= 0 || !A || !dA || !dout || !du || !ddelta || !dB || !dC) return 1;
    if (nthreads <= 0) nthreads = 1;
    for (int64_t i = 0; i < D * N; ++i) dA[i] = 0.0;
    if (dDskip) for (int64_t i = 0; i < D; ++i) dDskip[i] = 0.0;
    if (dbias) for (int64_t i = 0; i < D; ++i) dbias[i] = 0.0;
    for (int64_t i = 0; i < batch * L * N; ++i) { dB[i] = 0.0; dC[i] = 0.0; }
    int bad = 0;
    /* channels in parallel; the reductions over channels (dB, dC) and over
       (batch, token) (dA, dDskip, dbias) are accumulated per thread and added
       under a critical section in channel order per thread */
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
    {
        double* hs = (double*)malloc((size_t)(L + 1) * N * sizeof(double)); /* h_{-1..L-1} */
        double* g = (double*)malloc((size_t)N * sizeof(double));
        double* dA_loc = (double*)calloc((size_t)D * N, sizeof(double));
        double* dD_loc = (double*)calloc((size_t)D, sizeof(double));
        double* db_loc = (double*)calloc((size_t)D, sizeof(double));
        double* dB_loc = (double*)calloc((size_t)batch * L * N, sizeof(double));
        double* dC_loc = (double*)calloc((size_t)batch * L * N, sizeof(double));
        if (!hs || !g || !dA_loc || !dD_loc || !db_loc || !dB_loc || !dC_loc) bad |= 1;
#pragma omp for schedule(static)
        for (int64_t unit = 0; unit < batch * D; ++unit) {
            if (bad) continue;
            int64_t b = unit / D, d = unit % D;
            const double* Ar = A + d * N;
            /* forward, keeping every state: row k of hs is h_{k-1} */
            for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                int64_t i = (b * L + t) * D + d;
                double dt = token_dt(delta[i], delta_bias, d, softplus_flag);
                for (int64_t n = 0; n < N; ++n) hs[(t + 1) * N + n] = hs[t * N + n];
                (void)s6_token(N, dt, u[i], Ar, B + (b * L + t) * N, C + (b * L + t) * N, hs + (t + 1) * N);
            }
            /* backward */
            for (int64_t n = 0; n < N; ++n) g[n] = dlast ? dlast[(b * D + d) * N + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                int64_t i = (b * L + t) * D + d;
                const double* Bt = B + (b * L + t) * N;
                const double* Ct = C + (b * L + t) * N;
                const double* h_t = hs + (t + 1) * N;
                const double* h_p = hs + t * N;
                double v = delta[i] + (delta_bias ? delta_bias[d] : 0.0);
                double dt = softplus_flag ? softplus_exact(v) : v;
                double x = u[i];
                double y = 0.0;
                for (int64_t n = 0; n < N; ++n) y += Ct[n] * h_t[n];
                double o = y + (Dskip ? Dskip[d] * x : 0.0);
                double dy;
                if (z) {
                    double s = sigmoid(z[i]);
                    if (dz) dz[i] = dout[i] * o * (s + z[i] * s * (1.0 - s));
                    dy = dout[i] * z[i] * s;
                } else {
                    dy = dout[i];
                }
                double dx = Dskip ? Dskip[d] * dy : 0.0;
                if (Dskip) dD_loc[d] += dy * x;
                double ddt = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    double xa = dt * Ar[n];
                    double a = exp(xa);
                    double phi = (xa == 0.0) ? 1.0 : expm1(xa) / xa;
                    double beta = phi * dt;
                    g[n] += dy * Ct[n];                 /* dL/dh_t */
                    dC_loc[(b * L + t) * N + n] += dy * h_t[n];
                    double da = g[n] * h_p[n];
                    double dbeta = g[n] * Bt[n] * x;
                    dB_loc[(b * L + t) * N + n] += g[n] * beta * x;
                    dx += g[n] * beta * Bt[n];
                    ddt += da * Ar[n] * a + dbeta * a;
                    dA_loc[d * N + n] += da * dt * a + dbeta * dt * dt * psi_fn(xa);
                    g[n] *= a;                          /* dL/dh_{t-1} from h_t */
                }
                du[i] = dx;
                double dv = softplus_flag ? ddt * sigmoid(v) : ddt;
                ddelta[i] = dv;
                db_loc[d] += dv;
            }
            if (dh0) for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = g[n];
        }
#pragma omp critical
        {
            if (!bad) {
                for (int64_t k = 0; k < D * N; ++k) dA[k] += dA_loc[k];
                if (dDskip) for (int64_t k = 0; k < D; ++k) dDskip[k] += dD_loc[k];
                if (dbias) for (int64_t k = 0; k < D; ++k) dbias[k] += db_loc[k];
                for (int64_t k = 0; k < batch * L * N; ++k) { dB[k] += dB_loc[k]; dC[k] += dC_loc[k]; }
            }
        }
        free(hs); free(g); free(dA_loc); free(dD_loc); free(db_loc); free(dB_loc); free(dC_loc);
    }
    return bad ? 2 : 0;
}

/* ------------------------------------------------------------------------
 * Complex diagonal A (the -1/2 + ni row of the A-initialisation table of the
 * same page).  The page gives only the values of A; the reading taken here is
 * the plainest one the rest supports: delta, x, B and C stay real, A_n is
 * complex, so the state is complex with
 *     Abar_n = exp(dt A_n),   Bbar_n = (exp(dt A_n) - 1)/(dt A_n) * dt * B_n
 *     h_t = Abar h_{t-1} + Bbar x_t,   y_t = Re(sum_n C_n h_t[n])
 * (eq. (2), (3a), (3b) with complex A), then the same skip and gate.
 * A is given as (D, N, 2) = (re, im); h0 and last_state as (batch, D, N, 2).
 * ------------------------------------------------------------------------ */
#include <complex.h>

static double complex phi1c(double complex a) {
    /* (e^a - 1)/a, limit 1 at a = 0.  Below |a| = 1e-2 its Taylor series
     * 1 + a/2 + a^2/6 + a^3/24 + a^4/120 (next term |a|^5/720 < 1.4e-13);
     * above, the quotient, whose cancellation costs at most ~2e-14. */
    if (cabs(a) < 1e-2) return 1.0 + a * (1.0 / 2.0 + a * (1.0 / 6.0 + a * (1.0 / 24.0 + a / 120.0)));
    return (cexp(a) - 1.0) / a;
}

int s6_oracle_scan_complex(int64_t batch, int64_t L, int64_t D, int64_t N,
                           const double* u, const double* delta, const double* delta_bias,
                           const double* A, const double* B, const double* C,
                           const double* Dskip, const double* z, int softplus_flag,
                           const double* h0, double* out, double* last_state, int nthreads) {
    if (batch < 0 || L < 0 || D < 0 || N <= 0 || !A || !out) return 1;
    if (L > 0 && (!u || !delta || !B || !C)) return 1;
    if (nthreads <= 0) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : bad)
    for (int64_t unit = 0; unit < batch * D; ++unit) {
        int64_t b = unit / D, d = unit % D;
        double complex* h = (double complex*)malloc((size_t)N * sizeof(double complex));
        if (!h) { bad |= 1; continue; }
        for (int64_t n = 0; n < N; ++n)
            h[n] = h0 ? h0[((b * D + d) * N + n) * 2] + I * h0[((b * D + d) * N + n) * 2 + 1] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            int64_t i = (b * L + t) * D + d;
            double dt = token_dt(delta[i], delta_bias, d, softplus_flag);
            double x = u[i];
            double y = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double complex An = A[(d * N + n) * 2] + I * A[(d * N + n) * 2 + 1];
                double complex a = dt * An;                     /* dt*A_n             */
                double complex abar = cexp(a);                  /* eq. (2), Abar      */
                double complex bbar = phi1c(a) * dt * B[(b * L + t) * N + n];
                h[n] = abar * h[n] + bbar * x;                  /* eq. (3a)           */
                y += C[(b * L + t) * N + n] * creal(h[n]);     /* eq. (3b), real part */
            }
            out[i] = finish(y, x, Dskip, d, z ? z + i : NULL);
        }
        if (last_state)
            for (int64_t n = 0; n < N; ++n) {
                last_state[((b * D + d) * N + n) * 2] = creal(h[n]);
                last_state[((b * D + d) * N + n) * 2 + 1] = cimag(h[n]);
            }
        free(h);
    }
    return bad ? 2 : 0;
}
