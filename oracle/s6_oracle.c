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
