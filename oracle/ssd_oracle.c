/*
 * ssd_oracle.c -- plain, slow, float64 CPU oracle for the selective state-space
 * (SSD) scan.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark call it; the product library never links,
 * loads or calls it, and it shares no code, header or table with the HIP path.
 *
 * It evaluates the recurrences exactly as defined, one time step after the
 * other, in double precision.  No chunking, blocking or re-association: the
 * chunked GPU algorithm is checked against this definition.
 *
 * Sources (page titles and sections):
 *  - Mamba-3-Lite README, section on the classical Mamba-2 recurrence and its
 *    complex promotion: h_t = exp(A dt) h_{t-1} + B x_t, y_t = C h_t, and the
 *    complex form with A = A_re + i A_im, B, C complex.
 *  - "Block Anatomy, Numerical Stability & Scaling", section 4.4 (the per-head
 *    complex A used through exp(softplus(dt) * A)) and the Numerical Stability
 *    doc, section 4 (softplus is ln(1 + e^x); per-step factor |a| <= 1 when
 *    Re A <= 0).
 *  - The real form used here is the usual Mamba-2 discretisation with the
 *    step size on the input term as well, h_t = exp(A dt) h_{t-1} +
 *    dt B_t x_t^T, y_t = C_t^T h_t + D x_t, A one scalar per head (the README
 *    shorthand writes the input term as B x_t).
 *
 * Readings where the pages leave a step open (each is listed in the design doc):
 *  - real form: the input term carries the step size (dt * B * x); the
 *    complex form does not (B * x), as the complex recurrence on the README
 *    page writes it;
 *  - y_t reads the state after the update at step t (y_t = C h_t);
 *  - complex readout: y = Re(sum_n C_n h_n) with no conjugation (the page's
 *    real-GEMM expansion subtracts the imag*imag product);
 *  - x is real in the complex form; there is no D skip in the complex form;
 *  - dt processing: delta = clamp(softplus(dt + dt_bias), dt_min, dt_max);
 *  - head h reads B/C group g = h / (H / G).
 *
 * Layouts (row-major, last index fastest):
 *   x  (Bsz,T,H,P)  dt (Bsz,T,H)  B,C (Bsz,T,G,N)[,2]  y (Bsz,T,H,P)
 *   h0, h_final (Bsz,H,P,N)[,2]   A (H) or (H,2)      D, dt_bias (H)
 * x/B/C may be float32 (dtype 0) or bfloat16 bit patterns (dtype 1); they are
 * widened exactly to double.  Outputs are double.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads_used = 1;

int ssd_oracle_threads_used(void) { return g_threads_used; }

/* Set the OpenMP thread count for later calls (n <= 0 leaves it alone). */
void ssd_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Read element i of an array of float32 (dtype 0) or bfloat16 (dtype 1).
 * A bfloat16 value is the top half of a float32 bit pattern, so the
 * widening is exact. */
static double load_in(const void *p, size_t i, int dtype)
{
    if (dtype == 0)
        return (double)((const float *)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* softplus(z) = ln(1 + e^z), evaluated without overflow as
 * max(z,0) + ln(1 + e^{-|z|}). */
double ssd_oracle_softplus(double z)
{
    double m = z > 0.0 ? z : 0.0;
    return m + log1p(exp(-fabs(z)));
}

/* Step size for one (token, head): softplus of the biased raw value, then
 * the clamp [dt_min, dt_max]. */
double ssd_oracle_delta(double dt_raw, double bias, double dt_min, double dt_max)
{
    double d = ssd_oracle_softplus(dt_raw + bias);
    if (d < dt_min) d = dt_min;
    if (d > dt_max) d = dt_max;
    return d;
}

static void record_threads(void)
{
#ifdef _OPENMP
    g_threads_used = omp_get_num_threads();
#else
    g_threads_used = 1;
#endif
}

/*
 * Real Mamba-2 recurrence, sequential over t, for every (b, h):
 *   delta = clamp(softplus(dt + dt_bias))
 *   S[p][n] <- exp(A_h * delta) * S[p][n] + delta * x[p] * B[n]
 *   y[p]     = sum_n C[n] * S[p][n] + D_h * x[p]
 * S starts at h0 (zeros when h0 is NULL).  state is caller-owned scratch of
 * Bsz*H*P*N doubles.  Returns 0, or 1 on invalid sizes.
 */
int ssd_oracle_fwd(const void *x, const float *dt, const float *A,
                   const void *B, const void *C, const float *D,
                   const float *dt_bias, double dt_min, double dt_max,
                   const float *h0, double *y, double *h_final,
                   int Bsz, int T, int H, int P, int G, int N, int dtype,
                   double *state /* Bsz*H*P*N doubles, caller-owned */)
{
    if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G)
        return 1;
    const int hpg = H / G;
    const long long BH = (long long)Bsz * H;
#pragma omp parallel
    {
#pragma omp single
        record_threads();
#pragma omp for schedule(dynamic, 1)
        for (long long bh = 0; bh < BH; ++bh) {
            const int b = (int)(bh / H), h = (int)(bh % H), g = h / hpg;
            double *S = state + (size_t)bh * P * N;
            for (int i = 0; i < P * N; ++i)
                S[i] = h0 ? (double)h0[(size_t)bh * P * N + i] : 0.0;
            const double Ah = (double)A[h];
            const double Dh = D ? (double)D[h] : 0.0;
            const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t tok = (size_t)b * T + t;
                const double delta =
                    ssd_oracle_delta((double)dt[tok * H + h], bias, dt_min, dt_max);
                const double a = exp(Ah * delta);
                const size_t xo = (tok * H + h) * (size_t)P;
                const size_t bo = (tok * G + g) * (size_t)N;
                for (int p = 0; p < P; ++p) {
                    const double xp = load_in(x, xo + p, dtype);
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n) {
                        double *s = &S[(size_t)p * N + n];
                        *s = a * (*s) + delta * xp * load_in(B, bo + n, dtype);
                        acc += load_in(C, bo + n, dtype) * (*s);
                    }
                    y[xo + p] = acc + Dh * xp;
                }
            }
            if (h_final)
                memcpy(h_final + (size_t)bh * P * N, S, sizeof(double) * P * N);
        }
    }
    return 0;
}

/*
 * Complex (Mamba-3-Lite) recurrence, sequential over t, for every (b, h):
 *   delta = clamp(softplus(dt + dt_bias))
 *   a     = exp((alpha_h + i beta_h) * delta)
 *   S[p][n] <- a * S[p][n] + B[n] * x[p]          (complex, no delta factor)
 *   y[p]     = Re( sum_n C[n] * S[p][n] )          (unconjugated C)
 * x is real float32; A, B, C, h0, h_final are (re, im) float pairs.  The
 * complex arithmetic is written out on (re, im) doubles.  state must hold
 * Bsz*H*P*N*2 doubles.
 */
int ssd_oracle_complex_fwd(const float *x, const float *dt, const float *A,
                           const float *B, const float *C,
                           const float *dt_bias, double dt_min, double dt_max,
                           const float *h0, double *y, double *h_final,
                           int Bsz, int T, int H, int P, int G, int N,
                           double *state)
{
    if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G)
        return 1;
    const int hpg = H / G;
    const long long BH = (long long)Bsz * H;
#pragma omp parallel
    {
#pragma omp single
        record_threads();
#pragma omp for schedule(dynamic, 1)
        for (long long bh = 0; bh < BH; ++bh) {
            const int b = (int)(bh / H), h = (int)(bh % H), g = h / hpg;
            double *S = state + (size_t)bh * P * N * 2;
            for (int i = 0; i < P * N * 2; ++i)
                S[i] = h0 ? (double)h0[(size_t)bh * P * N * 2 + i] : 0.0;
            const double al = (double)A[2 * h], be = (double)A[2 * h + 1];
            const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t tok = (size_t)b * T + t;
                const double delta =
                    ssd_oracle_delta((double)dt[tok * H + h], bias, dt_min, dt_max);
                const double mag = exp(al * delta);
                const double are = mag * cos(be * delta), aim = mag * sin(be * delta);
                const size_t xo = (tok * H + h) * (size_t)P;
                const size_t bo = (tok * G + g) * (size_t)N * 2;
                for (int p = 0; p < P; ++p) {
                    const double xp = (double)x[xo + p];
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n) {
                        double *s = &S[((size_t)p * N + n) * 2];
                        const double br = B[bo + 2 * n], bi = B[bo + 2 * n + 1];
                        const double sr = are * s[0] - aim * s[1] + br * xp;
                        const double si = are * s[1] + aim * s[0] + bi * xp;
                        s[0] = sr;
                        s[1] = si;
                        const double cr = C[bo + 2 * n], ci = C[bo + 2 * n + 1];
                        acc += cr * sr - ci * si; /* Re(c * s) */
                    }
                    y[xo + p] = acc;
                }
            }
            if (h_final)
                memcpy(h_final + (size_t)bh * P * N * 2, S, sizeof(double) * P * N * 2);
        }
    }
    return 0;
}

/*
 * One real recurrent step (single-token decode) on a float64 state held by
 * the caller, updated in place:
 *   h[b,h,p,n] <- exp(A_h delta) h + delta x[b,h,p] B[b,g,n]
 *   y[b,h,p]    = sum_n C[b,g,n] h[b,h,p,n] + D_h x[b,h,p]
 * x (Bsz,H,P), dt (Bsz,H), B/C (Bsz,G,N) are float32.
 */
int ssd_oracle_step(double *hstate, const float *x, const float *dt, const float *A,
                    const float *B, const float *C, const float *D,
                    const float *dt_bias, double dt_min, double dt_max,
                    double *y, int Bsz, int H, int P, int G, int N)
{
    if (Bsz <= 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G)
        return 1;
    const int hpg = H / G;
    const long long BH = (long long)Bsz * H;
#pragma omp parallel
    {
#pragma omp single
        record_threads();
#pragma omp for schedule(static)
        for (long long bh = 0; bh < BH; ++bh) {
            const int b = (int)(bh / H), h = (int)(bh % H), g = h / hpg;
            const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
            const double delta = ssd_oracle_delta((double)dt[bh], bias, dt_min, dt_max);
            const double a = exp((double)A[h] * delta);
            const double Dh = D ? (double)D[h] : 0.0;
            const float *Bv = B + ((size_t)b * G + g) * N;
            const float *Cv = C + ((size_t)b * G + g) * N;
            for (int p = 0; p < P; ++p) {
                const double xp = (double)x[(size_t)bh * P + p];
                double *s = hstate + ((size_t)bh * P + p) * N;
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    s[n] = a * s[n] + delta * xp * (double)Bv[n];
                    acc += (double)Cv[n] * s[n];
                }
                y[(size_t)bh * P + p] = acc + Dh * xp;
            }
        }
    }
    return 0;
}

/*
 * One complex recurrent step (single-token decode, Mamba-3-Lite README: the
 * complex promotion of the recurrence) on a float64 complex state held by the
 * caller as (re, im) pairs, updated in place:
 *   h[b,h,p,n] <- exp((alpha_h + i beta_h) delta) h + B[b,g,n] x[b,h,p]
 *   y[b,h,p]    = Re(sum_n C[b,g,n] h[b,h,p,n])
 * (no step factor on the input, no D, readout after the update -- the
 * readings of the complex forward above).  x (Bsz,H,P), dt (Bsz,H) float32;
 * A (H,2), B/C (Bsz,G,N,2) float32 (re, im); h (Bsz,H,P,N,2).
 */
int ssd_oracle_complex_step(double *hstate, const float *x, const float *dt, const float *A,
                            const float *B, const float *C, const float *dt_bias,
                            double dt_min, double dt_max, double *y,
                            int Bsz, int H, int P, int G, int N)
{
    if (Bsz <= 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G)
        return 1;
    const int hpg = H / G;
    const long long BH = (long long)Bsz * H;
#pragma omp parallel
    {
#pragma omp single
        record_threads();
#pragma omp for schedule(static)
        for (long long bh = 0; bh < BH; ++bh) {
            const int b = (int)(bh / H), h = (int)(bh % H), g = h / hpg;
            const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
            const double delta = ssd_oracle_delta((double)dt[bh], bias, dt_min, dt_max);
            const double mag = exp((double)A[2 * h] * delta);
            const double ar = mag * cos((double)A[2 * h + 1] * delta);
            const double ai = mag * sin((double)A[2 * h + 1] * delta);
            const float *Bv = B + ((size_t)b * G + g) * N * 2;
            const float *Cv = C + ((size_t)b * G + g) * N * 2;
            for (int p = 0; p < P; ++p) {
                const double xp = (double)x[(size_t)bh * P + p];
                double *s = hstate + ((size_t)bh * P + p) * N * 2;
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    const double sr = ar * s[2 * n] - ai * s[2 * n + 1] + (double)Bv[2 * n] * xp;
                    const double si = ar * s[2 * n + 1] + ai * s[2 * n] + (double)Bv[2 * n + 1] * xp;
                    s[2 * n] = sr;
                    s[2 * n + 1] = si;
                    acc += (double)Cv[2 * n] * sr - (double)Cv[2 * n + 1] * si; /* Re(c * s) */
                }
                y[(size_t)bh * P + p] = acc;
            }
        }
    }
    return 0;
}

/*
 * Depthwise causal convolution of the Mamba-1/2 layer (Mamba-3-Lite block
 * page, section 5.1 "Zero causal convolution": before the scan, each channel's
 * value at position t is replaced by a learned combination of that channel's
 * values at positions t-K+1 .. t, K = 4).  Written out as the definition:
 *
 *   v[b,t,c]   = bias[c] + sum_{j=0..K-1} w[c,j] * in[b, t-K+1+j, c]
 *   out[b,t,c] = act ? v / (1 + exp(-v)) : v        (SiLU when act = 1)
 *
 * where in[b,p,c] for p < 0 is state_in[b, K-1+p, c] (the inputs that preceded
 * this segment; zero when state_in is NULL).  state_out[b,j,c] receives the raw
 * input at position T-K+1+j (j = 0..K-2), taken from state_in when that
 * position is negative, so that a sequence cut into segments gives the same
 * output as the whole.
 *
 *   xbc (Bsz,T,ld) of dtype 0 (float32) or 1 (bfloat16 bits), channels
 *   0..Ch-1 of each row used; w (Ch,K), bias (Ch) or NULL, state_in/state_out
 *   (Bsz,K-1,Ch) or NULL; out (Bsz,T,Ch) double.
 *
 * Readings: the bias and the SiLU are those of the usual Mamba-2 layer (the
 * pages name only the learned combination); the state holds raw inputs.
 */
int ssd_oracle_conv1d(const void *xbc, long long ld, const float *w, const float *bias,
                      const float *state_in, int act, double *out, double *state_out,
                      int Bsz, int T, int Ch, int K, int dtype)
{
    if (Bsz <= 0 || T < 0 || Ch <= 0 || K <= 0 || ld < Ch)
        return 1;
    const long long BC = (long long)Bsz * Ch;
#pragma omp parallel
    {
#pragma omp single
        record_threads();
#pragma omp for schedule(static)
        for (long long bc = 0; bc < BC; ++bc) {
            const int b = (int)(bc / Ch), c = (int)(bc % Ch);
            for (int t = 0; t < T; ++t) {
                double v = bias ? (double)bias[c] : 0.0;
                for (int j = 0; j < K; ++j) {
                    const long long p = (long long)t - (K - 1) + j;
                    double in;
                    if (p >= 0)
                        in = load_in(xbc, ((size_t)b * T + (size_t)p) * (size_t)ld + c, dtype);
                    else
                        in = state_in ? (double)state_in[((size_t)b * (K - 1) + (K - 1 + p)) * Ch + c] : 0.0;
                    v += (double)w[(size_t)c * K + j] * in;
                }
                if (act == 1)
                    v = v / (1.0 + exp(-v));
                out[((size_t)b * T + t) * Ch + c] = v;
            }
            if (state_out) {
                for (int j = 0; j < K - 1; ++j) {
                    const long long p = (long long)T - (K - 1) + j;
                    double in;
                    if (p >= 0)
                        in = load_in(xbc, ((size_t)b * T + (size_t)p) * (size_t)ld + c, dtype);
                    else
                        in = state_in ? (double)state_in[((size_t)b * (K - 1) + (K - 1 + p)) * Ch + c] : 0.0;
                    state_out[((size_t)b * (K - 1) + j) * Ch + c] = in;
                }
            }
        }
    }
    return 0;
}

/*
 * Reverse-mode derivative of the real recurrence (ssd_oracle_fwd) for the
 * scalar   loss = sum_t dy_t . y_t + <dh_final, h_final>,
 * by the adjoint recurrence run backwards in time (the definition of the
 * gradient of the recurrence of the Mamba-3-Lite README's classical Mamba-2
 * form, with the step size on the input term and y_t read after the update).
 * For every (b, h), with a_t = exp(A_h delta_t), u_t = delta_t x_t B_t^T:
 *   G = dh_final                       (adjoint of h_{T-1}; 0 when NULL)
 *   for t = T-1 .. 0:
 *     G        += dy_t C_t^T           (y_t = h_t C_t + D x_t)
 *     dC_t     += h_t^T dy_t
 *     dx_t      = delta_t G B_t + D dy_t
 *     dB_t     += delta_t G^T x_t
 *     ddelta_t  = <G, x_t B_t^T> + A_h a_t <G, h_{t-1}>
 *     dA_h     += delta_t a_t <G, h_{t-1}>
 *     dD_h     += dy_t . x_t
 *     ddt_t     = ddelta_t softplus'(z_t) [dt_min <= softplus(z_t) <= dt_max]
 *     ddt_bias_h += ddt_t
 *     G         = a_t G                (adjoint of h_{t-1})
 *   dh0 = G.
 * z_t = dt_t + dt_bias_h; softplus'(z) = 1 / (1 + e^-z); the clamp passes the
 * derivative on its closed interval and stops it outside.  dB and dC sum over
 * the heads of a group.  dy has the dtype of x.  Outputs are double: dx, dy-
 * shaped (Bsz,T,H,P); ddt (Bsz,T,H); dB, dC (Bsz,T,G,N); dA, dD, ddt_bias (H);
 * dh0 (Bsz,H,P,N) or NULL; da (Bsz,T,H) or NULL receives the gradient of
 * the step's log-decay A_h delta_t, a_t <G, h_{t-1}> (dA_h sums delta_t da_t).
 * The states h_0 .. h_{T-1} of one (b, h) are kept
 * (T P N doubles per thread); each thread sums dB and dC over its heads
 * and the sums are added at the end.
 */
int ssd_oracle_bwd(const void *x, const float *dt, const float *A, const void *B,
                   const void *C, const float *D, const float *dt_bias, double dt_min,
                   double dt_max, const float *h0, const void *dy, const float *dh_final,
                   double *dx, double *ddt, double *dA, double *dB, double *dC, double *dD,
                   double *ddt_bias, double *dh0, double *da, int Bsz, int T, int H, int P,
                   int G, int N, int dtype)
{
    if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G)
        return 1;
    const int hpg = H / G;
    const size_t PN = (size_t)P * N;
    memset(dB, 0, sizeof(double) * (size_t)Bsz * T * G * N);
    memset(dC, 0, sizeof(double) * (size_t)Bsz * T * G * N);
    int fail = 0;
    /* per head: sums over the batch, reduced after the parallel loop */
    double *pA = calloc((size_t)Bsz * H, sizeof(double));
    double *pD = calloc((size_t)Bsz * H, sizeof(double));
    double *pbias = calloc((size_t)Bsz * H, sizeof(double));
    if (!pA || !pD || !pbias) {
        free(pA); free(pD); free(pbias);
        return 2;
    }
    const long long BH = (long long)Bsz * H;
    const size_t nbc = (size_t)Bsz * T * G * N;
#pragma omp parallel
    {
#pragma omp single
        record_threads();
        double *hist = malloc(sizeof(double) * ((size_t)T + 1) * PN);
        double *Gm = malloc(sizeof(double) * PN);
        double *dlt = malloc(sizeof(double) * ((size_t)T + 1));
        /* this thread's sums over its heads of dB and dC */
        double *dBt = calloc(nbc ? nbc : 1, sizeof(double));
        double *dCt = calloc(nbc ? nbc : 1, sizeof(double));
        const int ok = hist && Gm && dlt && dBt && dCt;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic)
        for (long long bh = 0; bh < BH; ++bh) {
            if (!ok)
                continue;
            const int b = (int)(bh / H), h = (int)(bh % H), g = h / hpg;
            {
                const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
                const double Ah = (double)A[h];
                const double Dh = D ? (double)D[h] : 0.0;
                /* forward: hist[0] = h0, hist[t+1] = h_t */
                for (size_t i = 0; i < PN; ++i)
                    hist[i] = h0 ? (double)h0[((size_t)b * H + h) * PN + i] : 0.0;
                for (int t = 0; t < T; ++t) {
                    const size_t row = (size_t)b * T + t;
                    const double delta = ssd_oracle_delta((double)dt[row * H + h], bias, dt_min, dt_max);
                    dlt[t] = delta;
                    const double a = exp(Ah * delta);
                    const double *hp = hist + (size_t)t * PN;
                    double *hn = hist + ((size_t)t + 1) * PN;
                    for (int p = 0; p < P; ++p) {
                        const double xp = load_in(x, (row * H + h) * P + p, dtype);
                        for (int n = 0; n < N; ++n)
                            hn[(size_t)p * N + n] = a * hp[(size_t)p * N + n] +
                                delta * xp * load_in(B, (row * G + g) * N + n, dtype);
                    }
                }
                /* backward */
                for (size_t i = 0; i < PN; ++i)
                    Gm[i] = dh_final ? (double)dh_final[((size_t)b * H + h) * PN + i] : 0.0;
                for (int t = T - 1; t >= 0; --t) {
                    const size_t row = (size_t)b * T + t;
                    const double delta = dlt[t];
                    const double a = exp(Ah * delta);
                    const double *ht = hist + ((size_t)t + 1) * PN;
                    const double *hprev = hist + (size_t)t * PN;
                    /* G += dy_t C_t^T ; dC_t += h_t^T dy_t */
                    for (int p = 0; p < P; ++p) {
                        const double dyp = load_in(dy, (row * H + h) * P + p, dtype);
                        for (int n = 0; n < N; ++n) {
                            Gm[(size_t)p * N + n] += dyp * load_in(C, (row * G + g) * N + n, dtype);
                            dCt[(row * G + g) * N + n] += ht[(size_t)p * N + n] * dyp;
                        }
                    }
                    double gx_b = 0.0, g_hprev = 0.0, dyx = 0.0;
                    for (int p = 0; p < P; ++p) {
                        const double xp = load_in(x, (row * H + h) * P + p, dtype);
                        const double dyp = load_in(dy, (row * H + h) * P + p, dtype);
                        double gb = 0.0;
                        for (int n = 0; n < N; ++n) {
                            const double bn = load_in(B, (row * G + g) * N + n, dtype);
                            const double gv = Gm[(size_t)p * N + n];
                            gb += gv * bn;
                            dBt[(row * G + g) * N + n] += delta * gv * xp;
                            g_hprev += gv * hprev[(size_t)p * N + n];
                        }
                        dx[(row * H + h) * P + p] = delta * gb + Dh * dyp;
                        gx_b += xp * gb;
                        dyx += dyp * xp;
                    }
                    const double ddelta = gx_b + Ah * a * g_hprev;
                    if (da)
                        da[row * H + h] = a * g_hprev;
                    pA[(size_t)b * H + h] += delta * a * g_hprev;
                    pD[(size_t)b * H + h] += dyx;
                    const double z = (double)dt[row * H + h] + bias;
                    const double sp = ssd_oracle_softplus(z);
                    const double pass = (sp >= dt_min && sp <= dt_max) ? 1.0 : 0.0;
                    const double d = ddelta * pass / (1.0 + exp(-z));
                    ddt[row * H + h] = d;
                    pbias[(size_t)b * H + h] += d;
                    for (size_t i = 0; i < PN; ++i)
                        Gm[i] *= a;
                }
                if (dh0)
                    for (size_t i = 0; i < PN; ++i)
                        dh0[((size_t)b * H + h) * PN + i] = Gm[i];
            }
        }
#pragma omp critical
        if (ok) {
            for (size_t i = 0; i < nbc; ++i) {
                dB[i] += dBt[i];
                dC[i] += dCt[i];
            }
        }
        free(hist);
        free(Gm);
        free(dlt);
        free(dBt);
        free(dCt);
    }
    for (int h = 0; h < H; ++h) {
        double sa = 0.0, sd = 0.0, sb = 0.0;
        for (int b = 0; b < Bsz; ++b) {
            sa += pA[(size_t)b * H + h];
            sd += pD[(size_t)b * H + h];
            sb += pbias[(size_t)b * H + h];
        }
        dA[h] = sa;
        dD[h] = sd;
        ddt_bias[h] = sb;
    }
    free(pA);
    free(pD);
    free(pbias);
    return fail ? 2 : 0;
}

/*
 * Gradient of  loss = sum_t dy_t . y_t + <dh_final, h_final>_R  through the
 * complex recurrence of ssd_oracle_complex_fwd (Mamba-3-Lite README, the
 * complex recurrence; Block Anatomy, section 7, pitfall 7: the gradient of
 * the complex A is complex).  <u, v>_R = sum Re(conj(u) v), the real inner
 * product of the arrays as (re, im) pairs.  Every complex gradient is
 * returned as (dL/d re, dL/d im).  The reverse-mode derivative, one step at a
 * time from the last token:
 *   G      = dL/dh_t  (starts as dh_final, gains dy_t conj(C_t) at step t,
 *            and reaches h_{t-1} as conj(a_t) G)
 *   dx_t   = Re(sum_n conj(G[p][n]) B_t[n])
 *   dB_t   = sum_p x_t[p] G[p][n]          dC_t = sum_p dy_t[p] conj(h_t[p][n])
 *   q_t    = conj(a_t) sum G conj(h_{t-1})  (the gradient of the step's
 *            exponent A delta_t)
 *   dA    += delta_t q_t,   d delta_t = Re(A conj(q_t)),   dh0 = G after t = 0,
 * and the clamp and softplus of the step size as in ssd_oracle_bwd.
 * Layouts as ssd_oracle_complex_fwd; outputs double: dx (Bsz,T,H,P), ddt
 * (Bsz,T,H), dA (H,2), dB/dC (Bsz,T,G,N,2), ddt_bias (H), dh0 (Bsz,H,P,N,2)
 * (may be NULL), q (Bsz,T,H,2) (may be NULL).
 */
int ssd_oracle_complex_bwd(const float *x, const float *dt, const float *A, const float *B,
                           const float *C, const float *dt_bias, double dt_min, double dt_max,
                           const float *h0, const float *dy, const float *dh_final,
                           double *dx, double *ddt, double *dA, double *dB, double *dC,
                           double *ddt_bias, double *dh0, double *qout, int Bsz, int T, int H,
                           int P, int G, int N)
{
    if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G)
        return 1;
    const int hpg = H / G;
    const size_t PN2 = (size_t)P * N * 2;
    const size_t nbc = (size_t)Bsz * T * G * N * 2;
    memset(dB, 0, sizeof(double) * nbc);
    memset(dC, 0, sizeof(double) * nbc);
    int fail = 0;
    double *pA = calloc((size_t)Bsz * H * 2, sizeof(double));
    double *pbias = calloc((size_t)Bsz * H, sizeof(double));
    if (!pA || !pbias) {
        free(pA); free(pbias);
        return 2;
    }
    const long long BH = (long long)Bsz * H;
#pragma omp parallel
    {
#pragma omp single
        record_threads();
        double *hist = malloc(sizeof(double) * ((size_t)T + 1) * PN2);
        double *Gm = malloc(sizeof(double) * PN2);
        double *dlt = malloc(sizeof(double) * ((size_t)T + 1));
        double *dBt = calloc(nbc ? nbc : 1, sizeof(double));
        double *dCt = calloc(nbc ? nbc : 1, sizeof(double));
        const int ok = hist && Gm && dlt && dBt && dCt;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic)
        for (long long bh = 0; bh < BH; ++bh) {
            if (!ok)
                continue;
            const int b = (int)(bh / H), h = (int)(bh % H), g = h / hpg;
            const double al = (double)A[2 * h], be = (double)A[2 * h + 1];
            const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
            /* forward: hist[0] = h0, hist[t+1] = h_t */
            for (size_t i = 0; i < PN2; ++i)
                hist[i] = h0 ? (double)h0[(size_t)bh * PN2 + i] : 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t row = (size_t)b * T + t;
                const double delta = ssd_oracle_delta((double)dt[row * H + h], bias, dt_min, dt_max);
                dlt[t] = delta;
                const double mag = exp(al * delta);
                const double ar = mag * cos(be * delta), ai = mag * sin(be * delta);
                const double *hp = hist + (size_t)t * PN2;
                double *hn = hist + ((size_t)t + 1) * PN2;
                const size_t bo = (row * G + g) * (size_t)N * 2;
                for (int p = 0; p < P; ++p) {
                    const double xp = (double)x[(row * H + h) * P + p];
                    for (int n = 0; n < N; ++n) {
                        const size_t e = ((size_t)p * N + n) * 2;
                        hn[e] = ar * hp[e] - ai * hp[e + 1] + xp * B[bo + 2 * n];
                        hn[e + 1] = ar * hp[e + 1] + ai * hp[e] + xp * B[bo + 2 * n + 1];
                    }
                }
            }
            /* backward */
            for (size_t i = 0; i < PN2; ++i)
                Gm[i] = dh_final ? (double)dh_final[(size_t)bh * PN2 + i] : 0.0;
            for (int t = T - 1; t >= 0; --t) {
                const size_t row = (size_t)b * T + t;
                const double delta = dlt[t];
                const double mag = exp(al * delta);
                const double ar = mag * cos(be * delta), ai = mag * sin(be * delta);
                const double *ht = hist + ((size_t)t + 1) * PN2;
                const double *hprev = hist + (size_t)t * PN2;
                const size_t bo = (row * G + g) * (size_t)N * 2;
                /* G += dy_t conj(C_t);  dC_t += dy_t conj(h_t) */
                for (int p = 0; p < P; ++p) {
                    const double dyp = (double)dy[(row * H + h) * P + p];
                    for (int n = 0; n < N; ++n) {
                        const size_t e = ((size_t)p * N + n) * 2;
                        Gm[e] += dyp * C[bo + 2 * n];
                        Gm[e + 1] -= dyp * C[bo + 2 * n + 1];
                        dCt[bo + 2 * n] += dyp * ht[e];
                        dCt[bo + 2 * n + 1] -= dyp * ht[e + 1];
                    }
                }
                double gar = 0.0, gai = 0.0; /* sum G conj(h_{t-1}) */
                for (int p = 0; p < P; ++p) {
                    const double xp = (double)x[(row * H + h) * P + p];
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n) {
                        const size_t e = ((size_t)p * N + n) * 2;
                        const double gr = Gm[e], gi = Gm[e + 1];
                        acc += gr * B[bo + 2 * n] + gi * B[bo + 2 * n + 1]; /* Re(conj(G) B) */
                        dBt[bo + 2 * n] += xp * gr;
                        dBt[bo + 2 * n + 1] += xp * gi;
                        gar += gr * hprev[e] + gi * hprev[e + 1];
                        gai += gi * hprev[e] - gr * hprev[e + 1];
                    }
                    dx[(row * H + h) * P + p] = acc;
                }
                /* q = conj(a) Ga */
                const double qr = ar * gar + ai * gai, qi = ar * gai - ai * gar;
                if (qout) {
                    qout[(row * H + h) * 2] = qr;
                    qout[(row * H + h) * 2 + 1] = qi;
                }
                pA[((size_t)b * H + h) * 2] += delta * qr;
                pA[((size_t)b * H + h) * 2 + 1] += delta * qi;
                const double ddelta = al * qr + be * qi; /* Re(A conj(q)) */
                const double z = (double)dt[row * H + h] + bias;
                const double sp = ssd_oracle_softplus(z);
                const double pass = (sp >= dt_min && sp <= dt_max) ? 1.0 : 0.0;
                const double d = ddelta * pass / (1.0 + exp(-z));
                ddt[row * H + h] = d;
                pbias[(size_t)b * H + h] += d;
                /* G reaches h_{t-1}: G <- conj(a) G */
                for (size_t e = 0; e < PN2; e += 2) {
                    const double gr = Gm[e], gi = Gm[e + 1];
                    Gm[e] = ar * gr + ai * gi;
                    Gm[e + 1] = ar * gi - ai * gr;
                }
            }
            if (dh0)
                memcpy(dh0 + (size_t)bh * PN2, Gm, sizeof(double) * PN2);
        }
#pragma omp critical
        if (ok) {
            for (size_t i = 0; i < nbc; ++i) {
                dB[i] += dBt[i];
                dC[i] += dCt[i];
            }
        }
        free(hist);
        free(Gm);
        free(dlt);
        free(dBt);
        free(dCt);
    }
    for (int h = 0; h < H; ++h) {
        double sr = 0.0, si = 0.0, sb = 0.0;
        for (int b = 0; b < Bsz; ++b) {
            sr += pA[((size_t)b * H + h) * 2];
            si += pA[((size_t)b * H + h) * 2 + 1];
            sb += pbias[(size_t)b * H + h];
        }
        dA[2 * h] = sr;
        dA[2 * h + 1] = si;
        ddt_bias[h] = sb;
    }
    free(pA);
    free(pbias);
    return fail ? 2 : 0;
}
