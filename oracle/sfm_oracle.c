/*
 * sfm_oracle.c -- plain, slow, scalar fp64 CPU oracle for the folded, segmented
 * selective scan and its companions (aux pad, aux swap, boundary-masked
 * depthwise conv1d).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code, header,
 * table or helper with the HIP path, and neither side includes the other.
 *
 * Every array is float64, C-contiguous.  Values that stand for bf16 / f32
 * tensors are passed already upcast (exactly) to float64.  Build with
 * -O2 -ffp-contract=off and no fast-math, so every operation below is one
 * IEEE-754 double operation in the order written.
 *
 * Sources (web pages on SF-Mamba; cited by page title and section):
 *  [SBW]  "Seeing Both Ways, Running One Way" (sungsoo.github.io analysis of
 *         SF-Mamba), section 3.1 (selective SSM recurrence), 3.2 (aux tokens
 *         and swap), 3.3 (batch folding and the periodic reset), 8.1 (method
 *         list: aux init, swap, folding, reset, boundary-safe conv, adaptive B1).
 *  [TL]   "SF-Mamba：重新思考视觉 Mamba 的信息流与并行效率" (techloop.online
 *         walkthrough), sections "第一个模块：Auxiliary Patch Swapping",
 *         "第二个模块：Batch Folding with Periodic State Reset" and its
 *         sub-section on convolution boundaries.
 *  [GS]   "SF-Mamba: Rethinking State Space Model for Vision" (gist.science
 *         summary), Technische Zusammenfassung 2.B (folding equivalence).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - discretization: Abar = exp(Delta*A), Bbar*x = Delta*B*x (zero-order hold of
 *    Mamba, the background model the [SBW] sources name);
 *  - Delta = softplus(delta + bias) with PyTorch's documented softplus
 *    (beta = 1, threshold = 20); optional (softplus_on = 0 gives Delta = delta + bias);
 *  - skip term y += D*u;
 *  - the reset period is the scanned per-sample length L = T + 2 and the reset
 *    falls on the first token of every sample (t mod L == 0);
 *  - the reset re-initialises the state (h <- Bbar*x), which equals Abar = 0 for
 *    finite states;
 *  - fold order: sample b = b1*B2 + j sits at folded positions [j*L, (j+1)*L).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* io rounding codes for values that are stored into an io tensor */
#define ORC_IO_F64 0
#define ORC_IO_F32 1
#define ORC_IO_BF16 2

/* ---------------------------------------------------------------- helpers */

/* Round a double to the nearest bfloat16 value, ties to even, in ONE rounding
 * (bfloat16: 8 exponent bits as float32, 8 significant bits). */
static double round_to_bf16(double v) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    int e;
    frexp(v, &e);                        /* |v| = m * 2^e with m in [0.5, 1) */
    int q = e - 8;                       /* weight of the last kept bit       */
    if (q < -133) q = -133;              /* bf16 subnormal spacing is 2^-133  */
    double scaled = ldexp(v, -q);        /* exact: power-of-two scaling       */
    double r = nearbyint(scaled);        /* default rounding mode: to even    */
    double out = ldexp(r, q);
    if (fabs(out) > 3.3895313892515355e38) out = copysign(INFINITY, v);
    return out;
}

static double round_io(double v, int io) {
    if (io == ORC_IO_F32) return (double)(float)v;
    if (io == ORC_IO_BF16) return round_to_bf16(v);
    return v;
}

/* PyTorch's documented softplus with beta = 1 and threshold = 20 */
static double softplus(double v) {
    return v > 20.0 ? v : log1p(exp(v));
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int oracle_threads(int nthreads) { return set_threads(nthreads); }

int oracle_round_io(const double* in, double* out, int64_t n, int io) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_io(in[i], io);
    return 0;
}

/* ------------------------------------------------------------------ aux pad
 * [SBW] 3.2 and [TL] "第一个模块": the sequence (x_1..x_T) gets a head and a
 * tail aux token, both initialised with the mean of the patch tokens, so the
 * scanned length becomes T + 2.  Mean: float64 sum in index order, divided by
 * T, rounded once to the io type.
 */
int oracle_aux_pad(const double* x, double* out, int64_t B, int64_t D, int64_t T, int io) {
    if (T < 1) return 2;
    const int64_t L = T + 2;
    for (int64_t r = 0; r < B * D; ++r) {
        const double* xr = x + r * T;
        double* o = out + r * L;
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t) s += xr[t];
        double m = round_io(s / (double)T, io);
        o[0] = m;
        for (int64_t t = 0; t < T; ++t) o[1 + t] = xr[t];
        o[T + 1] = m;
    }
    return 0;
}

/* ----------------------------------------------------------------- aux swap
 * [SBW] 3.2 and [TL] "第一个模块": the next layer's head token is this layer's
 * tail output and the next layer's tail token is this layer's head output.
 */
int oracle_aux_swap(const double* y, double* out, int64_t B, int64_t D, int64_t L) {
    for (int64_t r = 0; r < B * D; ++r) {
        const double* yr = y + r * L;
        double* o = out + r * L;
        for (int64_t t = 0; t < L; ++t) o[t] = yr[t];
        o[0] = yr[L - 1];
        o[L - 1] = yr[0];
    }
    return 0;
}

/* ----------------------------------------------- boundary-masked dwconv1d
 * [TL] sub-section on convolution boundaries and [SBW] 8.1 item 5: the block's
 * depthwise 1-D convolution must not reach across sample boundaries of the
 * folded data.  Per sample that is a zero-padded depthwise conv:
 *   out[b,d,t] = act(bias[d] + sum_j w[d,j] * x[b,d,t+j-P]),
 * with x taken as 0 outside [0, L).  act: 0 = identity, 1 = SiLU.
 */
int oracle_dwconv1d(const double* x, const double* w, const double* bias, double* out,
                    int64_t B, int64_t D, int64_t L, int64_t K, int64_t P, int act, int nthreads) {
    if (K < 1 || P < 0 || P >= K) return 2;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < B * D; ++r) {
        const int64_t d = r % D;
        const double* xr = x + r * L;
        double* o = out + r * L;
        for (int64_t t = 0; t < L; ++t) {
            double acc = bias ? bias[d] : 0.0;
            for (int64_t j = 0; j < K; ++j) {
                int64_t src = t + j - P;
                double xv = (src >= 0 && src < L) ? xr[src] : 0.0;
                acc += w[d * K + j] * xv;
            }
            if (act == 1) acc = acc / (1.0 + exp(-acc));
            o[t] = acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------ selective scan, per sample
 * [SBW] 3.1: h_t = Abar_t h_{t-1} + Bbar_t x_t,  y_t = C_t h_t, here with
 * Abar = exp(Delta*A[d,n]), Bbar_t x_t = Delta*B[b,n,t]*u[b,d,t], plus D*u.
 * Each sample starts from h = 0, which is what the periodic reset of the
 * folded form reproduces ([SBW] 3.3, [GS] 2.B).
 * Layouts: u, delta, y [B,D,L]; Bm, Cm [B,N,L]; A [D,N]; Dskip, bias [D] (may be NULL).
 */
int oracle_selective_scan(const double* u, const double* delta, const double* A,
                          const double* Bm, const double* Cm, const double* Dskip,
                          const double* delta_bias, int softplus_on, double* y,
                          int64_t B, int64_t D, int64_t N, int64_t L, int nthreads) {
    if (N < 1 || N > 64 || L < 1) return 2;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < B * D; ++r) {
        const int64_t b = r / D, d = r % D;
        double h[64];
        for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double ut = u[r * L + t];
            double v = delta[r * L + t] + (delta_bias ? delta_bias[d] : 0.0);
            const double dt = softplus_on ? softplus(v) : v;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(dt * A[d * N + n]);
                const double bx = dt * Bm[(b * N + n) * L + t] * ut;
                h[n] = abar * h[n] + bx;
                acc += Cm[(b * N + n) * L + t] * h[n];
            }
            y[r * L + t] = acc + (Dskip ? Dskip[d] : 0.0) * ut;
        }
    }
    return 0;
}

/* ------------------------------------------------------ selective scan, folded
 * [SBW] 3.3 / [TL] "第二个模块": Z in R^{B x D x L} viewed as R^{B1 x D x (B2*L)}
 * (B = B1*B2, sample b = b1*B2 + j occupies folded positions [j*L, (j+1)*L)),
 * scanned as ONE long sequence per (b1, d) with Abar set to zero at every
 * position s with s mod L == 0, realised as state re-initialisation.
 * Kept as a separate code path so the test suite can check that folding with
 * the reset reproduces the per-sample result exactly ([GS] 2.B).
 */
int oracle_selective_scan_folded(const double* u, const double* delta, const double* A,
                                 const double* Bm, const double* Cm, const double* Dskip,
                                 const double* delta_bias, int softplus_on, double* y,
                                 int64_t B1, int64_t B2, int64_t D, int64_t N, int64_t L,
                                 int nthreads) {
    if (N < 1 || N > 64 || L < 1 || B1 < 1 || B2 < 1) return 2;
    set_threads(nthreads);
    const int64_t S = B2 * L;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < B1 * D; ++row) {
        const int64_t b1 = row / D, d = row % D;
        double h[64];
        for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
        for (int64_t s = 0; s < S; ++s) {
            const int64_t b = b1 * B2 + s / L;   /* fold index map */
            const int64_t t = s % L;
            const int reset = (s % L) == 0;       /* Abar_s = 0 at sample starts */
            const int64_t ix = (b * D + d) * L + t;
            const double ut = u[ix];
            double v = delta[ix] + (delta_bias ? delta_bias[d] : 0.0);
            const double dt = softplus_on ? softplus(v) : v;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double bx = dt * Bm[(b * N + n) * L + t] * ut;
                if (reset) {
                    h[n] = bx;
                } else {
                    const double abar = exp(dt * A[d * N + n]);
                    h[n] = abar * h[n] + bx;
                }
                acc += Cm[(b * N + n) * L + t] * h[n];
            }
            y[ix] = acc + (Dskip ? Dskip[d] : 0.0) * ut;
        }
    }
    return 0;
}

/* ================================================================ backward
 * Gradients of the per-sample forward above with respect to all of its inputs,
 * for an upstream gradient dy = dLoss/dy.  The pages give the forward only (the
 * method is trained end to end, [SBW] 3.3 / [TL] "第二个模块"); the backward
 * here is the chain rule applied to exactly that definition, written out in
 * reverse time for each (sample, channel):
 *   z_t = cb + sum_j w_j x~_{t+j-P}, u_t = act(z_t)   (u_t = x_t without conv)
 *   v_t = delta_t + bias, Delta_t = softplus(v_t)     (or v_t)
 *   h_0 = Delta_0 B_0 u_0 (reset), h_t = a_t h_{t-1} + Delta_t B_t u_t, a_t = exp(Delta_t A)
 *   y_t = sum_n C_t h_t + D u_t
 * G_t = dLoss/dh_t collects dy_t C_t and, through h_{t+1} = a_{t+1} h_t + ..,
 * a_{t+1} G_{t+1}; nothing flows across the reset into the previous sample.
 * Softplus keeps PyTorch's threshold: its derivative is exactly 1 above 20.
 * Per-channel gradients (dA, dD, dbias, dw, dcb) are summed over samples and
 * positions, dB and dC over channels, each in increasing index order.
 * Layouts as the forward; outputs are overwritten.  Pass conv_w = NULL for no
 * conv (then dx is du); dconv_w / dconv_b are then not touched.
 */
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

int oracle_selective_scan_bwd(const double* x, const double* delta, const double* A,
                              const double* Bm, const double* Cm, const double* Dskip,
                              const double* delta_bias, int softplus_on,
                              const double* conv_w, const double* conv_b, int64_t K, int64_t P, int act,
                              const double* dy,
                              double* dx, double* ddelta, double* dA, double* dBm, double* dCm,
                              double* dDskip, double* ddelta_bias, double* dconv_w, double* dconv_b,
                              int64_t B, int64_t D, int64_t N, int64_t L, int nthreads) {
    if (N < 1 || N > 64 || L < 1) return 2;
    if (conv_w && (K < 1 || P < 0 || P >= K)) return 2;
    const int64_t KK = conv_w ? K : 0;
    set_threads(nthreads);
    /* per-(b, d) partial sums of the per-channel gradients, reduced afterwards in
     * increasing b so the result does not depend on the thread count */
    const int64_t pc = N + 2 + KK + (conv_w ? 1 : 0);
    double* part = (double*)calloc((size_t)(B * D * pc), sizeof(double));
    /* per-(b, d) contributions to dB, dC: [B, D, N, L] */
    double* pbc = (double*)calloc((size_t)(2 * B * D * N * L), sizeof(double));
    int fail = (part == NULL || pbc == NULL);
    if (!fail) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < B * D; ++r) {
            const int64_t b = r / D, d = r % D;
            double* z = (double*)malloc((size_t)L * sizeof(double));
            double* u = (double*)malloc((size_t)L * sizeof(double));
            double* v = (double*)malloc((size_t)L * sizeof(double));
            double* dt = (double*)malloc((size_t)L * sizeof(double));
            double* h = (double*)malloc((size_t)(L * N) * sizeof(double));   /* h[t*N + n] */
            double* a = (double*)malloc((size_t)(L * N) * sizeof(double));   /* a[t*N + n] */
            double* du = (double*)malloc((size_t)L * sizeof(double));
            double* dz = (double*)malloc((size_t)L * sizeof(double));
            double G[64];
            const double* xr = x + r * L;
            /* forward, keeping every intermediate */
            for (int64_t t = 0; t < L; ++t) {
                if (conv_w) {
                    double acc = conv_b ? conv_b[d] : 0.0;
                    for (int64_t j = 0; j < K; ++j) {
                        const int64_t s = t + j - P;
                        acc += conv_w[d * K + j] * ((s >= 0 && s < L) ? xr[s] : 0.0);
                    }
                    z[t] = acc;
                    u[t] = act == 1 ? acc * sigmoid(acc) : acc;
                } else {
                    z[t] = xr[t];
                    u[t] = xr[t];
                }
                v[t] = delta[r * L + t] + (delta_bias ? delta_bias[d] : 0.0);
                dt[t] = softplus_on ? softplus(v[t]) : v[t];
                for (int64_t n = 0; n < N; ++n) {
                    const double bx = dt[t] * Bm[(b * N + n) * L + t] * u[t];
                    if (t == 0) {
                        a[n] = 0.0;
                        h[n] = bx;
                    } else {
                        a[t * N + n] = exp(dt[t] * A[d * N + n]);
                        h[t * N + n] = a[t * N + n] * h[(t - 1) * N + n] + bx;
                    }
                }
            }
            /* reverse time */
            double* pr = part + r * pc;   /* [dA (N), dD, dbias, dw (KK), dcb] */
            for (int64_t n = 0; n < N; ++n) G[n] = 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const double g = dy[r * L + t];
                double ddt = 0.0;
                du[t] = (Dskip ? Dskip[d] : 0.0) * g;
                pr[N] += g * u[t];
                for (int64_t n = 0; n < N; ++n) {
                    const double Bv = Bm[(b * N + n) * L + t], Cv = Cm[(b * N + n) * L + t];
                    /* G_t = dy_t C_t + a_{t+1} G_{t+1}  (G holds a_{t+1} G_{t+1} here) */
                    G[n] = g * Cv + G[n];
                    pbc[((r * 2 + 1) * N + n) * L + t] = g * h[t * N + n];          /* dC */
                    pbc[((r * 2 + 0) * N + n) * L + t] = G[n] * dt[t] * u[t];       /* dB */
                    du[t] += G[n] * dt[t] * Bv;
                    ddt += G[n] * Bv * u[t];
                    if (t > 0) {
                        const double dat = G[n] * h[(t - 1) * N + n];               /* dLoss/da_t */
                        ddt += dat * a[t * N + n] * A[d * N + n];
                        pr[n] += dat * a[t * N + n] * dt[t];
                        G[n] = a[t * N + n] * G[n];                                 /* -> a_t G_t */
                    } else {
                        G[n] = 0.0;                                                 /* reset */
                    }
                }
                const double dv = softplus_on ? (v[t] > 20.0 ? ddt : ddt * sigmoid(v[t])) : ddt;
                ddelta[r * L + t] = dv;
                pr[N + 1] += dv;
                if (conv_w) {
                    double dact = 1.0;
                    if (act == 1) {
                        const double s = sigmoid(z[t]);
                        dact = s + z[t] * s * (1.0 - s);
                    }
                    dz[t] = du[t] * dact;
                } else {
                    dz[t] = du[t];
                }
            }
            if (conv_w) {
                for (int64_t s = 0; s < L; ++s) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < K; ++j) {
                        const int64_t t = s + P - j;
                        if (t >= 0 && t < L) acc += conv_w[d * K + j] * dz[t];
                    }
                    dx[r * L + s] = acc;
                }
                for (int64_t j = 0; j < K; ++j) {
                    double acc = 0.0;
                    for (int64_t t = 0; t < L; ++t) {
                        const int64_t s = t + j - P;
                        if (s >= 0 && s < L) acc += dz[t] * xr[s];
                    }
                    pr[N + 2 + j] = acc;
                }
                double acc = 0.0;
                for (int64_t t = 0; t < L; ++t) acc += dz[t];
                pr[N + 2 + K] = acc;
            } else {
                for (int64_t t = 0; t < L; ++t) dx[r * L + t] = dz[t];
            }
            free(z); free(u); free(v); free(dt); free(h); free(a); free(du); free(dz);
        }
        /* reductions in increasing index order */
        for (int64_t d = 0; d < D; ++d) {
            for (int64_t k = 0; k < pc; ++k) {
                double acc = 0.0;
                for (int64_t b = 0; b < B; ++b) acc += part[(b * D + d) * pc + k];
                if (k < N) dA[d * N + k] = acc;
                else if (k == N) { if (dDskip) dDskip[d] = acc; }
                else if (k == N + 1) { if (ddelta_bias) ddelta_bias[d] = acc; }
                else if (k < N + 2 + KK) dconv_w[d * K + (k - N - 2)] = acc;
                else if (dconv_b) dconv_b[d] = acc;
            }
        }
        for (int64_t b = 0; b < B; ++b)
            for (int64_t n = 0; n < N; ++n)
                for (int64_t t = 0; t < L; ++t) {
                    double sb = 0.0, sc = 0.0;
                    for (int64_t d = 0; d < D; ++d) {
                        const int64_t r = b * D + d;
                        sb += pbc[((r * 2 + 0) * N + n) * L + t];
                        sc += pbc[((r * 2 + 1) * N + n) * L + t];
                    }
                    dBm[(b * N + n) * L + t] = sb;
                    dCm[(b * N + n) * L + t] = sc;
                }
    }
    free(part);
    free(pbc);
    return fail ? 3 : 0;
}

/* Backward of the aux pad: the mean feeds both end tokens, so each unpadded
 * token receives its own padded gradient plus (g_0 + g_{L-1}) / T.  The io
 * rounding of the mean is passed through as the identity. */
int oracle_aux_pad_bwd(const double* dxp, double* dx, int64_t B, int64_t D, int64_t T) {
    if (T < 1) return 2;
    const int64_t L = T + 2;
    for (int64_t r = 0; r < B * D; ++r) {
        const double* g = dxp + r * L;
        const double ends = (g[0] + g[L - 1]) / (double)T;
        for (int64_t t = 0; t < T; ++t) dx[r * T + t] = g[1 + t] + ends;
    }
    return 0;
}
