/*
 * gn_oracle.c -- plain fp64 CPU reference for 3D GroupNorm forward and backward.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU library never links, includes
 * or calls it, and it shares no code, header, table or helper with the GPU path.
 *
 * What it computes (the GroupNorm definition, written out with no blocking,
 * fusion or reordering):
 *   - "Optimize GroupNorm" (LBANN/ScaFFold pull 93), paragraph on ATen's
 *     per-(batch, group) statistics and FastGroupNorm: statistics are taken per
 *     (sample n, group g) over the group's C/G channels and all D*H*W voxels.
 *   - Same page, paragraph on the independent review: a single-element group has
 *     rstd = 316, i.e. rstd = 1/sqrt(var + eps) with eps = 1e-5 inside the square
 *     root and the biased (divide by M) variance; its input gradient is exactly 0.
 *   - "Preserve GroupNorm dtype" (LBANN/ScaFFold pull 105), first paragraph: the
 *     normalized value is the unrounded answer, rounded once to the output dtype.
 *     Here that answer is computed in fp64 and the rounding helpers below round
 *     straight from fp64 (never through fp32).
 *   - Optional ReLU after the affine ("Optimize GroupNorm", paragraphs on the rung ladder
 *     with the fused ReLU and on the NaN-correct ReLU): relu(v) = 0 where v < 0, else v, so
 *     NaN, +Inf and -0.0 pass unchanged and -Inf becomes 0, as torch's F.relu does; its
 *     gradient passes where the relu result is > 0 or NaN and is 0 where it is <= 0.
 *   - The backward is the calculus of the forward (the pages print no formula):
 *       xhat = (x - mu) * rstd
 *       s1[n,c] = sum_s dy,   s2[n,c] = sum_s dy * xhat
 *       c1[n,g] = (1/M) sum_{c in g} gamma_c s1[n,c]
 *       c2[n,g] = (1/M) sum_{c in g} gamma_c s2[n,c]
 *       dx = rstd * (gamma_c * dy - c1 - xhat * c2)
 *       dgamma_c = sum_n s2[n,c],  dbeta_c = sum_n s1[n,c]
 *     With the ReLU, dy above is replaced by the gated gradient g = gate(relu(pre)) * dy,
 *     pre = gamma_c * xhat + beta_c.
 *
 * Layout: NCDHW contiguous; S = D*H*W; group (n, g) is the contiguous run of
 * M = (C/G)*S elements that starts at (n*C + g*C/G)*S.
 *
 * Inputs are decoded exactly to fp64: fp32, bf16 (the upper half of an fp32) and fp16
 * (IEEE binary16) widen exactly; fp64 input is taken as is (used by the
 * finite-difference pins).
 * gamma/beta are fp32 as the GPU receives them; eps is the fp32 value widened.
 *
 * Parity pins live in tests/test_oracle.py (closed forms, an independent library,
 * exact rational brute force, finite differences).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GNO_F32 0
#define GNO_BF16 1
#define GNO_F64 2
#define GNO_F16 3

/*
 * IEEE binary16: sign bit, 5 exponent bits with bias 15, 10 fraction bits. Exponent 0
 * holds zero and the subnormals fraction * 2^-24; exponent 31 holds the infinities
 * (fraction 0) and NaN; otherwise the value is (1024 + fraction) * 2^(exponent - 25).
 */
static double gno_f16_value(uint16_t h)
{
    const int e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(f + 1024), e - 25);
    return (h & 0x8000) ? -v : v;
}

void gno_f16_decode_array(const uint16_t* h, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = gno_f16_value(h[i]);
}

static double gno_load(const void* p, int dt, int64_t i)
{
    if (dt == GNO_F32) return (double)((const float*)p)[i];
    if (dt == GNO_F16) return gno_f16_value(((const uint16_t*)p)[i]);
    if (dt == GNO_BF16) {
        uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return ((const double*)p)[i];
}

static double gno_gamma(const float* gamma, int64_t c) { return gamma ? (double)gamma[c] : 1.0; }
static double gno_beta(const float* beta, int64_t c) { return beta ? (double)beta[c] : 0.0; }

/* relu as torch's F.relu: 0 where v < 0, else v (NaN, +Inf, -0.0 unchanged). */
static double gno_relu(double v) { return v < 0.0 ? 0.0 : v; }

/* Gradient gate of the relu: blocks where the relu result r is <= 0, passes otherwise (NaN too). */
static double gno_gate(double r, double g) { return r <= 0.0 ? 0.0 : g; }

/* Shape check shared by every entry point of this file: C divisible by G, all positive. */
static int gno_shape_ok(int64_t N, int64_t C, int64_t S, int64_t G)
{
    return N > 0 && C > 0 && S > 0 && G > 0 && C % G == 0;
}

/*
 * Per-(n, g) statistics, two passes in fp64: the mean, then the biased variance
 * as the mean of squared deviations, then rstd = 1/sqrt(var + eps).
 * Outputs are [N*G]; any of them may be NULL.
 */
int gno_group_stats(const void* x, int x_dt, int64_t N, int64_t C, int64_t S, int64_t G,
                    float eps, double* mean, double* var, double* rstd)
{
    if (!gno_shape_ok(N, C, S, G)) return 1;
    const int64_t Cg = C / G, M = Cg * S;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t base = (n * C + g * Cg) * S;
            double sum = 0.0;
            for (int64_t i = 0; i < M; ++i) sum += gno_load(x, x_dt, base + i);
            const double mu = sum / (double)M;
            double ss = 0.0;
            for (int64_t i = 0; i < M; ++i) {
                const double d = gno_load(x, x_dt, base + i) - mu;
                ss += d * d;
            }
            const double v = ss / (double)M;
            const double r = 1.0 / sqrt(v + (double)eps);
            if (mean) mean[n * G + g] = mu;
            if (var) var[n * G + g] = v;
            if (rstd) rstd[n * G + g] = r;
        }
    }
    return 0;
}

/*
 * Forward: y[i] = gamma_c * (x[i] - mu) * rstd + beta_c for every element, in fp64, then
 * relu(y) if act is non-zero.
 * y is [N*C*S] fp64; mean, var, rstd are [N*G] and may be NULL.
 */
int gno_forward(const void* x, int x_dt, const float* gamma, const float* beta,
                int64_t N, int64_t C, int64_t S, int64_t G, float eps, int act,
                double* y, double* mean, double* var, double* rstd)
{
    if (!gno_shape_ok(N, C, S, G)) return 1;
    const int64_t Cg = C / G;
    double* mu = (double*)malloc(sizeof(double) * N * G);
    double* vr = (double*)malloc(sizeof(double) * N * G);
    double* rs = (double*)malloc(sizeof(double) * N * G);
    if (!mu || !vr || !rs) { free(mu); free(vr); free(rs); return 2; }
    gno_group_stats(x, x_dt, N, C, S, G, eps, mu, vr, rs);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t c = 0; c < C; ++c) {
            const int64_t ng = n * G + c / Cg;
            const double gm = gno_gamma(gamma, c), bt = gno_beta(beta, c);
            const int64_t base = (n * C + c) * S;
            for (int64_t s = 0; s < S; ++s) {
                const double xhat = (gno_load(x, x_dt, base + s) - mu[ng]) * rs[ng];
                const double pre = gm * xhat + bt;
                y[base + s] = act ? gno_relu(pre) : pre;
            }
        }
    }
    for (int64_t i = 0; i < N * G; ++i) {
        if (mean) mean[i] = mu[i];
        if (var) var[i] = vr[i];
        if (rstd) rstd[i] = rs[i];
    }
    free(mu); free(vr); free(rs);
    return 0;
}

/*
 * Forward at selected flat indices only, given statistics already computed by
 * gno_group_stats (for volumes whose fp64 output would not fit in memory).
 */
int gno_forward_at(const void* x, int x_dt, const float* gamma, const float* beta,
                   int64_t N, int64_t C, int64_t S, int64_t G, int act,
                   const double* mean, const double* rstd,
                   const int64_t* idx, int64_t n_idx, double* y_out)
{
    if (!gno_shape_ok(N, C, S, G)) return 1;
    const int64_t Cg = C / G;
    for (int64_t k = 0; k < n_idx; ++k) {
        const int64_t i = idx[k];
        const int64_t nc = i / S, n = nc / C, c = nc % C, ng = n * G + c / Cg;
        const double xhat = (gno_load(x, x_dt, i) - mean[ng]) * rstd[ng];
        const double pre = gno_gamma(gamma, c) * xhat + gno_beta(beta, c);
        y_out[k] = act ? gno_relu(pre) : pre;
    }
    return 0;
}

/*
 * Backward. Recomputes the statistics itself (it never takes them from a caller),
 * then the per-(n, c) sums, the per-(n, g) coefficients, dx, dgamma and dbeta.
 * dx is [N*C*S] fp64 or NULL (skipped); dgamma, dbeta are [C]; mean, rstd, c1, c2
 * are [N*G] and may be NULL.
 */
int gno_backward(const void* dy, int dy_dt, const void* x, int x_dt, const float* gamma,
                 const float* beta, int act,
                 int64_t N, int64_t C, int64_t S, int64_t G, float eps,
                 double* dx, double* dgamma, double* dbeta,
                 double* mean_out, double* rstd_out, double* c1_out, double* c2_out)
{
    if (!gno_shape_ok(N, C, S, G)) return 1;
    const int64_t Cg = C / G, M = Cg * S;
    double* mu = (double*)malloc(sizeof(double) * N * G);
    double* rs = (double*)malloc(sizeof(double) * N * G);
    double* s1 = (double*)malloc(sizeof(double) * N * C);
    double* s2 = (double*)malloc(sizeof(double) * N * C);
    double* c1 = (double*)malloc(sizeof(double) * N * G);
    double* c2 = (double*)malloc(sizeof(double) * N * G);
    if (!mu || !rs || !s1 || !s2 || !c1 || !c2) {
        free(mu); free(rs); free(s1); free(s2); free(c1); free(c2);
        return 2;
    }
    gno_group_stats(x, x_dt, N, C, S, G, eps, mu, NULL, rs);

    /* per-channel sums of dy and dy * xhat */
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t c = 0; c < C; ++c) {
            const int64_t ng = n * G + c / Cg;
            const int64_t base = (n * C + c) * S;
            const double gm = gno_gamma(gamma, c), bt = gno_beta(beta, c);
            double a = 0.0, b = 0.0;
            for (int64_t s = 0; s < S; ++s) {
                const double xhat = (gno_load(x, x_dt, base + s) - mu[ng]) * rs[ng];
                double g_ = gno_load(dy, dy_dt, base + s);
                if (act) g_ = gno_gate(gno_relu(gm * xhat + bt), g_);
                a += g_;
                b += g_ * xhat;
            }
            s1[n * C + c] = a;
            s2[n * C + c] = b;
        }
    }
    /* per-group coefficients */
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            double a = 0.0, b = 0.0;
            for (int64_t c = g * Cg; c < (g + 1) * Cg; ++c) {
                a += gno_gamma(gamma, c) * s1[n * C + c];
                b += gno_gamma(gamma, c) * s2[n * C + c];
            }
            c1[n * G + g] = a / (double)M;
            c2[n * G + g] = b / (double)M;
        }
    }
    /* input gradient */
    if (dx) {
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t c = 0; c < C; ++c) {
                const int64_t ng = n * G + c / Cg;
                const int64_t base = (n * C + c) * S;
                const double gm = gno_gamma(gamma, c), bt = gno_beta(beta, c);
                for (int64_t s = 0; s < S; ++s) {
                    const double xhat = (gno_load(x, x_dt, base + s) - mu[ng]) * rs[ng];
                    double g_ = gno_load(dy, dy_dt, base + s);
                    if (act) g_ = gno_gate(gno_relu(gm * xhat + bt), g_);
                    dx[base + s] = rs[ng] * (gm * g_ - c1[ng] - xhat * c2[ng]);
                }
            }
        }
    }
    /* parameter gradients */
    for (int64_t c = 0; c < C; ++c) {
        double a = 0.0, b = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            a += s2[n * C + c];
            b += s1[n * C + c];
        }
        if (dgamma) dgamma[c] = a;
        if (dbeta) dbeta[c] = b;
    }
    for (int64_t i = 0; i < N * G; ++i) {
        if (mean_out) mean_out[i] = mu[i];
        if (rstd_out) rstd_out[i] = rs[i];
        if (c1_out) c1_out[i] = c1[i];
        if (c2_out) c2_out[i] = c2[i];
    }
    free(mu); free(rs); free(s1); free(s2); free(c1); free(c2);
    return 0;
}

/*
 * Input gradient at selected flat indices, given the statistics and the
 * coefficients gno_backward returned.
 */
int gno_backward_at(const void* dy, int dy_dt, const void* x, int x_dt, const float* gamma,
                    const float* beta, int act, int64_t N, int64_t C, int64_t S, int64_t G,
                    const double* mean, const double* rstd, const double* c1, const double* c2,
                    const int64_t* idx, int64_t n_idx, double* dx_out)
{
    if (!gno_shape_ok(N, C, S, G)) return 1;
    const int64_t Cg = C / G;
    for (int64_t k = 0; k < n_idx; ++k) {
        const int64_t i = idx[k];
        const int64_t nc = i / S, n = nc / C, c = nc % C, ng = n * G + c / Cg;
        const double xhat = (gno_load(x, x_dt, i) - mean[ng]) * rstd[ng];
        const double gm = gno_gamma(gamma, c);
        double g_ = gno_load(dy, dy_dt, i);
        if (act) g_ = gno_gate(gno_relu(gm * xhat + gno_beta(beta, c)), g_);
        dx_out[k] = rstd[ng] * (gm * g_ - c1[ng] - xhat * c2[ng]);
    }
    return 0;
}

/*
 * Rounding once from fp64 to bf16 (round to nearest, ties to even), straight from
 * the fp64 value. bf16 keeps fp32's 8-bit exponent and 8 significant bits, so:
 * normal results are multiples of 2^(e-7) for 2^e <= |v| < 2^(e+1); results below
 * 2^-126 are multiples of 2^-133 (subnormals); magnitudes that round to 2^128 or
 * more overflow to infinity. NaN becomes the quiet NaN with its sign; infinities
 * keep their sign. Returns the bf16 bit pattern.
 */
static uint16_t gno_bf16_bits_of_exact(double r)
{
    /* r is exactly representable in bf16 (hence in fp32): take the fp32's top half */
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

uint16_t gno_round_bf16(double v)
{
    if (isnan(v)) return signbit(v) ? 0xFFC0 : 0x7FC0;
    const int neg = signbit(v) ? 1 : 0;
    const double a = fabs(v);
    if (isinf(a)) return neg ? 0xFF80 : 0x7F80;
    if (a == 0.0) return neg ? 0x8000 : 0x0000;
    int e;
    frexp(a, &e);            /* a = m * 2^e, 0.5 <= m < 1, so 2^(e-1) <= a < 2^e */
    int q = (e - 1) - 7;     /* quantum exponent for 8 significant bits */
    if (q < -133) q = -133;  /* subnormal range: fixed quantum 2^-133 */
    double k = nearbyint(ldexp(a, -q)); /* exact scaling; default mode rounds ties to even */
    double r = ldexp(k, q);
    if (r >= ldexp(1.0, 128)) return neg ? 0xFF80 : 0x7F80;
    uint16_t bits = gno_bf16_bits_of_exact(r);
    return (uint16_t)(bits | (neg ? 0x8000 : 0));
}

void gno_round_bf16_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = gno_round_bf16(v[i]);
}

/*
 * Rounding once from fp64 to fp16 (round to nearest, ties to even), straight from the
 * fp64 value: 11 significant bits, so normal results are multiples of 2^(e-10) for
 * 2^e <= |v| < 2^(e+1); results below 2^-14 are multiples of 2^-24 (subnormals);
 * magnitudes that round to 2^16 or more overflow to infinity (the largest finite value
 * is 65504). NaN becomes the quiet NaN with its sign. Returns the fp16 bit pattern.
 */
uint16_t gno_round_f16(double v)
{
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00);
    const double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);            /* 2^(e-1) <= a < 2^e */
    int q = (e - 1) - 10;    /* quantum exponent for 11 significant bits */
    if (q < -24) q = -24;    /* subnormal range: fixed quantum 2^-24 */
    const double k = nearbyint(ldexp(a, -q)); /* exact scaling; default mode rounds ties to even */
    const double r = ldexp(k, q);
    if (r >= 65536.0) return (uint16_t)(sign | 0x7C00);
    if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(r, 24)); /* subnormal */
    int er;
    const double m = frexp(r, &er);          /* r = m * 2^er, 0.5 <= m < 1 */
    const int expo = er - 1 + 15;            /* biased exponent of 2^(er-1) */
    const int frac = (int)ldexp(m, 11) - 1024;
    return (uint16_t)(sign | (uint16_t)(expo << 10) | (uint16_t)frac);
}

void gno_round_f16_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = gno_round_f16(v[i]);
}

/* Rounding once from fp64 to fp32: the C conversion rounds to nearest-even. */
void gno_round_f32_array(const double* v, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (float)v[i];
}

/*
 * Per-channel sums of |g| and |g * xhat| (xhat from the given statistics, g = dy or the
 * relu-gated dy): the magnitudes that bound the rounding error of any fp32 summation of
 * dbeta and dgamma.
 */
int gno_channel_abs_sums(const void* dy, int dy_dt, const void* x, int x_dt,
                         const float* gamma, const float* beta, int act,
                         int64_t N, int64_t C, int64_t S, int64_t G,
                         const double* mean, const double* rstd, double* abs_dy, double* abs_dyxhat)
{
    if (!gno_shape_ok(N, C, S, G)) return 1;
    const int64_t Cg = C / G;
    for (int64_t c = 0; c < C; ++c) { abs_dy[c] = 0.0; abs_dyxhat[c] = 0.0; }
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t c = 0; c < C; ++c) {
            const int64_t ng = n * G + c / Cg;
            const int64_t base = (n * C + c) * S;
            double a = 0.0, b = 0.0;
            for (int64_t s = 0; s < S; ++s) {
                const double xhat = (gno_load(x, x_dt, base + s) - mean[ng]) * rstd[ng];
                double g_ = gno_load(dy, dy_dt, base + s);
                if (act) g_ = gno_gate(gno_relu(gno_gamma(gamma, c) * xhat + gno_beta(beta, c)), g_);
                a += fabs(g_);
                b += fabs(g_ * xhat);
            }
            abs_dy[c] += a;
            abs_dyxhat[c] += b;
        }
    }
    return 0;
}

/* The relu and its gradient gate on single values (exposed for their own pins). */
double gno_relu_value(double v) { return gno_relu(v); }
double gno_gate_value(double r, double g) { return gno_gate(r, g); }
