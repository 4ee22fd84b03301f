/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the
 * memory-bound transformer ops: RMSNorm, fused add+RMSNorm, RoPE, fused
 * RMSNorm+RoPE (QK-norm), SiLU-mul, add, embedding gather, greedy argmax.
 *
 * TEST INFRASTRUCTURE ONLY.  The product library never links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no source with the HIP kernels.
 *
 * Also the next rows built after those: softmax over the last axis with a
 * temperature; LayerNorm; GELU-gated multiply (GeGLU, erf and tanh forms);
 * RoPE from a precomputed cos/sin cache; multi-axis RoPE.
 *
 * Sources (web pages; sections named, never line numbers):
 *   [OPS]  "Operations" (glia runtime op spec): 2 Normalization / RmsNorm,
 *          LayerNorm;
 *          3 Position encoding / Rope; 4 Activation / Silu, Gelu, SwiGlu,
 *          GeGlu, Softmax;
 *          5 Attention / QK-norm; 8 Sampling / Greedy; 10 Fused ops.
 *   [ELT]  "Elementwise kernels in C: RMSNorm, RoPE, SiLU-mul, embedding,
 *          add, argmax": 2.1 RMSNorm; 2.2 RoPE; 2.3 SiLU-mul (SwiGLU);
 *          2.4 Embedding, add, argmax; 4 The interface.
 *   [DNN]  "ruDNN User Guide": 7 LayerNorm, RMSNorm, and Softmax.
 *
 * Storage: f32, bf16 or IEEE f16 ([OPS] gives F16 tolerances).
 *
 * Arithmetic: every input is widened exactly to f64; all math is IEEE f64
 * with libm sqrt/exp/sin/cos; every stored output is rounded once (RNE),
 * straight from f64 to the storage type.  Build with
 * -O2 -fno-fast-math -ffp-contract=off so that no fused multiply-add or
 * reassociation changes what is written here.  Rows (tokens) are
 * independent, so the OpenMP loops change no result.
 *
 * Parity: every function is pinned by the CPU tests (worked examples of
 * [ELT] section 3, closed forms, invariants, brute force, library routines,
 * and the mutants of [ELT] section 5).  No function here is parity unpinned.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- storage */

/* IEEE binary16 bits to f64, exactly: sign, 5-bit biased exponent (bias
 * 15), 10-bit fraction; exponent 0 holds the subnormals f * 2^-24, exponent
 * 31 infinity (f = 0) and NaN. */
static double f16_to_f64(uint16_t h) {
    const int sgn = h >> 15, ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + fr), ex - 25);
    return sgn ? -v : v;
}

/* Widen element i of a dt-typed array to f64 (exact for all three types). */
static double ld(int dt, const void* p, int64_t i) {
    if (dt == ORC_BF16) {
        uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dt == ORC_F16) return f16_to_f64(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

/* Round-to-nearest-even from f64 straight to bfloat16 (8 significant bits,
 * the exponent range of f32).  A value in binade e (2^e <= |v| < 2^(e+1))
 * is rounded to a multiple of 2^(e-7); below 2^-126 the spacing stays 2^-133
 * (bf16 subnormals).  Results of magnitude 2^128 or more are infinite. */
uint16_t orc_bf16_from_f64(double v) {
    if (isnan(v)) return signbit(v) ? 0xFFC0u : 0x7FC0u;
    if (isinf(v)) return signbit(v) ? 0xFF80u : 0x7F80u;
    if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
    int e;
    frexp(v, &e);                 /* |v| = m * 2^e with 0.5 <= m < 1 */
    int binade = e - 1;
    if (binade < -126) binade = -126;
    const double q = ldexp(1.0, binade - 7);
    const double r = nearbyint(v / q) * q;   /* ties to even (default mode) */
    const float f = (float)r;                /* exact, or +-inf past 2^128 */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Round-to-nearest-even from f64 straight to IEEE binary16 (11 significant
 * bits, normal exponents -14..15).  A value in binade e is rounded to a
 * multiple of 2^(e-10); below 2^-14 the spacing stays 2^-24 (subnormals).
 * A result of 2^16 or more (|v| >= 65520, halfway past the largest finite
 * 65504, rounds up) is infinite. */
uint16_t orc_f16_from_f64(double v) {
    if (isnan(v)) return signbit(v) ? 0xFE00u : 0x7E00u;
    const uint16_t sign = signbit(v) ? 0x8000u : 0x0000u;
    const double a = fabs(v);
    if (isinf(a)) return sign | 0x7C00u;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a = m * 2^e with 0.5 <= m < 1 */
    int binade = e - 1;
    if (binade < -14) binade = -14;
    const double q = ldexp(1.0, binade - 10);
    const double r = nearbyint(a / q) * q;   /* ties to even (default mode) */
    if (r >= 65536.0) return sign | 0x7C00u;
    if (r < ldexp(1.0, -14))                 /* subnormal: r = k * 2^-24, k < 1024 */
        return sign | (uint16_t)ldexp(r, 24);
    frexp(r, &e);
    const int ex = e - 1;                    /* binade of the rounded value */
    const int fr = (int)(ldexp(r, 10 - ex) - 1024.0);
    return sign | (uint16_t)(((ex + 15) << 10) | fr);
}

/* Store v into element i, rounded once to the storage type. */
static void st(int dt, void* p, int64_t i, double v) {
    if (dt == ORC_BF16)
        ((uint16_t*)p)[i] = orc_bf16_from_f64(v);
    else if (dt == ORC_F16)
        ((uint16_t*)p)[i] = orc_f16_from_f64(v);
    else
        ((float*)p)[i] = (float)v;           /* C conversion: RNE */
}

/* The storage rounding of n values, exported for the tests. */
void orc_round_to(int dt, const double* v, int64_t n, void* out) {
    for (int64_t i = 0; i < n; ++i) st(dt, out, i, v[i]);
}

/* Quiet NaN in the storage type (the row an out-of-range id produces). */
static void st_nan(int dt, void* p, int64_t i) {
    if (dt == ORC_BF16) {
        ((uint16_t*)p)[i] = 0x7FC0u;
    } else if (dt == ORC_F16) {
        ((uint16_t*)p)[i] = 0x7E00u;
    } else {
        const uint32_t u = 0x7FC00000u;
        memcpy((float*)p + i, &u, sizeof u);
    }
}

static double* row_buffer(int64_t n) {
    double* b = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!b) abort();
    return b;
}

/* ---------------------------------------------------------------- RMSNorm */

/* The pages' normalisation statistics are single-precision sums ([ELT] 2.1
 * accumulates the squares in a float; [DNN] 7 keeps its statistics in F32).
 * Where such a sum, or LayerNorm's deviation x - mu, passes the f32 range
 * the single-precision value is +-inf, and so is it here: f32_range maps an
 * f64 value to +-inf from 2^128 - 2^103 on, where round-to-nearest f32
 * overflows.  Below that the f64 value stands (the order of the f32 partial
 * sums is the kernels' own, and a sum whose terms have mixed signs may
 * overflow in a partial sum first: no single value is right there). */
static double f32_range(double v) {
    if (v >= 0x1.ffffffp127) return INFINITY;
    if (v <= -0x1.ffffffp127) return -INFINITY;
    return v;
}

/* [OPS] RmsNorm; [ELT] 2.1: y_i = x_i / sqrt(mean(x^2) + eps) * w_i, with eps
 * inside the root and the mean taken over the row's d entries.  The row is
 * given in f64 and normalised in place; a sum of squares past the f32 range
 * is +inf (f32_range), so the row then maps to x * 0 (NaN where x is
 * infinite). */
static void normalize_row(double* v, int64_t d, int dt, const void* w,
                          float eps) {
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i) ss += v[i] * v[i];
    ss = f32_range(ss);
    const double ms = ss / (double)d;
    const double inv = 1.0 / sqrt(ms + (double)eps);
    for (int64_t i = 0; i < d; ++i) v[i] = v[i] * inv * ld(dt, w, i);
}

void orc_rmsnorm(int dt, const void* x, const void* w, int64_t rows,
                 int64_t d, float eps, double* y64, void* y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double* v = row_buffer(d);
        for (int64_t i = 0; i < d; ++i) v[i] = ld(dt, x, r * d + i);
        normalize_row(v, d, dt, w, eps);
        for (int64_t i = 0; i < d; ++i) {
            if (y64) y64[r * d + i] = v[i];
            if (y) st(dt, y, r * d + i, v[i]);
        }
        free(v);
    }
}

/* [OPS] 10 Fused ops, FusedSkipNorm: h = x + skip (the stored sum, rounded to
 * the storage type) and y = RmsNorm(h); both are returned.  y is the unfused
 * composition, so it normalises h as stored. */
void orc_add_rmsnorm(int dt, const void* x, const void* res, const void* w,
                     int64_t rows, int64_t d, float eps, double* y64, void* y,
                     void* h) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double* v = row_buffer(d);
        for (int64_t i = 0; i < d; ++i) {
            const double hv = ld(dt, x, r * d + i) + ld(dt, res, r * d + i);
            st(dt, h, r * d + i, hv);
        }
        for (int64_t i = 0; i < d; ++i) v[i] = ld(dt, h, r * d + i);
        normalize_row(v, d, dt, w, eps);
        for (int64_t i = 0; i < d; ++i) {
            if (y64) y64[r * d + i] = v[i];
            if (y) st(dt, y, r * d + i, v[i]);
        }
        free(v);
    }
}

/* ------------------------------------------------------------------- RoPE */

/* [ELT] 2.2: the angle of pair i at token t is p_t * w_i formed once in f64
 * and rounded to f32 (equal to f32(p) * f32(w) whenever |p| < 2^24). */
float orc_rope_angle(int32_t p, float w) {
    return (float)((double)p * (double)w);
}

/* [ELT] 2.2: which two entries of a head form pair i.  Layout 0 ("half")
 * pairs (x_i, x_{i+r/2}); layout 1 ("interleaved") pairs (x_2i, x_2i+1). */
static void rope_pair(int layout, int64_t r, int64_t i, int64_t* ia,
                      int64_t* ib) {
    if (layout == 0) {
        *ia = i;
        *ib = i + r / 2;
    } else {
        *ia = 2 * i;
        *ib = 2 * i + 1;
    }
}

/* [ELT] 2.2 and [OPS] Rope: rotate the first r entries of each of the H head
 * rows of one token (f64, rows[h*D + j]) in place:
 *   a' = mu (a cos t - b sin t),  b' = mu (a sin t + b cos t),
 * reading both members before writing either; entries r..D-1 are untouched.
 * Loop order token, pair, head: one angle serves every head. */
static void rope_token(double* rows, int64_t H, int64_t D, int64_t r,
                       int32_t p, const float* inv_freq, float mu_f,
                       int layout) {
    const int64_t rr = r;
    const double mu = (double)mu_f;
    for (int64_t i = 0; i < rr / 2; ++i) {
        const double ang = (double)orc_rope_angle(p, inv_freq[i]);
        const double c = cos(ang);
        const double s = sin(ang);
        int64_t ia, ib;
        rope_pair(layout, rr, i, &ia, &ib);
        for (int64_t h = 0; h < H; ++h) {
            double* v = rows + h * D;
            const double a = v[ia];
            const double b = v[ib];
            const double an = mu * (a * c - b * s);
            const double bn = mu * (a * s + b * c);
            v[ia] = an;
            v[ib] = bn;
        }
    }
}

/* In place on x [T, H, D]; only the first r entries of each head are
 * written.  y64 (optional) receives all D entries (the tail as given). */
void orc_rope(int dt, void* x, const int32_t* pos, int64_t T, int64_t H,
              int64_t D, int64_t r, const float* inv_freq, float mu,
              int layout, double* y64) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const int64_t base = t * H * D;
        double* v = row_buffer(H * D);
        for (int64_t j = 0; j < H * D; ++j) v[j] = ld(dt, x, base + j);
        rope_token(v, H, D, r, pos[t], inv_freq, mu, layout);
        for (int64_t h = 0; h < H; ++h)
            for (int64_t j = 0; j < D; ++j) {
                if (j < r) st(dt, x, base + h * D + j, v[h * D + j]);
                if (y64) y64[base + h * D + j] = v[h * D + j];
            }
        free(v);
    }
}

/* [OPS] 5 QK-norm: per (token, head) row of length D, RmsNorm over all D
 * entries with the per-head gain g [D], then Rope on the normalised row.  The
 * intermediate stays in f64; every entry is rounded once at the end. */
void orc_rmsnorm_rope(int dt, void* x, const void* g, float eps,
                      const int32_t* pos, int64_t T, int64_t H, int64_t D,
                      int64_t r, const float* inv_freq, float mu, int layout,
                      double* y64) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const int64_t base = t * H * D;
        double* v = row_buffer(H * D);
        for (int64_t j = 0; j < H * D; ++j) v[j] = ld(dt, x, base + j);
        for (int64_t h = 0; h < H; ++h) normalize_row(v + h * D, D, dt, g, eps);
        rope_token(v, H, D, r, pos[t], inv_freq, mu, layout);
        for (int64_t j = 0; j < H * D; ++j) {
            st(dt, x, base + j, v[j]);
            if (y64) y64[base + j] = v[j];
        }
        free(v);
    }
}

/* --------------------------------------------------------------- SiLU-mul */

/* [ELT] 2.3 and [OPS] Silu, SwiGlu: y = g / (1 + e^-g) * u.  The page's
 * single-precision exponential overflows to +inf once e^-g passes the f32
 * range, giving g / inf = -0 for very negative g; the f64 value is taken to
 * +inf at the same point so that limit is kept. */
void orc_silu_mul(int dt, const void* gate, const void* up, int64_t n,
                  double* y64, void* y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const double gv = ld(dt, gate, i);
        const double u = ld(dt, up, i);
        double e = exp(-gv);
        if (e > FLT_MAX) e = INFINITY;
        const double s = gv / (1.0 + e);
        const double v = s * u;
        if (y64) y64[i] = v;
        if (y) st(dt, y, i, v);
    }
}

/* ------------------------------------------------------------ add, gather */

/* [ELT] 2.4 and [OPS] Add: y = a + b, the exact sum rounded once. */
void orc_add(int dt, const void* a, const void* b, int64_t n, void* y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        st(dt, y, i, ld(dt, a, i) + ld(dt, b, i));
}

/* [ELT] 2.4 and [OPS] TokenEmbed: out[t, :] = table[ids[t], :], the source
 * row starting at element ids[t] * d; a bit copy.  An id outside [0, V) gives
 * a row of quiet NaN (the kernels' documented behaviour for bad ids). */
void orc_embedding(int dt, const void* table, int64_t V, const int32_t* ids,
                   int64_t n, int64_t d, void* out) {
    const size_t es = (dt == ORC_F32) ? 4 : 2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        char* dst = (char*)out + (size_t)t * (size_t)d * es;
        if (ids[t] < 0 || (int64_t)ids[t] >= V) {
            for (int64_t j = 0; j < d; ++j) st_nan(dt, out, t * d + j);
            continue;
        }
        const size_t off = (size_t)ids[t] * (size_t)d;
        memcpy(dst, (const char*)table + off * es, (size_t)d * es);
    }
}

/* ----------------------------------------------------------------- argmax */

/* [ELT] 2.4 and [OPS] 8 Sampling, Greedy: scan forward keeping the first
 * strictly greater value; NaN entries are skipped; -1 when the row holds no
 * number (empty or all NaN). */
void orc_argmax(int dt, const void* x, int64_t rows, int64_t n,
                int32_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int32_t best = -1;
        double bv = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double v = ld(dt, x, r * n + i);
            if (isnan(v)) continue;
            if (best < 0 || v > bv) {
                best = (int32_t)i;
                bv = v;
            }
        }
        out[r] = best;
    }
}

/* ---------------------------------------------------------------- softmax */

/* [OPS] 4 Activation / Softmax and 8 Sampling / Temperature; [DNN] 7: over
 * each row, z_i = x_i / t, m = max_i z_i, e_i = exp(z_i - m),
 * y_i = e_i / sum_j e_j.  The max is subtracted so that large logits do not
 * overflow.  z is the f64 quotient, except that a quotient beyond the f32
 * range is taken to +-inf, as the single-precision division the pages'
 * statistics use would give.  Special values follow the formula: a NaN
 * anywhere in a row, or a row whose max is +-inf, makes the whole row NaN. */
void orc_softmax(int dt, const void* x, int64_t rows, int64_t n, float t,
                 double* y64, void* y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double* z = row_buffer(n);
        double m = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            double v = ld(dt, x, r * n + i) / (double)t;
            if (v > FLT_MAX) v = INFINITY;
            if (v < -FLT_MAX) v = -INFINITY;
            z[i] = v;
            if (isnan(v) || isnan(m)) m = NAN;
            else if (v > m) m = v;
        }
        double sum = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            z[i] = exp(z[i] - m);
            sum += z[i];
        }
        for (int64_t i = 0; i < n; ++i) {
            const double v = z[i] / sum;
            if (y64) y64[r * n + i] = v;
            if (y) st(dt, y, r * n + i, v);
        }
        free(z);
    }
}

/* -------------------------------------------------------------- LayerNorm */

/* [OPS] 2 Normalization / LayerNorm; [DNN] 7: mu = mean(x),
 * var = mean((x - mu)^2), y = (x - mu) / sqrt(var + eps) * g + b over the
 * last axis (the two-pass variance, as written).  b may be NULL (no bias,
 * [DNN] 7's optional beta).  The sum of x, each deviation x - mu and the sum
 * of squared deviations are taken to +-inf past the f32 range (f32_range):
 * a row whose squared deviations overflow maps to the bias, one whose sum
 * overflows to NaN. */
void orc_layernorm(int dt, const void* x, const void* g, const void* b,
                   int64_t rows, int64_t d, float eps, double* y64, void* y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double sum = 0.0;
        for (int64_t i = 0; i < d; ++i) sum += ld(dt, x, r * d + i);
        const double mu = f32_range(sum) / (double)d;
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            const double c = f32_range(ld(dt, x, r * d + i) - mu);
            ss += c * c;
        }
        const double var = f32_range(ss) / (double)d;
        const double inv = 1.0 / sqrt(var + (double)eps);
        for (int64_t i = 0; i < d; ++i) {
            double v = f32_range(ld(dt, x, r * d + i) - mu) * inv * ld(dt, g, i);
            if (b) v += ld(dt, b, i);
            if (y64) y64[r * d + i] = v;
            if (y) st(dt, y, r * d + i, v);
        }
    }
}

/* ------------------------------------------------------------------ GeGLU */

/* [OPS] 4 Activation / Gelu and GeGlu: y = Gelu(gate) * up with
 *   form 0 (exact):  Gelu(x) = x * 0.5 * (1 + erf(x / sqrt(2)))
 *   form 1 (tanh):   Gelu(x) = 0.5 * x * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))
 * (the page's constant inside the tanh form is garbled; it is 2/pi, the
 * form's published definition).  Each is evaluated through an exact
 * identity that avoids the cancellation of 1 + (-1 + tiny) for negative x:
 * 1 + erf(z) = erfc(-z), and (1 + tanh(u)) / 2 = 1 / (1 + e^(-2u)).
 * f64 throughout with libm erfc and exp; as for SiLU, e^(-2u) is taken to
 * +inf once it passes the f32 range (x / inf = -0 far below zero). */
void orc_geglu(int dt, const void* gate, const void* up, int64_t n, int form,
               double* y64, void* y) {
    const double k = sqrt(2.0 / acos(-1.0));   /* acos(-1) is pi rounded to f64 */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const double x = ld(dt, gate, i);
        double gl;
        if (form == 0) {
            gl = x * 0.5 * erfc(-x / sqrt(2.0));
        } else {
            double e = exp(-2.0 * k * (x + 0.044715 * x * x * x));
            if (e > FLT_MAX) e = INFINITY;  /* the f32 exponential's limit, as for SiLU */
            gl = x / (1.0 + e);
        }
        const double u = ld(dt, up, i);
        double v = gl * u;
        /* Phi(x) > 0 for every finite x, so x Phi(x) is nonzero, with the sign
         * of x, also where erfc underflows f64 (x below about -38.6): its
         * product with an infinite up is the infinity of that sign, not
         * 0 * inf.  (x = +-0 and x = -inf, where Phi is 0, stay NaN.) */
        if (form == 0 && isinf(u) && isfinite(x) && x != 0.0)
            v = ((x > 0.0) == (u > 0.0)) ? INFINITY : -INFINITY;
        if (y64) y64[i] = v;
        if (y) st(dt, y, i, v);
    }
}

/* ------------------------------------------------------------ RoPE cache */

/* [OPS] 3 Rope, "Cos/sin cache": cos[p, i] and sin[p, i] for every position
 * p < max_pos and pair i < r/2, of the angle [ELT] 2.2 defines (the f32
 * product, R1), in f64 and rounded once to f32.  Layout [max_pos, r/2]. */
void orc_rope_cache(const float* inv_freq, int64_t max_pos, int64_t r,
                    float* cos_c, float* sin_c) {
    const int64_t half = r / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < max_pos; ++p)
        for (int64_t i = 0; i < half; ++i) {
            const double ang = (double)orc_rope_angle((int32_t)p, inv_freq[i]);
            cos_c[p * half + i] = (float)cos(ang);
            sin_c[p * half + i] = (float)sin(ang);
        }
}

/* RoPE with the rotation read from a cache instead of computed: for pair i
 * of token t, c = cos[pos[t], i] and s = sin[pos[t], i] as given (f32,
 * widened), then a' = mu (a c - b s), b' = mu (a s + b c) in f64.  A
 * position outside [0, max_pos) (the pages make it an error: no angle is
 * defined for it) is never looked up; that token's rotated entries become
 * quiet NaN, its other entries stay as given. */
void orc_rope_cached(int dt, void* x, const int32_t* pos, int64_t T,
                     int64_t H, int64_t D, int64_t r, const float* cos_c,
                     const float* sin_c, int64_t max_pos, float mu_f,
                     int layout, double* y64) {
    const int64_t half = r / 2;
    const double mu = (double)mu_f;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const int64_t base = t * H * D;
        const int32_t p = pos[t];
        const int ok = p >= 0 && (int64_t)p < max_pos;
        double* v = row_buffer(H * D);
        for (int64_t j = 0; j < H * D; ++j) v[j] = ld(dt, x, base + j);
        for (int64_t i = 0; i < half; ++i) {
            const double c = ok ? (double)cos_c[(int64_t)p * half + i] : NAN;
            const double sn = ok ? (double)sin_c[(int64_t)p * half + i] : NAN;
            int64_t ia, ib;
            rope_pair(layout, r, i, &ia, &ib);
            for (int64_t h = 0; h < H; ++h) {
                double* w = v + h * D;
                const double a = w[ia];
                const double b = w[ib];
                w[ia] = mu * (a * c - b * sn);
                w[ib] = mu * (a * sn + b * c);
            }
        }
        for (int64_t h = 0; h < H; ++h)
            for (int64_t j = 0; j < D; ++j) {
                if (j < r) st(dt, x, base + h * D + j, v[h * D + j]);
                if (y64) y64[base + h * D + j] = v[h * D + j];
            }
        free(v);
    }
}

/* ------------------------------------------------------- multi-axis RoPE */

/* [OPS] 3 Rope, multi-axis RoPE (3D, for video diffusion transformers):
 * token t has a position vector pos[t * A + a], a < A.  The head is cut into
 * consecutive sub-ranges of dims[a] entries (each even; they need not fill
 * the head), axis a starting at o_a = dims[0] + ... + dims[a-1].  Axis a
 * applies RoPE on its own sub-range, as if that were a whole head of
 * dims[a] entries: its position pos[t * A + a], its own frequencies
 * inv_freq[h_a + j], j < dims[a]/2, h_a = (dims[0] + ... + dims[a-1]) / 2
 * (so each axis may have its own base), the angle of [ELT] 2.2 (R1), and
 * the pairing of layout inside the sub-range: half (o_a + j, o_a + j +
 * dims[a]/2) or interleaved (o_a + 2j, o_a + 2j + 1).  Entries past the last
 * sub-range are not touched. */
void orc_rope_multi(int dt, void* x, const int32_t* pos, int64_t T,
                    int64_t H, int64_t D, int64_t A, const int64_t* dims,
                    const float* inv_freq, float mu_f, int layout,
                    double* y64) {
    const double mu = (double)mu_f;
    int64_t span = 0;
    for (int64_t a = 0; a < A; ++a) span += dims[a];
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const int64_t base = t * H * D;
        double* v = row_buffer(H * D);
        for (int64_t j = 0; j < H * D; ++j) v[j] = ld(dt, x, base + j);
        int64_t off = 0;    /* o_a: first entry of this axis's sub-range */
        int64_t foff = 0;   /* h_a: first frequency of this axis */
        for (int64_t a = 0; a < A; ++a) {
            const int64_t da = dims[a];
            const int32_t p = pos[t * A + a];
            for (int64_t j = 0; j < da / 2; ++j) {
                const double ang = (double)orc_rope_angle(p, inv_freq[foff + j]);
                const double ca = cos(ang);
                const double sa = sin(ang);
                int64_t ia, ib;
                rope_pair(layout, da, j, &ia, &ib);
                for (int64_t h = 0; h < H; ++h) {
                    double* w = v + h * D + off;
                    const double x1 = w[ia];
                    const double x2 = w[ib];
                    w[ia] = mu * (x1 * ca - x2 * sa);
                    w[ib] = mu * (x1 * sa + x2 * ca);
                }
            }
            off += da;
            foff += da / 2;
        }
        for (int64_t h = 0; h < H; ++h)
            for (int64_t j = 0; j < D; ++j) {
                if (j < span) st(dt, x, base + h * D + j, v[h * D + j]);
                if (y64) y64[base + h * D + j] = v[h * D + j];
            }
        free(v);
    }
}
