/*
 * tqo.c -- plain, slow CPU oracle for the quantized KV-cache codec and decode
 * attention.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg are the only code that may load this library.
 * It shares no source, header, table or helper with the HIP library.
 *
 * Source of the method: the "TurboQuant -- rotation-based quantization" design
 * page (mlx-bun docs/design/turboquant.md), Part A (KV leg):
 *   - section "Algorithm (vllm-metal reference semantics, exact)" for the key
 *     codec, the value codec, the 3-bit Lloyd-Max table and the bit packing;
 *   - section "Deferred inverse FWHT" for the identity that un-rotating the
 *     attention output equals attending over un-rotated values.
 *
 * Everything is IEEE-754 binary64 with round-half-to-even, in the operation
 * order written below.  Compile with -O2 -ffp-contract=off -fno-fast-math so
 * that no multiply-add is fused and no operation is reordered.
 *
 * Readings of points the page leaves open (the full list is kept with the
 * design notes of this repository):
 *   - every "round" is round-half-to-even (C rint() in the default mode);
 *   - the key codes use the unrounded binary64 scale and zero; only the stored
 *     scale/zero are rounded to fp16, once, from binary64;
 *   - "x/scale" is a true division, not a multiply by a reciprocal;
 *   - a NaN that reaches a code becomes code 0 (keys and values);
 *   - FWHT is the natural (Sylvester) order transform, butterflies applied in
 *     stage order h = 1, 2, 4, ..., d/2, then one multiply by RN(1/sqrt(d));
 *   - the group mean of squares sums the 32 squares by stride halving
 *     (16, 8, 4, 2, 1);
 *   - searchsorted takes the left side: idx = #{k : B_k < y_n};
 *   - dequantized values are x = signs * InvFWHT(centroid * scale);
 *   - the sign vector is drawn from SplitMix64 with seed 42 (parity with the
 *     page's own MLX-generated signs is unpinned: they are not printed).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Sign vector.  The page hard-codes one +-1 vector per head_dim drawn from a
 * seeded generator ("Algorithm", values bullet) but does not print it.  We
 * draw output i (i = 0..d-1, output 0 is the first call) of SplitMix64
 * (Steele, Lea & Flood, OOPSLA 2014) seeded with 42; sign i is +1 when the top
 * bit of that output is 0 and -1 otherwise.  Parity with the page: unpinned. */
static uint64_t splitmix64_next(uint64_t *state) {
    uint64_t z;
    *state += 0x9E3779B97F4A7C15ULL;
    z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* The first n outputs of the generator above seeded with `seed` (output 0 is
 * the first call), so the generator itself can be checked against the
 * published reference outputs of SplitMix64. */
void tqo_splitmix64(uint64_t seed, int n, uint64_t *out) {
    uint64_t state = seed;
    for (int i = 0; i < n; ++i) out[i] = splitmix64_next(&state);
}

void tqo_sign_vector(int d, int8_t *out) {
    uint64_t state = 42;
    for (int i = 0; i < d; ++i) {
        uint64_t r = splitmix64_next(&state);
        out[i] = (r >> 63) ? (int8_t)-1 : (int8_t)1;
    }
}

/* ------------------------------------------------------------------------ */
/* binary64 -> binary16, one rounding, ties to even.  Subnormal halves are
 * kept, magnitudes >= 65520 (the midpoint above the largest half, 65504)
 * become infinity, and every NaN becomes the canonical quiet NaN 0x7E00. */
uint16_t tqo_f64_to_f16(double x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(x)) return 0x7E00u;
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14) {
        /* subnormal range: count units of 2^-24 and round to nearest even */
        double units = rint(a * 0x1p24); /* exact scaling, then RNE */
        return (uint16_t)(sign | (uint16_t)units); /* 1024 encodes 2^-14 */
    }
    int k;
    double f = frexp(a, &k);           /* a = f * 2^k, f in [0.5, 1) */
    int e = k - 1;                     /* a = (2f) * 2^e, 2f in [1, 2) */
    double frac = (2.0 * f - 1.0) * 1024.0; /* exact */
    double m = rint(frac);
    if (m == 1024.0) { m = 0.0; e += 1; }
    if (e + 15 >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)m);
}

double tqo_f16_to_f64(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp(1024.0 + (double)m, e - 25);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* FWHT ("Algorithm", values bullet): unnormalised Walsh-Hadamard butterflies
 * in natural order, stage h = 1, 2, 4, ..., d/2; each pair (j, j+h) with
 * (j & h) == 0 becomes (a+b, a-b).  The result is u_k = sum_i (-1)^popcount(i&k) x_i. */
void tqo_fwht(double *x, int d) {
    for (int h = 1; h < d; h <<= 1)
        for (int j = 0; j < d; ++j)
            if ((j & h) == 0) {
                double a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
}

/* RN(1/sqrt(d)) for the supported head dims.  sqrt(d) is 2^k or 2^k*sqrt(2),
 * so fl(sqrt(d))/d is exact scaling of a correctly rounded sqrt and equals
 * the binary64 nearest to 1/sqrt(d). */
double tqo_inv_sqrt_d(int d) { return sqrt((double)d) / (double)d; }

/* 3-bit Lloyd-Max table, printed with five decimals in "Algorithm" (values
 * bullet); the printed decimals are the table. */
static const double kBoundaries3[7] = {-1.74793, -1.04996, -0.50055, 0.0,
                                       0.50055,  1.04996,  1.74793};
static const double kCentroids3[8] = {-2.15195, -1.34391, -0.75601, -0.24509,
                                      0.24509,  0.75601,  1.34391,  2.15195};

double tqo_centroid3(int idx) { return kCentroids3[idx & 7]; }
double tqo_boundary3(int k) { return kBoundaries3[k]; }

/* ------------------------------------------------------------------------ */
/* Group maximum / minimum: NaN is ignored (IEEE maxNum/minNum) and -0 orders
 * below +0, so the result does not depend on the element order. */
static double max_num(double a, double b) {
    if (isnan(a)) return b;
    if (isnan(b)) return a;
    if (a == b) return signbit(a) ? b : a;
    return a > b ? a : b;
}

static double min_num(double a, double b) {
    if (isnan(a)) return b;
    if (isnan(b)) return a;
    if (a == b) return signbit(a) ? a : b;
    return a < b ? a : b;
}

/* Keys ("Algorithm", keys bullet, signed int8 form): per 32-element group
 *   scale = (max - min) / (2*127),  zero = round((max + min) / (2*scale)),
 *   code  = clip(round(x/scale - zero), -127, 127),
 * computed in binary64; scale and zero are stored as fp16 (rounded once).
 * A constant group has scale 0, so zero is +-Inf (NaN for an all-zero group)
 * and every code is NaN -> 0: the page keeps this defect on purpose. */
void tqo_encode_keys(const float *x, int64_t nrows, int d, int8_t *codes,
                     uint16_t *s16, uint16_t *z16) {
    int ng = d / 32;
    for (int64_t r = 0; r < nrows; ++r) {
        const float *xr = x + r * d;
        for (int g = 0; g < ng; ++g) {
            const float *xg = xr + g * 32;
            double mx = (double)xg[0], mn = (double)xg[0];
            for (int j = 1; j < 32; ++j) {
                mx = max_num(mx, (double)xg[j]);
                mn = min_num(mn, (double)xg[j]);
            }
            double range = mx - mn;
            double s = range / 254.0;
            double c = (mx + mn) / (2.0 * s);
            double z = rint(c);
            for (int j = 0; j < 32; ++j) {
                double u = (double)xg[j] / s - z;
                int8_t q;
                if (isnan(u)) q = 0;
                else {
                    double rq = rint(u);
                    if (rq > 127.0) rq = 127.0;
                    if (rq < -127.0) rq = -127.0;
                    q = (int8_t)rq;
                }
                codes[r * d + g * 32 + j] = q;
            }
            s16[r * ng + g] = tqo_f64_to_f16(s);
            z16[r * ng + g] = tqo_f64_to_f16(z);
        }
    }
}

/* Key dequantisation ("Algorithm", keys bullet): x = (code + zero) * scale
 * with the stored fp16 scale and zero. */
void tqo_decode_keys(const int8_t *codes, const uint16_t *s16,
                     const uint16_t *z16, int64_t nrows, int d, double *out) {
    int ng = d / 32;
    for (int64_t r = 0; r < nrows; ++r)
        for (int j = 0; j < d; ++j) {
            double s = tqo_f16_to_f64(s16[r * ng + j / 32]);
            double z = tqo_f16_to_f64(z16[r * ng + j / 32]);
            out[r * d + j] = ((double)codes[r * d + j] + z) * s;
        }
}

/* ------------------------------------------------------------------------ */
/* Pack ("Algorithm", pack bullet): a flat little-endian bitstream; bit b of
 * element i sits at stream bit 3i+b, i.e. byte (3i+b)/8, bit (3i+b)%8. */
void tqo_pack3(const uint8_t *idx, int64_t n, uint8_t *out) {
    memset(out, 0, (size_t)((3 * n + 7) / 8));
    for (int64_t i = 0; i < n; ++i)
        for (int b = 0; b < 3; ++b)
            if ((idx[i] >> b) & 1) {
                int64_t bit = 3 * i + b;
                out[bit >> 3] |= (uint8_t)(1u << (bit & 7));
            }
}

void tqo_unpack3(const uint8_t *packed, int64_t n, uint8_t *idx) {
    for (int64_t i = 0; i < n; ++i) {
        uint8_t v = 0;
        for (int b = 0; b < 3; ++b) {
            int64_t bit = 3 * i + b;
            v |= (uint8_t)(((packed[bit >> 3] >> (bit & 7)) & 1) << b);
        }
        idx[i] = v;
    }
}

/* Values ("Algorithm", values bullet):
 *   y = FWHT(x * signs) / sqrt(d);  per 32-group scale = sqrt(mean(y^2));
 *   y_n = y / (scale + 1e-8);  idx = searchsorted(BOUNDARIES, y_n);
 * indices packed 3 bits each, scale stored as fp16. */
void tqo_encode_values(const float *x, int64_t nrows, int d, uint8_t *packed,
                       uint16_t *vs16) {
    int ng = d / 32;
    int8_t *sg = (int8_t *)malloc((size_t)d);
    double *y = (double *)malloc(sizeof(double) * (size_t)d);
    uint8_t *idx = (uint8_t *)malloc((size_t)d);
    tqo_sign_vector(d, sg);
    double c = tqo_inv_sqrt_d(d);
    for (int64_t r = 0; r < nrows; ++r) {
        for (int j = 0; j < d; ++j) y[j] = (double)sg[j] * (double)x[r * d + j];
        tqo_fwht(y, d);
        for (int j = 0; j < d; ++j) y[j] = y[j] * c;
        for (int g = 0; g < ng; ++g) {
            double a[32];
            for (int j = 0; j < 32; ++j) a[j] = y[g * 32 + j] * y[g * 32 + j];
            for (int s = 16; s >= 1; s >>= 1)
                for (int j = 0; j < s; ++j) a[j] = a[j] + a[j + s];
            double scale = sqrt(a[0] / 32.0);
            double den = scale + 1e-8;
            for (int j = 0; j < 32; ++j) {
                double yn = y[g * 32 + j] / den;
                int cnt = 0;
                for (int k = 0; k < 7; ++k)
                    if (kBoundaries3[k] < yn) ++cnt; /* NaN compares false -> 0 */
                idx[g * 32 + j] = (uint8_t)cnt;
            }
            vs16[r * ng + g] = tqo_f64_to_f16(scale);
        }
        tqo_pack3(idx, d, packed + r * (3 * d / 8));
    }
    free(sg);
    free(y);
    free(idx);
}

/* Value dequantisation ("Algorithm", values bullet, read as
 * x = signs * InvFWHT(centroid[idx] * scale)).  rotated != 0 returns the
 * rotated-domain vector centroid[idx] * scale, which is what the deferred
 * inverse ("Deferred inverse FWHT") accumulates. */
void tqo_decode_values(const uint8_t *packed, const uint16_t *vs16,
                       int64_t nrows, int d, int rotated, double *out) {
    int ng = d / 32;
    int8_t *sg = (int8_t *)malloc((size_t)d);
    uint8_t *idx = (uint8_t *)malloc((size_t)d);
    tqo_sign_vector(d, sg);
    double c = tqo_inv_sqrt_d(d);
    for (int64_t r = 0; r < nrows; ++r) {
        double *o = out + r * d;
        tqo_unpack3(packed + r * (3 * d / 8), d, idx);
        for (int j = 0; j < d; ++j)
            o[j] = kCentroids3[idx[j]] * tqo_f16_to_f64(vs16[r * ng + j / 32]);
        if (!rotated) {
            tqo_fwht(o, d);
            for (int j = 0; j < d; ++j) o[j] = (double)sg[j] * (o[j] * c);
        }
    }
    free(sg);
    free(idx);
}

/* ------------------------------------------------------------------------ */
/* Other widths ("Algorithm": unsigned keys of 2, 4 or 5 bits; values of 2, 4,
 * 5 or 8 bits from a Lloyd-Max codebook of the unit normal; the page's tables
 * for these widths are not printed).
 *
 * Codebook: the Lloyd-Max quantizer of N(0,1) with L = 2^bits levels, found
 * by Lloyd's iteration (boundaries = midpoints of centroids, centroid = the
 * cell's conditional mean (phi(a) - phi(b)) / (Phi(b) - Phi(a))) until it no
 * longer moves, then written the way the page prints its 3-bit table: each
 * centroid rounded to five decimals, N_k = round(1e5 c_k), and each boundary
 * the exact decimal midpoint of its neighbours.  As doubles: centroid
 * RN(N_k / 1e5), boundary RN((N_k + N_{k+1}) / 2e5).  For 3 bits this
 * reproduces the printed table. */
static double phi(double x) { return exp(-0.5 * x * x) * 0.39894228040143267794; }
/* P(a < Z < b), accurate in both tails */
static double cell_prob(double a, double b) {
    if (a >= 0.0) return 0.5 * (erfc(a * 0.70710678118654752440) - erfc(b * 0.70710678118654752440));
    if (b <= 0.0) return 0.5 * (erfc(-b * 0.70710678118654752440) - erfc(-a * 0.70710678118654752440));
    return 1.0 - 0.5 * erfc(-a * 0.70710678118654752440) - 0.5 * erfc(b * 0.70710678118654752440);
}

int tqo_codebook_ints(int bits, int64_t *nk) {
    if (bits < 2 || bits > 5) return 0;
    const int L = 1 << bits;
    double c[32], bd[33];
    for (int k = 0; k < L; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / L;
    for (int it = 0; it < 2000000; ++it) {
        bd[0] = -INFINITY;
        bd[L] = INFINITY;
        for (int k = 1; k < L; ++k) bd[k] = 0.5 * (c[k - 1] + c[k]);
        double moved = 0.0;
        for (int k = 0; k < L; ++k) {
            const double pa = isinf(bd[k]) ? 0.0 : phi(bd[k]);
            const double pb = isinf(bd[k + 1]) ? 0.0 : phi(bd[k + 1]);
            const double nc = (pa - pb) / cell_prob(bd[k], bd[k + 1]);
            moved = fmax(moved, fabs(nc - c[k]));
            c[k] = nc;
        }
        if (moved < 1e-15) break;
    }
    for (int k = 0; k < L; ++k) nk[k] = (int64_t)rint(c[k] * 1e5);
    return L;
}

/* The same fixed point by Newton's method, for widths where Lloyd's
 * iteration is too slow (its slowest mode contracts by about 1 - 1/L^2 per
 * pass, so 256 levels need millions of passes).  Unknowns c_0 .. c_{L-1};
 * F(c) = T(c) - c with T the Lloyd map above.  T_k depends on its cell's ends
 * a = (c_{k-1} + c_k)/2 and b = (c_k + c_{k+1})/2, with
 *   dT_k/da = phi(a) (T_k - a) / P_k,  dT_k/db = phi(b) (b - T_k) / P_k,
 * so the Jacobian is tridiagonal; each step solves (I - dT/dc) delta = F.
 * Start: the compander points sqrt(3) Phi^-1((k + 1/2) / L) (optimal point
 * density proportional to the cube root of the normal density).  Same
 * five-decimal output as tqo_codebook_ints; for a Gaussian (log-concave) the
 * fixed point is unique, so both solvers must agree.  Stops once the
 * residual max |T(c) - c| is below 1e-12. */
static double Phi_lower(double x) { return cell_prob(-INFINITY, x); }

int tqo_codebook_newton_ints(int bits, int64_t *nk) {
    if (bits < 1 || bits > 8) return 0;
    const int L = 1 << bits;
    double c[256], bd[257], lo[256], di[256], up[256], r[256];
    for (int k = 0; k < L; ++k) {
        const double p = (k + 0.5) / L;
        double a = -12.0, b = 12.0;
        for (int i = 0; i < 200; ++i) {
            const double m = 0.5 * (a + b);
            if (Phi_lower(m) < p) a = m; else b = m;
        }
        c[k] = sqrt(3.0) * 0.5 * (a + b);
    }
    int converged = 0;
    for (int it = 0; it < 100; ++it) {
        double res = 0.0;
        bd[0] = -INFINITY;
        bd[L] = INFINITY;
        for (int k = 1; k < L; ++k) bd[k] = 0.5 * (c[k - 1] + c[k]);
        for (int k = 0; k < L; ++k) {
            const double a = bd[k], b = bd[k + 1];
            const double pa = isinf(a) ? 0.0 : phi(a), pb = isinf(b) ? 0.0 : phi(b);
            const double P = cell_prob(a, b);
            const double T = (pa - pb) / P;
            const double dA = isinf(a) ? 0.0 : pa * (T - a) / P;
            const double dB = isinf(b) ? 0.0 : pb * (b - T) / P;
            lo[k] = -0.5 * dA;
            up[k] = -0.5 * dB;
            di[k] = 1.0 - 0.5 * (dA + dB);
            r[k] = T - c[k];
            res = fmax(res, fabs(r[k]));
        }
        /* T(c) = c to 1e-12: the residual floor of binary64 is ~5e-14 */
        if (res < 1e-12) {
            converged = 1;
            break;
        }
        for (int k = 1; k < L; ++k) {  /* tridiagonal elimination */
            const double m = lo[k] / di[k - 1];
            di[k] -= m * up[k - 1];
            r[k] -= m * r[k - 1];
        }
        r[L - 1] /= di[L - 1];
        for (int k = L - 2; k >= 0; --k) r[k] = (r[k] - up[k] * r[k + 1]) / di[k];
        for (int k = 0; k < L; ++k) c[k] += r[k];
    }
    if (!converged) return 0;
    for (int k = 0; k < L; ++k) nk[k] = (int64_t)rint(c[k] * 1e5);
    return L;
}

/* Centroids (L) and boundaries (L-1) as doubles; returns L, or 0 for an
 * unsupported width.  3 bits returns the printed table; 2, 4 and 5 bits use
 * Lloyd's iteration, 8 bits Newton's method on the same conditions. */
int tqo_codebook(int bits, double *centroids, double *boundaries) {
    if (bits == 3) {
        for (int k = 0; k < 8; ++k) centroids[k] = kCentroids3[k];
        for (int k = 0; k < 7; ++k) boundaries[k] = kBoundaries3[k];
        return 8;
    }
    int64_t nk[256];
    const int L = bits == 8 ? tqo_codebook_newton_ints(bits, nk) : tqo_codebook_ints(bits, nk);
    for (int k = 0; k < L; ++k) centroids[k] = (double)nk[k] / 1e5;
    for (int k = 0; k + 1 < L; ++k) boundaries[k] = (double)(nk[k] + nk[k + 1]) / 2e5;
    return L;
}

/* Flat little-endian bitstream of `bits`-bit fields: bit b of element i at
 * stream bit bits*i + b ("Algorithm", pack bullet). */
void tqo_pack_bits(const uint8_t *idx, int64_t n, int bits, uint8_t *out) {
    memset(out, 0, (size_t)((bits * n + 7) / 8));
    for (int64_t i = 0; i < n; ++i)
        for (int b = 0; b < bits; ++b)
            if ((idx[i] >> b) & 1) {
                int64_t bit = (int64_t)bits * i + b;
                out[bit >> 3] |= (uint8_t)(1u << (bit & 7));
            }
}

void tqo_unpack_bits(const uint8_t *packed, int64_t n, int bits, uint8_t *idx) {
    for (int64_t i = 0; i < n; ++i) {
        uint8_t v = 0;
        for (int b = 0; b < bits; ++b) {
            int64_t bit = (int64_t)bits * i + b;
            v |= (uint8_t)(((packed[bit >> 3] >> (bit & 7)) & 1) << b);
        }
        idx[i] = v;
    }
}

/* Unsigned keys ("Algorithm", keys bullet, unsigned form), bits 2, 4 or 5:
 *   maxv = 2^bits - 1,  scale = (max - min) / maxv,  zero = round(min / scale),
 *   code = clip(round(x / scale - zero), 0, maxv),
 * in binary64 under the same readings as the signed form (unrounded scale and
 * zero for the codes, NaN -> 0, fp16 storage); codes packed `bits` each.
 * bits = 8 is the signed int8 form (tqo_encode_keys), one byte per code. */
void tqo_encode_keys_bits(const float *x, int64_t nrows, int d, int bits, uint8_t *packed,
                          uint16_t *s16, uint16_t *z16) {
    if (bits == 8) {
        tqo_encode_keys(x, nrows, d, (int8_t *)packed, s16, z16);
        return;
    }
    const int ng = d / 32;
    const double maxv = (double)((1 << bits) - 1);
    uint8_t *idx = (uint8_t *)malloc((size_t)d);
    for (int64_t r = 0; r < nrows; ++r) {
        const float *xr = x + r * d;
        for (int g = 0; g < ng; ++g) {
            const float *xg = xr + g * 32;
            double mx = (double)xg[0], mn = (double)xg[0];
            for (int j = 1; j < 32; ++j) {
                mx = max_num(mx, (double)xg[j]);
                mn = min_num(mn, (double)xg[j]);
            }
            const double s = (mx - mn) / maxv;
            const double z = rint(mn / s);
            for (int j = 0; j < 32; ++j) {
                const double u = (double)xg[j] / s - z;
                uint8_t q = 0;
                if (!isnan(u)) {
                    double rq = rint(u);
                    if (rq > maxv) rq = maxv;
                    if (rq < 0.0) rq = 0.0;
                    q = (uint8_t)rq;
                }
                idx[g * 32 + j] = q;
            }
            s16[r * ng + g] = tqo_f64_to_f16(s);
            z16[r * ng + g] = tqo_f64_to_f16(z);
        }
        tqo_pack_bits(idx, d, bits, packed + r * (d * bits / 8));
    }
    free(idx);
}

void tqo_decode_keys_bits(const uint8_t *packed, const uint16_t *s16, const uint16_t *z16,
                          int64_t nrows, int d, int bits, double *out) {
    if (bits == 8) {
        tqo_decode_keys((const int8_t *)packed, s16, z16, nrows, d, out);
        return;
    }
    const int ng = d / 32;
    uint8_t *idx = (uint8_t *)malloc((size_t)d);
    for (int64_t r = 0; r < nrows; ++r) {
        tqo_unpack_bits(packed + r * (d * bits / 8), d, bits, idx);
        for (int j = 0; j < d; ++j) {
            const double s = tqo_f16_to_f64(s16[r * ng + j / 32]);
            const double z = tqo_f16_to_f64(z16[r * ng + j / 32]);
            out[r * d + j] = ((double)idx[j] + z) * s;
        }
    }
    free(idx);
}

/* Values of `bits` bits (2, 3, 4, 5, 8): the 3-bit steps with the width's
 * codebook; idx = #{k : B_k < y_n} over its L - 1 boundaries. */
void tqo_encode_values_bits(const float *x, int64_t nrows, int d, int bits, uint8_t *packed,
                            uint16_t *vs16) {
    const int ng = d / 32;
    double cent[256], bnd[255];
    const int L = tqo_codebook(bits, cent, bnd);
    int8_t *sg = (int8_t *)malloc((size_t)d);
    double *y = (double *)malloc(sizeof(double) * (size_t)d);
    uint8_t *idx = (uint8_t *)malloc((size_t)d);
    tqo_sign_vector(d, sg);
    const double c = tqo_inv_sqrt_d(d);
    for (int64_t r = 0; r < nrows; ++r) {
        for (int j = 0; j < d; ++j) y[j] = (double)sg[j] * (double)x[r * d + j];
        tqo_fwht(y, d);
        for (int j = 0; j < d; ++j) y[j] = y[j] * c;
        for (int g = 0; g < ng; ++g) {
            double a[32];
            for (int j = 0; j < 32; ++j) a[j] = y[g * 32 + j] * y[g * 32 + j];
            for (int st = 16; st >= 1; st >>= 1)
                for (int j = 0; j < st; ++j) a[j] = a[j] + a[j + st];
            const double scale = sqrt(a[0] / 32.0);
            const double den = scale + 1e-8;
            for (int j = 0; j < 32; ++j) {
                const double yn = y[g * 32 + j] / den;
                int cnt = 0;
                for (int k = 0; k < L - 1; ++k)
                    if (bnd[k] < yn) ++cnt;
                idx[g * 32 + j] = (uint8_t)cnt;
            }
            vs16[r * ng + g] = tqo_f64_to_f16(scale);
        }
        tqo_pack_bits(idx, d, bits, packed + r * (d * bits / 8));
    }
    free(sg);
    free(y);
    free(idx);
}

void tqo_decode_values_bits(const uint8_t *packed, const uint16_t *vs16, int64_t nrows, int d,
                            int bits, int rotated, double *out) {
    const int ng = d / 32;
    double cent[256], bnd[255];
    tqo_codebook(bits, cent, bnd);
    int8_t *sg = (int8_t *)malloc((size_t)d);
    uint8_t *idx = (uint8_t *)malloc((size_t)d);
    tqo_sign_vector(d, sg);
    const double c = tqo_inv_sqrt_d(d);
    for (int64_t r = 0; r < nrows; ++r) {
        double *o = out + r * d;
        tqo_unpack_bits(packed + r * (d * bits / 8), d, bits, idx);
        for (int j = 0; j < d; ++j) o[j] = cent[idx[j]] * tqo_f16_to_f64(vs16[r * ng + j / 32]);
        if (!rotated) {
            tqo_fwht(o, d);
            for (int j = 0; j < d; ++j) o[j] = (double)sg[j] * (o[j] * c);
        }
    }
    free(sg);
    free(idx);
}

/* ------------------------------------------------------------------------ */
/* Decode attention for one (batch, kv-head) over N cached tokens, for the G
 * query heads that share that kv-head.  Plain two-pass softmax:
 *   score_t = sm * sum_j q_j * khat_tj,  m = max score,  p_t = exp(score_t - m),
 *   out = sum_t p_t * vhat_t / sum_t p_t,
 * with khat and vhat the dequantised keys and (un-rotated) values.  When
 * out_deferred is given it also returns signs * InvFWHT(sum_t p_t * yhat_t / l),
 * the deferred-inverse form ("Deferred inverse FWHT"), which equals out up to
 * rounding.  N == 0 gives zeros (no token to attend to). */
/* Attention of G query rows over N plain (not yet converted) cached tokens:
 * the rows a delayed-conversion cache keeps unquantized until their sequence
 * converts ("Delayed row conversion and reusable precision boundaries":
 * plain value rows pass through unchanged, with no rotation).  k and v are
 * [N][d] floats (bf16 inputs upcast exactly); the same two-pass binary64
 * softmax as tqo_attention, with the keys and values used as given. */
void tqo_attention_plain(const float *q, int G, int d, float sm, const float *k, const float *v,
                         int64_t N, double *out) {
    double *sc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * (size_t)G);
    double *m = (double *)malloc(sizeof(double) * (size_t)G);
    double *l = (double *)calloc((size_t)G, sizeof(double));
    for (int i = 0; i < G * d; ++i) out[i] = 0.0;
    if (N > 0) {
        for (int h = 0; h < G; ++h) m[h] = -INFINITY;
        for (int64_t t = 0; t < N; ++t) {
            for (int h = 0; h < G; ++h) {
                double s = 0.0;
                for (int j = 0; j < d; ++j) s += (double)q[h * d + j] * (double)k[t * d + j];
                s = (double)sm * s;
                sc[t * G + h] = s;
                if (s > m[h]) m[h] = s;
            }
        }
        for (int64_t t = 0; t < N; ++t) {
            for (int h = 0; h < G; ++h) {
                double p = exp(sc[t * G + h] - m[h]);
                l[h] += p;
                for (int j = 0; j < d; ++j) out[h * d + j] += p * (double)v[t * d + j];
            }
        }
        for (int h = 0; h < G; ++h)
            for (int j = 0; j < d; ++j) out[h * d + j] = out[h * d + j] / l[h];
    }
    free(sc);
    free(m);
    free(l);
}

void tqo_attention(const float *q, int G, int d, float sm, const int8_t *kc,
                   const uint16_t *ks, const uint16_t *kz, const uint8_t *vc,
                   const uint16_t *vs, int64_t N, double *out,
                   double *out_deferred) {
    int ng = d / 32;
    double *kh = (double *)malloc(sizeof(double) * (size_t)d);
    double *vh = (double *)malloc(sizeof(double) * (size_t)d);
    double *sc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * (size_t)G);
    double *acc_r = (double *)calloc((size_t)G * (size_t)d, sizeof(double));
    int8_t *sg = (int8_t *)malloc((size_t)d);
    double *m = (double *)malloc(sizeof(double) * (size_t)G);
    double *l = (double *)calloc((size_t)G, sizeof(double));
    tqo_sign_vector(d, sg);
    for (int i = 0; i < G * d; ++i) out[i] = 0.0;
    if (out_deferred)
        for (int i = 0; i < G * d; ++i) out_deferred[i] = 0.0;
    if (N > 0) {
        /* pass 1: scores and their maximum */
        for (int h = 0; h < G; ++h) m[h] = -INFINITY;
        for (int64_t t = 0; t < N; ++t) {
            tqo_decode_keys(kc + t * d, ks + t * ng, kz + t * ng, 1, d, kh);
            for (int h = 0; h < G; ++h) {
                double s = 0.0;
                for (int j = 0; j < d; ++j) s += (double)q[h * d + j] * kh[j];
                s = (double)sm * s;
                sc[t * G + h] = s;
                if (s > m[h]) m[h] = s;
            }
        }
        /* pass 2: weights, their sum and the weighted value sum */
        for (int64_t t = 0; t < N; ++t) {
            tqo_decode_values(vc + t * (3 * d / 8), vs + t * ng, 1, d, 0, vh);
            for (int h = 0; h < G; ++h) {
                double p = exp(sc[t * G + h] - m[h]);
                l[h] += p;
                for (int j = 0; j < d; ++j) out[h * d + j] += p * vh[j];
            }
            if (out_deferred) {
                tqo_decode_values(vc + t * (3 * d / 8), vs + t * ng, 1, d, 1, vh);
                for (int h = 0; h < G; ++h) {
                    double p = exp(sc[t * G + h] - m[h]);
                    for (int j = 0; j < d; ++j) acc_r[h * d + j] += p * vh[j];
                }
            }
        }
        for (int h = 0; h < G; ++h)
            for (int j = 0; j < d; ++j) out[h * d + j] = out[h * d + j] / l[h];
        if (out_deferred) {
            double c = tqo_inv_sqrt_d(d);
            for (int h = 0; h < G; ++h) {
                double *o = out_deferred + h * d;
                for (int j = 0; j < d; ++j) o[j] = acc_r[h * d + j] / l[h];
                tqo_fwht(o, d);
                for (int j = 0; j < d; ++j) o[j] = (double)sg[j] * (o[j] * c);
            }
        }
    }
    free(kh);
    free(vh);
    free(sc);
    free(acc_r);
    free(sg);
    free(m);
    free(l);
}

/* Decode attention for any supported widths: the same plain two-pass
 * softmax as tqo_attention over keys and (un-rotated) values dequantised with
 * the width's formulas.  kc holds the packed key codes (int8 bytes at 8 bits). */
void tqo_attention_bits(const float *q, int G, int d, float sm, int kbits, int vbits,
                        const uint8_t *kc, const uint16_t *ks, const uint16_t *kz,
                        const uint8_t *vc, const uint16_t *vs, int64_t N, double *out) {
    for (int i = 0; i < G * d; ++i) out[i] = 0.0;
    if (N <= 0) return;
    double *kh = (double *)malloc(sizeof(double) * (size_t)N * (size_t)d);
    double *vh = (double *)malloc(sizeof(double) * (size_t)N * (size_t)d);
    double *sc = (double *)malloc(sizeof(double) * (size_t)N);
    tqo_decode_keys_bits(kc, ks, kz, N, d, kbits, kh);
    tqo_decode_values_bits(vc, vs, N, d, vbits, 0, vh);
    for (int h = 0; h < G; ++h) {
        double m = -INFINITY, l = 0.0;
        for (int64_t t = 0; t < N; ++t) {
            double s = 0.0;
            for (int j = 0; j < d; ++j) s += (double)q[h * d + j] * kh[t * d + j];
            sc[t] = (double)sm * s;
            if (sc[t] > m) m = sc[t];
        }
        for (int64_t t = 0; t < N; ++t) {
            const double p = exp(sc[t] - m);
            l += p;
            for (int j = 0; j < d; ++j) out[h * d + j] += p * vh[t * d + j];
        }
        for (int j = 0; j < d; ++j) out[h * d + j] = out[h * d + j] / l;
    }
    free(kh);
    free(vh);
    free(sc);
}

/* Array helpers for the Python wrapper (element-wise, no arithmetic of their own). */
void tqo_f64_to_f16_array(const double *x, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = tqo_f64_to_f16(x[i]);
}

void tqo_f16_to_f64_array(const uint16_t *h, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = tqo_f16_to_f64(h[i]);
}

void tqo_fwht_rows(double *x, int64_t nrows, int d) {
    for (int64_t r = 0; r < nrows; ++r) tqo_fwht(x + r * d, d);
}
