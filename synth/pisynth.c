/*
 * pisynth.c -- seeded synthetic workload generator for the predictor-gated sparse FFN.
 *
 * This module produces INPUTS only: fp16 weight matrices, Q4_0 weight rows, token
 * vectors and per-neuron predictor offsets.  It contains none of the arithmetic of the
 * method itself (no predictor evaluation, no masking, no FFN).  Both the CPU oracle and
 * the HIP path consume the bytes written here, so the two see identical inputs.
 *
 * Every value is a pure function of (seed, layer, tensor, row, col) through a
 * counter-based hash built from the SplitMix64 output finalizer (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).  Output therefore does
 * not depend on the number of threads or on the order rows are produced in.
 *
 * Normal draws use the Irwin-Hall sum of four uniform 16-bit integers, centred and scaled
 * to unit variance (bounded at +-sqrt(12) sigma); the integer sum is exact, it is scaled
 * by one fp32 multiply and rounded to fp16 with round-to-nearest-even as IEEE 754
 * binary16 defines it.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- hashing */

static inline uint64_t ps_mix64(uint64_t z) {
    /* SplitMix64 output function (Steele et al. 2014). */
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

#define PS_GOLDEN 0x9E3779B97F4A7C15ull

/* Hash prefix for one (seed, layer, tensor, row); finish with ps_hash_col. */
static inline uint64_t ps_hash_row(uint64_t seed, uint32_t layer, uint32_t tensor, uint64_t row) {
    uint64_t h = ps_mix64(seed + PS_GOLDEN);
    h = ps_mix64(h ^ (((uint64_t)layer << 32) | (uint64_t)tensor));
    h = ps_mix64(h + PS_GOLDEN * (row + 1));
    return h;
}

static inline uint64_t ps_hash_col(uint64_t row_hash, uint64_t col) {
    return ps_mix64(row_hash ^ (PS_GOLDEN * (col + 1)));
}

uint64_t ps_hash(uint64_t seed, uint32_t layer, uint32_t tensor, uint64_t row, uint64_t col) {
    return ps_hash_col(ps_hash_row(seed, layer, tensor, row), col);
}

/* ------------------------------------------------------- fp32 -> binary16 */

/* Round an fp32 value to IEEE 754 binary16, round-to-nearest, ties to even. */
uint16_t ps_f32_to_f16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t exp = (u >> 23) & 0xFFu;
    uint32_t man = u & 0x7FFFFFu;
    if (exp == 0xFFu) {                       /* inf / NaN */
        if (man == 0) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | 0x7E00u | (man >> 13));
    }
    int32_t e = (int32_t)exp - 127 + 15;       /* biased binary16 exponent */
    if (e >= 31) return (uint16_t)(sign | 0x7C00u);   /* overflow -> inf */
    if (e <= 0) {
        /* subnormal (or zero) in binary16: value = m * 2^-24 with m < 1024 */
        if (e < -10) return (uint16_t)sign;    /* rounds to zero (below half of min subnormal) */
        uint32_t full = man | 0x800000u;       /* 24-bit significand */
        uint32_t shift = (uint32_t)(14 - e);   /* bits to drop: 13 + (1 - e) */
        uint32_t q = full >> shift;
        uint32_t rem = full & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) q += 1u;
        return (uint16_t)(sign | q);           /* q may carry into the exponent field: correct */
    }
    uint32_t q = ((uint32_t)e << 10) | (man >> 13);
    uint32_t rem = man & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q += 1u;  /* carry may reach inf: correct */
    return (uint16_t)(sign | q);
}

/* --------------------------------------------------------------- normals */

/* Irwin-Hall(4) normal from the four 16-bit fields of one hash: an integer in
 * [-131070, 131070], of variance 4*(65536^2-1)/12. */
static inline int32_t ps_ih4(uint64_t h) {
    int32_t s = (int32_t)(h & 0xFFFFu) + (int32_t)((h >> 16) & 0xFFFFu) +
                (int32_t)((h >> 32) & 0xFFFFu) + (int32_t)((h >> 48) & 0xFFFFu);
    return s - 131070;
}

static float ps_ih4_scale(double sigma) {
    /* sqrt(3)/65536 maps the Irwin-Hall(4) sum to (nearly) unit variance. */
    return (float)(sigma * sqrt(3.0) / 65536.0);
}

/*
 * Fill an fp16 matrix.  Output row k (k < nrows) holds generator row rows[k] (or row0+k
 * when rows == NULL), columns 0..ncols-1, at out + k*out_stride (stride in elements).
 */
void ps_normal_f16(uint64_t seed, uint32_t layer, uint32_t tensor, const int32_t *rows,
                   int64_t row0, int64_t nrows, int64_t ncols, double sigma,
                   uint16_t *out, int64_t out_stride) {
    const float k = ps_ih4_scale(sigma);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        uint64_t grow = rows ? (uint64_t)rows[r] : (uint64_t)(row0 + r);
        uint64_t hr = ps_hash_row(seed, layer, tensor, grow);
        uint16_t *o = out + r * out_stride;
        for (int64_t c = 0; c < ncols; ++c)
            o[c] = ps_f32_to_f16((float)ps_ih4(ps_hash_col(hr, (uint64_t)c)) * k);
    }
}

/* Same draws widened to fp32 without fp16 rounding (used for statistics checks). */
void ps_normal_f32(uint64_t seed, uint32_t layer, uint32_t tensor, int64_t row0, int64_t nrows,
                   int64_t ncols, double sigma, float *out) {
    const float k = ps_ih4_scale(sigma);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        uint64_t hr = ps_hash_row(seed, layer, tensor, (uint64_t)(row0 + r));
        for (int64_t c = 0; c < ncols; ++c)
            out[r * ncols + c] = (float)ps_ih4(ps_hash_col(hr, (uint64_t)c)) * k;
    }
}

/*
 * Q4_0 rows (32-weight blocks, one fp16 scale each).  Storage per row of d weights:
 *   d/2 code bytes  -- byte j holds weight 2j in its low nibble, weight 2j+1 in its high nibble
 *   d/32 fp16 scales -- little-endian, block b covers weights 32b..32b+31
 * for 9d/16 bytes per row.  Codes are uniform on [0,15]; the block scale is
 * fp16((0.75 + 0.5u) / sqrt(21.5 d)) with u uniform on [0,1), so that weights
 * scale*(code-8) have variance near 1/d (21.5 is the mean of (code-8)^2).
 * code_tensor and code_tensor+1 are the hash streams of codes and scales.
 */
void ps_q4_0_rows(uint64_t seed, uint32_t layer, uint32_t code_tensor, const int32_t *rows,
                  int64_t row0, int64_t nrows, int64_t d, uint8_t *out, int64_t out_stride_bytes) {
    const double inv = 1.0 / sqrt(21.5 * (double)d);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        uint64_t grow = rows ? (uint64_t)rows[r] : (uint64_t)(row0 + r);
        uint8_t *o = out + r * out_stride_bytes;
        uint64_t hc = ps_hash_row(seed, layer, code_tensor, grow);
        int64_t nbytes = d / 2;
        for (int64_t j = 0; j < nbytes; j += 8) {
            uint64_t h = ps_hash_col(hc, (uint64_t)(j / 8));
            for (int64_t t = 0; t < 8 && j + t < nbytes; ++t) o[j + t] = (uint8_t)(h >> (8 * t));
        }
        uint64_t hs = ps_hash_row(seed, layer, code_tensor + 1, grow);
        uint16_t *sc = (uint16_t *)(o + nbytes);
        for (int64_t b = 0; b < d / 32; ++b) {
            double u = (double)(ps_hash_col(hs, (uint64_t)b) >> 11) * (1.0 / 9007199254740992.0);
            sc[b] = ps_f32_to_f16((float)((0.75 + 0.5 * u) * inv));
        }
    }
}

/* ------------------------------------------------ Zipf firing frequencies */

/* p_k = min(cap, A k^-s) for ranks k = 1..f. */
static double ps_zipf_mean(int64_t f, double s, double A, double cap) {
    double acc = 0.0;
    for (int64_t k = 1; k <= f; ++k) {
        double p = A * pow((double)k, -s);
        acc += p < cap ? p : cap;
    }
    return acc / (double)f;
}

static double ps_zipf_share(int64_t f, double s, double A, double cap, int64_t ntop) {
    double top = 0.0, all = 0.0;
    for (int64_t k = 1; k <= f; ++k) {
        double p = A * pow((double)k, -s);
        p = p < cap ? p : cap;
        all += p;
        if (k <= ntop) top += p;
    }
    return top / all;
}

/* For a given exponent s, the amplitude A giving mean frequency `density` (bisection). */
static double ps_zipf_amp(int64_t f, double s, double density, double cap) {
    double lo = 0.0, hi = 1.0;
    while (ps_zipf_mean(f, s, hi, cap) < density) hi *= 2.0;
    for (int it = 0; it < 100; ++it) {
        double mid = 0.5 * (lo + hi);
        if (ps_zipf_mean(f, s, mid, cap) < density) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

/*
 * Solve (s, A) so that the mean firing frequency is `density` and the hottest
 * ntop = round(top_frac*f) neurons carry `share` of all firings.  Returns 0 on success.
 */
int ps_zipf_solve(int64_t f, double density, double top_frac, double share, double cap,
                  double *s_out, double *A_out) {
    int64_t ntop = (int64_t)llround(top_frac * (double)f);
    if (ntop < 1 || ntop >= f || density <= 0.0 || density >= cap) return -1;
    double lo = 0.0, hi = 4.0;
    for (int it = 0; it < 80; ++it) {
        double mid = 0.5 * (lo + hi);
        double A = ps_zipf_amp(f, mid, density, cap);
        if (ps_zipf_share(f, mid, A, cap, ntop) < share) lo = mid; else hi = mid;
    }
    *s_out = 0.5 * (lo + hi);
    *A_out = ps_zipf_amp(f, *s_out, density, cap);
    return 0;
}

/*
 * Per-neuron firing frequency p[i] for one layer: rank k (1-based) is given to neuron
 * perm[k-1], where perm is a seeded Fisher-Yates shuffle of 0..f-1.  rank_of[i] (may be
 * NULL) receives neuron i's rank.
 */
void ps_zipf_freq(uint64_t seed, uint32_t layer, uint32_t perm_tensor, int64_t f, double s,
                  double A, double cap, int32_t *perm, double *p, int32_t *rank_of) {
    for (int64_t i = 0; i < f; ++i) perm[i] = (int32_t)i;
    uint64_t hr = ps_hash_row(seed, layer, perm_tensor, 0);
    for (int64_t i = f - 1; i > 0; --i) {
        int64_t j = (int64_t)(ps_hash_col(hr, (uint64_t)i) % (uint64_t)(i + 1));
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
    for (int64_t k = 1; k <= f; ++k) {
        double v = A * pow((double)k, -s);
        int32_t i = perm[k - 1];
        p[i] = v < cap ? v : cap;
        if (rank_of) rank_of[i] = (int32_t)k;
    }
}

/* ------------------------------------------------------ predictor offsets */

/* Standard normal quantile by bisection on the library erfc (Phi(x) = erfc(-x/sqrt2)/2). */
static double ps_norm_quantile(double p) {
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 200; ++it) {
        double mid = 0.5 * (lo + hi);
        if (0.5 * erfc(-mid / sqrt(2.0)) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

static double ps_f16_bits_to_double(uint16_t h) {
    /* Widening of binary16 for the offset calibration (generator-side, not the oracle's). */
    int e = (h >> 10) & 31, m = h & 1023;
    double v = e == 0 ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
    return (h & 0x8000) ? -v : v;
}

/*
 * Offsets c_i that make neuron i's logit positive with probability about p_i, under the
 * workload's own law: with z = ReLU of near-N(0,1) pre-activations, the row product
 * P2[i]·z is close to normal with mean 0.39894*sum(P2[i,:]) and variance
 * 0.34085*sum(P2[i,:]^2) (mean and variance of a rectified standard normal).  So
 * c_i = s_i*quantile(p_i) - mu_i.  P2 is read as stored (fp16 bits, [f][r] row-major).
 */
void ps_offsets(const uint16_t *p2, int64_t f, int64_t r, const double *p, uint16_t *c_out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < f; ++i) {
        double s1 = 0.0, s2 = 0.0;
        for (int64_t j = 0; j < r; ++j) {
            double w = ps_f16_bits_to_double(p2[i * r + j]);
            s1 += w;
            s2 += w * w;
        }
        double mu = 0.3989422804014327 * s1;
        double sd = sqrt(0.3408450569081046 * s2);
        double ci = sd * ps_norm_quantile(p[i]) - mu;
        c_out[i] = ps_f32_to_f16((float)ci);
    }
}

int ps_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
