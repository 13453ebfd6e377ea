/*
 * pi_oracle.c -- CPU oracle for the predictor-gated, neuron-aware sparse FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this
 * file's library; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (PowerInfer, arXiv 2312.12456; abstract and "method" section of the
 * summary page): a predictor decides, per token, which FFN neurons fire; a neuron-aware
 * operator then computes only those neurons; a GPU placement index restricts the work to
 * the neurons resident on the device.  Written out plainly:
 *
 *   z_b  = max(0, P1 x_b)                        predictor hidden layer (rank r)
 *   l_b  = P2 z_b + c                            per-neuron logits with offset c
 *   m_b  = [l_b > 0];  M = OR_b m_b              firing prediction, union over the batch
 *   M'   = M restricted to resident neurons      placement index (NULL = all resident)
 *   idx  = ascending members of M'
 *   h_bk = max(0, W_up[i] x_b + b_up[i])                 (ReLU FFN)
 *        = max(0, W_gate[i] x_b) * (W_up[i] x_b)         (ReGLU FFN)      with i = idx[k]
 *   y_b  = b_down + sum_k h_bk W_down^T[i]       summed in ascending k
 *
 * Every fp16 value is widened exactly to double; Q4_0 weights are scale*(code-8), also
 * exact in double; all sums are taken in double in the order written above.  The caller
 * rounds y to fp32.  Nothing is blocked, fused or reordered beyond that definition;
 * OpenMP only splits independent outputs across threads, so results do not depend on the
 * thread count.
 */
#include "pi_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------ binary16 */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double pio_half(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                   /* zero / subnormal: m * 2^-24 */
    else if (e == 31)
        v = m == 0 ? INFINITY : NAN;                 /* infinity / NaN */
    else
        v = ldexp((double)(1024 + m), e - 25);       /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double g_half[65536];
static int g_half_ready = 0;

static void pio_init(void) {
    if (g_half_ready) return;
    for (int i = 0; i < 65536; ++i) g_half[i] = pio_half((uint16_t)i);
    g_half_ready = 1;
}

/* ------------------------------------------------------------ weight rows */

/* Bytes of one stored row of d weights. */
int64_t pio_row_bytes(int wtype, int64_t d) {
    return wtype == PIO_F16 ? 2 * d : (d / 2 + 2 * (d / 32));
}

/*
 * Weight t of one stored row.
 * fp16: the t-th binary16 value.
 * Q4_0 (32-weight blocks, one fp16 scale each): byte t/2 of the code area holds weight t in
 * its low nibble when t is even and in its high nibble when t is odd; the d/32 scales follow
 * the d/2 code bytes; the weight is scale[t/32] * (code - 8).
 */
static inline double pio_weight(const uint8_t *row, int wtype, int64_t d, int64_t t) {
    if (wtype == PIO_F16) {
        uint16_t v;
        memcpy(&v, row + 2 * t, 2);
        return g_half[v];
    }
    uint8_t byte = row[t / 2];
    int code = (t & 1) ? (byte >> 4) : (byte & 0x0F);
    uint16_t sbits;
    memcpy(&sbits, row + d / 2 + 2 * (t / 32), 2);
    return g_half[sbits] * (double)(code - 8);
}

void pio_decode_row(const void *row, int wtype, int64_t d, double *w) {
    pio_init();
    for (int64_t t = 0; t < d; ++t) w[t] = pio_weight((const uint8_t *)row, wtype, d, t);
}

static double pio_dot_row(const uint8_t *row, int wtype, int64_t d, const uint16_t *x) {
    double acc = 0.0;
    for (int64_t t = 0; t < d; ++t) acc += pio_weight(row, wtype, d, t) * g_half[x[t]];
    return acc;
}

/* ------------------------------------------------------------ predictor */

int pio_predict(int64_t d, int64_t f, int64_t r, const uint16_t *p1, const uint16_t *p2,
                const uint16_t *c, const uint16_t *x, int64_t B, double *logits,
                uint8_t *mask_tok, uint8_t *mask) {
    if (d <= 0 || f <= 0 || r <= 0 || B <= 0 || !p1 || !p2 || !c || !x || !mask) return -1;
    pio_init();
    double *z = (double *)malloc(sizeof(double) * (size_t)r);
    double *l = (double *)malloc(sizeof(double) * (size_t)f);
    if (!z || !l) { free(z); free(l); return -2; }
    memset(mask, 0, (size_t)f);
    for (int64_t b = 0; b < B; ++b) {
        const uint16_t *xb = x + b * d;
        /* z = max(0, P1 x_b) */
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < d; ++k) acc += g_half[p1[j * d + k]] * g_half[xb[k]];
            z[j] = acc > 0.0 ? acc : 0.0;
        }
        /* l = P2 z + c */
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < f; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < r; ++j) acc += g_half[p2[i * r + j]] * z[j];
            l[i] = acc + g_half[c[i]];
        }
        for (int64_t i = 0; i < f; ++i) {
            uint8_t m = l[i] > 0.0;                  /* strict: a zero logit does not fire */
            if (logits) logits[b * f + i] = l[i];
            if (mask_tok) mask_tok[b * f + i] = m;
            mask[i] = (uint8_t)(mask[i] | m);        /* union over the batch */
        }
    }
    free(z);
    free(l);
    return 0;
}

/* ------------------------------------------------------------ compaction */

int pio_compact(const uint8_t *mask, int64_t f, const int32_t *slot_of, int32_t *idx,
                int32_t *counts) {
    if (!mask || !idx || !counts || f < 0) return -1;
    int32_t n = 0, n_pred = 0;
    for (int64_t i = 0; i < f; ++i) {
        if (!mask[i]) continue;
        n_pred++;
        if (slot_of == NULL || slot_of[i] >= 0) idx[n++] = (int32_t)i;
    }
    counts[0] = n;
    counts[1] = n_pred;
    return 0;
}

/* ------------------------------------------------------------ sparse FFN */

int pio_sparse_ffn(int64_t d, int64_t f, int gated, int wtype, int64_t n_slots,
                   const int32_t *slot_of, const void *w_in, const void *w_down_t,
                   const uint16_t *b_up, const uint16_t *b_down, const uint16_t *x, int64_t B,
                   const int32_t *idx, int64_t n, double *h_out, double *y) {
    if (d <= 0 || f <= 0 || B <= 0 || n < 0 || n > f || !w_in || !w_down_t || !x || !y) return -1;
    if (n > 0 && !idx) return -1;
    if (wtype != PIO_F16 && wtype != PIO_Q4_0) return -3;
    if (wtype == PIO_Q4_0 && d % 32 != 0) return -3;
    if (gated < 0 || gated > PIO_SQUARED_RELU) return -3;
    if (gated == PIO_REGLU && b_up) return -3;       /* the gated form has no up bias */
    pio_init();
    const int64_t rb = pio_row_bytes(wtype, d);
    const int64_t in_rows = gated == PIO_REGLU ? 2 : 1;
    const uint8_t *win = (const uint8_t *)w_in;
    const uint8_t *wdn = (const uint8_t *)w_down_t;

    int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    double *h = (double *)malloc(sizeof(double) * (size_t)(B * (n > 0 ? n : 1)));
    if (!slot || !h) { free(slot); free(h); return -2; }
    for (int64_t k = 0; k < n; ++k) {
        int64_t i = idx[k];
        int64_t s = slot_of ? slot_of[i] : i;
        if (i < 0 || i >= f || s < 0 || s >= n_slots) { free(slot); free(h); return -2; }
        slot[k] = s;
    }

    /* h_bk for every active neuron k (independent outputs). */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t k = 0; k < n; ++k) {
        const uint8_t *row = win + slot[k] * in_rows * rb;
        for (int64_t b = 0; b < B; ++b) {
            const uint16_t *xb = x + b * d;
            double hv;
            if (gated == PIO_REGLU) {
                double g = pio_dot_row(row, wtype, d, xb);        /* gate row first */
                double u = pio_dot_row(row + rb, wtype, d, xb);   /* then the up row */
                hv = (g > 0.0 ? g : 0.0) * u;
            } else {
                double u = pio_dot_row(row, wtype, d, xb);
                if (b_up) u += g_half[b_up[slot[k]]];
                hv = u > 0.0 ? u : 0.0;
                if (gated == PIO_SQUARED_RELU) hv = hv * hv;     /* squared ReLU: ReLU(u)^2 */
            }
            h[b * n + k] = hv;
        }
    }

    /* y_b = b_down + sum over ascending k of h_bk * W_down^T[slot_k]; columns split
     * across threads, every column summed in the same ascending order. */
    const int64_t CB = 256;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j0 = 0; j0 < d; j0 += CB) {
        int64_t j1 = j0 + CB < d ? j0 + CB : d;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t j = j0; j < j1; ++j) y[b * d + j] = b_down ? g_half[b_down[j]] : 0.0;
        for (int64_t k = 0; k < n; ++k) {
            const uint8_t *row = wdn + slot[k] * rb;
            for (int64_t j = j0; j < j1; ++j) {
                double w = pio_weight(row, wtype, d, j);
                for (int64_t b = 0; b < B; ++b) y[b * d + j] += h[b * n + k] * w;
            }
        }
    }
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)(B * n));
    free(slot);
    free(h);
    return 0;
}

/* Dense FFN over all f neurons (identity slots) -- the plain MLP the sparse form must equal. */
int pio_dense_ffn(int64_t d, int64_t f, int gated, int wtype, const void *w_in,
                  const void *w_down_t, const uint16_t *b_up, const uint16_t *b_down,
                  const uint16_t *x, int64_t B, uint8_t *true_mask, double *y) {
    if (d <= 0 || f <= 0 || B <= 0 || !w_in || !w_down_t || !x || !y) return -1;
    int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)f);
    double *h = (double *)malloc(sizeof(double) * (size_t)(B * f));
    if (!all || !h) { free(all); free(h); return -2; }
    for (int64_t i = 0; i < f; ++i) all[i] = (int32_t)i;
    int rc = pio_sparse_ffn(d, f, gated, wtype, f, NULL, w_in, w_down_t, b_up, b_down, x, B, all, f,
                            h, y);
    if (rc == 0 && true_mask)
        for (int64_t t = 0; t < B * f; ++t) true_mask[t] = h[t] != 0.0;
    free(all);
    free(h);
    return rc;
}

/* ------------------------------------------------------------ whole layer */

int pio_ffn_layer(int64_t d, int64_t f, int64_t r, const uint16_t *p1, const uint16_t *p2,
                  const uint16_t *c, int gated, int wtype, int64_t n_slots, const int32_t *slot_of,
                  const void *w_in, const void *w_down_t, const uint16_t *b_up,
                  const uint16_t *b_down, const uint16_t *x, int64_t B, double *logits,
                  uint8_t *mask, int32_t *idx, int32_t *counts, double *y) {
    if (!mask || !idx || !counts) return -1;
    int rc = pio_predict(d, f, r, p1, p2, c, x, B, logits, NULL, mask);
    if (rc) return rc;
    rc = pio_compact(mask, f, slot_of, idx, counts);
    if (rc) return rc;
    return pio_sparse_ffn(d, f, gated, wtype, n_slots, slot_of, w_in, w_down_t, b_up, b_down, x, B,
                          idx, counts[0], NULL, y);
}

int pio_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void pio_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
