// pi_cold.cpp -- the host half of the hybrid neuron split (PowerInfer, arXiv 2312.12456, method
// section and abstract: hot neurons are preloaded on the GPU, the cold ones are computed on the
// CPU, and the two partial results are combined).  The neurons that are predicted to fire but are
// not resident on the device are computed here, on the host's cores, over the same neuron-major
// rows the device kernels read; the caller adds the returned y to the device's y.
//
// For the listed neurons i (mask[i] != 0 and held here, ascending), slot s:
//   h[b] = max(0, W_up[s] x_b + b_up[s])  (squared for squared ReLU)  or  max(0, W_gate[s] x_b) * (W_up[s] x_b)
//   y[b] = sum over listed i of h[b] W_down^T[s]      (no b_down: the device half adds it once)
//
// The list is cut into kChunks fixed chunks; each chunk's partial y is summed in ascending order
// by whichever thread takes it, and the chunk partials are added in chunk order, so y does not
// depend on the number of threads.  fp16 rows are widened with F16C and accumulated in fp32 with
// FMA; Q4_0 codes are decoded exactly (scale * (code - 8)).  Host code only: no HIP call.
#include <immintrin.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "pi_sparse_ffn.h"

namespace {

constexpr int kChunks = 64;

size_t align64(size_t x) { return (x + 63) / 64 * 64; }

float hsum(__m256 v) {
    __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
    s = _mm_add_ps(s, _mm_movehl_ps(s, s));
    s = _mm_add_ss(s, _mm_shuffle_ps(s, s, 1));
    return _mm_cvtss_f32(s);
}

__m256 load_f16x8(const uint16_t *p) { return _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i *>(p))); }

float half_to_float(uint16_t h) { return _cvtsh_ss(h); }

// The 32 weights of Q4_0 block q of a row (d/2 code bytes, then d/32 fp16 scales), as
// (code - 8) in four vectors of 8 consecutive weights, and the block's scale.
void q4_block(const uint8_t *row, int d, int q, __m256 (&v)[4], float &scale) {
    const __m128i c = _mm_loadu_si128(reinterpret_cast<const __m128i *>(row + (size_t)q * 16));
    const __m128i lo = _mm_and_si128(c, _mm_set1_epi8(0x0F));                    // weights 2j
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(c, 4), _mm_set1_epi8(0x0F));  // weights 2j+1
    const __m128i w0 = _mm_unpacklo_epi8(lo, hi), w1 = _mm_unpackhi_epi8(lo, hi); // weights 0..15, 16..31
    const __m256 eight = _mm256_set1_ps(8.f);
    v[0] = _mm256_sub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(w0)), eight);
    v[1] = _mm256_sub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(w0, 8))), eight);
    v[2] = _mm256_sub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(w1)), eight);
    v[3] = _mm256_sub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(w1, 8))), eight);
    uint16_t s;
    memcpy(&s, row + (size_t)d / 2 + (size_t)q * 2, 2);
    scale = half_to_float(s);
}

// Four rows at a time: the dots of four fp16 rows with one x (each x vector loaded once for all
// four), and y += sum_r h[r] * row_r (y loaded and stored once per four rows).  A missing row is
// passed as a copy of row 0 with h = 0, which adds exact zeros.
void dot4_f16(const uint16_t *const (&w)[4], const float *x, int d, float (&out)[4]) {
    __m256 a[4][2];
    for (int r = 0; r < 4; ++r) a[r][0] = a[r][1] = _mm256_setzero_ps();
    int j = 0;
    for (; j + 16 <= d; j += 16) {
        const __m256 x0 = _mm256_loadu_ps(x + j), x1 = _mm256_loadu_ps(x + j + 8);
        for (int r = 0; r < 4; ++r) {
            a[r][0] = _mm256_fmadd_ps(load_f16x8(w[r] + j), x0, a[r][0]);
            a[r][1] = _mm256_fmadd_ps(load_f16x8(w[r] + j + 8), x1, a[r][1]);
        }
    }
    if (j < d) {                                                  // d % 16 == 8
        const __m256 x0 = _mm256_loadu_ps(x + j);
        for (int r = 0; r < 4; ++r) a[r][0] = _mm256_fmadd_ps(load_f16x8(w[r] + j), x0, a[r][0]);
    }
    for (int r = 0; r < 4; ++r) out[r] = hsum(_mm256_add_ps(a[r][0], a[r][1]));
}

void axpy4_f16(const float (&h)[4], const uint16_t *const (&w)[4], float *y, int d) {
    const __m256 h0 = _mm256_set1_ps(h[0]), h1 = _mm256_set1_ps(h[1]), h2 = _mm256_set1_ps(h[2]),
                 h3 = _mm256_set1_ps(h[3]);
    for (int j = 0; j < d; j += 8) {
        __m256 acc = _mm256_loadu_ps(y + j);
        acc = _mm256_fmadd_ps(h0, load_f16x8(w[0] + j), acc);
        acc = _mm256_fmadd_ps(h1, load_f16x8(w[1] + j), acc);
        acc = _mm256_fmadd_ps(h2, load_f16x8(w[2] + j), acc);
        acc = _mm256_fmadd_ps(h3, load_f16x8(w[3] + j), acc);
        _mm256_storeu_ps(y + j, acc);
    }
}

void dot4_q4(const uint8_t *const (&w)[4], const float *x, int d, float (&out)[4]) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < d / 32; ++q) {
        const float *xq = x + (size_t)q * 32;
        const __m256 x0 = _mm256_loadu_ps(xq), x1 = _mm256_loadu_ps(xq + 8), x2 = _mm256_loadu_ps(xq + 16),
                     x3 = _mm256_loadu_ps(xq + 24);
        for (int r = 0; r < 4; ++r) {
            __m256 v[4];
            float sc;
            q4_block(w[r], d, q, v, sc);
            __m256 t = _mm256_mul_ps(v[0], x0);
            t = _mm256_fmadd_ps(v[1], x1, t);
            t = _mm256_fmadd_ps(v[2], x2, t);
            t = _mm256_fmadd_ps(v[3], x3, t);
            acc[r] += sc * hsum(t);
        }
    }
    for (int r = 0; r < 4; ++r) out[r] = acc[r];
}

void axpy4_q4(const float (&h)[4], const uint8_t *const (&w)[4], float *y, int d) {
    for (int q = 0; q < d / 32; ++q) {
        float *yq = y + (size_t)q * 32;
        __m256 acc[4];
        for (int k = 0; k < 4; ++k) acc[k] = _mm256_loadu_ps(yq + 8 * k);
        for (int r = 0; r < 4; ++r) {
            __m256 v[4];
            float sc;
            q4_block(w[r], d, q, v, sc);
            const __m256 hs = _mm256_set1_ps(h[r] * sc);
            for (int k = 0; k < 4; ++k) acc[k] = _mm256_fmadd_ps(hs, v[k], acc[k]);
        }
        for (int k = 0; k < 4; ++k) _mm256_storeu_ps(yq + 8 * k, acc[k]);
    }
}

int check_host_ffn(const pi_ffn *f) {
    if (!f) return PI_ERR_NULL;
    if (!f->w_in || !f->w_down_t) return PI_ERR_NULL;
    if (f->wtype != PI_F16 && f->wtype != PI_Q4_0) return PI_ERR_DTYPE;
    if (f->gated != 0 && f->gated != 1) return PI_ERR_DTYPE;
    if (f->gated && f->wtype == PI_Q4_0) return PI_ERR_DTYPE;
    if (f->gated && f->b_up) return PI_ERR_DTYPE;
    if (f->act != PI_ACT_RELU && f->act != PI_ACT_SQUARED_RELU) return PI_ERR_DTYPE;
    if (f->gated && f->act != PI_ACT_RELU) return PI_ERR_DTYPE;
    if (f->b_down) return PI_ERR_DTYPE;                           // the device half adds b_down
    if (f->d_ffn < 1 || f->d_ffn > PI_MAX_D_FFN || f->n_slots < 0 || f->n_slots > f->d_ffn) return PI_ERR_SHAPE;
    if (!f->slot_of && f->n_slots != f->d_ffn) return PI_ERR_SHAPE;
    if (f->d_model > PI_MAX_D_MODEL) return PI_ERR_SHAPE;
    if (f->wtype == PI_F16 && (f->d_model < 8 || f->d_model % 8 != 0)) return PI_ERR_SHAPE;
    if (f->wtype == PI_Q4_0 && (f->d_model < 256 || f->d_model % 256 != 0)) return PI_ERR_SHAPE;
    return PI_OK;
}

struct ColdScratch {
    float *xf;       // [B][d] x widened to fp32
    float *part;     // [kChunks][B][d] chunk partials
    int32_t *list;   // [d_ffn] listed neuron ids, ascending
};

ColdScratch cold_scratch(const pi_ffn *f, int B, void *ws) {
    char *p = static_cast<char *>(ws);
    const size_t bd = (size_t)B * f->d_model * sizeof(float);
    ColdScratch s;
    s.xf = reinterpret_cast<float *>(p);
    s.part = reinterpret_cast<float *>(p + align64(bd));
    s.list = reinterpret_cast<int32_t *>(p + align64(bd) + align64(kChunks * bd));
    return s;
}

}  // namespace

extern "C" {

size_t pi_cold_workspace_bytes(const pi_ffn *ffn, int32_t batch) {
    if (check_host_ffn(ffn) != PI_OK || batch < 1 || batch > PI_MAX_BATCH) return 0;
    const size_t bd = (size_t)batch * ffn->d_model * sizeof(float);
    return align64(bd) + align64(kChunks * bd) + align64((size_t)ffn->d_ffn * sizeof(int32_t));
}

int pi_cold_ffn_host(const pi_ffn *ffn, const void *x, int32_t batch, const uint8_t *mask, float *y,
                     int32_t *n_computed, void *ws, size_t ws_bytes, int32_t n_threads) {
    int rc = check_host_ffn(ffn);
    if (rc) return rc;
    if (batch < 1 || batch > PI_MAX_BATCH) return PI_ERR_BATCH;
    if (!x || !mask || !y) return PI_ERR_NULL;
    if (n_threads < 0) return PI_ERR_SHAPE;
    if (!ws || ws_bytes < pi_cold_workspace_bytes(ffn, batch)) return PI_ERR_WORKSPACE;
    const int B = batch, d = ffn->d_model, f = ffn->d_ffn, ns = ffn->n_slots;
    const bool q4 = ffn->wtype == PI_Q4_0, gated = ffn->gated != 0, sq = ffn->act == PI_ACT_SQUARED_RELU;
    const size_t rb = q4 ? (size_t)d * 9 / 16 : (size_t)d * 2;
    const size_t in_stride = gated ? 2 * rb : rb;
    const uint8_t *w_in = static_cast<const uint8_t *>(ffn->w_in), *w_dn = static_cast<const uint8_t *>(ffn->w_down_t);
    const uint16_t *b_up = static_cast<const uint16_t *>(ffn->b_up);
    const ColdScratch sc = cold_scratch(ffn, B, ws);

    // the listed neurons, ascending: predicted and held here
    int n = 0;
    for (int i = 0; i < f; ++i) {
        if (!mask[i]) continue;
        const int s = ffn->slot_of ? ffn->slot_of[i] : i;
        if (s >= 0 && s < ns) sc.list[n++] = i;
    }
    if (n_computed) *n_computed = n;
    const uint16_t *xh = static_cast<const uint16_t *>(x);
    for (size_t j = 0; j < (size_t)B * d; j += 8) _mm256_storeu_ps(sc.xf + j, load_f16x8(xh + j));
    const int nthr = n_threads > 0 ? n_threads : omp_get_max_threads();
    const size_t bd = (size_t)B * d;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthr)
    for (int c = 0; c < kChunks; ++c) {
        float *yc = sc.part + (size_t)c * bd;
        memset(yc, 0, bd * sizeof(float));
        const int k0 = (int)((int64_t)n * c / kChunks), k1 = (int)((int64_t)n * (c + 1) / kChunks);
        // neurons four at a time (gated: two, as four rows); a missing neuron repeats the first
        // with h = 0
        const int G = gated ? 2 : 4;
        for (int k = k0; k < k1; k += G) {
            const int m = k1 - k < G ? k1 - k : G;
            int sl[4];
            for (int i = 0; i < 4; ++i) {
                const int id = sc.list[k + (i < m ? i : 0)];
                sl[i] = ffn->slot_of ? ffn->slot_of[id] : id;
            }
            float h[PI_MAX_BATCH][4];
            bool any = false;
            for (int b = 0; b < B; ++b) {
                const float *xb = sc.xf + (size_t)b * d;
                float u[4], g[4];
                if (q4) {
                    const uint8_t *const rows[4] = {w_in + (size_t)sl[0] * in_stride, w_in + (size_t)sl[1] * in_stride,
                                                    w_in + (size_t)sl[2] * in_stride, w_in + (size_t)sl[3] * in_stride};
                    dot4_q4(rows, xb, d, u);
                } else if (gated) {
                    // rows: gate and up of neurons 0 and 1
                    const uint16_t *const rows[4] = {
                        reinterpret_cast<const uint16_t *>(w_in + (size_t)sl[0] * in_stride),
                        reinterpret_cast<const uint16_t *>(w_in + (size_t)sl[0] * in_stride + rb),
                        reinterpret_cast<const uint16_t *>(w_in + (size_t)sl[1] * in_stride),
                        reinterpret_cast<const uint16_t *>(w_in + (size_t)sl[1] * in_stride + rb)};
                    float gu[4];
                    dot4_f16(rows, xb, d, gu);
                    g[0] = gu[0]; u[0] = gu[1]; g[1] = gu[2]; u[1] = gu[3];
                } else {
                    const uint16_t *const rows[4] = {reinterpret_cast<const uint16_t *>(w_in + (size_t)sl[0] * in_stride),
                                                     reinterpret_cast<const uint16_t *>(w_in + (size_t)sl[1] * in_stride),
                                                     reinterpret_cast<const uint16_t *>(w_in + (size_t)sl[2] * in_stride),
                                                     reinterpret_cast<const uint16_t *>(w_in + (size_t)sl[3] * in_stride)};
                    dot4_f16(rows, xb, d, u);
                }
                for (int i = 0; i < 4; ++i) {
                    float hv = 0.f;
                    if (i < m) {
                        if (gated) {
                            hv = (g[i] > 0.f ? g[i] : 0.f) * u[i];
                        } else {
                            const float v = u[i] + (b_up ? half_to_float(b_up[sl[i]]) : 0.f);
                            hv = v > 0.f ? v : 0.f;
                            if (sq) hv *= hv;
                        }
                    }
                    h[b][i] = hv;
                    any |= hv != 0.f;
                }
            }
            if (!any) continue;                                  // adds exact zeros
            for (int b = 0; b < B; ++b) {
                float *yb = yc + (size_t)b * d;
                const float hb[4] = {h[b][0], h[b][1], h[b][2], h[b][3]};
                if (q4) {
                    const uint8_t *const rows[4] = {w_dn + (size_t)sl[0] * rb, w_dn + (size_t)sl[1] * rb,
                                                    w_dn + (size_t)sl[2] * rb, w_dn + (size_t)sl[3] * rb};
                    axpy4_q4(hb, rows, yb, d);
                } else {
                    const uint16_t *const rows[4] = {reinterpret_cast<const uint16_t *>(w_dn + (size_t)sl[0] * rb),
                                                     reinterpret_cast<const uint16_t *>(w_dn + (size_t)sl[1] * rb),
                                                     reinterpret_cast<const uint16_t *>(w_dn + (size_t)sl[2] * rb),
                                                     reinterpret_cast<const uint16_t *>(w_dn + (size_t)sl[3] * rb)};
                    axpy4_f16(hb, rows, yb, d);
                }
            }
        }
    }
    // chunk partials in chunk order
#pragma omp parallel for schedule(static) num_threads(nthr)
    for (size_t j = 0; j < bd; j += 8) {
        __m256 s = _mm256_loadu_ps(sc.part + j);
        for (int c = 1; c < kChunks; ++c) s = _mm256_add_ps(s, _mm256_loadu_ps(sc.part + (size_t)c * bd + j));
        _mm256_storeu_ps(y + j, s);
    }
    return PI_OK;
}

}  // extern "C"
