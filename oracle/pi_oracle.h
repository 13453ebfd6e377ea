/*
 * pi_oracle.h -- CPU oracle of the predictor-gated sparse FFN (TEST INFRASTRUCTURE ONLY).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may use this.
 * It shares nothing with the HIP library.  All pointers are host memory owned by the
 * caller; fp16 values are passed as their uint16 bit patterns.  Functions return 0 on
 * success, -1 for a null pointer or a non-positive size, -2 for an out-of-range index or
 * an allocation failure, -3 for an unsupported weight kind.
 */
#ifndef PI_ORACLE_H
#define PI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { PIO_F16 = 1, PIO_Q4_0 = 2 };
/* FFN kinds (the `gated` argument below): ReLU(W_up x + b_up), ReGLU ReLU(W_gate x) (W_up x), and
 * squared ReLU ReLU(W_up x + b_up)^2 (README FAQ: the activations the method supports). */
enum { PIO_RELU = 0, PIO_REGLU = 1, PIO_SQUARED_RELU = 2 };

/* IEEE 754 binary16 bit pattern -> double (exact). */
double pio_half(uint16_t h);

/* Bytes of one stored row of d weights (fp16: 2d; Q4_0: d/2 code bytes + d/32 fp16 scales). */
int64_t pio_row_bytes(int wtype, int64_t d);

/* Widen one stored row to d doubles. */
void pio_decode_row(const void *row, int wtype, int64_t d, double *w);

/* Predictor: logits [B][f] (nullable), per-token masks [B][f] (nullable), union mask [f]. */
int pio_predict(int64_t d, int64_t f, int64_t r, const uint16_t *p1, const uint16_t *p2,
                const uint16_t *c, const uint16_t *x, int64_t B, double *logits,
                uint8_t *mask_tok, uint8_t *mask);

/* Ascending active ids of mask restricted to slot_of >= 0 (slot_of NULL: all resident).
 * counts[0] = number listed, counts[1] = number predicted (mask popcount). */
int pio_compact(const uint8_t *mask, int64_t f, const int32_t *slot_of, int32_t *idx,
                int32_t *counts);

/* Sparse FFN over neuron ids idx[0..n).  gated: the FFN kind (PIO_RELU, PIO_REGLU or
 * PIO_SQUARED_RELU).  Weight rows are neuron-major and indexed by slot (slot_of[i], or i when
 * slot_of is NULL): w_in row = gate row then up row for ReGLU.
 * h_out [B][n] (nullable) receives the activations; y [B][d] receives the output. */
int pio_sparse_ffn(int64_t d, int64_t f, int gated, int wtype, int64_t n_slots,
                   const int32_t *slot_of, const void *w_in, const void *w_down_t,
                   const uint16_t *b_up, const uint16_t *b_down, const uint16_t *x, int64_t B,
                   const int32_t *idx, int64_t n, double *h_out, double *y);

/* Dense FFN over all f neurons; true_mask [B][f] (nullable) = [h != 0]. */
int pio_dense_ffn(int64_t d, int64_t f, int gated, int wtype, const void *w_in,
                  const void *w_down_t, const uint16_t *b_up, const uint16_t *b_down,
                  const uint16_t *x, int64_t B, uint8_t *true_mask, double *y);

/* predict -> compact -> sparse FFN. */
int pio_ffn_layer(int64_t d, int64_t f, int64_t r, const uint16_t *p1, const uint16_t *p2,
                  const uint16_t *c, int gated, int wtype, int64_t n_slots, const int32_t *slot_of,
                  const void *w_in, const void *w_down_t, const uint16_t *b_up,
                  const uint16_t *b_down, const uint16_t *x, int64_t B, double *logits,
                  uint8_t *mask, int32_t *idx, int32_t *counts, double *y);

int pio_num_threads(void);
void pio_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
