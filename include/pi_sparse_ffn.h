/*
 * pi_sparse_ffn.h -- C ABI of the predictor-gated, neuron-aware sparse FFN for MI355X (gfx950).
 *
 * The operation (PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU,
 * arXiv 2312.12456 -- abstract, and the "method" and "key results" sections of the summary
 * page): in a ReLU-family FFN only a small, input-dependent set of neurons fires for a token.
 * A small predictor decides which ones will fire; a neuron-aware sparse operator then reads
 * and computes only those neurons; a GPU placement index (the ".gpuidx" file of the project
 * README's model-weights section) names the neurons whose weights are resident on the device,
 * and the device computes only predicted neurons that are resident.  The README's FAQ lists
 * ReLU / ReGLU activations and its quantization section Q4_0 INT4 weights.
 *
 * For tokens x_b (b < batch), with d = d_model, f = d_ffn, r = rank:
 *   z_b  = max(0, P1 x_b)                       P1 [r][d]
 *   l_b  = P2 z_b + c                           P2 [f][r], c [f]
 *   M    = { i : l_b,i > 0 for some b }         strict threshold, union over the batch
 *   M'   = { i in M : slot_of[i] >= 0 }         (all of M when slot_of is NULL)
 *   idx  = members of M' in ascending order, n = |M'|
 *   h_bk = max(0, W_up[s] x_b + b_up[s])                 gated == 0
 *        = max(0, W_gate[s] x_b) * (W_up[s] x_b)         gated == 1      s = slot of idx[k]
 *   y_b  = b_down + sum_k h_bk W_down^T[s]
 *
 * Conventions for every entry point:
 *  - All pointers are DEVICE memory owned by the caller (e.g. torch tensors' data_ptr()),
 *    except the descriptor structs themselves, which are host memory read during the call.
 *    The library never allocates or frees; scratch comes from the caller's workspace `ws`
 *    of `ws_bytes` bytes, which must stay alive and unused by others until the enqueued
 *    work has finished.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default stream) and never
 *    synchronize.  Device-side counts stay on the device.  The enqueued kernels contain no
 *    memset nodes, so the calls may be captured into a HIP graph.
 *  - A nonzero return means nothing was enqueued (argument errors are detected on the host
 *    before any HIP call), except PI_ERR_HIP, which reports a launch failure.
 *  - fp16 is IEEE binary16.  y is fp32.  Accumulation is fp32.
 *  - Layout: weights are neuron-major -- row s of w_in holds the input weights of the neuron
 *    in slot s (gate row then up row when gated), row s of w_down_t holds its output
 *    weights -- so each active neuron is one contiguous read.
 *  - Q4_0 rows (32-weight blocks, one fp16 scale per block) of d weights are d/2 code bytes
 *    (byte j: weight 2j in the low nibble, weight 2j+1 in the high nibble; weight value
 *    scale*(code-8)) followed by d/32 fp16 scales: 9d/16 bytes per row.
 *  - Alignment: p1, p2, x, w_in, w_down_t must be 16-byte aligned.  Shapes: 1 <= batch <= 16,
 *    d_model % 8 == 0 (fp16) or d_model % 256 == 0 (Q4_0), d_model <= 2^24, rank % 8 == 0 and
 *    rank <= 2048, 1 <= d_ffn <= 2^26, 0 <= n_slots <= d_ffn.
 */
#ifndef PI_SPARSE_FFN_H
#define PI_SPARSE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PI_OK = 0,
    PI_ERR_NULL = -1,       /* a required pointer is NULL */
    PI_ERR_SHAPE = -2,      /* a size is out of range or inconsistent */
    PI_ERR_DTYPE = -3,      /* unsupported weight kind or kind/gating combination */
    PI_ERR_BATCH = -4,      /* batch outside [1, PI_MAX_BATCH] */
    PI_ERR_WORKSPACE = -5,  /* ws NULL or ws_bytes < pi_workspace_bytes(...) */
    PI_ERR_ALIGN = -6,      /* a pointer or row is not 16-byte aligned */
    PI_ERR_HIP = -7         /* a HIP launch failed */
} pi_status;

typedef enum { PI_F16 = 1, PI_Q4_0 = 2 } pi_wtype;
/* Activation of a non-gated layer (README FAQ: the supported activations are ReLU, ReGLU and
 * squared ReLU). */
typedef enum { PI_ACT_RELU = 0, PI_ACT_SQUARED_RELU = 1 } pi_act;

#define PI_MAX_BATCH 16
#define PI_MAX_WIDE_BATCH 16      /* pi_sparse_ffn_wide */
#define PI_MAX_RANK 2048
#define PI_MAX_D_MODEL (1 << 24)  /* kernels address one token vector or row with 32-bit offsets */
#define PI_MAX_D_FFN (1 << 26)    /* ... and the mask with 32-bit offsets */

/* Low-rank predictor of one layer (the "adaptive predictor" of the method section; its shape
 * -- a rank-r ReLU MLP with a per-neuron offset on the logits -- is this library's reading). */
typedef struct pi_predictor {
    int32_t d_model, d_ffn, rank;
    const void *p1;   /* [rank][d_model] fp16, row-major */
    const void *p2;   /* [d_ffn][rank]   fp16, row-major */
    const void *c;    /* [d_ffn]         fp16 per-neuron logit offset */
} pi_predictor;

/* Resident FFN weights of one layer. */
typedef struct pi_ffn {
    int32_t d_model, d_ffn;
    int32_t gated;             /* 0: ReLU(W_up x + b_up); 1: ReLU(W_gate x) * (W_up x) (ReGLU) */
    int32_t wtype;             /* pi_wtype */
    int32_t n_slots;           /* resident rows; must equal d_ffn when slot_of is NULL */
    const int32_t *slot_of;    /* [d_ffn] slot of neuron i, -1 = not resident; NULL = identity */
    const void *w_in;          /* [n_slots][gated ? 2 : 1][row] */
    const void *w_down_t;      /* [n_slots][row] */
    const void *b_up;          /* [n_slots] fp16, or NULL; must be NULL when gated */
    const void *b_down;        /* [d_model] fp16, or NULL */
    int32_t act;               /* pi_act: PI_ACT_SQUARED_RELU makes h = max(0, W_up x + b_up)^2;
                                  must be PI_ACT_RELU when gated.  A neuron is active iff h != 0. */
} pi_ffn;

/* Bytes of workspace the calls below need for this layer and batch (either descriptor may be
 * NULL when only the other one's calls are used).  0 on invalid arguments. */
size_t pi_workspace_bytes(const pi_predictor *pred, const pi_ffn *ffn, int32_t batch);

/* Predictor (method section: online prediction of the neurons that fire).
 * x [batch][d_model] fp16.  mask [d_ffn] u8 receives the batch union {0,1}.  logits
 * [batch][d_ffn] fp32 receives l_b when non-NULL.  Uses the workspace for z (and, past 8 tokens, for
 * the column-chunk sums of z that the MFMA form adds in order). */
int pi_predict(const pi_predictor *pred, const void *x, int32_t batch, uint8_t *mask,
               float *logits, void *ws, size_t ws_bytes, void *stream);

/* Placement restriction and compaction (README: GPU index of resident neurons).
 * mask [d_ffn] u8 (nonzero = predicted); slot_of [d_ffn] or NULL.  idx [d_ffn] receives the
 * ascending ids of predicted resident neurons (the first n entries are valid);
 * counts [2] receives {n, number predicted}.  Single kernel, no workspace. */
int pi_compact(const uint8_t *mask, int32_t d_ffn, const int32_t *slot_of, int32_t *idx,
               int32_t *counts, void *stream);

/* Neuron-aware sparse FFN over idx[0..counts[0]) (method section: sparse operators that
 * compute only the active neurons).  idx and counts are device memory (as pi_compact writes
 * them); n is clamped to [0, n_slots] and entries whose neuron or slot is out of range are
 * skipped.  y [batch][d_model] fp32 is overwritten.
 * At batch <= 2 (and d_model <= 32768 for fp16 rows, <= 65536 for Q4_0) this is three kernels over
 * (column slab x list chunk) workgroups: partial dot products of each slab, then h and the rows of
 * W_down^T, then the sum of the chunks' partial y in a fixed order.  Other batches run two kernels
 * (h, then the rows of W_down^T; from batch 3 for gated or Q4_0 rows and from batch 6 for other
 * fp16 rows, the MFMA kernels of pi_sparse_ffn_wide).  None of these kernels waits on another
 * workgroup; y is deterministic.  The workspace starts with a 512-byte control block whose int32 at
 * byte offset 384 is a sticky status word: the MFMA form hands h to its second kernel as an fp16
 * pair, so an |h| of 65504 or more cannot be carried -- it ORs 64 into the status word and that
 * call's y is invalid; the other forms have no such limit and leave the word untouched.  Zero-fill
 * the workspace once to read the status; the calls themselves need no zero fill.  A workspace must
 * not be shared by calls in flight at the same time. */
int pi_sparse_ffn(const pi_ffn *ffn, const void *x, int32_t batch, const int32_t *idx,
                  const int32_t *counts, float *y, void *ws, size_t ws_bytes, void *stream);

/* The same sparse FFN at batches of up to 16 tokens on MFMA (matrix-core) tiles, for prefill-like
 * batches where the per-token GEMV form would be bound by the vector ALU (the method's sparse
 * operator over the predicted neurons, method section, computed as [16 x n] and [16 x d]
 * products over the gathered rows with the batch padded to 16).  Arguments, idx/counts rules and
 * y as in pi_sparse_ffn, with 1 <= batch <= PI_MAX_WIDE_BATCH (PI_ERR_BATCH otherwise); fp16 and
 * Q4_0 rows (Q4_0 weights enter the MFMA as fp16 scale * (code - 8), rounded once to fp16).
 * Two kernels; the workspace of
 * pi_sparse_ffn_wide_workspace_bytes(ffn, batch) bytes (16-byte aligned) must not be shared by calls
 * in flight at the same time.  h passes between the kernels as an fp16 pair (h = hi + lo), so |h|
 * must stay below 65504: a larger one ORs 64 into the sticky status word that is the workspace's
 * first int32 (zero-fill the workspace once to read it; the calls need no zero fill otherwise) and
 * that call's y is invalid.  y is deterministic (fixed summation order).  The workspace-size call
 * returns 0 on invalid arguments. */
size_t pi_sparse_ffn_wide_workspace_bytes(const pi_ffn *ffn, int32_t batch);
int pi_sparse_ffn_wide(const pi_ffn *ffn, const void *x, int32_t batch, const int32_t *idx,
                       const int32_t *counts, float *y, void *ws, size_t ws_bytes, void *stream);

/* Whole layer (the decode step of one FFN layer as the method section describes it: the online
 * predictor picks the neurons that fire, the GPU index restricts them to the resident ones, and the
 * neuron-aware operator computes only those): the result of pi_predict -> pi_compact ->
 * pi_sparse_ffn, stream-ordered.  pred and ffn must agree on d_model and d_ffn.  mask_out [d_ffn],
 * idx_out [d_ffn] and counts_out [2] receive the intermediate results when non-NULL (otherwise they
 * live in the workspace; the list is only built when idx_out or counts_out is given -- the sparse
 * FFN itself reads the predictor's listed flags).
 * The workspace must be zero-filled before the first call that uses it; each call leaves it ready
 * for the next one (never clear or share it while a call is in flight; after a call that returned
 * an error, zero-fill it again).
 * For layers of at most 12288 neurons at batch <= 3 whose x and z fit one workgroup's LDS
 * (pi_layer_path == 1), everything after the first predictor matrix is ONE persistent kernel whose
 * workgroups hand the mask and h to each other through the workspace.  The int32 at byte offset
 * 384 of the workspace is a sticky status word: nonzero means a cross-workgroup wait ran out its
 * time limit (20 ms) and the outputs of that call are invalid.  Every wait inside the kernel is
 * bounded.  At the
 * batches where the sparse FFN runs on the MFMA form, an |h| of 65504 or more ORs 64 into the same
 * status word (see pi_sparse_ffn).
 * One workspace may serve several layers, one call at a time, when their pi_ffn descriptors agree
 * in d_model, d_ffn, n_slots, gated, wtype and act and the batch is the same: their predictors may
 * differ in rank (size it by the largest rank; what carries state between calls does not move with
 * the rank).  A layer of another FFN shape needs a workspace of its own, or a zero fill first. */
int pi_ffn_layer(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int32_t batch,
                 float *y, uint8_t *mask_out, int32_t *idx_out, int32_t *counts_out, void *ws,
                 size_t ws_bytes, void *stream);

/* The layer in two steps, split where pi_ffn_layer's first kernel ends (for callers that time or
 * schedule the steps separately).  pi_predict_hidden writes z = max(0, P1 x_b) as fp32
 * [batch][rank] to z (device, 16-byte aligned, caller-owned; no workspace).
 * pi_ffn_layer_from_hidden then runs the rest of the layer from that z: logits, mask, placement
 * restriction and the sparse FFN, with the arguments, workspace rules and results of pi_ffn_layer.
 * pi_ffn_layer(...) is exactly pi_predict_hidden followed by pi_ffn_layer_from_hidden. */
int pi_predict_hidden(const pi_predictor *pred, const void *x, int32_t batch, float *z, void *stream);
int pi_ffn_layer_from_hidden(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int32_t batch,
                             const float *z, float *y, uint8_t *mask_out, int32_t *idx_out, int32_t *counts_out,
                             void *ws, size_t ws_bytes, void *stream);

/* Which launches pi_ffn_layer_from_hidden makes for this layer and batch: 1 = one persistent kernel
 * (logits, mask and sparse FFN together; x, z and the kernel's arrays fit one workgroup's LDS and
 * d_ffn <= 12288, batch <= 3), 2 = separate kernels (at batch <= 2: logits, mask and up rows in
 * one kernel, then the down rows and the sum of their partials; otherwise logits and mask, then
 * the sparse FFN).  0 on invalid arguments. */
int pi_layer_path(const pi_predictor *pred, const pi_ffn *ffn, int32_t batch);

/* Diagnostics: where a pi_sparse_ffn call leaves h (list position k, token b) in its workspace,
 * for callers that count the rows of W_down^T that had to be read (h != 0 for some token).
 * Returns the byte offset of the table inside a pi_sparse_ffn workspace and sets *kind:
 *  1 = slab x chunk kernels (batch <= 2): fp32 h at offset + 4*(b*d_ffn + k);
 *  2 = two-kernel form: fp32 h at offset + 4*(b*max(n_slots, 1) + k);
 *  3 = MFMA form (the batches named above): h = hi + lo, in 16-byte units: unit u = (k/4)*16 + b at
 *      offset + 16*u holds the fp16 hi parts of positions 4(k/4) .. +3 of token b, then their fp16
 *      lo parts (hi at offset + 16*u + 2*(k%4), lo 8 bytes further); max(n_slots, 1) rounded up to 32
 *      positions (64 bytes each).
 * Positions k >= counts[0] hold stale values.  Returns (size_t)-1 on invalid arguments. */
size_t pi_sparse_ffn_h_offset(const pi_ffn *ffn, int32_t batch, int32_t *kind);

/* ---- host half of the hybrid split (method section and abstract: hot neurons are preloaded on
 * the GPU, cold ones are computed on the CPU, and the partial results are combined) ----
 *
 * pi_cold_ffn_host computes, on the host's cores, the neurons that are predicted (mask[i] != 0)
 * and held in host memory (ffn->slot_of[i] >= 0, or every neuron when slot_of is NULL), in
 * ascending id order:  y[b] = sum_i h[b][i] W_down^T[slot_i],  h as in pi_sparse_ffn.  No b_down:
 * the device half (pi_ffn_layer over the resident neurons) adds it, and the caller adds the two
 * y's.  Every pointer is HOST memory owned by the caller (ffn's rows and slot_of too, in the
 * layouts above; no alignment needed); x is [batch][d_model] fp16, mask [d_ffn] u8 (e.g. the
 * device's mask_out, copied back), y [batch][d_model] fp32 (overwritten).  *n_computed (if
 * non-NULL) receives the number of neurons computed.  ffn->b_down must be NULL (PI_ERR_DTYPE).
 * ws is a host workspace of pi_cold_workspace_bytes(ffn, batch) bytes (no zero fill needed).
 * n_threads = 0 uses the OpenMP default; the result does not depend on it (the neuron list is cut
 * into 64 fixed chunks, added in chunk order).  Synchronous; returns a pi_status, and nothing is
 * written on an error.  Needs an x86-64 host with AVX2, FMA and F16C. */
size_t pi_cold_workspace_bytes(const pi_ffn *ffn, int32_t batch);   /* 0 on invalid arguments */
int pi_cold_ffn_host(const pi_ffn *ffn, const void *x, int32_t batch, const uint8_t *mask, float *y,
                     int32_t *n_computed, void *ws, size_t ws_bytes, int32_t n_threads);

/* ---- offline placement (method section: an offline policy, an integer linear program over
 * activation frequency and hardware bandwidth, chooses the neurons preloaded on the GPU; README:
 * the result is the GPU index, sized by a VRAM budget) ----
 *
 * pi_place chooses, for n_layers layers of d_ffn[l] neurons of neuron_bytes[l] bytes each (all of
 * a neuron's rows in that layer's format) with firing frequencies freq (concatenated per layer,
 * each in [0, 1]), the neurons to keep on the device so that the expected time of a token,
 * sum_l max(device bytes_l / gpu_bytes_per_s, host bytes_l / host_bytes_per_s) with the bytes of
 * a neuron counted at its firing frequency, is smallest under sum_l neuron_bytes[l] * placed_l <=
 * budget_bytes.  Output: slot_of (concatenated per layer, [d_ffn[l]] each: the neuron's slot, in
 * ascending id order among the placed ones, or -1) -- the layer's pi_ffn.slot_of -- n_placed
 * [n_layers], and *expected_s (if non-NULL) the model's expected seconds per token.  Greedy by
 * marginal gain per byte over the most frequent remaining neuron of each layer.  Among placements
 * that keep each layer's most frequent neurons it is exact when all neurons have the same size
 * (within one neuron's time otherwise); those include the optimum while the host side of every
 * layer dominates, and are within one neuron's time per layer of it in general.  Host memory,
 * synchronous; returns a pi_status. */
int pi_place(int32_t n_layers, const int32_t *d_ffn, const int64_t *neuron_bytes, const float *freq,
             int64_t budget_bytes, double gpu_bytes_per_s, double host_bytes_per_s, int32_t *slot_of,
             int32_t *n_placed, double *expected_s);

/* ---- adaptive predictor size (methodology and core innovations: adaptive predictors per layer,
 * kept small in GPU memory) ----
 *
 * pi_predictor_ranks chooses the rank of each of n_layers layers' predictors (d_model[l],
 * d_ffn[l]; freq: the firing frequencies, concatenated per layer, each in [0, 1]) under a budget
 * for all predictor matrices, sum_l 2 rank[l] (d_model[l] + d_ffn[l]) <= budget_bytes (P1 and P2
 * in fp16).  A layer's share follows the entropy of its firing pattern, H_l = sum_i h(p_i) bits
 * (h the binary entropy, H_l rounded to 1/1024 bit): rank[l] is the largest of r_min, r_min +
 * r_step, ..., r_max not above max(r_min, lambda H_l), for the largest lambda the budget allows;
 * at equal lambda the lower layer is raised first, and raising stops at the first raise that
 * does not fit.  Sparser and more skewed layers (lower H) get smaller predictors; a layer with
 * H = 0 keeps r_min.  r_min, r_step: multiples of 8, r_min >= 8, r_max <= PI_MAX_RANK, r_max -
 * r_min a multiple of r_step.  Outputs rank [n_layers] and, if non-NULL, entropy_bits [n_layers]
 * (the rounded H_l).  PI_ERR_SHAPE if the budget cannot hold r_min in every layer or an argument
 * is out of range (nothing written).  Host memory, synchronous; returns a pi_status. */
int pi_predictor_ranks(int32_t n_layers, const int32_t *d_model, const int32_t *d_ffn, const float *freq,
                       int64_t budget_bytes, int32_t r_min, int32_t r_max, int32_t r_step, int32_t *rank,
                       double *entropy_bits);

/* ---- the same sparse FFN without a caller workspace ----
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  pi_sparse_ffn_noalloc is pi_sparse_ffn (same arguments, kernels
 * and results, bit for bit) with its scratch in a device array that the library holds, one copy per
 * GPU, from the first call on that GPU until the process ends; it calls no hipMalloc, hipFree or
 * allocating routine.  The layer and batch must need at most PI_NOALLOC_SCRATCH_BYTES of scratch
 * (pi_workspace_bytes(NULL, ffn, batch) <= PI_NOALLOC_SCRATCH_BYTES), else PI_ERR_WORKSPACE and
 * nothing is enqueued; PI_ERR_HIP if the array's address cannot be obtained.  Every call on one GPU
 * uses the same array, so calls that overlap in time on one GPU (two streams, or two host threads
 * without ordering) race and must not be made; calls ordered on one stream are fine.  The array
 * needs no clearing: each call writes every scratch value before reading it. */
#define PI_NOALLOC_SCRATCH_BYTES (32u << 20)
int pi_sparse_ffn_noalloc(const pi_ffn *ffn, const void *x, int32_t batch, const int32_t *idx,
                          const int32_t *counts, float *y, void *stream);

/* Human-readable name of a pi_status value (static storage). */
const char *pi_status_string(int status);

/* ABI version of this header (major*100 + minor). */
int pi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PI_SPARSE_FFN_H */
