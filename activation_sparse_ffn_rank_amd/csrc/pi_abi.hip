// pi_abi.hip -- host side of the C ABI declared in include/pi_sparse_ffn.h.
//
// Every entry point validates its arguments on the host before touching HIP, then enqueues
// stream-ordered kernel launches on the caller's stream.  Nothing here allocates, frees,
// synchronizes or issues memset/memcpy nodes, so the calls are safe inside HIP graph capture.
// No C++ exception crosses the ABI.
#include "pi_sparse_ffn.h"
#include "pi_kernels.hpp"
#include "pi_split.hpp"
#include "pi_tail.hpp"
#include "pi_wide.hpp"
#include "pi_occupancy.hpp"

#include <algorithm>
#include <mutex>

// Scratch of pi_sparse_ffn_noalloc: a file-scope device array, one copy per GPU, held until the
// process ends.  Host code never uses this name as an address (on the host it is a stand-in for the
// device symbol); it asks for each device's address with hipGetSymbolAddress and passes that.
static __device__ __align__(256) uint8_t scratch[PI_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace pik;

constexpr size_t kAlign = 256;
constexpr int kLdsXBytes = 64 * 1024;   // per-workgroup LDS budget for staged token vectors
constexpr int kUpMaxGroups = 512;       // workgroups of k_sparse_up
constexpr int kDownTargetTiles = 768;   // (slab, chunk) tiles of k_sparse_down

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

int check_batch(int32_t B) { return (B >= 1 && B <= PI_MAX_BATCH) ? PI_OK : PI_ERR_BATCH; }
// The GEMV kernels (first predictor matrix, tail kernel, GEMV sparse FFN) are instantiated for up to
// 8 tokens; past that the first predictor matrix runs in two passes and the rest on MFMA.
constexpr int kGemvMaxBatch = 8;
// From this batch on the second predictor matrix runs on MFMA (k_pred_l2_mfma_s, or k_pred_l2_mfma
// past rank 1024): the GEMV form's vector-ALU work per weight grows with the batch (measured
// crossovers on MI355X, rank 1024: batch 3 at 28672 and 49152 neurons, batch 6 at 11008).
inline int pred_mfma_from(int d_ffn) { return d_ffn >= 16384 ? 3 : 6; }

int check_pred(const pi_predictor *p) {
    if (!p) return PI_ERR_NULL;
    if (!p->p1 || !p->p2 || !p->c) return PI_ERR_NULL;
    if (p->d_model < 8 || p->d_model % 8 != 0 || p->d_model > PI_MAX_D_MODEL || p->d_ffn < 1 ||
        p->d_ffn > PI_MAX_D_FFN || p->rank < 8 ||
        p->rank % 8 != 0 || p->rank > PI_MAX_RANK)
        return PI_ERR_SHAPE;
    if (!aligned16(p->p1) || !aligned16(p->p2)) return PI_ERR_ALIGN;
    return PI_OK;
}

int64_t row_bytes_of(const pi_ffn *f) {
    return f->wtype == PI_F16 ? 2 * (int64_t)f->d_model : (int64_t)f->d_model * 9 / 16;
}

int check_ffn(const pi_ffn *f) {
    if (!f) return PI_ERR_NULL;
    if (!f->w_in || !f->w_down_t) return PI_ERR_NULL;
    if (f->wtype != PI_F16 && f->wtype != PI_Q4_0) return PI_ERR_DTYPE;
    if (f->gated != 0 && f->gated != 1) return PI_ERR_DTYPE;
    if (f->gated && f->wtype == PI_Q4_0) return PI_ERR_DTYPE;      // not a configuration of this library
    if (f->gated && f->b_up) return PI_ERR_DTYPE;                  // the gated form has no up bias
    if (f->act != PI_ACT_RELU && f->act != PI_ACT_SQUARED_RELU) return PI_ERR_DTYPE;
    if (f->gated && f->act != PI_ACT_RELU) return PI_ERR_DTYPE;     // ReGLU has its own form
    if (f->d_ffn < 1 || f->d_ffn > PI_MAX_D_FFN || f->n_slots < 0 || f->n_slots > f->d_ffn) return PI_ERR_SHAPE;
    if (!f->slot_of && f->n_slots != f->d_ffn) return PI_ERR_SHAPE;
    if (f->d_model > PI_MAX_D_MODEL) return PI_ERR_SHAPE;
    if (f->wtype == PI_F16 && (f->d_model < 8 || f->d_model % 8 != 0)) return PI_ERR_SHAPE;
    if (f->wtype == PI_Q4_0 && (f->d_model < 256 || f->d_model % 256 != 0)) return PI_ERR_SHAPE;
    if (!aligned16(f->w_in) || !aligned16(f->w_down_t)) return PI_ERR_ALIGN;
    return PI_OK;
}

// Column chunk of staged token vectors: all of d when B*d fp16 fit the LDS budget.
int x_chunk(int d, int B) {
    const int fit = kLdsXBytes / (2 * B);
    if (d <= fit) return d;
    return std::max(512, fit / 512 * 512);
}

int down_slabs(int d) { return ceil_div(d, 512); }

// Workspace of pi_sparse_ffn_wide: a status word (its first int32; 256 bytes reserved), slab
// tickets, h as fp16 hi and lo parts (the interleaved table of wide_h_store, 64*hs bytes over the
// hi and lo regions), the chunk partials [C][B][d] fp32, and x in the up step's operand order.
constexpr int kWideTargetGroups = 256;   // (slab, chunk) workgroups of k_wide_down (8 waves each)
constexpr size_t kWideStatusBytes = 256;
struct WideGeom {
    int S, C, hs;
    size_t tick, hi, lo, part, xmf, total;
};
WideGeom wide_geom(const pi_ffn *fn, int B) {
    WideGeom g{};
    const int d = fn->d_model;
    g.S = ceil_div(d, 16 * wide_down_cpl(fn->wtype == PI_Q4_0 ? WT_Q4_0 : WT_F16));
    g.C = std::min(kWideMaxChunks, std::max(1, ceil_div(kWideTargetGroups, g.S)));
    // room for the chunk partials of up to 8 chunks on Q4_0 rows (the launch itself takes as many
    // chunks as fit one workgroup per compute unit, 5 at d = 12288)
    if (fn->wtype == PI_Q4_0) g.C = std::min(kWideMaxChunks, (g.C + 7) / 8 * 8);
    g.hs = ceil_div(std::max(fn->n_slots, 1), 32) * 32;    // k_wide_up writes whole 32-position groups
    g.tick = kWideStatusBytes;
    g.hi = g.tick + align_up((size_t)g.S * 4);
    g.lo = g.hi + align_up((size_t)kWideB * g.hs * 2);
    g.part = g.lo + align_up((size_t)kWideB * g.hs * 2);
    g.xmf = g.part + align_up((size_t)g.C * B * d * 4);
    g.total = g.xmf + align_up((size_t)wide_xmf_vectors(d, fn->wtype == PI_Q4_0) * 16);
    return g;
}
int check_wide_batch(int32_t B) { return (B >= 1 && B <= PI_MAX_WIDE_BATCH) ? PI_OK : PI_ERR_BATCH; }

int down_chunks(int d) {
    return std::min(kDownMaxChunks, std::max(1, ceil_div(kDownTargetTiles, down_slabs(d))));
}

// The first predictor matrix on MFMA (k_pred_l1_mfma, split over d into KS column chunks of cw, then
// k_zsum) past the GEMV kernels' 8 tokens, where the caller gives a workspace for the chunk sums
// (pi_predict, the layer entry points; pi_predict_hidden has none and runs the GEMV form in two
// passes).  Measured on MI355X, pi_predict at 16 tokens: 54.7 -> 48.3 us (49152 neurons), 24.7 ->
// 21.7 (11008); at 8 tokens the single GEMV pass is as fast.
constexpr int pred_l1_mfma_from() { return kGemvMaxBatch + 1; }
struct L1Geom {
    int KS, cw;
};
L1Geom l1_geom(const pi_predictor *p) {
    const int groups = ceil_div(p->rank, 64);
    int KS = std::min(64, std::max(1, ceil_div(512, groups)));
    const int cw = ceil_div(ceil_div(p->d_model, KS), 32) * 32;
    KS = ceil_div(p->d_model, cw);
    return L1Geom{KS, cw};
}
// z [B][r] fp32, then (batches on MFMA) the chunk sums [KS][B][r]
size_t pred_ws(const pi_predictor *p, int B) {
    size_t n = align_up((size_t)B * p->rank * sizeof(float));
    if (B >= pred_l1_mfma_from()) n += align_up((size_t)l1_geom(p).KS * B * p->rank * sizeof(float));
    return n;
}
float *pred_zpart(const pi_predictor *p, int B, float *z) {
    return B >= pred_l1_mfma_from() ? z + align_up((size_t)B * p->rank * sizeof(float)) / sizeof(float) : nullptr;
}

// Sparse-FFN scratch: h [B][max(n_slots,1)] fp32, chunk partials [C][B][d] fp32, slab tickets.
struct FfnScratch {
    float *h;
    float *part;
    int32_t *tickets;
};

size_t ffn_h_bytes(const pi_ffn *f, int B) { return align_up((size_t)B * std::max(f->n_slots, 1) * sizeof(float)); }
size_t ffn_part_bytes(const pi_ffn *f, int B) {
    return align_up((size_t)down_chunks(f->d_model) * B * f->d_model * sizeof(float));
}
size_t ffn_legacy_ws(const pi_ffn *f, int B) {
    return ffn_h_bytes(f, B) + ffn_part_bytes(f, B) + align_up((size_t)down_slabs(f->d_model) * sizeof(int32_t));
}

// The control block shared by every persistent launch on a workspace (pi_sync.hpp): epoch, exit
// count, abort flag, status word (byte offset 384).
size_t ctl_bytes(int) { return align_up((size_t)CTL_WORDS * sizeof(int32_t)); }

// Scratch of the (column slab x list chunk) kernels of pi_split.hpp, batch <= 2: partial dot
// products [positions][S][B*G] fp32, chunk partials of y [kSplitMaxChunks][B][d] fp32 (the chunk
// count is chosen at launch), and h per position [B][d_ffn] fp32 (diagnostics).
struct SplitGeom {
    int S;
    size_t part, ypart, hout;
};
SplitGeom split_geom(const pi_ffn *fn, int B) {
    SplitGeom g;
    const int wt = fn->wtype == PI_Q4_0 ? WT_Q4_0 : WT_F16;
    g.S = split_slabs(fn->d_model, wt);
    g.part = align_up((size_t)fn->d_ffn * g.S * B * (fn->gated ? 2 : 1) * sizeof(float));
    g.ypart = align_up((size_t)kSplitMaxChunks * B * fn->d_model * sizeof(float));
    g.hout = align_up((size_t)B * fn->d_ffn * sizeof(float));
    return g;
}
// Batches 1 and 2 run the split kernels whenever the slab count allows (d_model up to 32768 for fp16
// rows, 65536 for Q4_0); they need no copy of x in LDS.
bool sparse_split(const pi_ffn *fn, int B) {
    return B <= 2 && split_slabs(fn->d_model, fn->wtype == PI_Q4_0 ? WT_Q4_0 : WT_F16) <= kSplitMaxSlabs;
}
int mask_words(int f) { return ceil_div(f, 32); }
// In a layer, the split kernels read the predictor's listed-flag words directly (no compaction).
bool layer_split(const pi_ffn *fn, int B) { return sparse_split(fn, B) && mask_words(fn->d_ffn) <= kSplitMaxWords; }
// ... and when x and z fit one workgroup's LDS and the matrices stay below the 32-bit offsets of its
// buffer loads, the second predictor matrix and the up rows run as one kernel (k_pred_up).
bool layer_pred_up(const pi_predictor *p, const pi_ffn *fn, int B) {
    const int64_t in_bytes = (int64_t)fn->n_slots * row_bytes_of(fn) * (fn->gated ? 2 : 1);
    const int64_t p2_bytes = (int64_t)p->d_ffn * p->rank * 2;
    return layer_split(fn, B) && in_bytes < (int64_t)kBufMax && p2_bytes < (int64_t)kBufMax &&
           pred_up_lds(B, fn->d_model, p->rank) <= (size_t)kLdsXBytes + 16 * 1024;
}

// The tail kernel (second predictor matrix + mask + sparse FFN) keeps x [B][d] fp16 and z [B][r]
// fp32 in dynamic LDS next to its static arrays (wave partials of the down tiles, the list of a
// down tile's neurons, a few words); all of it must fit one workgroup.  It is used while every
// 32-neuron tile can have an up workgroup of its own (d_ffn <= 32 * kTailMaxTiles).  Larger layers
// at batch <= 2 run k_pred_up and the split kernels instead (measured on MI355X: 9% faster than
// this kernel at 28672 neurons, 14% at 32768; at 11008 this kernel is 11% faster).  Past 3 tokens
// the separate predictor, compaction and sparse-FFN kernels win (11008 neurons: 81.9 -> 50.1 us
// per layer at 4 tokens, 118.2 -> 55.0 at 6; at 3 the tail kernel still leads, 42.3 vs 46.7).
constexpr int kTailMaxBatch = 3;
bool tail_persistent(const pi_predictor *p, const pi_ffn *fn, int B) {
    if (B > kTailMaxBatch) return false;
    const size_t stat = (size_t)4 * B * kTailCPL * 64 * 4 + (size_t)B * kTailSlab * 4 + (size_t)kTailListMax * 4 + 512;
    // the kernel reads through 32-bit buffer offsets: every matrix (and the partials) must stay
    // below kBufMax bytes
    const int64_t in_bytes = (int64_t)fn->n_slots * row_bytes_of(fn) * (fn->gated ? 2 : 1);
    const int64_t p2_bytes = (int64_t)p->d_ffn * p->rank * 2;
    const int64_t part_bytes = (int64_t)kSparseMaxChunks * B * fn->d_model * 8;
    if (in_bytes >= (int64_t)kBufMax || p2_bytes >= (int64_t)kBufMax || part_bytes >= (int64_t)kBufMax) return false;
    const int tiles = ceil_div(fn->d_ffn, 32);
    if (tiles > kTailMaxTiles) return false;
    return (size_t)B * fn->d_model * 2 <= (size_t)kLdsXBytes &&
           tail_dyn_lds(B, fn->d_model, p->rank) + stat <= 160 * 1024;
}

// Scratch of the tail kernel (after the shared control block): a stamped word per 32-neuron tile,
// (1 + B) stamped words per neuron (slot, h per token), stamped chunk partials.
struct TailGeom {
    int slabs, NTL;
    size_t tword, ent, part;
};

TailGeom tail_geom(const pi_ffn *fn, int B) {
    TailGeom g;
    g.slabs = ceil_div(fn->d_model, kTailSlab);
    g.NTL = ceil_div(fn->d_ffn, 32);
    g.tword = align_up((size_t)g.NTL * sizeof(uint64_t));
    g.ent = align_up((size_t)fn->d_ffn * (1 + B) * sizeof(uint64_t));
    g.part = align_up((size_t)kSparseMaxChunks * B * fn->d_model * sizeof(uint64_t));
    return g;
}

size_t tail_ws(const pi_ffn *fn, int B) {
    const TailGeom g = tail_geom(fn, B);
    return g.tword + g.ent + g.part;
}

// From these batches on the sparse FFN runs on MFMA tiles (k_wide_up / k_wide_down), where the
// GEMV kernels become bound by the vector ALU: batch 3 for gated (two dot products per neuron) and
// Q4_0 rows (decode work per weight), batch 6 for plain fp16 rows (measured crossovers).
int wide_from_batch(const pi_ffn *f) { return (f->gated || f->wtype == PI_Q4_0) ? 3 : 6; }
bool sparse_wide(const pi_ffn *f, int B) { return B >= wide_from_batch(f) && !sparse_split(f, B); }

// Scratch of pi_sparse_ffn: a control block first on every path, so that the status word sits at
// a fixed offset (the kernels that never wait leave it as they found it), then the split kernel's
// regions, the MFMA form's, or the GEMV two-kernel form's.
size_t ffn_ws(const pi_ffn *f, int B) {
    if (sparse_split(f, B)) {
        const SplitGeom g = split_geom(f, B);
        return ctl_bytes(f->d_model) + g.part + g.ypart + g.hout;
    }
    if (sparse_wide(f, B)) return ctl_bytes(f->d_model) + wide_geom(f, B).total;
    return ctl_bytes(f->d_model) + ffn_legacy_ws(f, B);
}

FfnScratch ffn_scratch(const pi_ffn *f, int B, void *base) {
    char *p = static_cast<char *>(base);
    FfnScratch s;
    s.h = reinterpret_cast<float *>(p);
    s.part = reinterpret_cast<float *>(p + ffn_h_bytes(f, B));
    s.tickets = reinterpret_cast<int32_t *>(p + ffn_h_bytes(f, B) + ffn_part_bytes(f, B));
    return s;
}


int launch_status() { return hipGetLastError() == hipSuccess ? PI_OK : PI_ERR_HIP; }

// ------------------------------------------------------------------ enqueue helpers

// bits (optional, with slot_of/n_slots): the placement-restricted listed flags, one word per 32 rows.
template <int B>
int enqueue_pred_l2_b(const pi_predictor *p, const float *z, uint8_t *mask, float *logits, uint32_t *bits,
                      const int32_t *slot_of, int n_slots, hipStream_t st) {
    const int r = p->rank, f = p->d_ffn;
    constexpr int R = 8;                               // predictor rows per wave
    const int groups = ceil_div(f, 4 * R);
    const uint16_t *p2 = static_cast<const uint16_t *>(p->p2), *c = static_cast<const uint16_t *>(p->c);
    const size_t zb = (size_t)B * r * sizeof(float);       // z staged in LDS (<= 64 KB)
    if (r <= 512)
        hipLaunchKernelGGL((k_pred_l2<B, 1, R>), dim3(groups), dim3(256), zb, st, p2, c, z, r, f, logits, mask, bits,
                           slot_of, n_slots);
    else if (r <= 1024)
        hipLaunchKernelGGL((k_pred_l2<B, 2, R>), dim3(groups), dim3(256), zb, st, p2, c, z, r, f, logits, mask, bits,
                           slot_of, n_slots);
    else
        hipLaunchKernelGGL((k_pred_l2<B, 4, R>), dim3(groups), dim3(256), zb, st, p2, c, z, r, f, logits, mask, bits,
                           slot_of, n_slots);
    return launch_status();
}

// Whether enqueue_pred_l2 runs k_pred_l2_mfma_s (which can also lay out x for the Q4_0 up step).
bool pred_l2_staged(const pi_predictor *p, int B) {
    return B >= pred_mfma_from(p->d_ffn) && p->rank <= kPredL2StagedMaxRank;
}

// x, d, xmf: with pred_l2_staged, also write x [B][d] in the Q4_0 up step's operand order to xmf.
int enqueue_pred_l2(const pi_predictor *p, const float *z, int B, uint8_t *mask, float *logits, hipStream_t st,
                    uint32_t *bits = nullptr, const int32_t *slot_of = nullptr, int n_slots = 0,
                    const void *x = nullptr, uint4 *xmf = nullptr, bool xq4 = true) {
    if (B >= pred_mfma_from(p->d_ffn)) {
        const int r = p->rank, f = p->d_ffn;
        const uint16_t *p2 = static_cast<const uint16_t *>(p->p2), *c = static_cast<const uint16_t *>(p->c);
        const dim3 grid(ceil_div(f, 64));
        if (r <= kPredL2StagedMaxRank)
            hipLaunchKernelGGL(k_pred_l2_mfma_s<8>, dim3(ceil_div(f, 16 * kPredL2Waves)), dim3(kPredL2Waves * kWave),
                               (size_t)ceil_div(r, 32) * 2 * kWave * 16, st, p2, c, z, B, r, f, logits, mask, bits,
                               slot_of, n_slots, static_cast<const uint16_t *>(x), p->d_model, xq4 ? 1 : 0, xmf);
        else if (r >= 256)
            hipLaunchKernelGGL(k_pred_l2_mfma<8>, grid, dim3(256), 0, st, p2, c, z, B, r, f, logits, mask, bits, slot_of,
                               n_slots);
        else
            hipLaunchKernelGGL(k_pred_l2_mfma<4>, grid, dim3(256), 0, st, p2, c, z, B, r, f, logits, mask, bits, slot_of,
                               n_slots);
        return launch_status();
    }
    switch (B) {
        case 1: return enqueue_pred_l2_b<1>(p, z, mask, logits, bits, slot_of, n_slots, st);
        case 2: return enqueue_pred_l2_b<2>(p, z, mask, logits, bits, slot_of, n_slots, st);
        case 3: return enqueue_pred_l2_b<3>(p, z, mask, logits, bits, slot_of, n_slots, st);
        case 4: return enqueue_pred_l2_b<4>(p, z, mask, logits, bits, slot_of, n_slots, st);
        case 5: return enqueue_pred_l2_b<5>(p, z, mask, logits, bits, slot_of, n_slots, st);
        case 6: return enqueue_pred_l2_b<6>(p, z, mask, logits, bits, slot_of, n_slots, st);
        case 7: return enqueue_pred_l2_b<7>(p, z, mask, logits, bits, slot_of, n_slots, st);
        case 8: return enqueue_pred_l2_b<8>(p, z, mask, logits, bits, slot_of, n_slots, st);
    }
    return PI_ERR_BATCH;
}

template <int B, int U>
void enqueue_pred_l1_bu(const pi_predictor *p, const uint16_t *x, float *z, hipStream_t st) {
    constexpr int RW = pred_l1_rows(B);
    hipLaunchKernelGGL((k_pred_l1<B, RW, U>), dim3(ceil_div(p->rank, RW)), dim3(256), 0, st,
                       static_cast<const uint16_t *>(p->p1), x, z, p->d_model, p->rank);
}

// One pass of k_pred_l1 covers U*2048 columns: as many as d needs (loads past d touch no memory
// but take issue slots), at most 8/RW loads per thread per row.
template <int B>
void enqueue_pred_l1_b(const pi_predictor *p, const uint16_t *x, float *z, hipStream_t st) {
    constexpr int UMAX = 8 / pred_l1_rows(B);
    const int need = ceil_div(p->d_model, 2048);
    if (need <= 1 || UMAX == 1) enqueue_pred_l1_bu<B, 1>(p, x, z, st);
    else if (need <= 2 || UMAX == 2) enqueue_pred_l1_bu<B, 2>(p, x, z, st);
    else if (need <= 4 || UMAX == 4) enqueue_pred_l1_bu<B, (UMAX >= 4 ? 4 : 2)>(p, x, z, st);
    else enqueue_pred_l1_bu<B, UMAX>(p, x, z, st);
}

int enqueue_pred_l1(const pi_predictor *p, const void *x, int B, float *z, hipStream_t st, float *zpart = nullptr) {
    const uint16_t *xx = static_cast<const uint16_t *>(x);
    if (zpart != nullptr && B >= pred_l1_mfma_from()) {
        const L1Geom g = l1_geom(p);
        hipLaunchKernelGGL(k_pred_l1_mfma<4>, dim3(ceil_div(p->rank, 64), g.KS), dim3(256), 0, st,
                           static_cast<const uint16_t *>(p->p1), xx, B, p->d_model, p->rank, g.cw, zpart);
        if (hipGetLastError() != hipSuccess) return PI_ERR_HIP;
        hipLaunchKernelGGL(k_zsum, dim3(ceil_div(B * p->rank, 256)), dim3(256), 0, st, zpart, g.KS, B * p->rank, z);
        return launch_status();
    }
    if (B > kGemvMaxBatch) {
        // tokens 0..7, then the rest: P1 is read twice, x and z rows are offset
        int rc = enqueue_pred_l1(p, x, kGemvMaxBatch, z, st);
        if (rc) return rc;
        return enqueue_pred_l1(p, xx + (size_t)kGemvMaxBatch * p->d_model, B - kGemvMaxBatch,
                               z + (size_t)kGemvMaxBatch * p->rank, st);
    }
    switch (B) {
        case 1: enqueue_pred_l1_b<1>(p, xx, z, st); break;
        case 2: enqueue_pred_l1_b<2>(p, xx, z, st); break;
        case 3: enqueue_pred_l1_b<3>(p, xx, z, st); break;
        case 4: enqueue_pred_l1_b<4>(p, xx, z, st); break;
        case 5: enqueue_pred_l1_b<5>(p, xx, z, st); break;
        case 6: enqueue_pred_l1_b<6>(p, xx, z, st); break;
        case 7: enqueue_pred_l1_b<7>(p, xx, z, st); break;
        case 8: enqueue_pred_l1_b<8>(p, xx, z, st); break;
        default: return PI_ERR_BATCH;
    }
    return launch_status();
}

int enqueue_predict(const pi_predictor *p, const void *x, int B, uint8_t *mask, float *logits, float *z,
                    hipStream_t st) {
    int rc = enqueue_pred_l1(p, x, B, z, st, pred_zpart(p, B, z));
    return rc ? rc : enqueue_pred_l2(p, z, B, mask, logits, st);
}

// The tail kernel: z (from k_pred_l1) -> mask -> sparse FFN -> y; ctl is the shared control block,
// data the tail scratch (tail_ws bytes); mask (optional) receives the fired flags.
int enqueue_tail(const pi_predictor *p, const pi_ffn *fn, const void *x, int B, const float *z, float *y,
                 uint8_t *mask, int32_t *ctl, char *data, hipStream_t st, uint64_t *trace = nullptr) {
    const TailGeom g = tail_geom(fn, B);
    TailArgs a{};
    a.d = fn->d_model; a.f = fn->d_ffn; a.r = p->rank; a.n_slots = fn->n_slots; a.slabs = g.slabs; a.NTL = g.NTL;
    a.row_bytes = row_bytes_of(fn);
    a.act = fn->act;
    a.p2 = static_cast<const uint16_t *>(p->p2); a.c = static_cast<const uint16_t *>(p->c); a.z = z;
    a.w_in = static_cast<const uint8_t *>(fn->w_in); a.w_dn = static_cast<const uint8_t *>(fn->w_down_t);
    a.b_up = static_cast<const uint16_t *>(fn->b_up); a.b_down = static_cast<const uint16_t *>(fn->b_down);
    a.slot_of = fn->slot_of;
    a.x = static_cast<const uint16_t *>(x); a.y = y; a.mask = mask;
    a.ctl = ctl;
    a.tword = reinterpret_cast<uint64_t *>(data); data += g.tword;
    a.ent = reinterpret_cast<uint64_t *>(data); data += g.ent;
    a.part = reinterpret_cast<uint64_t *>(data);
#ifdef PIK_TRACE
    a.trace = trace;
#else
    (void)trace;
#endif
    const int wt = fn->wtype == PI_Q4_0 ? WT_Q4_0 : WT_F16;
    const int NT = p->rank <= 512 ? 1 : (p->rank <= 1024 ? 2 : 4);
    int rc;
    switch (B) {
        case 1: rc = launch_tail_batch<1>(a, wt, fn->gated, NT, st); break;
        case 2: rc = launch_tail_batch<2>(a, wt, fn->gated, NT, st); break;
        case 3: rc = launch_tail_batch<3>(a, wt, fn->gated, NT, st); break;
        case 4: rc = launch_tail_batch<4>(a, wt, fn->gated, NT, st); break;
        case 5: rc = launch_tail_batch<5>(a, wt, fn->gated, NT, st); break;
        case 6: rc = launch_tail_batch<6>(a, wt, fn->gated, NT, st); break;
        case 7: rc = launch_tail_batch<7>(a, wt, fn->gated, NT, st); break;
        case 8: rc = launch_tail_batch<8>(a, wt, fn->gated, NT, st); break;
        default: return PI_ERR_BATCH;
    }
    return rc == 0 ? PI_OK : PI_ERR_HIP;
}

int enqueue_compact(const uint8_t *mask, int f, const int32_t *slot_of, int32_t *idx, int32_t *counts,
                    hipStream_t st) {
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, mask, f, slot_of, idx, counts);
    return launch_status();
}

template <int B, bool GATED, int WT>
int enqueue_sparse_b(const pi_ffn *fn, const uint16_t *x, const int32_t *idx, const int32_t *counts, float *y,
                     const FfnScratch &sc, hipStream_t st) {
    const int d = fn->d_model, f = fn->d_ffn, ns = fn->n_slots;
    const int64_t rb = row_bytes_of(fn);
    const int xch = x_chunk(d, B);
    const int G = std::max(1, std::min(kUpMaxGroups, ceil_div(ns, 4 * UpStep<GATED, WT>::R)));
    const int h_stride = std::max(ns, 1);
    const int slabs = down_slabs(d), C = down_chunks(d);
    hipLaunchKernelGGL((k_sparse_up<B, GATED, WT>), dim3(G), dim3(256), (size_t)B * xch * 2, st,
                       static_cast<const uint8_t *>(fn->w_in), rb, d, static_cast<const uint16_t *>(fn->b_up), x,
                       idx, counts, fn->slot_of, f, ns, sc.h, h_stride, xch, sc.tickets, slabs, fn->act);
    hipLaunchKernelGGL((k_sparse_down<B, WT>), dim3(slabs, C), dim3(256), 0, st,
                       static_cast<const uint8_t *>(fn->w_down_t), rb, d, idx, counts, fn->slot_of, f, ns, sc.h,
                       h_stride, sc.part, C, sc.tickets, static_cast<const uint16_t *>(fn->b_down), y);
    return launch_status();
}

template <int B>
int enqueue_sparse_bt(const pi_ffn *fn, const uint16_t *x, const int32_t *idx, const int32_t *counts, float *y,
                      const FfnScratch &sc, hipStream_t st) {
    if (fn->wtype == PI_Q4_0) return enqueue_sparse_b<B, false, WT_Q4_0>(fn, x, idx, counts, y, sc, st);
    if (fn->gated) return enqueue_sparse_b<B, true, WT_F16>(fn, x, idx, counts, y, sc, st);
    return enqueue_sparse_b<B, false, WT_F16>(fn, x, idx, counts, y, sc, st);
}

int enqueue_sparse_legacy(const pi_ffn *fn, const void *x, int B, const int32_t *idx, const int32_t *counts, float *y,
                          const FfnScratch &sc, hipStream_t st) {
    const uint16_t *xx = static_cast<const uint16_t *>(x);
    switch (B) {
        case 1: return enqueue_sparse_bt<1>(fn, xx, idx, counts, y, sc, st);
        case 2: return enqueue_sparse_bt<2>(fn, xx, idx, counts, y, sc, st);
        case 3: return enqueue_sparse_bt<3>(fn, xx, idx, counts, y, sc, st);
        case 4: return enqueue_sparse_bt<4>(fn, xx, idx, counts, y, sc, st);
        case 5: return enqueue_sparse_bt<5>(fn, xx, idx, counts, y, sc, st);
        case 6: return enqueue_sparse_bt<6>(fn, xx, idx, counts, y, sc, st);
        case 7: return enqueue_sparse_bt<7>(fn, xx, idx, counts, y, sc, st);
        case 8: return enqueue_sparse_bt<8>(fn, xx, idx, counts, y, sc, st);
    }
    return PI_ERR_BATCH;
}

// The split kernels on a pi_sparse_ffn workspace `w` (past its control block).  Positions from
// idx/counts, or (bits != nullptr) from the listed-flag words.
int enqueue_split(const pi_ffn *fn, const void *x, int B, const int32_t *idx, const int32_t *counts,
                  const uint32_t *bits, float *y, char *w, hipStream_t st, uint64_t *trace = nullptr) {
    const SplitGeom g = split_geom(fn, B);
    SplitArgs a{};
    a.d = fn->d_model; a.f = fn->d_ffn; a.n_slots = fn->n_slots; a.S = g.S; a.act = fn->act;
    a.nwords = bits != nullptr ? mask_words(fn->d_ffn) : 0;
    a.row_bytes = row_bytes_of(fn);
    a.w_in = static_cast<const uint8_t *>(fn->w_in); a.w_dn = static_cast<const uint8_t *>(fn->w_down_t);
    a.b_up = static_cast<const uint16_t *>(fn->b_up); a.b_down = static_cast<const uint16_t *>(fn->b_down);
    a.slot_of = fn->slot_of;
    a.x = static_cast<const uint16_t *>(x); a.y = y;
    a.idx = idx; a.counts = counts; a.bits = bits;
    a.part = reinterpret_cast<float *>(w); w += g.part;
    a.ypart = reinterpret_cast<float *>(w); w += g.ypart;
    a.hout = reinterpret_cast<float *>(w);
#ifdef PIK_TRACE
    a.trace = trace;
#else
    (void)trace;
#endif
    const int wt = fn->wtype == PI_Q4_0 ? WT_Q4_0 : WT_F16;
    return launch_split(a, B, wt, fn->gated, st) == 0 ? PI_OK : PI_ERR_HIP;
}

// The MFMA form of the sparse FFN (k_wide_up, then k_wide_down) on a wide workspace at w; status:
// the sticky status word that an h outside the fp16 pair's range is reported in (NULL: the wide
// workspace's own).
// Whether the Q4_0 up step runs k_wide_up_q4 (one workgroup per compute unit; *cus set).
bool wide_up_q4(const pi_ffn *fn, int *cus) {
    int per_cu = 0;
    return fn->wtype == PI_Q4_0 && (int64_t)fn->n_slots * row_bytes_of(fn) < (int64_t)kBufMax &&
           resident_slots(reinterpret_cast<const void *>(k_wide_up_q4), kWideUpWaves * kWave, 0, cus, &per_cu) == 0;
}
// Whether k_wide_up_q4 can take the positions from the predictor's flag words itself (every neuron
// resident, the words and a workgroup's run within its limits), so the layer needs no k_compact_bits.
bool wide_up_from_bits(const pi_ffn *fn, int B) {
    int cus = 0;
    const int f = fn->d_ffn;
    return sparse_wide(fn, B) && fn->slot_of == nullptr && fn->n_slots == f && wide_up_q4(fn, &cus) &&
           mask_words(f) <= kWideUpWordsPerThread * kWideUpWaves * kWave &&
           ceil_div(ceil_div(f, 16), cus) * 16 <= kWideUpRunIds;
}

// bits, idx_w, counts_w: with wide_up_from_bits, the predictor's flag words; the positions and counts
// are then written to idx_w / counts_w (the same arrays as idx / counts) by k_wide_up_q4.
int enqueue_wide(const pi_ffn *fn, const void *x, int B, const int32_t *idx, const int32_t *counts, float *y, char *w,
                 hipStream_t st, int32_t *status = nullptr, bool xmf_ready = false, const uint32_t *bits = nullptr,
                 int32_t *idx_w = nullptr, int32_t *counts_w = nullptr) {
    const WideGeom g = wide_geom(fn, B);
    int32_t *tickets = reinterpret_cast<int32_t *>(w + g.tick);
    if (status == nullptr) status = reinterpret_cast<int32_t *>(w);
    uint16_t *h_hi = reinterpret_cast<uint16_t *>(w + g.hi);     // the h table (hi and lo regions together)
    float *part = reinterpret_cast<float *>(w + g.part);
    const int d = fn->d_model, f = fn->d_ffn, ns = fn->n_slots;
    const int64_t rb = row_bytes_of(fn);
    const uint8_t *w_in = static_cast<const uint8_t *>(fn->w_in);
    const uint16_t *xx = static_cast<const uint16_t *>(x), *b_up = static_cast<const uint16_t *>(fn->b_up);
    const dim3 up_grid(std::max(1, ceil_div(ns, 16)));
    const bool q4 = fn->wtype == PI_Q4_0;
    // x in the up step's operand order: always for Q4_0 rows; for fp16 rows when the predictor's grid
    // wrote it, or past 8 tokens (a launch of its own costs more than it saves below that: measured,
    // the 11008-neuron layer at 4 tokens 50.6 -> 53.5 us per layer; the 28672-neuron one at 16 tokens
    // 158.7 -> 132.0, its 16 token rows 14336 bytes apart)
    const bool use_xmf = q4 || xmf_ready || B > kGemvMaxBatch;
    uint4 *xmf = reinterpret_cast<uint4 *>(w + g.xmf);
    if (use_xmf && !xmf_ready)
        hipLaunchKernelGGL(k_wide_xmf, dim3(ceil_div(wide_xmf_vectors(d, q4), 256)), dim3(256), 0, st, xx, B, d,
                           q4 ? 1 : 0, xmf);
    if (q4) {
        int cus = 0;
        if (wide_up_q4(fn, &cus)) {
            WideUpQ4Args ua{w_in, rb, d, B, f, ns, g.hs, fn->act, b_up, xmf, idx, fn->slot_of, h_hi, status,
                            bits, mask_words(f), idx_w, counts_w};
            hipLaunchKernelGGL(k_wide_up_q4, dim3(cus), dim3(kWideUpWaves * kWave), 0, st, ua, counts, tickets, g.S);
        }
        else
            hipLaunchKernelGGL((k_wide_up<false, WT_Q4_0, 2>), dim3(std::max(1, ceil_div(ns, 32))), dim3(kWideThreads),
                               0, st, w_in, rb, d, b_up, xx, xmf, B, idx, counts, fn->slot_of, f, ns, h_hi, g.hs,
                               tickets, g.S, fn->act, status);
    } else if (fn->gated) {
        hipLaunchKernelGGL((k_wide_up<true, WT_F16, 1>), up_grid, dim3(kWideThreads), 0, st, w_in, rb, d, b_up, xx,
                           use_xmf ? xmf : nullptr, B, idx, counts, fn->slot_of, f, ns, h_hi, g.hs,
                           tickets, g.S, fn->act, status);
    } else {
        hipLaunchKernelGGL((k_wide_up<false, WT_F16, 1>), up_grid, dim3(kWideThreads), 0, st, w_in, rb, d, b_up, xx,
                           use_xmf ? xmf : nullptr, B, idx, counts, fn->slot_of, f, ns, h_hi, g.hs,
                           tickets, g.S, fn->act, status);
    }
    const uint8_t *w_dn = static_cast<const uint8_t *>(fn->w_down_t);
    const uint16_t *b_dn = static_cast<const uint16_t *>(fn->b_down);
    if (fn->wtype == PI_Q4_0) {
        // as many (slab, chunk) workgroups as compute units, at most: one each, none drawing two
        // (measured on the 49152-neuron layer: 5 chunks of 12 waves instead of 8 chunks of 8 waves,
        // 123.1 -> 118.1 us per layer at batch 8, 163.6 -> 159.8 at 16)
        int cus = 0, per_cu = 0;
        int C = g.C;
        if (resident_slots(reinterpret_cast<const void *>(k_wide_down<WT_Q4_0, kWideDownWaves>), kWideDownWaves * kWave,
                           0, &cus, &per_cu) == 0)
            C = std::max(1, std::min(g.C, cus / g.S));
        const int pairs = ceil_div(g.S, 8) * C;
        hipLaunchKernelGGL((k_wide_down<WT_Q4_0, kWideDownWaves>), dim3(64 * ceil_div(pairs, 8)),
                           dim3(kWideDownWaves * kWave), 0, st, w_dn, rb, d, B, idx, counts, fn->slot_of, f, ns, h_hi,
                           g.hs, part, C, tickets, b_dn, y, 1, g.S);
    } else {
        // 12 waves (measured on the 11008-neuron layer at 16 tokens: 81.7 -> 79.7 us per layer)
        hipLaunchKernelGGL((k_wide_down<WT_F16, kWideDownWaves>), dim3(g.S, g.C), dim3(kWideDownWaves * kWave), 0, st,
                           w_dn, rb, d, B, idx, counts, fn->slot_of, f, ns, h_hi, g.hs, part, g.C, tickets, b_dn,
                           y, 0, g.S);
    }
    return launch_status();
}

// pi_sparse_ffn's work on a workspace laid out by ffn_ws; bits: listed-flag words to take the
// positions from instead of idx/counts; status: the status word to report in (NULL: the
// workspace's own, at byte offset 384).
int enqueue_sparse(const pi_ffn *fn, const void *x, int B, const int32_t *idx, const int32_t *counts, float *y,
                   void *ws, hipStream_t st, const uint32_t *bits = nullptr, int32_t *status = nullptr,
                   bool xmf_ready = false, const uint32_t *up_bits = nullptr, int32_t *idx_w = nullptr,
                   int32_t *counts_w = nullptr) {
    char *w = static_cast<char *>(ws);
    if (sparse_split(fn, B))
        return enqueue_split(fn, x, B, idx, counts, bits, y, w + ctl_bytes(fn->d_model), st);
    if (status == nullptr) status = reinterpret_cast<int32_t *>(w) + CTL_STATUS;
    if (sparse_wide(fn, B))
        return enqueue_wide(fn, x, B, idx, counts, y, w + ctl_bytes(fn->d_model), st, status, xmf_ready, up_bits,
                            idx_w, counts_w);
    return enqueue_sparse_legacy(fn, x, B, idx, counts, y, ffn_scratch(fn, B, w + ctl_bytes(fn->d_model)), st);
}

// Layout of a pi_ffn_layer workspace: the shared control block, the sparse-FFN scratch (ffn_ws),
// the tail kernel's scratch (tail_ws), the union mask [f] u8, idx [f] and counts [2] int32, the
// listed-bit words [ceil(f/32)], z [B][r] fp32.  Everything that carries state from one call to
// the next (the epoch, stamped words, slab tickets) sits at offsets that depend on the FFN
// descriptor and the batch only; z, the one rank-dependent part, comes last, so layers whose
// predictors differ in rank can share one workspace sized for the largest rank.
struct LayerWs {
    int32_t *ctl;
    float *z;
    uint8_t *mask;
    int32_t *idx, *counts;
    uint32_t *bits;
    char *ffn, *tail;
};
size_t layer_ws_bytes(const pi_predictor *p, const pi_ffn *fn, int B) {
    return ctl_bytes(p->d_model) + pred_ws(p, B) + align_up((size_t)p->d_ffn) + align_up((size_t)p->d_ffn * 4) +
           align_up(2 * sizeof(int32_t)) + align_up((size_t)mask_words(p->d_ffn) * 4) + ffn_ws(fn, B) + tail_ws(fn, B);
}
LayerWs layer_ws(const pi_predictor *p, const pi_ffn *fn, int B, void *ws) {
    LayerWs L;
    char *q = static_cast<char *>(ws);
    L.ctl = reinterpret_cast<int32_t *>(q); q += ctl_bytes(p->d_model);
    L.ffn = q; q += ffn_ws(fn, B);
    L.tail = q; q += tail_ws(fn, B);
    L.mask = reinterpret_cast<uint8_t *>(q); q += align_up((size_t)p->d_ffn);
    L.idx = reinterpret_cast<int32_t *>(q); q += align_up((size_t)p->d_ffn * 4);
    L.counts = reinterpret_cast<int32_t *>(q); q += align_up(2 * sizeof(int32_t));
    L.bits = reinterpret_cast<uint32_t *>(q); q += align_up((size_t)mask_words(p->d_ffn) * 4);
    L.z = reinterpret_cast<float *>(q);
    return L;
}

}  // namespace

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// Address of the current device's copy of `scratch` (looked up once per device), or nullptr.
void *noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace

// ==================================================================== C ABI

extern "C" {

size_t pi_workspace_bytes(const pi_predictor *pred, const pi_ffn *ffn, int32_t batch) {
    if (check_batch(batch) != PI_OK || (!pred && !ffn)) return 0;
    if (pred && check_pred(pred) != PI_OK) return 0;
    if (ffn && check_ffn(ffn) != PI_OK) return 0;
    if (pred && ffn) {
        if (pred->d_model != ffn->d_model || pred->d_ffn != ffn->d_ffn) return 0;
        return layer_ws_bytes(pred, ffn, batch);
    }
    return pred ? pred_ws(pred, batch) : ffn_ws(ffn, batch);
}

int pi_predict(const pi_predictor *pred, const void *x, int32_t batch, uint8_t *mask, float *logits, void *ws,
               size_t ws_bytes, void *stream) {
    int rc = check_pred(pred);
    if (rc) return rc;
    if ((rc = check_batch(batch))) return rc;
    if (!x || !mask) return PI_ERR_NULL;
    if (!aligned16(x)) return PI_ERR_ALIGN;
    if (!ws || ws_bytes < pred_ws(pred, batch)) return PI_ERR_WORKSPACE;
    if (!aligned16(ws)) return PI_ERR_ALIGN;
    return enqueue_predict(pred, x, batch, mask, logits, static_cast<float *>(ws), static_cast<hipStream_t>(stream));
}

int pi_compact(const uint8_t *mask, int32_t d_ffn, const int32_t *slot_of, int32_t *idx, int32_t *counts,
               void *stream) {
    if (!mask || !idx || !counts) return PI_ERR_NULL;
    if (d_ffn < 1 || d_ffn > PI_MAX_D_FFN) return PI_ERR_SHAPE;
    return enqueue_compact(mask, d_ffn, slot_of, idx, counts, static_cast<hipStream_t>(stream));
}

int pi_sparse_ffn(const pi_ffn *ffn, const void *x, int32_t batch, const int32_t *idx, const int32_t *counts,
                  float *y, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_ffn(ffn);
    if (rc) return rc;
    if ((rc = check_batch(batch))) return rc;
    if (!x || !idx || !counts || !y) return PI_ERR_NULL;
    if (!aligned16(x)) return PI_ERR_ALIGN;
    if (!ws || ws_bytes < ffn_ws(ffn, batch)) return PI_ERR_WORKSPACE;
    if (!aligned16(ws)) return PI_ERR_ALIGN;
    return enqueue_sparse(ffn, x, batch, idx, counts, y, ws, static_cast<hipStream_t>(stream));
}

size_t pi_sparse_ffn_wide_workspace_bytes(const pi_ffn *ffn, int32_t batch) {
    if (check_ffn(ffn) != PI_OK || check_wide_batch(batch) != PI_OK) return 0;
    return wide_geom(ffn, batch).total;
}

int pi_sparse_ffn_wide(const pi_ffn *ffn, const void *x, int32_t batch, const int32_t *idx, const int32_t *counts,
                       float *y, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_ffn(ffn);
    if (rc) return rc;
    if ((rc = check_wide_batch(batch))) return rc;
    if (!x || !idx || !counts || !y) return PI_ERR_NULL;
    if (!aligned16(x)) return PI_ERR_ALIGN;
    const WideGeom g = wide_geom(ffn, batch);
    if (!ws || ws_bytes < g.total) return PI_ERR_WORKSPACE;
    if (!aligned16(ws)) return PI_ERR_ALIGN;
    return enqueue_wide(ffn, x, batch, idx, counts, y, static_cast<char *>(ws), static_cast<hipStream_t>(stream));
}

int pi_predict_hidden(const pi_predictor *pred, const void *x, int32_t batch, float *z, void *stream) {
    int rc = check_pred(pred);
    if (rc) return rc;
    if ((rc = check_batch(batch))) return rc;
    if (!x || !z) return PI_ERR_NULL;
    if (!aligned16(x) || !aligned16(z)) return PI_ERR_ALIGN;
    return enqueue_pred_l1(pred, x, batch, z, static_cast<hipStream_t>(stream));
}

namespace {

// The layer path of batches <= 2 on layers too large for the tail kernel: k_pred_up (logits, mask,
// live flags, h of the listed neurons), then k_down_split on the live neurons and k_sum_split.
int enqueue_pred_up(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int B, const float *z, float *y,
                    uint8_t *mask, const LayerWs &L, hipStream_t st, uint64_t *trace = nullptr) {
    const int f = pred->d_ffn;
    const SplitGeom g = split_geom(ffn, B);
    PredUpArgs p{};
    p.d = pred->d_model; p.f = f; p.r = pred->rank; p.n_slots = ffn->n_slots; p.act = ffn->act;
    p.row_bytes = row_bytes_of(ffn);
    p.p2 = static_cast<const uint16_t *>(pred->p2); p.c = static_cast<const uint16_t *>(pred->c); p.z = z;
    p.w_in = static_cast<const uint8_t *>(ffn->w_in); p.b_up = static_cast<const uint16_t *>(ffn->b_up);
    p.slot_of = ffn->slot_of; p.x = static_cast<const uint16_t *>(x);
    p.mask = mask; p.bits = L.bits;
    char *w = L.ffn + ctl_bytes(ffn->d_model);
    SplitArgs a{};
    a.d = ffn->d_model; a.f = f; a.n_slots = ffn->n_slots; a.S = g.S; a.act = ffn->act;
    a.nwords = mask_words(f);
    a.row_bytes = row_bytes_of(ffn);
    a.w_in = static_cast<const uint8_t *>(ffn->w_in); a.w_dn = static_cast<const uint8_t *>(ffn->w_down_t);
    a.b_up = p.b_up; a.b_down = static_cast<const uint16_t *>(ffn->b_down);
    a.slot_of = ffn->slot_of; a.x = p.x; a.y = y; a.bits = L.bits;
    a.part = reinterpret_cast<float *>(w);
    a.ypart = reinterpret_cast<float *>(w + g.part);
    a.hout = nullptr;
    p.h = reinterpret_cast<float *>(w + g.part + g.ypart);        // the hout region: [B][f]
    a.hin = p.h;
#ifdef PIK_TRACE
    a.trace = trace;
    p.trace = trace != nullptr ? trace + 8192 * 8 : nullptr;
#else
    (void)trace;
#endif
    const int wt = ffn->wtype == PI_Q4_0 ? WT_Q4_0 : WT_F16;
    const int NT = pred->rank <= 512 ? 1 : (pred->rank <= 1024 ? 2 : 4);
    return launch_pred_up_split(p, a, B, wt, ffn->gated, NT, st) ? PI_ERR_HIP : PI_OK;
}

// The layer from z on (mask, placement restriction, sparse FFN) on a layer workspace.
int layer_from_hidden(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int32_t batch, const float *z,
                      float *y, uint8_t *mask_out, int32_t *idx_out, int32_t *counts_out, void *ws, hipStream_t st) {
    const int f = pred->d_ffn;
    const LayerWs L = layer_ws(pred, ffn, batch, ws);
    uint8_t *mask = mask_out ? mask_out : L.mask;
    int32_t *idx = idx_out ? idx_out : L.idx;
    int32_t *counts = counts_out ? counts_out : L.counts;
    const bool want_list = idx_out != nullptr || counts_out != nullptr;
    int rc;
    if (tail_persistent(pred, ffn, batch)) {
        // one kernel for the mask and the sparse FFN; the list only when it is asked for
        if ((rc = enqueue_tail(pred, ffn, x, batch, z, y, (mask_out || want_list) ? mask : nullptr, L.ctl, L.tail, st)))
            return rc;
        return want_list ? enqueue_compact(mask, f, ffn->slot_of, idx, counts, st) : PI_OK;
    }
    if (layer_pred_up(pred, ffn, batch)) {
        // logits, mask, live flags and h of the listed neurons in one kernel, then the down rows
        if ((rc = enqueue_pred_up(pred, ffn, x, batch, z, y, mask, L, st))) return rc;
        return want_list ? enqueue_compact(mask, f, ffn->slot_of, idx, counts, st) : PI_OK;
    }
    if (layer_split(ffn, batch)) {
        // the predictor leaves the listed flags as bit words, which the sparse FFN reads directly
        if ((rc = enqueue_pred_l2(pred, z, batch, mask, nullptr, st, L.bits, ffn->slot_of, ffn->n_slots))) return rc;
        if ((rc = enqueue_sparse(ffn, x, batch, nullptr, nullptr, y, L.ffn, st, L.bits))) return rc;
        return want_list ? enqueue_compact(mask, f, ffn->slot_of, idx, counts, st) : PI_OK;
    }
    // the up step's copy of x (MFMA form) comes from the predictor's grid when it runs k_pred_l2_mfma_s
    uint4 *xmf = nullptr;
    if (sparse_wide(ffn, batch) && pred_l2_staged(pred, batch))
        xmf = reinterpret_cast<uint4 *>(static_cast<char *>(L.ffn) + ctl_bytes(ffn->d_model) + wide_geom(ffn, batch).xmf);
    if (mask_words(f) <= 4096) {
        // the list from the predictor's flag words (unrestricted: the placement is applied while
        // listing), a 32-fold smaller read than the mask bytes
        if ((rc = enqueue_pred_l2(pred, z, batch, mask, nullptr, st, L.bits, nullptr, f, x, xmf,
                                  ffn->wtype == PI_Q4_0)))
            return rc;
        if (wide_up_from_bits(ffn, batch))                     // the up step lists the positions itself
            return enqueue_sparse(ffn, x, batch, idx, counts, y, L.ffn, st, nullptr, L.ctl + CTL_STATUS,
                                  xmf != nullptr, L.bits, idx, counts);
        hipLaunchKernelGGL(k_compact_bits, dim3(1), dim3(1024), 0, st, L.bits, mask_words(f), ffn->slot_of,
                           ffn->n_slots, idx, counts);
        if ((rc = launch_status())) return rc;
    } else {
        if ((rc = enqueue_pred_l2(pred, z, batch, mask, nullptr, st, nullptr, nullptr, 0, x, xmf, ffn->wtype == PI_Q4_0)))
            return rc;
        if ((rc = enqueue_compact(mask, f, ffn->slot_of, idx, counts, st))) return rc;
    }
    return enqueue_sparse(ffn, x, batch, idx, counts, y, L.ffn, st, nullptr, L.ctl + CTL_STATUS, xmf != nullptr);
}

int check_layer(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int32_t batch, const float *y,
                const void *ws, size_t ws_bytes) {
    int rc = check_pred(pred);
    if (rc) return rc;
    if ((rc = check_ffn(ffn))) return rc;
    if ((rc = check_batch(batch))) return rc;
    if (pred->d_model != ffn->d_model || pred->d_ffn != ffn->d_ffn) return PI_ERR_SHAPE;
    if (!x || !y) return PI_ERR_NULL;
    if (!aligned16(x)) return PI_ERR_ALIGN;
    if (!ws || ws_bytes < pi_workspace_bytes(pred, ffn, batch)) return PI_ERR_WORKSPACE;
    if (!aligned16(ws)) return PI_ERR_ALIGN;
    return PI_OK;
}

}  // namespace

int pi_layer_path(const pi_predictor *pred, const pi_ffn *ffn, int32_t batch) {
    if (check_pred(pred) != PI_OK || check_ffn(ffn) != PI_OK || check_batch(batch) != PI_OK) return 0;
    if (pred->d_model != ffn->d_model || pred->d_ffn != ffn->d_ffn) return 0;
    return tail_persistent(pred, ffn, batch) ? 1 : 2;
}

int pi_ffn_layer_from_hidden(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int32_t batch,
                             const float *z, float *y, uint8_t *mask_out, int32_t *idx_out, int32_t *counts_out,
                             void *ws, size_t ws_bytes, void *stream) {
    int rc = check_layer(pred, ffn, x, batch, y, ws, ws_bytes);
    if (rc) return rc;
    if (!z) return PI_ERR_NULL;
    if (!aligned16(z)) return PI_ERR_ALIGN;
    return layer_from_hidden(pred, ffn, x, batch, z, y, mask_out, idx_out, counts_out, ws,
                             static_cast<hipStream_t>(stream));
}

int pi_ffn_layer(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int32_t batch, float *y,
                 uint8_t *mask_out, int32_t *idx_out, int32_t *counts_out, void *ws, size_t ws_bytes,
                 void *stream) {
    int rc = check_layer(pred, ffn, x, batch, y, ws, ws_bytes);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const LayerWs L = layer_ws(pred, ffn, batch, ws);
    if ((rc = enqueue_pred_l1(pred, x, batch, L.z, st, pred_zpart(pred, batch, L.z)))) return rc;
    return layer_from_hidden(pred, ffn, x, batch, L.z, y, mask_out, idx_out, counts_out, ws, st);
}

size_t pi_sparse_ffn_h_offset(const pi_ffn *ffn, int32_t batch, int32_t *kind) {
    if (check_ffn(ffn) != PI_OK || check_batch(batch) != PI_OK || !kind) return (size_t)-1;
    if (sparse_split(ffn, batch)) {
        const SplitGeom g = split_geom(ffn, batch);
        *kind = 1;
        return ctl_bytes(ffn->d_model) + g.part + g.ypart;
    }
    if (sparse_wide(ffn, batch)) {
        *kind = 3;
        return ctl_bytes(ffn->d_model) + wide_geom(ffn, batch).hi;
    }
    *kind = 2;
    return ctl_bytes(ffn->d_model);
}

int pi_sparse_ffn_noalloc(const pi_ffn *ffn, const void *x, int32_t batch, const int32_t *idx, const int32_t *counts,
                          float *y, void *stream) {
    int rc = check_ffn(ffn);
    if (rc) return rc;
    if ((rc = check_batch(batch))) return rc;
    if (!x || !idx || !counts || !y) return PI_ERR_NULL;
    if (!aligned16(x)) return PI_ERR_ALIGN;
    if (ffn_ws(ffn, batch) > (size_t)PI_NOALLOC_SCRATCH_BYTES) return PI_ERR_WORKSPACE;
    void *ws = noalloc_scratch();
    if (ws == nullptr) return PI_ERR_HIP;
    // every form of the sparse FFN writes each scratch value before reading it within the call, so
    // the array's contents from earlier calls never matter and nothing is cleared
    return enqueue_sparse(ffn, x, batch, idx, counts, y, ws, static_cast<hipStream_t>(stream));
}

const char *pi_status_string(int status) {
    switch (status) {
        case PI_OK: return "ok";
        case PI_ERR_NULL: return "a required pointer is NULL";
        case PI_ERR_SHAPE: return "a size is out of range or inconsistent";
        case PI_ERR_DTYPE: return "unsupported weight kind or gating combination";
        case PI_ERR_BATCH: return "batch outside [1, 16]";
        case PI_ERR_WORKSPACE: return "workspace missing or too small";
        case PI_ERR_ALIGN: return "pointer or row not 16-byte aligned";
        case PI_ERR_HIP: return "HIP kernel launch failed";
    }
    return "unknown status";
}

int pi_version(void) { return 200; }

#ifdef PIK_TRACE
// Diagnostic build only: the tail kernel and the split kernel with per-workgroup timestamps.
int pi_trace_tail(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int32_t batch, float *y, void *ws,
                  uint64_t *trace, void *stream) {
    if (!tail_persistent(pred, ffn, batch)) return PI_ERR_SHAPE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const LayerWs L = layer_ws(pred, ffn, batch, ws);
    int rc = enqueue_pred_l1(pred, x, batch, L.z, st);
    if (rc) return rc;
    return enqueue_tail(pred, ffn, x, batch, L.z, y, nullptr, L.ctl, L.tail, st, trace);
}

int pi_trace_layer_split(const pi_predictor *pred, const pi_ffn *ffn, const void *x, int32_t batch, float *y,
                         void *ws, uint64_t *trace, void *stream) {
    if (tail_persistent(pred, ffn, batch) || !layer_pred_up(pred, ffn, batch)) return PI_ERR_SHAPE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const LayerWs L = layer_ws(pred, ffn, batch, ws);
    int rc = enqueue_pred_l1(pred, x, batch, L.z, st);
    if (rc) return rc;
    return enqueue_pred_up(pred, ffn, x, batch, L.z, y, L.mask, L, st, trace);
}

int pi_trace_sparse(const pi_ffn *ffn, const void *x, int32_t batch, const int32_t *idx, const int32_t *counts,
                    float *y, void *ws, uint64_t *trace, void *stream) {
    if (!sparse_split(ffn, batch)) return PI_ERR_SHAPE;
    char *w = static_cast<char *>(ws);
    return enqueue_split(ffn, x, batch, idx, counts, nullptr, y, w + ctl_bytes(ffn->d_model),
                         static_cast<hipStream_t>(stream), trace);
}
#endif

}  // extern "C"
