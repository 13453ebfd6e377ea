// pi_split.hpp -- the neuron-aware sparse FFN at batch <= 2 as two launches of (column slab x list
// chunk) workgroups (PowerInfer, arXiv 2312.12456, method section: operators that compute only the
// neurons predicted to fire, each neuron's weights read as contiguous rows).
//
// For list positions k < n, slot s_k of neuron idx[k]:
//   h[b][k] = act(W_up[s_k] x_b + b_up[s_k])  or  max(0, W_gate[s_k] x_b) * (W_up[s_k] x_b)
//   y[b]    = b_down + sum_k h[b][k] W_down^T[s_k]
//
// At batch 1 the operator reads a few thousand scattered rows once each: tens of MB, a few
// microseconds of HBM time, so what bounds it is the number of dependent round trips between the
// first load and y, and how evenly the bytes spread over the compute units.  Workgroup (slab s,
// chunk c) owns columns [s*SLAB, (s+1)*SLAB) of every row of list positions [n*c/C, n*(c+1)/C):
// every workgroup moves the same bytes, and the x values a lane needs -- its own columns -- sit in
// its registers, so nothing is staged.
//   k_up_split    loads its columns of the input row(s) of its positions (all at once), forms the
//                 partial dot products (one wave-wide reduction per row) and stores them:
//                 part[k][s][b*G + g].
//   k_down_split  reads the S partial products of each of its positions (written by the previous
//                 launch; those loads go out first, so h is ready early), issues the loads of its
//                 columns of the W_down^T rows, sums the partials in slab order, applies bias and
//                 activation, accumulates h times its columns as the rows arrive (rows whose h is
//                 zero for every token are skipped: exact zeros), reduces its four waves in LDS and
//                 stores its chunk partial of y.
//   k_sum_split   one thread per output: the C chunk partials in chunk order, plus b_down.
// The kernel boundaries are the only hand-offs: no workgroup waits on another, so any grid works,
// and every sum runs in an order fixed by the list and the launch shape, so y is deterministic.
// (Measured on MI355X: a kernel boundary costs less than making the last workgroups of a slab wait
// for the others inside one launch, and far less than polling stamped words.)
// Positions come from a device list (idx, counts: pi_sparse_ffn) or from the listed-flag words the
// predictor wrote (each workgroup counts the set bits of all words and finds its positions by a
// prefix sum: the ascending ranks of the set bits, exactly the list pi_compact would build).  When
// k_pred_up has already formed h (the layer path), the down kernel's chunks are ranges of flag
// words instead, so a workgroup reads only its own words (range mode).
#pragma once

#include "pi_sync.hpp"

namespace pik {

constexpr int kSplitMaxSlabs = 64;
constexpr int kSplitMaxChunks = 64;
constexpr int kSplitMaxWords = 4096;            // mask words a workgroup scans (d_ffn <= 131072)
constexpr int kSplitThreads = 256;
constexpr int kRangeMaxWords = kSplitThreads;   // live-flag words of one chunk in range mode

// Columns of a slab: 64 lanes x CPL (fp16: one 16-byte vector of 8 columns per row; Q4_0: 8 code
// bytes = 16 columns, half of a 32-weight block, plus that block's scale).
template <int WT>
struct SplitCols {
    static constexpr int CPL = WT == WT_F16 ? 8 : 16;
    static constexpr int SLAB = CPL * kWave;
};
// Rows per wave per round (a round covers 4*NR positions), bounded by the registers that hold a
// round's row pieces.
template <int B, bool GATED, int WT>
struct SplitRows {
    static constexpr int NR = GATED ? 8 : 16;
};

__host__ __device__ inline int split_slab_cols(int wt) {
    return wt == WT_F16 ? SplitCols<WT_F16>::SLAB : SplitCols<WT_Q4_0>::SLAB;
}
__host__ __device__ inline int split_slabs(int d, int wt) { return (d + split_slab_cols(wt) - 1) / split_slab_cols(wt); }
// dynamic LDS of either kernel: the mask words and their prefix sums (bits mode; in range mode the
// ids of the chunk's live neurons, at most 32 per word of its range); the down kernel reuses it for
// the four waves' partials of its slab
__host__ __device__ inline size_t split_dyn_lds(int B, int wt, int nwords, bool down, int range_words = 0) {
    const size_t scan = range_words > 0 ? (size_t)32 * range_words * sizeof(int)
                                        : (size_t)2 * (nwords > 0 ? nwords : 0) * sizeof(int);
    const size_t red = down ? (size_t)4 * B * split_slab_cols(wt) * sizeof(float) : 0;
    const size_t m = scan > red ? scan : red;
    return m > 0 ? m : 16;
}

struct SplitArgs {
    int d, f, n_slots, S, C, act, nwords;   // nwords > 0: positions from `bits`, else from idx/counts
    int64_t row_bytes;
    const uint8_t *w_in, *w_dn;
    const uint16_t *b_up, *b_down;
    const int32_t *slot_of;
    const uint16_t *x;
    float *y;
    const int32_t *idx, *counts;            // list mode
    const uint32_t *bits;                   // bits mode: bit i%32 of word i/32 = neuron i is listed
    float *part;                            // [position][S][B*G] partial dot products
    float *ypart;                           // [C][B][d] chunk partials of y
    float *hout;                            // [B][d_ffn] h per position (slab 0 writes it), or nullptr
    const float *hin;                       // [B][d_ffn] h by neuron id (k_pred_up wrote it; bits mode),
                                            // or nullptr: h from the partial products of k_up_split
#ifdef PIK_TRACE
    uint64_t *trace;                        // [grid][8] timestamps
#endif
};

#ifdef PIK_TRACE
#define SPLIT_TRACE_AT(row0, slot)                                                                  \
    do {                                                                                            \
        if (a.trace != nullptr && threadIdx.x == 0)                                                 \
            a.trace[((size_t)(row0) + blockIdx.x) * 8 + (slot)] = wall_clock64();                   \
    } while (0)
#else
#define SPLIT_TRACE_AT(row0, slot) ((void)0)
#endif
#define SPLIT_TRACE(slot) SPLIT_TRACE_AT(0, slot)
#define DOWN_TRACE(slot) SPLIT_TRACE_AT(4096, slot)

// Position of the k-th (0-based) set bit of w; w has more than k bits set.
__device__ __forceinline__ int select_bit(uint32_t w, int k) {
    int pos = 0, c;
    c = __popc(w & 0xFFFFu); if (k >= c) { k -= c; w >>= 16; pos += 16; }
    c = __popc(w & 0xFFu);   if (k >= c) { k -= c; w >>= 8;  pos += 8; }
    c = __popc(w & 0xFu);    if (k >= c) { k -= c; w >>= 4;  pos += 4; }
    c = __popc(w & 0x3u);    if (k >= c) { k -= c; w >>= 2;  pos += 2; }
    if (k >= (int)(w & 1u)) pos += 1;
    return pos;
}

// Exclusive prefix of v over the workgroup (4 waves) and the total; s_w holds 4 ints.
__device__ __forceinline__ int block_excl_scan(int v, int *s_w, int lane, int wave, int &total) {
    const int incl = wave_incl_scan(v);
    if (lane == kWave - 1) s_w[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        before += w < wave ? s_w[w] : 0;
        total += s_w[w];
    }
    return before + incl - v;
}

// The list of a launch: n, and in bits mode the mask words and their inclusive popcount prefix in
// LDS (dyn: [nwords] words then [nwords] prefix).  Workgroup-uniform result.
__device__ __forceinline__ int split_count(const SplitArgs &a, int *dyn, int *s_w, int tid, int lane, int wave) {
    if (a.nwords <= 0) return __builtin_amdgcn_readfirstlane(min(max(a.counts[0], 0), a.n_slots));
    int *s_words = dyn, *s_scan = dyn + a.nwords;
    // thread t owns words [t*per, (t+1)*per): counts, a block scan, then inclusive prefixes
    const int per = (a.nwords + kSplitThreads - 1) / kSplitThreads;        // <= 16
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(a.bits, (uint32_t)a.nwords * 4u);
    uint32_t wv[16];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int wi = tid * per + i;
        wv[i] = bld4(rw, (i < per && wi < a.nwords) ? (uint32_t)wi * 4u : kOOB);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) cnt += __popc(wv[i]);
    int total;
    int run = block_excl_scan(cnt, s_w, lane, wave, total);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int wi = tid * per + i;
        run += __popc(wv[i]);
        if (i < per && wi < a.nwords) {
            s_words[wi] = (int)wv[i];
            s_scan[wi] = run;
        }
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(total);
}

// Slot of list position q (the q-th listed neuron), or -1; *id_out receives the neuron id.
__device__ __forceinline__ int split_slot(const SplitArgs &a, const int *dyn, int q, int *id_out = nullptr) {
    int id;
    if (a.nwords > 0) {
        const int *s_words = dyn, *s_scan = dyn + a.nwords;
        int lo = 0, hi = a.nwords - 1;                       // first word whose prefix exceeds q
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_scan[mid] > q) hi = mid; else lo = mid + 1;
        }
        const int before = lo > 0 ? s_scan[lo - 1] : 0;
        id = lo * 32 + select_bit((uint32_t)s_words[lo], q - before);
    } else {
        id = a.idx[q];
    }
    if (id_out != nullptr) *id_out = id;
    return slot_of_id(id, a.slot_of, a.f, a.n_slots);
}

// Range mode (h by id): chunk c owns the flag words [c*nwords/C, (c+1)*nwords/C) (at most
// kRangeMaxWords), and its positions are the set bits of those words in ascending id order.  Writes
// their ids to ids[0..n) (LDS) and returns n (workgroup-uniform).  No scan over the whole mask and
// no search per position; the chunks hold unequal numbers of neurons (as many as fired in their id
// range), and every sum still runs in an order fixed by the ids.
__device__ __forceinline__ int split_range(const SplitArgs &a, int c, int *ids, int *s_w, int tid, int lane,
                                           int wave) {
    const int w0 = (int)((int64_t)a.nwords * c / a.C), w1 = (int)((int64_t)a.nwords * (c + 1) / a.C);
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(a.bits, (uint32_t)a.nwords * 4u);
    const uint32_t wv = bld4(rw, w0 + tid < w1 ? (uint32_t)(w0 + tid) * 4u : kOOB);
    int total;
    int pos = block_excl_scan(__popc(wv), s_w, lane, wave, total);
    for (uint32_t m = wv; m != 0u; m &= m - 1u) ids[pos++] = (w0 + tid) * 32 + __builtin_ctz(m);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(total);
}

// ------------------------------------------------------------------------------ up: partial dots

template <int B, bool GATED, int WT>
__global__ __launch_bounds__(kSplitThreads) void k_up_split(SplitArgs a) {
    constexpr int CPL = SplitCols<WT>::CPL, SLAB = SplitCols<WT>::SLAB;
    constexpr int G = GATED ? 2 : 1, BG = B * G;
    constexpr int NR = SplitRows<B, GATED, WT>::NR, RMAX = 4 * NR;
    constexpr int XV = WT == WT_F16 ? 1 : 2;              // 16-byte x vectors per lane per token
    extern __shared__ __align__(16) int dyn[];
    __shared__ int s_slot[RMAX];
    __shared__ int s_w[4];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int s = blockIdx.x % a.S, c = blockIdx.x / a.S;
    SPLIT_TRACE(1);
    const int col = s * SLAB + lane * CPL;
    const bool colok = col < a.d;
    const int cc = colok ? col : 0;                       // a lane past d reads column 0, adds zeros
    const int64_t rb = a.row_bytes;
    const int64_t in_stride = GATED ? 2 * rb : rb;
    // this lane's columns of x; loaded now, used (zeroed past d, q4-paired for Q4_0 rows) only after
    // the row loads are out, so the latencies overlap
    uint4 xr[B][XV];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int v = 0; v < XV; ++v) xr[b][v] = ld16(a.x + (size_t)b * a.d + cc + 8 * v);
    bool x_ready = false;

    const int n = split_count(a, dyn, s_w, tid, lane, wave);
    const int p0 = (int)((int64_t)n * c / a.C), p1 = (int)((int64_t)n * (c + 1) / a.C);
    SPLIT_TRACE(2);
    for (int r0 = p0; r0 < p1; r0 += RMAX) {
        const int nr = min(RMAX, p1 - r0);
        if (tid < nr) s_slot[tid] = split_slot(a, dyn, r0 + tid);
        __syncthreads();
        // this wave's rows j = wave + 4i: its columns of the input row(s)
        uint4 wu[WT == WT_F16 ? NR : 1], wg[GATED ? NR : 1];
        uint2 qu[WT == WT_Q4_0 ? NR : 1];
        uint16_t su[WT == WT_Q4_0 ? NR : 1];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int j = wave + 4 * i;
            const int sl = j < nr ? s_slot[j] : -1;          // wave-uniform
            const int64_t so = sl > 0 ? sl : 0;               // an absent row reads row 0 and is dropped
            const uint8_t *ri = a.w_in + so * in_stride;
            if (WT == WT_F16) {
                wu[WT == WT_F16 ? i : 0] = ld16(ri + (GATED ? rb : 0) + (int64_t)cc * 2);
                if (GATED) wg[GATED ? i : 0] = ld16(ri + (int64_t)cc * 2);
            } else {
                qu[WT == WT_Q4_0 ? i : 0] = *reinterpret_cast<const uint2 *>(ri + cc / 2);
                su[WT == WT_Q4_0 ? i : 0] = *reinterpret_cast<const uint16_t *>(ri + a.d / 2 + (cc / 32) * 2);
            }
        }
        SPLIT_TRACE(3);
        if (!x_ready) {
            x_ready = true;
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int v = 0; v < XV; ++v) xr[b][v] = colok ? (WT == WT_Q4_0 ? pair_for_q4(xr[b][v]) : xr[b][v]) : zero4();
        }
        float pv[BG][NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (WT == WT_F16) {
                    pv[b * G + G - 1][i] = dot8(wu[WT == WT_F16 ? i : 0], xr[b][0], 0.f);
                    if (GATED) pv[b * G][i] = dot8(wg[GATED ? i : 0], xr[b][0], 0.f);
                } else {
                    const uint2 q = qu[WT == WT_Q4_0 ? i : 0];
                    float t = 0.f;
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const uint32_t w = k == 0 ? q.x : q.y;
                        const uint4 xv = xr[b][WT == WT_Q4_0 ? k : 0];
                        t = fdot2(q4pair(w, 0), xv.x, t);
                        t = fdot2(q4pair(w, 4), xv.y, t);
                        t = fdot2(q4pair(w, 8), xv.z, t);
                        t = fdot2(q4pair(w, 12), xv.w, t);
                    }
                    pv[b][i] = t * half_to_float(su[WT == WT_Q4_0 ? i : 0]);
                }
            }
        }
        // one reduce-scatter per component: lane l then holds row l / (64/NR)'s sum
#pragma unroll
        for (int k = 0; k < BG; ++k) {
            const float tot = reduce_scatter<NR>(pv[k], lane);
            const int j = wave + 4 * (lane / (kWave / NR));
            if ((lane % (kWave / NR)) == 0 && j < nr) a.part[((size_t)(r0 + j) * a.S + s) * BG + k] = tot;
        }
        __syncthreads();                                       // s_slot is refilled next round
    }
    SPLIT_TRACE(0);
}

// ------------------------------------------------------------------------------ down: h, y

// HID: h by neuron id (k_pred_up formed it; positions in range mode), else h from the partial
// products of k_up_split (list or bits mode).
template <int B, bool GATED, int WT, bool HID>
__global__ __launch_bounds__(kSplitThreads) void k_down_split(SplitArgs a) {
    constexpr int CPL = SplitCols<WT>::CPL, SLAB = SplitCols<WT>::SLAB;
    constexpr int G = GATED ? 2 : 1, BG = B * G;
    constexpr int NR = SplitRows<B, GATED, WT>::NR, RMAX = 4 * NR;
    static_assert(RMAX * BG <= kSplitThreads, "one thread per (position, component) in the gather");
    extern __shared__ __align__(16) int dyn[];            // scan (bits mode) | wave partials of y
    __shared__ int s_slot[RMAX];
    __shared__ int s_id[RMAX];
    __shared__ float s_hc[RMAX][BG];
    __shared__ float s_h[RMAX][B];
    __shared__ int s_w[4];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int s = blockIdx.x % a.S, c = blockIdx.x / a.S;
    DOWN_TRACE(1);
    const int col = s * SLAB + lane * CPL;
    const int cc = col < a.d ? col : 0;
    constexpr bool hmode = HID;
    constexpr bool range = HID;                             // positions: the live ids of this chunk's range
    const int64_t rb = a.row_bytes;

    int p0, p1;
    if (range) {
        p0 = 0;
        p1 = split_range(a, c, dyn, s_w, tid, lane, wave);
    } else {
        const int n = split_count(a, dyn, s_w, tid, lane, wave);
        p0 = (int)((int64_t)n * c / a.C);
        p1 = (int)((int64_t)n * (c + 1) / a.C);
    }
    DOWN_TRACE(2);
    float acc[B][CPL];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < CPL; ++t) acc[b][t] = 0.f;

    for (int r0 = p0; r0 < p1; r0 += RMAX) {
        const int nr = min(RMAX, p1 - r0);
        if (tid < nr) {
            int id;
            if (range) {
                id = dyn[r0 + tid];
                s_slot[tid] = slot_of_id(id, a.slot_of, a.f, a.n_slots);
            } else {
                s_slot[tid] = split_slot(a, dyn, r0 + tid, &id);
            }
            s_id[tid] = id;
        }
        __syncthreads();
        // h mode: thread (j, b) reads h of position j's neuron, token b (goes out before the rows)
        float hpre = 0.f;
        if (hmode && tid < nr * B) {
            const int j = tid / B, b = tid - j * B;
            hpre = a.hin[(size_t)b * a.f + s_id[j]];
        }
        // thread (j, k) reads component k of position j from every slab; these loads go out before
        // the row loads, so they return first and h is ready while the rows still stream
        // (through a buffer resource over the round's partials: no branch, an absent one reads 0)
        const bool mine = !hmode && tid < nr * BG;
        const int jh = mine ? tid / BG : 0, kh = tid - jh * BG;
        const __amdgpu_buffer_rsrc_t rp = buf_rsrc(a.part + (size_t)r0 * a.S * BG, (uint32_t)(nr * a.S * BG) * 4u);
        auto part_off = [&](int u) -> uint32_t {
            return (mine && u < a.S) ? (uint32_t)((jh * a.S + u) * BG + kh) * 4u : kOOB;
        };
        float pv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) pv[u] = __builtin_bit_cast(float, bld4(rp, part_off(u)));
        // this wave's rows j = wave + 4i: its columns of the W_down^T rows
        uint4 wd[WT == WT_F16 ? NR : 1];
        uint2 qd[WT == WT_Q4_0 ? NR : 1];
        uint16_t sd[WT == WT_Q4_0 ? NR : 1];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int j = wave + 4 * i;
            const int sl = j < nr ? s_slot[j] : -1;           // wave-uniform
            const int64_t so = sl > 0 ? sl : 0;
            const uint8_t *rd = a.w_dn + so * rb;
            if (WT == WT_F16) {
                wd[WT == WT_F16 ? i : 0] = ld16(rd + (int64_t)cc * 2);
            } else {
                qd[WT == WT_Q4_0 ? i : 0] = *reinterpret_cast<const uint2 *>(rd + cc / 2);
                sd[WT == WT_Q4_0 ? i : 0] = *reinterpret_cast<const uint16_t *>(rd + a.d / 2 + (cc / 32) * 2);
            }
        }
        float sum = 0.f;                                        // slab order
#pragma unroll
        for (int u = 0; u < 16; ++u) sum += pv[u];
        for (int s0 = 16; !hmode && s0 < a.S; s0 += 16) {       // more than 16 slabs (wide rows)
#pragma unroll
            for (int u = 0; u < 16; ++u) pv[u] = __builtin_bit_cast(float, bld4(rp, part_off(s0 + u)));
#pragma unroll
            for (int u = 0; u < 16; ++u) sum += pv[u];
        }
        if (mine) s_hc[jh][kh] = sum;
        __syncthreads();
        if (tid < nr * B) {
            const int j = tid / B, b = tid - j * B;
            const int sl = s_slot[j];
            float hv;
            if (hmode) {
                hv = hpre;
            } else if (GATED) {
                hv = fmaxf(s_hc[j][b * 2], 0.f) * s_hc[j][b * 2 + 1];
            } else {
                const float bias = (a.b_up != nullptr && sl >= 0) ? half_to_float(a.b_up[sl]) : 0.f;
                hv = fmaxf(s_hc[j][b] + bias, 0.f);
                if (a.act) hv *= hv;                          // squared ReLU
            }
            if (sl < 0) hv = 0.f;
            s_h[j][b] = hv;
            if (s == 0 && a.hout != nullptr) a.hout[(size_t)b * a.f + r0 + j] = hv;
        }
        __syncthreads();
        DOWN_TRACE(3);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int j = wave + 4 * i;
            if (j >= nr) break;                                 // wave-uniform
            float hb[B];
            bool any = false;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                hb[b] = s_h[j][b];
                any |= hb[b] != 0.f;
            }
            if (!any) continue;                                 // adds exact zeros
            if (WT == WT_F16) {
                const uint4 w = wd[WT == WT_F16 ? i : 0];
                const uint32_t wq[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const h2 pr = __builtin_bit_cast(h2, wq[p]);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        acc[b][2 * p] = fmaf(hb[b], (float)pr.x, acc[b][2 * p]);
                        acc[b][2 * p + 1] = fmaf(hb[b], (float)pr.y, acc[b][2 * p + 1]);
                    }
                }
            } else {
                const float sc = half_to_float(sd[WT == WT_Q4_0 ? i : 0]);
                const uint2 q = qd[WT == WT_Q4_0 ? i : 0];
                float cf[B];
#pragma unroll
                for (int b = 0; b < B; ++b) cf[b] = hb[b] * sc;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const uint32_t w = k == 0 ? q.x : q.y;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        // q4pair(w, 4p) = (code_p - 8, code_{p+4} - 8): columns 8k + p and 8k + p + 4
                        const h2 pr = __builtin_bit_cast(h2, q4pair(w, 4 * p));
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            acc[b][8 * k + p] = fmaf(cf[b], (float)pr.x, acc[b][8 * k + p]);
                            acc[b][8 * k + p + 4] = fmaf(cf[b], (float)pr.y, acc[b][8 * k + p + 4]);
                        }
                    }
                }
            }
        }
        __syncthreads();                                        // s_slot and s_h are refilled next round
    }
    DOWN_TRACE(4);

    // The chunk partial of this slab: the four waves meet in LDS (fixed order), then plain stores.
    float *s_red = reinterpret_cast<float *>(dyn);             // [4][B][CPL][64]
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < CPL; ++t) s_red[((wave * B + b) * CPL + t) * kWave + lane] = acc[b][t];
    __syncthreads();
    for (int o = tid; o < B * SLAB; o += kSplitThreads) {
        const int b = o / SLAB, ci = o - b * SLAB;
        const int ln = ci / CPL, t = ci - ln * CPL;
        const int e = (b * CPL + t) * kWave + ln;
        const int gcol = s * SLAB + ci;
        if (gcol < a.d)
            a.ypart[((size_t)c * B + b) * a.d + gcol] = s_red[e] + s_red[B * CPL * kWave + e] +
                                                          s_red[2 * B * CPL * kWave + e] + s_red[3 * B * CPL * kWave + e];
    }
    DOWN_TRACE(0);
}

// ------------------------------------------------------------------------------ sum of the chunks

// y[o] = b_down + sum over chunks q, in order, of ypart[q][o] (o = b*d + column); one thread per
// output, all C loads in flight at once.  Launched as one-wave workgroups, so the loads spread over
// four times as many compute units as 256-thread ones would use (measured on the 12288-wide layer
// at batch 1: 47.3 -> 47.1 us per layer).
static __global__ __launch_bounds__(kSplitThreads) void k_sum_split(const float *__restrict__ ypart, int C, int Bd,
                                                                    int d, const uint16_t *__restrict__ b_down,
                                                                    float *__restrict__ y) {
    const int o = blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= Bd) return;
    float v[kSplitMaxChunks];
#pragma unroll
    for (int q = 0; q < kSplitMaxChunks; ++q) v[q] = q < C ? ypart[(size_t)q * Bd + o] : 0.f;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < kSplitMaxChunks; ++q) sum += v[q];
    y[o] = sum + (b_down != nullptr ? half_to_float(b_down[o % d]) : 0.f);
}

// ------------------------------------------------------------------------------ predictor + up

// The second predictor matrix, the mask and the up rows in one launch (layer path, batch <= 2):
// 32-neuron tiles, workgroup g taking tiles g, g + grid, g + 2 grid, ... (the grid is sized so that
// the workgroups fit on the chip together and each gets the same number of tiles, or one fewer, at
// most kPredUpMaxTiles).  A workgroup stages x and z in LDS once, while its first tile's rows of P2
// stream in.  Per tile: each wave forms the partial logits of its eight rows in two halves,
// reloading a half's registers with the next tile's rows as soon as that half is consumed (so P2
// keeps streaming while it computes), sums them with one reduce-scatter, writes the union mask and
// records the tile's listed neurons (fired and resident) in LDS.  After the last tile, the listed
// neurons of all the workgroup's tiles go to the waves, two rows per wave at once where one pass
// covers a row; each reads the input row(s) against x and stores h by neuron id.  Last, each tile's
// word of live flags (listed, and h nonzero for some token) is stored.  Taking the up rows after
// the last tile (one round trip per workgroup, instead of one per tile behind the next tile's P2
// rows) was measured faster on the 49152-neuron layer (42.2 -> 40.5 us for the three kernels of
// the layer path).  k_down_split then visits the live neurons only (a row whose h is zero for every
// token adds exact zeros), reads h by id (hin) and needs no partial products.
struct PredUpArgs {
    int d, f, r, n_slots, act;
    int64_t row_bytes;
    const uint16_t *p2, *c;
    const float *z;                         // [B][r]
    const uint8_t *w_in;
    const uint16_t *b_up;
    const int32_t *slot_of;
    const uint16_t *x;
    uint8_t *mask;                          // [f] union flags
    uint32_t *bits;                         // [ceil(f/32)] live flags (listed, h nonzero for some token)
    float *h;                               // [B][f] h of listed neurons by id (others untouched)
#ifdef PIK_TRACE
    uint64_t *trace;                        // [grid][8] timestamps
#endif
};

// Dynamic LDS of k_pred_up: x [B][d] fp16 (q4-paired for Q4_0), then z [B][r] fp32.
__host__ __device__ inline size_t pred_up_lds(int B, int d, int r) {
    return ((size_t)B * d * 2 + 15) / 16 * 16 + (size_t)B * r * 4;
}

// Tiles of P2 one k_pred_up workgroup takes at most: their listed neurons are handled together
// after the last tile's logits.
constexpr int kPredUpMaxTiles = 8;

template <int B, bool GATED, int WT, int NT>
__global__ __launch_bounds__(256) void k_pred_up(PredUpArgs a) {
    constexpr int R = 8, RH = 4;                          // P2 rows per wave (the tile: 4 x 8), in two halves
    extern __shared__ __align__(16) uint16_t dynx[];
    __shared__ uint32_t s_bytes[kPredUpMaxTiles][4];      // per tile, per wave: listed rows of the wave's eight
    __shared__ uint32_t s_live[kPredUpMaxTiles];
    __shared__ int s_slot[kPredUpMaxTiles][32];
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int ntiles = (a.f + 31) / 32;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.p2, (uint32_t)((size_t)a.f * a.r * 2));
    // the two halves of this wave's rows of P2 (rows 0-3 and 4-7 of its eight); each half is
    // reloaded with the next tile's rows as soon as its logits are formed, so a wave always has
    // P2 loads in flight while it computes (two tiles in flight measured slower: the registers
    // cost a third of the resident waves)
    uint4 w0[RH][NT], w1[RH][NT];
    auto issue = [&](uint4 (&w)[RH][NT], int t, int h) {
        const int row0 = t * 32 + wave * R + h * RH;
#pragma unroll
        for (int i = 0; i < RH; ++i)
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                const int row = row0 + i, col = lane * 8 + q * 512;
                w[i][q] = bld16(rs, (t < ntiles && row < a.f && col < a.r) ? ((uint32_t)row * a.r + col) * 2 : kOOB);
            }
    };
    // partial logits of a half: lane-wise dot products of its columns with z
    auto dots = [&](const uint4 (&w)[RH][NT], const float *zs, float (&v)[B][R], int h) {
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const int col = lane * 8 + q * 512;
            if (col < a.r) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float4 za = *reinterpret_cast<const float4 *>(zs + b * a.r + col);
                    const float4 zb = *reinterpret_cast<const float4 *>(zs + b * a.r + col + 4);
                    const float zr[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
#pragma unroll
                    for (int i = 0; i < RH; ++i) {
                        const uint32_t qq[4] = {w[i][q].x, w[i][q].y, w[i][q].z, w[i][q].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const h2 p = __builtin_bit_cast(h2, qq[e]);
                            v[b][h * RH + i] = fmaf((float)p.x, zr[2 * e], v[b][h * RH + i]);
                            v[b][h * RH + i] = fmaf((float)p.y, zr[2 * e + 1], v[b][h * RH + i]);
                        }
                    }
                }
            }
        }
    };
    const int G = gridDim.x;
    SPLIT_TRACE(1);
    if (threadIdx.x < kPredUpMaxTiles) s_live[threadIdx.x] = 0u;
    issue(w0, blockIdx.x, 0);
    issue(w1, blockIdx.x, 1);
    uint16_t *xs = dynx;
    float *zs = reinterpret_cast<float *>(dynx + ((size_t)B * a.d + 7) / 8 * 8);
    stage_x<B, WT == WT_Q4_0>(xs, a.x, a.d, 0, a.d, a.d);
    stage_vec16(zs, a.z, B * a.r / 4);
    __syncthreads();
    SPLIT_TRACE(2);
    // 1. the logits of every tile of this workgroup (tiles blockIdx.x, +G, +2G, ...): mask flags to
    //    memory, listed rows and their slots to LDS (entry nt for the nt-th tile); the waves need
    //    not meet between tiles
    int nt = 0;
    for (int t = blockIdx.x; t < ntiles && nt < kPredUpMaxTiles; t += G, ++nt) {   // the launch gives no workgroup more tiles
        // lanes 8j .. 8j+7 end up with row j of the wave's eight (reduce-scatter below); they load
        // that row's offset and slot now
        const int rowk = t * 32 + wave * R + (lane >> 3);
        const bool rok = rowk < a.f;
        const uint16_t cbits = rok ? a.c[rowk] : (uint16_t)0;
        const int slot = rok ? (a.slot_of ? a.slot_of[rowk] : rowk) : -1;
        float v[B][R];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int i = 0; i < R; ++i) v[b][i] = 0.f;
        dots(w0, zs, v, 0);
        issue(w0, t + G, 0);
        dots(w1, zs, v, 1);
        issue(w1, t + G, 1);
        const float ci = half_to_float(cbits);
        bool fired = false;
#pragma unroll
        for (int b = 0; b < B; ++b) fired |= reduce_scatter<R>(v[b], lane) + ci > 0.f;
        // bit 8j of the ballot = row j fired (its eight lanes agree)
        const uint64_t fb = __ballot(fired && rok);
        const bool resident = slot >= 0 && slot < a.n_slots;
        const uint64_t rb8 = __ballot(rok && resident);
        uint32_t mb = 0, byte = 0;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            mb |= (uint32_t)((fb >> (8 * j)) & 1u) << j;
            byte |= (uint32_t)((fb & rb8) >> (8 * j) & 1u) << j;
        }
        if ((lane & 7) == 0 && rok) a.mask[rowk] = (uint8_t)((mb >> (lane >> 3)) & 1u);
        if ((lane & 7) == 0) s_slot[nt][wave * R + (lane >> 3)] = resident ? slot : -1;
        if (lane == 0) s_bytes[nt][wave] = byte;
    }
    __syncthreads();
    SPLIT_TRACE(3);
    // 2. the listed neurons of all those tiles, tile by tile in ascending id: wave w takes the
    //    (8p+w)-th and (8p+w+4)-th for p = 0, 1, ... (two rows in flight per wave where one pass
    //    covers a row; the P2 registers are free by now), else the (4p+w)-th
    auto word_of = [&](int k) {
        return s_bytes[k][0] | (s_bytes[k][1] << 8) | (s_bytes[k][2] << 16) | (s_bytes[k][3] << 24);
    };
    int total = 0;
    for (int k = 0; k < nt; ++k) total += __builtin_popcount(word_of(k));
#ifdef PIK_TRACE
    if (a.trace != nullptr && threadIdx.x == 0) {
        a.trace[(size_t)blockIdx.x * 8 + 5] = (uint64_t)total;
        a.trace[(size_t)blockIdx.x * 8 + 6] = (uint64_t)nt;
    }
#endif
    // tile and bit of the j-th listed neuron (j < total)
    auto locate = [&](int j, int &k, int &bit) {
        for (k = 0;; ++k) {
            const uint32_t w = word_of(k);
            const int c = __builtin_popcount(w);
            if (j < c) {
                bit = select_bit(w, j);
                return;
            }
            j -= c;
        }
    };
    using P = RowPass<B, GATED, WT>;
    const int64_t in_stride = GATED ? 2 * a.row_bytes : a.row_bytes;
    const __amdgpu_buffer_rsrc_t rin = buf_rsrc(a.w_in, (uint32_t)(a.n_slots * in_stride));
    const bool pairs = P::extent(a.d) <= P::STEP;
    for (int j = wave; j < total; j += pairs ? 8 : 4) {
        const int j2 = j + 4;
        const bool two = pairs && j2 < total;
        int k1, bit1, k2 = 0, bit2 = 0;
        locate(j, k1, bit1);
        if (two) locate(j2, k2, bit2);
        const int s1 = s_slot[k1][bit1], s2 = two ? s_slot[k2][bit2] : 0;
        float ag[B], au[B], ag2[B], au2[B];
#pragma unroll
        for (int b = 0; b < B; ++b) ag[b] = au[b] = ag2[b] = au2[b] = 0.f;
        if (pairs) {
            const int d2 = two ? a.d : 0;                 // a missing second neuron reads nothing
            P q1, q2;
            q1.issue_buf(rin, (uint32_t)(s1 * in_stride), a.row_bytes, a.d, 0, lane);
            q2.issue_buf(rin, (uint32_t)(s2 * in_stride), a.row_bytes, d2, 0, lane);
            q1.consume(xs, a.d, a.d, 0, lane, ag, au);
            q2.consume(xs, a.d, d2, 0, lane, ag2, au2);
        } else {
            neuron_dots<B, GATED, WT>(a.w_in + (int64_t)s1 * in_stride, a.row_bytes, a.d, xs, a.d, lane, ag, au);
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            if (n == 1 && !two) break;                    // wave-uniform
            const int sl = n == 0 ? s1 : s2, kk = n == 0 ? k1 : k2, bit = n == 0 ? bit1 : bit2;
            const int id = (blockIdx.x + kk * G) * 32 + bit;
            const float bias = (!GATED && a.b_up != nullptr) ? half_to_float(a.b_up[sl]) : 0.f;
            bool live = false;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float u = wave_sum(n == 0 ? au[b] : au2[b]);
                float hv;
                if (GATED) {
                    hv = fmaxf(wave_sum(n == 0 ? ag[b] : ag2[b]), 0.f) * u;
                } else {
                    hv = fmaxf(u + bias, 0.f);
                    if (a.act) hv *= hv;                  // squared ReLU
                }
                live |= hv != 0.f;
                if (lane == 0) a.h[(size_t)b * a.f + id] = hv;
            }
            if (lane == 0 && live) atomicOr(&s_live[kk], 1u << bit);
        }
    }
    // 3. each tile's word of live flags (listed, and h nonzero for some token): the down rows to read
    __syncthreads();
    SPLIT_TRACE(4);
    if (threadIdx.x < nt) a.bits[blockIdx.x + threadIdx.x * G] = s_live[threadIdx.x];
    SPLIT_TRACE(0);
}

// Launch of the three kernels for batch width B in {1, 2}; C is chosen here.
int launch_split(SplitArgs &a, int B, int wtype, int gated, hipStream_t st);
// The layer path: k_pred_up (NT = rank / 512 rounded up to 1, 2 or 4), then k_down_split on h by
// id and k_sum_split.
int launch_pred_up_split(PredUpArgs &p, SplitArgs &a, int B, int wtype, int gated, int NT, hipStream_t st);

}  // namespace pik
