// pi_tail.hpp -- the second half of a layer as ONE persistent kernel: the predictor's second
// matrix and the firing mask, then the sparse FFN over the predicted, resident neurons.
// (PowerInfer, arXiv 2312.12456, method section: an online predictor picks the neurons that will
// fire and neuron-aware operators compute only those; README model-weights section: the GPU index
// of resident neurons.)
//
// Input: z = max(0, P1 x) from the first predictor kernel (a kernel boundary before this one, so z
// is read with ordinary loads and cached by every L2).  For each 32-neuron tile t:
//   l_b,i = P2[i] . z_b + c_i,   fired_i = OR_b [l_b,i > 0],   listed_i = fired_i and slot_of[i] >= 0
//   h_b,i = ReLU(W_up[s] x_b + b_up[s])  or  ReLU(W_gate[s] x_b) (W_up[s] x_b)     (listed i, slot s)
//   y_b   = b_down + sum over listed i, ascending, of h_b,i W_down^T[s]
//
// Workgroups, all resident at once:
//   up    (blockIdx < PU)  tiles t = blockIdx, blockIdx + PU, ...: the tile's 32 rows of P2 are
//                          loaded before anything else (they depend on nothing), z and x are staged
//                          in LDS, the tile's listed bits are published as a stamped word, then each
//                          listed neuron goes to one wave, which publishes its slot and h.
//   down  (NE = slabs * C) tile (column slab, chunk of consecutive neuron tiles): it polls the
//                          chunk's tile words, lists the listed neurons in ascending order, issues
//                          the loads of their W_down^T rows (its columns only) before h is known,
//                          then polls h, accumulates, and stores a partial; then each tile finishes
//                          its share of the slab's columns: the C partials in chunk order + b_down.
// No compaction pass is needed: a chunk's neurons are found from its own tile words, and every
// sum runs in an order fixed by the mask alone, so results do not depend on timing.
//
// Hand-offs use the stamped-word protocol of pi_sync.hpp; the workspace must be zero-filled
// before its first use, and every wait is bounded.
#pragma once

#include "pi_sync.hpp"

namespace pik {

constexpr int kSparseMaxChunks = 16;           // chunk partials per slab
constexpr int kTailListMax = 2048;             // listed neurons a down tile handles per round
constexpr int kTailMaxTiles = 384;             // neuron tiles up to which the tail kernel is used
constexpr int kTailCPL = 8;                    // columns per lane of a down tile (one 16-byte fp16
                                               // load or one Q4_0 code word per row)
constexpr int kTailSlab = kTailCPL * kWave;    // columns of a down tile

struct TailArgs {
    int d, f, r, n_slots, slabs, C, PU, NE, NTL;   // NTL: number of 32-neuron tiles
    int act;                                       // 1: squared ReLU (non-gated)
    int64_t row_bytes;
    const uint16_t *p2, *c;
    const float *z;                                // [B][r]
    const uint8_t *w_in, *w_dn;
    const uint16_t *b_up, *b_down;
    const int32_t *slot_of;
    const uint16_t *x;
    float *y;
    uint8_t *mask;                                 // [f] fired flags (0/1), or null
    int32_t *ctl;
    uint64_t *tword;                               // [NTL] listed bits of each tile, stamped
    uint64_t *ent;                                 // [f][1 + B] slot, then h per token, stamped
    uint64_t *part;                                // [C][B][d] chunk partials, stamped
#ifdef PIK_TRACE
    uint64_t *trace;                               // [P][16] timeline of each workgroup (100 MHz clock)
#endif
};

#ifdef PIK_TRACE
#define TAIL_TRACE(slot, val)                                                                          \
    do {                                                                                               \
        if (a.trace != nullptr && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * 16 + (slot)] = (val); \
    } while (0)
#else
#define TAIL_TRACE(slot, val) ((void)0)
#endif

// Dynamic LDS of the tail kernel: x [B][d] fp16 (q4-paired for Q4_0), then z [B][r] fp32.
__host__ __device__ inline size_t tail_dyn_lds(int B, int d, int r) {
    return ((size_t)B * d * 2 + 15) / 16 * 16 + (size_t)B * r * 4;
}

// ------------------------------------------------------------------------------ up workgroups

// The P2 rows of one 32-neuron tile (wave w: rows 8w .. 8w+7), plus the offset and slot of row i in
// lane i -- all loads issued together.
template <int B, int NT>
struct P2Tile {
    static constexpr int R = 8;
    uint4 w[R][NT];
    uint16_t c;
    int slot;
    __device__ __forceinline__ void issue(const TailArgs &a, int t, int wave, int lane) {
        const int row0 = t * 32 + wave * R;
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.p2, (uint32_t)((size_t)a.f * a.r * 2));
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                const int row = row0 + i, col = lane * 8 + q * 512;
                w[i][q] = bld16(rs, (row < a.f && col < a.r) ? ((uint32_t)row * a.r + col) * 2 : kOOB);
            }
        const int row = row0 + lane;                 // lane i < R: offset and slot of row i
        const bool mine = lane < R && row < a.f;
        c = mine ? a.c[row] : (uint16_t)0;
        slot = mine ? (a.slot_of ? a.slot_of[row] : row) : -1;
    }
};

// Finish one neuron's dots (wave sums, bias, ReLU or ReGLU) and publish its slot and h.
template <int B, bool GATED>
__device__ __forceinline__ void tail_publish(const TailArgs &a, int id, int s, float (&ag)[B], float (&au)[B],
                                             uint32_t stamp, int lane) {
    const float bias = (!GATED && a.b_up != nullptr) ? half_to_float(a.b_up[s]) : 0.f;
    uint64_t *e = a.ent + (size_t)id * (1 + B);
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float u = wave_sum(au[b]);
        float hv;
        if (GATED) {
            const float gv = wave_sum(ag[b]);
            hv = fmaxf(gv, 0.f) * u;
        } else {
            hv = fmaxf(u + bias, 0.f);
            if (a.act) hv *= hv;                        // squared ReLU
        }
        if (lane == 0) store_c64(e + 1 + b, stamped_f(hv, stamp));
    }
    if (lane == 0) store_c64(e, stamped((uint32_t)s, stamp));
}

template <int B, bool GATED, int WT, int NT>
__device__ __forceinline__ void tail_up(const TailArgs &a, uint32_t stamp, int lane, int wave, const uint16_t *xs, const float *zs,
                        uint32_t *s_words, int *s_slot, P2Tile<B, NT> &pt) {
    constexpr int R = P2Tile<B, NT>::R;
    const int64_t in_stride = GATED ? 2 * a.row_bytes : a.row_bytes;
    const __amdgpu_buffer_rsrc_t rin = buf_rsrc(a.w_in, (uint32_t)(a.n_slots * in_stride));
    bool first = true;
    for (int t = blockIdx.x; t < a.NTL; t += a.PU) {
        if (!first) pt.issue(a, t, wave, lane);
        first = false;
        const int row0 = t * 32 + wave * R;
        const float ci = half_to_float(pt.c);
        uint32_t mb = 0;                            // fired bits of the wave's rows (uniform)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float v[R];
#pragma unroll
            for (int i = 0; i < R; ++i) v[i] = 0.f;
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                const int col = lane * 8 + q * 512;
                if (col < a.r) {
                    const float4 za = *reinterpret_cast<const float4 *>(zs + b * a.r + col);
                    const float4 zb = *reinterpret_cast<const float4 *>(zs + b * a.r + col + 4);
                    const float zr[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const uint32_t qq[4] = {pt.w[i][q].x, pt.w[i][q].y, pt.w[i][q].z, pt.w[i][q].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const h2 p = __builtin_bit_cast(h2, qq[e]);
                            v[i] = fmaf((float)p.x, zr[2 * e], v[i]);
                            v[i] = fmaf((float)p.y, zr[2 * e + 1], v[i]);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float l = wave_sum(v[i]) + bcastf(ci, i);
                mb |= (uint32_t)(l > 0.f) << i;
            }
        }
        const int row = row0 + lane;
        const bool mine = lane < R && row < a.f;
        if (mine && a.mask != nullptr) a.mask[row] = (uint8_t)((mb >> lane) & 1u);
        const bool resident = pt.slot >= 0 && pt.slot < a.n_slots;
        if (lane < R) s_slot[wave * R + lane] = resident ? pt.slot : -1;
        // the tile's listed bits: wave w's rows are tile rows 8w .. 8w+7
        const uint32_t byte = mb & (uint32_t)__ballot(mine && resident);
        if (lane == 0) s_words[wave] = byte;
        if (t == (int)blockIdx.x) TAIL_TRACE(3, wall_clock64());
        __syncthreads();
        const uint32_t word = s_words[0] | (s_words[1] << 8) | (s_words[2] << 16) | (s_words[3] << 24);
        if (threadIdx.x == 0) store_c64(a.tword + t, stamped(word, stamp));
        if (t == (int)blockIdx.x) TAIL_TRACE(4, wall_clock64());
        // listed neurons of the tile in ascending order: wave w takes the w-th, (w+4)-th, ...; when
        // one pass covers a row, a wave reads two neurons' rows at once
        using P = RowPass<B, GATED, WT>;
        const int cnt = __builtin_popcount(word);
        const bool pairs = P::extent(a.d) <= P::STEP;
        for (int j = wave; j < cnt; j += pairs ? 8 : 4) {
            const int j2 = j + 4;
            const bool two = pairs && j2 < cnt;
            int bit = 0, bit2 = 0;
            {
                uint32_t bits = word;
                for (int q = 0; q < j; ++q) bits &= bits - 1;
                bit = __builtin_ctz(bits);
                if (two) {
                    for (int q = j; q < j2; ++q) bits &= bits - 1;
                    bit2 = __builtin_ctz(bits);
                }
            }
            const int s = s_slot[bit], s2 = two ? s_slot[bit2] : 0;
            float ag[B], au[B], ag2[B], au2[B];
#pragma unroll
            for (int b = 0; b < B; ++b) ag[b] = au[b] = ag2[b] = au2[b] = 0.f;
            if (pairs) {
                // (a missing second neuron reads nothing: its extent is 0)
                const int d2 = two ? a.d : 0;
                P p1, p2;
                p1.issue_buf(rin, (uint32_t)(s * in_stride), a.row_bytes, a.d, 0, lane);
                p2.issue_buf(rin, (uint32_t)(s2 * in_stride), a.row_bytes, d2, 0, lane);
                p1.consume(xs, a.d, a.d, 0, lane, ag, au);
                p2.consume(xs, a.d, d2, 0, lane, ag2, au2);
            } else {
                neuron_dots<B, GATED, WT>(a.w_in + (int64_t)s * in_stride, a.row_bytes, a.d, xs, a.d, lane, ag, au);
            }
            if (t == (int)blockIdx.x && j == wave) TAIL_TRACE(6, wall_clock64() + (ag[0] == 1e30f) + (au[0] == 1e30f));
            tail_publish<B, GATED>(a, t * 32 + bit, s, ag, au, stamp, lane);
            if (two) tail_publish<B, GATED>(a, t * 32 + bit2, s2, ag2, au2, stamp, lane);
        }
        __syncthreads();                               // s_words / s_slot are reused by the next tile
    }
}

// ------------------------------------------------------------------------------ down tiles

template <int B, int WT>
__device__ __forceinline__ void tail_down(const TailArgs &a, uint32_t stamp, int lane, int wave, int e, float *s_red, int *s_list,
                          int *s_cnt, float *s_own) {
    constexpr int CPL = kTailCPL, SLAB = kTailSlab;
    constexpr int U = 32;                               // rows in flight per wave
    constexpr int TPR = kTailListMax / 32;              // neuron tiles per round (one per lane)
    static_assert(TPR <= kWave, "one lane per tile");
    const int slab = e % a.slabs, ck = e / a.slabs;
    const int T0 = (int)((int64_t)a.NTL * ck / a.C), T1 = (int)((int64_t)a.NTL * (ck + 1) / a.C);
    const int col = slab * SLAB + lane * CPL;
    const bool colok = col < a.d;
    const __amdgpu_buffer_rsrc_t rdn = buf_rsrc(a.w_dn, (uint32_t)(a.n_slots * a.row_bytes));
    float acc[B][CPL];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < CPL; ++t) acc[b][t] = 0.f;

    for (int tb = T0; tb < T1; tb += TPR) {
        // wave 0 polls the round's tile words (one lane per tile) and lists the listed neurons
        if (wave == 0) {
            const int tt = tb + lane;
            const bool mine = lane < TPR && tt < T1;
            uint64_t w1[1];
            poll_words<1>(mine ? a.tword + tt : nullptr, stamp, a.ctl, lane, 16, w1);
            // only ids < f can be listed (a word left by an aborted wait is masked the same way)
            const int valid = mine ? min(32, a.f - tt * 32) : 0;
            const uint32_t word = mine ? (uint32_t)w1[0] & (valid >= 32 ? 0xFFFFFFFFu : ((1u << valid) - 1u)) : 0u;
            const int c = __builtin_popcount(word);
            const int incl = wave_incl_scan(c);
            int pos = incl - c;
            for (uint32_t bits = word; bits && pos < kTailListMax; bits &= bits - 1) s_list[pos++] = tt * 32 + __builtin_ctz(bits);
            if (lane == kWave - 1) *s_cnt = incl;
            if (tb == T0) TAIL_TRACE(2, wall_clock64());
        }
        __syncthreads();
        const int L = __builtin_amdgcn_readfirstlane(*s_cnt);
        // wave w takes list entries w, w + 4, ...: lane j of a round holds entry base + 4j
        for (int base = wave; base < L; base += 4 * kWave) {
            const int m = min(kWave, (L - base + 3) / 4);
            const int k = base + 4 * lane;
            const int id = lane < m ? s_list[k] : 0;
            const int s = lane < m ? slot_of_id(id, a.slot_of, a.f, a.n_slots) : -1;
            float hv[B];
            // byte offset of the row of the lane's entry (kOOB: none), and of this lane's columns
            const uint32_t rowoff = (lane < m && s >= 0) ? (uint32_t)s * (uint32_t)a.row_bytes : kOOB;
            const uint32_t cpart = colok ? (WT == WT_F16 ? (uint32_t)col * 2 : (uint32_t)col / 2) : kOOB;
            const uint32_t spart = colok ? (uint32_t)(a.d / 2) + (uint32_t)(col / 32) * 2 : kOOB;
            for (int j0 = 0; j0 < m; j0 += U) {
                uint4 wf[WT == WT_F16 ? U : 1];
                uint32_t wq[WT == WT_Q4_0 ? U : 1];
                uint16_t sq[WT == WT_Q4_0 ? U : 1];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t ro = (uint32_t)__builtin_amdgcn_readlane((int)rowoff, j0 + u);
                    if (WT == WT_F16) {
                        wf[WT == WT_F16 ? u : 0] = bld16(rdn, ro + cpart);
                    } else {
                        wq[WT == WT_Q4_0 ? u : 0] = bld4(rdn, ro + cpart);
                        sq[WT == WT_Q4_0 ? u : 0] = bld2(rdn, ro + spart);
                    }
                }
                if (j0 == 0) {
                    if (tb == T0 && base == 0) TAIL_TRACE(3, wall_clock64());
                    uint64_t hw[B];
                    poll_words<B>(lane < m ? a.ent + (size_t)id * (1 + B) + 1 : nullptr, stamp, a.ctl, lane, 2, hw);
#pragma unroll
                    for (int b = 0; b < B; ++b) hv[b] = lane < m ? word_f(hw[b]) : 0.f;
                    if (tb == T0 && base == 0) TAIL_TRACE(4, wall_clock64());
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int j = j0 + u;
                    if (j >= m) break;
                    float hb[B];
                    bool any = false;
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        hb[b] = bcastf(hv[b], j);
                        any |= hb[b] != 0.f;
                    }
                    if (!any) continue;                 // h = 0 for every token: adds exact zeros
                    if (WT == WT_F16) {
                        const uint4 w = wf[WT == WT_F16 ? u : 0];
                        const uint32_t wq4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const h2 pr = __builtin_bit_cast(h2, wq4[p]);
                            const float lo = (float)pr.x, hi = (float)pr.y;
#pragma unroll
                            for (int b = 0; b < B; ++b) {
                                acc[b][2 * p] = fmaf(hb[b], lo, acc[b][2 * p]);
                                acc[b][2 * p + 1] = fmaf(hb[b], hi, acc[b][2 * p + 1]);
                            }
                        }
                    } else {
                        const float scf = half_to_float(sq[WT == WT_Q4_0 ? u : 0]);
                        const uint32_t cw = wq[WT == WT_Q4_0 ? u : 0];
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const h2 pr = __builtin_bit_cast(h2, q4pair(cw, 4 * p));
                            const float lo = (float)pr.x, hi = (float)pr.y;
#pragma unroll
                            for (int b = 0; b < B; ++b) {
                                const float cf = hb[b] * scf;
                                acc[b][p] = fmaf(cf, lo, acc[b][p]);
                                acc[b][p + 4] = fmaf(cf, hi, acc[b][p + 4]);
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();                                // s_list / s_cnt are rewritten next round
    }

    // Reduction, scattered over the slab's tiles: the 4 waves meet in LDS, the tile stores its
    // stamped chunk partial, then tile ck finishes columns [ck*W, (ck+1)*W) of the slab: it polls
    // those columns' partials of every chunk, sums them in chunk order (its own from LDS), adds
    // b_down and writes y.  No ticket and no single workgroup reading the whole slab.
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < CPL; ++t) s_red[((wave * B + b) * CPL + t) * kWave + lane] = acc[b][t];
    __syncthreads();
    TAIL_TRACE(5, wall_clock64());
    const int Bd = B * a.d;
    for (int o = threadIdx.x; o < B * SLAB; o += blockDim.x) {
        const int b = o / SLAB, cc = o - b * SLAB;
        const int ln = cc / CPL, t = cc - ln * CPL;
        const int gcol = slab * SLAB + cc;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) sum += s_red[((w * B + b) * CPL + t) * kWave + ln];
        s_own[o] = sum;
        if (gcol < a.d) store_c64(a.part + (size_t)ck * Bd + (size_t)b * a.d + gcol, stamped_f(sum, stamp));
    }
    __syncthreads();
    TAIL_TRACE(6, wall_clock64());
    const int W = (SLAB + a.C - 1) / a.C;              // columns this tile finishes
    const int c0 = ck * W, nc = max(0, min(W, SLAB - c0));
    const int nout = B * nc;
    for (int o0 = 0; o0 < nout; o0 += blockDim.x) {    // one output (token, column) per thread
        const int o = o0 + threadIdx.x;
        const int b = o / nc, cc = c0 + (o - b * nc);
        const int gcol = slab * SLAB + cc;
        const bool ok = o < nout && gcol < a.d;
        const size_t off = (size_t)b * a.d + (ok ? gcol : 0);
        const float bd = (ok && a.b_down != nullptr) ? half_to_float(a.b_down[gcol]) : 0.f;
        uint64_t v[kSparseMaxChunks];
#pragma unroll
        for (int c = 0; c < kSparseMaxChunks; ++c)
            v[c] = (ok && c < a.C && c != ck) ? load_c64(a.part + (size_t)c * Bd + off) : stamped(0u, stamp);
        float bdv = bd;
        asm volatile("" : "+v"(bdv));                  // b_down arrives with the first partials
        const uint64_t t0 = wall_clock64();
        for (;;) {
            bool stale = false;
#pragma unroll
            for (int c = 0; c < kSparseMaxChunks; ++c) stale |= !fresh(v[c], stamp);
            if (__syncthreads_or(stale) == 0) break;
            // the abort word and the stale partials go out together: one round trip per poll
            const int ab = threadIdx.x == 0 ? load_coherent_i(a.ctl + CTL_ABORT) : 0;
#pragma unroll
            for (int c = 0; c < kSparseMaxChunks; ++c)
                if (!fresh(v[c], stamp)) v[c] = load_c64(a.part + (size_t)c * Bd + off);
            if (__syncthreads_or(ab)) break;
            if (wall_clock64() - t0 > kSpinTicks) {
                if (threadIdx.x == 0) {
                    store_coherent_i(a.ctl + CTL_ABORT, 1);
                    atomicOr(a.ctl + CTL_STATUS, 4);
                }
                break;
            }
        }
        if (o0 == 0) TAIL_TRACE(7, wall_clock64());
        if (ok) {
            float sum = 0.f;
#pragma unroll
            for (int c = 0; c < kSparseMaxChunks; ++c)
                if (c < a.C) sum += c == ck ? s_own[b * SLAB + cc] : word_f(v[c]);
            a.y[off] = sum + bdv;
        }
    }
    TAIL_TRACE(8, wall_clock64());
}

// ------------------------------------------------------------------------------ the kernel

template <int B, bool GATED, int WT, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_layer_tail(TailArgs a) {
    extern __shared__ __align__(16) uint16_t dyn[];
    __shared__ float s_red[4 * B * kTailCPL * kWave];
    __shared__ float s_own[B * kTailSlab];
    __shared__ int s_list[kTailListMax];
    __shared__ uint32_t s_words[4];
    __shared__ int s_slot[32];
    __shared__ int s_cnt;
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    TAIL_TRACE(1, wall_clock64());
    const uint32_t stamp = (uint32_t)load_coherent_i(a.ctl + CTL_EPOCH) + 1u;
    const bool up = (int)blockIdx.x < a.PU;
    if (up) {
        P2Tile<B, NT> pt;
        if ((int)blockIdx.x < a.NTL) pt.issue(a, blockIdx.x, wave, lane);      // before anything else
        uint16_t *xs = dyn;
        float *zs = reinterpret_cast<float *>(dyn + ((size_t)B * a.d + 7) / 8 * 8);
        stage_x<B, WT == WT_Q4_0>(xs, a.x, a.d, 0, a.d, a.d);
        stage_vec16(zs, a.z, B * a.r / 4);
        __syncthreads();
        TAIL_TRACE(2, wall_clock64());
        tail_up<B, GATED, WT, NT>(a, stamp, lane, wave, xs, zs, s_words, s_slot, pt);
    } else {
        tail_down<B, WT>(a, stamp, lane, wave, blockIdx.x - a.PU, s_red, s_list, &s_cnt, s_own);
    }
    TAIL_TRACE(0, up ? 1 : 2);
    TAIL_TRACE(9, wall_clock64());
    persistent_exit(a.ctl, stamp, a.PU + a.NE);   // the last workgroup out advances the epoch
}

// Launch of the tail kernel for batch width B (one translation unit per B); PU and C come from
// the device's occupancy so that every workgroup is resident at once.
template <int B>
int launch_tail_batch(TailArgs &a, int wtype, int gated, int NT, hipStream_t st);
template <> int launch_tail_batch<1>(TailArgs &, int, int, int, hipStream_t);
template <> int launch_tail_batch<2>(TailArgs &, int, int, int, hipStream_t);
template <> int launch_tail_batch<3>(TailArgs &, int, int, int, hipStream_t);
template <> int launch_tail_batch<4>(TailArgs &, int, int, int, hipStream_t);
template <> int launch_tail_batch<5>(TailArgs &, int, int, int, hipStream_t);
template <> int launch_tail_batch<6>(TailArgs &, int, int, int, hipStream_t);
template <> int launch_tail_batch<7>(TailArgs &, int, int, int, hipStream_t);
template <> int launch_tail_batch<8>(TailArgs &, int, int, int, hipStream_t);

}  // namespace pik
