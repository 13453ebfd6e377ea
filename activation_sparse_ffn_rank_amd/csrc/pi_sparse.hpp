// pi_sparse.hpp -- the neuron-aware sparse FFN over a device-side list of neurons as ONE
// persistent kernel (PowerInfer, arXiv 2312.12456, method section: operators that compute only
// the neurons predicted to fire, reading each neuron's weights as one contiguous row).
//
// For list positions k < n (n read from the device), slot s_k of neuron idx[k]:
//   h[b][k] = max(0, W_up[s_k] x_b + b_up[s_k])  or  max(0, W_gate[s_k] x_b) * (W_up[s_k] x_b)
//   y[b]    = b_down + sum_k h[b][k] W_down^T[s_k]
//
// Two kinds of workgroups share the launch, and all of them are resident at once:
//   up    (blockIdx < PD)  wave w of workgroup j takes positions 4j + w, 4(j + PD) + w, ...: it
//                          reads the neuron's input row(s) against x staged in LDS and publishes
//                          its slot and h as stamped words.
//   down  (NE = slabs * C) tile (column slab, chunk of the list): it looks up its positions' slots
//                          and issues the loads of their W_down^T rows, restricted to its columns,
//                          BEFORE h is known -- so the down rows stream while the up rows do --
//                          then polls h, accumulates, and stores its stamped chunk partial; each
//                          tile of a slab then finishes 1/C of the slab's columns, summing the C
//                          partials in chunk order, adding b_down and writing y.  Every result
//                          is independent of timing.
// Reading the down rows before h is known means rows whose h is zero for every token are read
// too (their products are skipped); it removes a dependent HBM round trip from the critical path.
//
// Hand-offs use the stamped-word protocol of pi_fused.hpp (agent-coherent 64-bit stores carrying
// the launch's stamp; consumers re-read stale words; bounded waits raise an abort flag and a
// sticky status word).  The workspace must be zero-filled before its first use.
#pragma once

#include "pi_fused.hpp"

namespace pik {

constexpr int kSparseMaxChunks = 16;           // chunk partials per slab

// Columns of one down tile: 64 lanes x CPL columns (fp16: 4 per lane, one 8-byte load per row;
// Q4_0: 8 per lane, one 4-byte code word and one scale per row).
template <int WT>
struct DownCols {
    static constexpr int CPL = WT == WT_F16 ? 4 : 8;
    static constexpr int SLAB = CPL * kWave;
};

__host__ __device__ inline int sparse_slab_cols(int wt) {
    return wt == WT_F16 ? DownCols<WT_F16>::SLAB : DownCols<WT_Q4_0>::SLAB;
}
__host__ __device__ inline int sparse_slabs(int d, int wt) { return (d + sparse_slab_cols(wt) - 1) / sparse_slab_cols(wt); }

struct SparseArgs {
    int d, f, n_slots, slabs, C, PD, NE;
    int act;             // 1: squared ReLU (non-gated)
    int64_t row_bytes;
    const uint8_t *w_in, *w_dn;
    const uint16_t *b_up, *b_down;
    const int32_t *slot_of;
    const uint16_t *x;
    float *y;
    const int32_t *idx, *counts;
    int32_t *ctl;        // control block (epoch, exit count, abort, status)
    uint64_t *ent;       // [n_slots][1 + B]: slot, then h per token, stamped
    uint64_t *part;      // [C][B][d] chunk partials, stamped
#ifdef PIK_TRACE
    uint64_t *trace;     // [P][8]: kind, entry, dependency met, exit, up: idx known, row dots done, x staged
#endif
};

// Wave-wide: load the W words p[0..W) of each lane (p == nullptr: nothing, counts as fresh) and
// re-read the stale ones until every lane holds current words (or the wait gives up).
template <int W>
__device__ __forceinline__ void poll_words(const uint64_t *p, uint32_t stamp, int32_t *ctl, int lane, int code,
                                           uint64_t (&w)[W]) {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = p ? load_c64(p + i) : stamped(0u, stamp);
    const uint64_t t0 = wall_clock64();
    for (;;) {
        bool stale = false;
#pragma unroll
        for (int i = 0; i < W; ++i) stale |= !fresh(w[i], stamp);
        if (__ballot(stale) == 0) break;
        // the abort word and the stale words go out together: one round trip per poll
        const int ab = lane == 0 ? load_coherent_i(ctl + CTL_ABORT) : 0;
#pragma unroll
        for (int i = 0; i < W; ++i)
            if (!fresh(w[i], stamp)) w[i] = load_c64(p + i);
        if (poll_stop(ab, t0, ctl, lane, code)) break;
    }
}

// ------------------------------------------------------------------------------ up workgroups

template <int B, bool GATED, int WT>
__device__ void sparse_up(const SparseArgs &a, int n, uint32_t stamp, int lane, int wave, uint16_t *xs) {
    const int64_t in_stride = GATED ? 2 * a.row_bytes : a.row_bytes;
    for (int k0 = blockIdx.x * 4; k0 < n; k0 += a.PD * 4) {
        const int k = k0 + wave;
        if (k >= n) continue;
        const int s = slot_of_id(a.idx[k], a.slot_of, a.f, a.n_slots);
#ifdef PIK_TRACE
        if (a.trace != nullptr && threadIdx.x == 0 && k0 == (int)blockIdx.x * 4) a.trace[(size_t)blockIdx.x * 8 + 4] = wall_clock64() + (s < -5 ? 1 : 0);
#endif
        float ag[B], au[B];
#pragma unroll
        for (int b = 0; b < B; ++b) ag[b] = au[b] = 0.f;
        if (s >= 0) neuron_dots<B, GATED, WT>(a.w_in + (int64_t)s * in_stride, a.row_bytes, a.d, xs, a.d, lane, ag, au);
#ifdef PIK_TRACE
        if (a.trace != nullptr && threadIdx.x == 0 && k0 == (int)blockIdx.x * 4) a.trace[(size_t)blockIdx.x * 8 + 5] = wall_clock64() + (ag[0] == 1e30f ? 1 : 0) + (au[0] == 1e30f ? 1 : 0);
#endif
        const float bias = (!GATED && a.b_up != nullptr && s >= 0) ? half_to_float(a.b_up[s]) : 0.f;
        uint64_t *e = a.ent + (size_t)k * (1 + B);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float u = wave_sum(au[b]);
            float hv;
            if (GATED) {
                const float gv = wave_sum(ag[b]);
                hv = fmaxf(gv, 0.f) * u;
            } else {
                hv = fmaxf(u + bias, 0.f);
                if (a.act) hv *= hv;                    // squared ReLU
            }
            if (lane == 0) store_c64(e + 1 + b, stamped_f(s >= 0 ? hv : 0.f, stamp));
        }
        if (lane == 0) store_c64(e, stamped((uint32_t)s, stamp));
    }
}

// ------------------------------------------------------------------------------ down tiles

template <int B, int WT>
__device__ void sparse_down(const SparseArgs &a, int n, uint32_t stamp, int lane, int wave, int e, float *s_red) {
    using DC = DownCols<WT>;
    constexpr int CPL = DC::CPL, SLAB = DC::SLAB;
    constexpr int U = 32;                               // rows in flight per wave
    const int slab = e % a.slabs, ck = e / a.slabs;
    const int p0 = (int)((int64_t)n * ck / a.C), p1 = (int)((int64_t)n * (ck + 1) / a.C);
    const int col = slab * SLAB + lane * CPL;
    const bool colok = col < a.d;
    // This lane's bytes of any row (a lane past d reads column 0 and never stores it): the loads
    // below are unconditional, so that the compiler issues all U of them before the first use.
    const int cc = colok ? col : 0;
    const uint8_t *wcol = a.w_dn + (WT == WT_F16 ? (int64_t)cc * 2 : (int64_t)cc / 2);
    const uint8_t *wsc = a.w_dn + a.d / 2 + (cc / 32) * 2;
    float acc[B][CPL];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < CPL; ++t) acc[b][t] = 0.f;

    // wave w takes positions p0 + w, p0 + w + 4, ...: lane j of a round holds position base + 4j
    for (int base = p0 + wave; base < p1; base += 4 * kWave) {
        const int m = min(kWave, (p1 - base + 3) / 4);  // lanes 0..m-1 hold a position
        const int k = base + 4 * lane;
        const int s = lane < m ? slot_of_id(a.idx[k], a.slot_of, a.f, a.n_slots) : -1;
        const int sr = s >= 0 ? s : 0;                  // an absent row reads row 0; its h is 0
        float hv[B];
        for (int j0 = 0; j0 < m; j0 += U) {
            // loads of the next U rows (restricted to this tile's columns) go out first
            uint2 wf[WT == WT_F16 ? U : 1];
            uint32_t wq[WT == WT_Q4_0 ? U : 1];
            uint16_t sq[WT == WT_Q4_0 ? U : 1];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t ro = (int64_t)__builtin_amdgcn_readlane(sr, j0 + u) * a.row_bytes;
                if (WT == WT_F16) {
                    wf[WT == WT_F16 ? u : 0] = *reinterpret_cast<const uint2 *>(wcol + ro);
                } else {
                    wq[WT == WT_Q4_0 ? u : 0] = *reinterpret_cast<const uint32_t *>(wcol + ro);
                    sq[WT == WT_Q4_0 ? u : 0] = *reinterpret_cast<const uint16_t *>(wsc + ro);
                }
            }
            if (j0 == 0) {
                // h of the round's positions, one lane per position
                uint64_t hw[B];
                poll_words<B>(lane < m ? a.ent + (size_t)k * (1 + B) + 1 : nullptr, stamp, a.ctl, lane, 2, hw);
#pragma unroll
                for (int b = 0; b < B; ++b) hv[b] = (s >= 0) ? word_f(hw[b]) : 0.f;
#ifdef PIK_TRACE
                if (a.trace != nullptr && threadIdx.x == 0 && base == p0) a.trace[(size_t)blockIdx.x * 8 + 2] = wall_clock64();
#endif
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
                if (!any) continue;                     // h = 0 for every token: adds exact zeros
                if (WT == WT_F16) {
                    const uint2 w = wf[WT == WT_F16 ? u : 0];
                    const h2 w01 = __builtin_bit_cast(h2, w.x), w23 = __builtin_bit_cast(h2, w.y);
                    const float wv[4] = {(float)w01.x, (float)w01.y, (float)w23.x, (float)w23.y};
#pragma unroll
                    for (int b = 0; b < B; ++b)
#pragma unroll
                        for (int t = 0; t < 4; ++t) acc[b][t] = fmaf(hb[b], wv[t], acc[b][t]);
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
#ifdef PIK_TRACE
    if (a.trace != nullptr && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * 8 + 4] = wall_clock64() + (acc[0][0] == 1e30f ? 1 : 0);
#endif

    // Reduction, scattered over the slab's tiles: the 4 waves meet in LDS, the tile stores its
    // stamped chunk partial, then tile ck finishes columns [ck*W, (ck+1)*W) of the slab: it polls
    // those columns' partials of every other chunk, sums all C in chunk order (its own from LDS),
    // adds b_down and writes y.  The tile's own partial of (token b, column ln*CPL + t) is kept
    // in wave 0's LDS entry for it, which only the thread that sums that entry touches.
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < CPL; ++t) s_red[((wave * B + b) * CPL + t) * kWave + lane] = acc[b][t];
    __syncthreads();
    const int Bd = B * a.d;
    for (int o = threadIdx.x; o < B * SLAB; o += blockDim.x) {
        const int b = o / SLAB, c = o - b * SLAB;
        const int ln = c / CPL, t = c - ln * CPL;
        const int gcol = slab * SLAB + c;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) sum += s_red[((w * B + b) * CPL + t) * kWave + ln];
        s_red[(b * CPL + t) * kWave + ln] = sum;
        if (gcol < a.d) store_c64(a.part + (size_t)ck * Bd + (size_t)b * a.d + gcol, stamped_f(sum, stamp));
    }
    __syncthreads();
#ifdef PIK_TRACE
    if (a.trace != nullptr && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * 8 + 5] = wall_clock64();
#endif
    const int W = (SLAB + a.C - 1) / a.C;              // columns this tile finishes
    const int c0 = ck * W, nc = max(0, min(W, SLAB - c0));
    const int nout = B * nc;
    for (int o0 = 0; o0 < nout; o0 += blockDim.x) {    // one output (token, column) per thread
        const int o = o0 + threadIdx.x;
        const int b = o / max(nc, 1), c = c0 + (o - b * nc);
        const int gcol = slab * SLAB + c;
        const bool ok = o < nout && gcol < a.d;
        const size_t off = (size_t)b * a.d + (ok ? gcol : 0);
        const float bd = (ok && a.b_down != nullptr) ? half_to_float(a.b_down[gcol]) : 0.f;
        uint64_t v[kSparseMaxChunks];
#pragma unroll
        for (int q = 0; q < kSparseMaxChunks; ++q)
            v[q] = (ok && q < a.C && q != ck) ? load_c64(a.part + (size_t)q * Bd + off) : stamped(0u, stamp);
        float bdv = bd;
        asm volatile("" : "+v"(bdv));                  // b_down arrives with the first partials
        const uint64_t t0 = wall_clock64();
        for (;;) {
            bool stale = false;
#pragma unroll
            for (int q = 0; q < kSparseMaxChunks; ++q) stale |= !fresh(v[q], stamp);
            if (__syncthreads_or(stale) == 0) break;
            // the abort word and the stale partials go out together: one round trip per poll
            const int ab = threadIdx.x == 0 ? load_coherent_i(a.ctl + CTL_ABORT) : 0;
#pragma unroll
            for (int q = 0; q < kSparseMaxChunks; ++q)
                if (!fresh(v[q], stamp)) v[q] = load_c64(a.part + (size_t)q * Bd + off);
            if (__syncthreads_or(ab)) break;
            if (wall_clock64() - t0 > kSpinTicks) {
                if (threadIdx.x == 0) {
                    store_coherent_i(a.ctl + CTL_ABORT, 1);
                    atomicOr(a.ctl + CTL_STATUS, 4);
                }
                break;
            }
        }
#ifdef PIK_TRACE
        if (a.trace != nullptr && threadIdx.x == 0 && o0 == 0) a.trace[(size_t)blockIdx.x * 8 + 6] = wall_clock64();
#endif
        if (ok) {
            const int ln = c / CPL, t = c - ln * CPL;
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < kSparseMaxChunks; ++q)
                if (q < a.C) sum += q == ck ? s_red[(b * CPL + t) * kWave + ln] : word_f(v[q]);
            a.y[off] = sum + bdv;
        }
    }
}

// ------------------------------------------------------------------------------ the kernel

template <int B, bool GATED, int WT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(B <= 2 ? 3 : 2))) void k_sparse_ffn(SparseArgs a) {
    extern __shared__ __align__(16) uint16_t xs[];              // x [B][d] (q4-paired for Q4_0), up only
    __shared__ float s_red[4 * B * DownCols<WT>::CPL * kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
#ifdef PIK_TRACE
    if (a.trace != nullptr && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * 8 + 1] = wall_clock64();
#endif
    const uint32_t stamp = (uint32_t)load_coherent_i(a.ctl + CTL_EPOCH) + 1u;
    const int n = __builtin_amdgcn_readfirstlane(min(max(a.counts[0], 0), a.n_slots));
    const bool up = (int)blockIdx.x < a.PD;
    if (up) {
        stage_x<B, WT == WT_Q4_0>(xs, a.x, a.d, 0, a.d, a.d);
        __syncthreads();
#ifdef PIK_TRACE
        if (a.trace != nullptr && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * 8 + 6] = wall_clock64() + (n < -5 ? 1 : 0);
#endif
        sparse_up<B, GATED, WT>(a, n, stamp, lane, wave, xs);
    } else {
        sparse_down<B, WT>(a, n, stamp, lane, wave, blockIdx.x - a.PD, s_red);
    }
#ifdef PIK_TRACE
    if (a.trace != nullptr && threadIdx.x == 0) {
        a.trace[(size_t)blockIdx.x * 8 + 0] = up ? 1 : 2;
        a.trace[(size_t)blockIdx.x * 8 + 3] = wall_clock64();
    }
#endif
    // leave: the last workgroup out advances the epoch
    __syncthreads();
    if (threadIdx.x == 0) {
        if (atomicAdd(a.ctl + CTL_EXIT, 1) == a.PD + a.NE - 1) {
            store_coherent_i(a.ctl + CTL_ABORT, 0);
            store_coherent_i(a.ctl + CTL_EXIT, 0);
            store_coherent_i(a.ctl + CTL_EPOCH, (int32_t)stamp);
        }
    }
}

// Launch of the sparse-FFN kernel for batch width B (one translation unit per B).  Picks PD and C
// from the device's occupancy so that every workgroup is resident at once.
template <int B>
int launch_sparse_batch(SparseArgs &a, int wtype, int gated, hipStream_t st);
template <> int launch_sparse_batch<1>(SparseArgs &, int, int, hipStream_t);
template <> int launch_sparse_batch<2>(SparseArgs &, int, int, hipStream_t);
template <> int launch_sparse_batch<3>(SparseArgs &, int, int, hipStream_t);
template <> int launch_sparse_batch<4>(SparseArgs &, int, int, hipStream_t);
template <> int launch_sparse_batch<5>(SparseArgs &, int, int, hipStream_t);
template <> int launch_sparse_batch<6>(SparseArgs &, int, int, hipStream_t);
template <> int launch_sparse_batch<7>(SparseArgs &, int, int, hipStream_t);
template <> int launch_sparse_batch<8>(SparseArgs &, int, int, hipStream_t);

}  // namespace pik
