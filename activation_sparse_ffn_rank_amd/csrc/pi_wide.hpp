// pi_wide.hpp -- the neuron-aware sparse FFN at batches of up to 16 tokens, on MFMA.
//
// The sparse operator of the method (PowerInfer, arXiv 2312.12456, method section: only the
// predicted neurons' rows are read and computed) is, at a batch of B tokens, a contraction over
// the gathered rows: H = act(X W_in[idx]^T + b) is [B x n], Y = H W_down^T[idx] is [B x d].  The
// GEMV kernels of pi_kernels.hpp spend vector-ALU work per weight that grows with B (at B = 16 the
// down step alone needs 16 FMAs per fp16 weight: 64 T FMA/s at 8 TB/s, most of the vector ALU's
// 78.6 T), so here both steps run on v_mfma_f32_16x16x16_f16 tiles with the batch padded to 16
// (tokens >= B read as zero and are never stored); pi_sparse_ffn uses these kernels from batch 3
// for gated or Q4_0 rows and from batch 6 for plain fp16 rows.
//
// Operand layout of a 16x16x16 f16 MFMA (wave64): lane l supplies A[m = l%16][k = 4(l/16)+v] and
// B[k = 4(l/16)+v][n = l%16] for v < 4, and receives D[m = 4(l/16)+v][n = l%16].  A contraction
// may assign its k indices to (lane group, v) slots in any order as long as A and B agree, which
// the kernels use to make every lane's loads contiguous.
//
// Kernels (stream-ordered):
//   k_wide_xmf   x copied once into the A-operand order of the up step's MFMAs (Q4_0 rows; fp16 rows
//                past 8 tokens or when the predictor's grid does it), so that each of the up step's
//                x loads is one contiguous 1 KB run for the wave (read in place, the 16 tokens'
//                rows made every load touch 16 to 32 cache lines).
//   k_wide_up    one workgroup per 16 listed neurons: H tile [16 tokens x 16 neurons] over all d,
//                the eight waves taking interleaved 256-column blocks, summed in LDS; writes h
//                as fp16 hi + fp16 lo parts (h = hi + lo to ~2^-22 relative), so that feeding h to
//                the f16 MFMA of the down step costs no accuracy.  On Q4_0 rows k_wide_up_q4 does
//                the same on one workgroup per compute unit, each taking an even run of tiles.
//   k_wide_down  (slab, neuron chunk) tiles: Y tile [16 tokens x 128 (Q4_0: 256) columns] over the
//                chunk's neurons, waves summed in LDS, chunk partials summed in chunk order by the
//                last workgroup of each slab (deterministic), plus b_down.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pi_kernels.hpp"

namespace pik {

constexpr int kWideB = 16;            // the padded batch: one MFMA M (or N) dimension
constexpr int kWideUpCols = 256;      // columns per k_wide_up block (8 column groups of 32)
constexpr int kStatusHRange = 64;     // status bit: some |h| reached 65504 (outside the fp16 pair)
// columns per lane per row in k_wide_down (a slab is 16 lanes wide)
constexpr int wide_down_cpl(int wt) { return wt == WT_Q4_0 ? 16 : 8; }
constexpr int kWideMaxChunks = 16;    // chunk partials per slab summed by the last workgroup
constexpr int kWideWaves = 8;         // waves per workgroup of k_wide_up
constexpr int kWideDownWaves = 12;    // ... and of k_wide_down
constexpr int kWideThreads = kWideWaves * kWave;

typedef f16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f4 c) {
    const h4 a = __builtin_bit_cast(h4, make_uint2(a0, a1));
    const h4 b = __builtin_bit_cast(h4, make_uint2(b0, b1));
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// x in k_wide_up's Q4_0 operand order: 16-byte vector ((kq*4 + i)*4 + g)*16 + r holds tokens r's
// columns 32(4kq + g) + 8i .. +8, re-paired for q4pair (pair_for_q4), or zeros for a token r >= B;
// 2d vectors (d*32 bytes), one thread each.  Lane r + 16g of a wave then reads the vectors of block
// 4kq + g for its token r: a wave's load for one (kq, i) is 64 consecutive vectors.
__device__ __forceinline__ void wide_xmf_vec(const uint16_t *__restrict__ x, int B, int d, uint4 *__restrict__ xmf,
                                             int v) {
    const int kq = v >> 8, i = (v >> 6) & 3, g = (v >> 4) & 3, r = v & 15;
    xmf[v] = r < B ? pair_for_q4(ld16(x + (size_t)r * d + (4 * kq + g) * 32 + 8 * i)) : zero4();
}
// The fp16-row counterpart: vector 64*k + L holds token L%16's columns 32k + 8(L/16) .. +8 (zeros for
// a token >= B or columns past d), the A operand of k_wide_up's step k; 64*ceil(d/32) vectors.
__device__ __forceinline__ void wide_xf16_vec(const uint16_t *__restrict__ x, int B, int d, uint4 *__restrict__ xmf,
                                              int v) {
    const int k = v >> 6, r = v & 15, col = 32 * k + 8 * ((v >> 4) & 3);
    xmf[v] = (r < B && col < d) ? ld16(x + (size_t)r * d + col) : zero4();
}
// Vectors of the layout for either row kind (Q4_0: 2d; fp16: 64*ceil(d/32)).
__host__ __device__ inline int wide_xmf_vectors(int d, bool q4) { return q4 ? 2 * d : 64 * ((d + 31) / 32); }

__global__ __launch_bounds__(256) void k_wide_xmf(const uint16_t *__restrict__ x, int B, int d, int q4,
                                                  uint4 *__restrict__ xmf) {
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v < wide_xmf_vectors(d, q4 != 0)) {
        if (q4) wide_xmf_vec(x, B, d, xmf, v);
        else wide_xf16_vec(x, B, d, xmf, v);
    }
}

// The table of h that the up kernels hand to k_wide_down, in the down step's operand order: for
// list position k and token b, the 16-byte unit (k/4)*16 + b holds the fp16 hi parts of positions
// 4(k/4) .. +3 of token b, then their lo parts (h = hi + lo to ~2^-22 relative).  A wave of the down
// kernel then reads one contiguous 1 KB run per step (lane 16g + r: positions 4g .. 4g+3 of the
// step, token r).  hs (positions, a multiple of 32) * 64 bytes.
__device__ __forceinline__ void wide_h_store(uint16_t *__restrict__ hl, int b, int k, float hv) {
    const f16 hi = (f16)hv;
    const f16 lo = (f16)(hv - (float)hi);
    uint16_t *u = hl + ((size_t)(k >> 2) * 16 + b) * 8 + (k & 3);
    u[0] = __builtin_bit_cast(uint16_t, hi);
    u[4] = __builtin_bit_cast(uint16_t, lo);
}

// h[b][k] for the listed neurons, as fp16 hi and lo parts in the table above.  Workgroup t holds
// list positions 16t .. 16t+15; lane l of every wave works on position 16t + l%16 and token l%16
// (the MFMA's n and m) and columns blk + 32j + 8(l/16) .. +8 of block blk (j < 8), so each of a
// row's 16-byte loads is contiguous with the next lane group's.  Row loads are unconditional (slot
// 0, column 0 stand in for an absent neuron or a column past d, and the value is zeroed), so all
// of a block's loads are in flight together; x is read through a buffer resource (a token >= B or
// a column past d reads zero).  Workgroup 0 also clears `zero_ptr[0..nzero)` (the down kernel's
// slab tickets); the down kernel always runs after this one on the same stream.
template <bool GATED, int WT, int NT, int W = kWideWaves>
__global__ __launch_bounds__(W * kWave) void k_wide_up(const uint8_t *__restrict__ w_in, int64_t row_bytes, int d,
                                                 const uint16_t *__restrict__ b_up, const uint16_t *__restrict__ x,
                                                 const uint4 *__restrict__ xmf, int B, const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ counts,
                                                 const int32_t *__restrict__ slot_of, int f, int n_slots,
                                                 uint16_t *__restrict__ hl, int hs,
                                                 int32_t *__restrict__ zero_ptr, int nzero, int act,
                                                 int32_t *__restrict__ status) {
    __shared__ f4 red[GATED ? 2 : NT][W][kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    if (blockIdx.x == 0)
        for (int t = tid; t < nzero; t += blockDim.x) zero_ptr[t] = 0;
    const int n = min(max(counts[0], 0), n_slots);
    const int t0 = blockIdx.x * 16 * NT;
    if (t0 >= n) return;                                         // workgroup-uniform
    const int r = lane & 15, g = lane >> 4;
    int sl[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int pu = t0 + 16 * u + r;
        sl[u] = pu < n ? slot_of_id(idx[pu], slot_of, f, n_slots) : -1;
    }
    const int s = sl[0];
    const int pos = t0 + r;
    const int64_t stride = row_bytes * (GATED ? 2 : 1);
    const uint8_t *row = w_in + (int64_t)(s >= 0 ? s : 0) * stride;
    const __amdgpu_buffer_rsrc_t xr = buf_rsrc(x, (uint32_t)B * (uint32_t)d * 2u);
    const uint32_t xrow = r < B ? (uint32_t)r * (uint32_t)d * 2u : kOOB;
    f4 au = {0.f, 0.f, 0.f, 0.f}, ag = {0.f, 0.f, 0.f, 0.f};
    f4 aq[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) aq[u] = f4{0.f, 0.f, 0.f, 0.f};
    for (int blk = wave * kWideUpCols; WT == WT_Q4_0 && blk < d; blk += W * kWideUpCols) {
        // Q4_0 (d % 256 == 0, so every block of the 256 columns exists): lane group g takes the
        // 32-weight blocks blk/32 + g + 4j (j < 2) of each of its NT rows, one 16-byte code load and
        // one scale each; the codes become exact fp16 (code - 8) pairs, times the block's scale (one
        // fp16 rounding), and x -- read once for the NT rows, from xmf, already re-paired to the
        // codes' order -- feeds two MFMAs per code word
        uint4 cw[NT][2], xq[2][4];
        uint32_t sc[NT][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kb = blk / 32 + g + 4 * j;
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const uint8_t *ru = w_in + (int64_t)(sl[u] >= 0 ? sl[u] : 0) * stride;
                cw[u][j] = ld16(ru + (int64_t)kb * 16);
                sc[u][j] = *reinterpret_cast<const uint16_t *>(ru + d / 2 + (int64_t)kb * 2);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) xq[j][i] = ld16(xmf + ((blk / 128 + j) * 4 + i) * kWave + lane);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 xp = xq[j][q];
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const h2 s2 = __builtin_bit_cast(h2, sl[u] >= 0 ? (sc[u][j] | (sc[u][j] << 16)) : 0u);
                    const uint32_t wd = q == 0 ? cw[u][j].x : q == 1 ? cw[u][j].y : q == 2 ? cw[u][j].z : cw[u][j].w;
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        w[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, q4pair(wd, 4 * p)) * s2);
                    aq[u] = mfma16(xp.x, xp.y, w[0], w[1], aq[u]);
                    aq[u] = mfma16(xp.z, xp.w, w[2], w[3], aq[u]);
                }
            }
        }
    }
    if (WT == WT_Q4_0) au = aq[0];
    for (int blk = wave * kWideUpCols; WT == WT_F16 && blk < d; blk += W * kWideUpCols) {
        uint4 wu[8], wg[8], xv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = blk + 32 * j + 8 * g;
            const bool ok = col < d;                             // d % 8 == 0: a vector is all in or all out
            const int64_t off = (int64_t)(ok ? col : 0) * 2;
            if (GATED) {
                wg[j] = ld16(row + off);
                wu[j] = ld16(row + row_bytes + off);
            } else {
                wu[j] = ld16(row + off);
            }
            // (a step past d reads the last step's x, clamped in bounds; its weights are zeroed below)
            xv[j] = xmf != nullptr ? ld16(xmf + min(blk / 32 + j, (d + 31) / 32 - 1) * kWave + lane)
                                   : bld16(xr, xrow + (ok ? (uint32_t)col * 2u : kOOB));
        }
        const bool live = s >= 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = live && blk + 32 * j + 8 * g < d;
            const uint4 u = ok ? wu[j] : zero4();
            au = mfma16(xv[j].x, xv[j].y, u.x, u.y, au);
            au = mfma16(xv[j].z, xv[j].w, u.z, u.w, au);
            if (GATED) {
                const uint4 q = ok ? wg[j] : zero4();
                ag = mfma16(xv[j].x, xv[j].y, q.x, q.y, ag);
                ag = mfma16(xv[j].z, xv[j].w, q.z, q.w, ag);
            }
        }
    }
    red[0][wave][lane] = au;
    if (GATED) red[GATED ? 1 : 0][wave][lane] = ag;
#pragma unroll
    for (int u = 1; u < NT; ++u) red[GATED ? 0 : u][wave][lane] = aq[u];
    __syncthreads();
    // thread (tile, v, l) of the first 4*NT waves: D element v of lane l of that tile = token
    // 4(l/16) + v, position t0 + 16*tile + l%16 -- a position whose slot this thread looked up
    // itself (sl[tile])
    if (tid >= 4 * NT * kWave) return;
    const int tile = tid / (4 * kWave), v = (tid / kWave) & 3, l = lane;
    const int b = 4 * (l >> 4) + v;
    float u = 0.f, gg = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        u += red[GATED ? 0 : tile][w][l][v];
        if (GATED) gg += red[GATED ? 1 : 0][w][l][v];
    }
    float hv;
    if (GATED) {
        hv = fmaxf(gg, 0.f) * u;
    } else {
        const int st = tile == 0 ? sl[0] : sl[NT - 1];
        const float bias = (b_up != nullptr && st >= 0) ? half_to_float(b_up[st]) : 0.f;
        hv = fmaxf(u + bias, 0.f);
        if (act) hv *= hv;                                       // squared ReLU
    }
    const int st = tile == 0 ? sl[0] : sl[NT - 1];
    if (st < 0 || b >= B) hv = 0.f;
    // h travels to the down kernel as an fp16 pair; beyond fp16's range the pair cannot hold it,
    // and y would not be finite: say so in the status word instead of failing silently
    if (!(fabsf(hv) < 65504.f)) atomicOr(status, kStatusHRange);
    wide_h_store(hl, b, pos + 16 * tile, hv);                   // pos + 16 tile < hs
}

// The Q4_0 form of k_wide_up on a grid of one kWideUpWaves-wave workgroup per compute unit: the
// ceil(n/16) 16-position tiles are split into gridDim.x contiguous, even runs (one tile more or
// less), and a workgroup sweeps d once per pass of NT tiles (3 or 4: its run in the fewest passes,
// evened out), the waves taking interleaved 256-column blocks and sharing each x load among the
// NT tiles as above.  On one workgroup per 32 neurons, the units that drew two workgroups set the
// time; here every unit gets the same count of neurons.  Rows are read through a buffer resource
// over w_in (n_slots * row_bytes < kBufMax), so absent positions read nothing.
constexpr int kWideUpWaves = 12;
constexpr int kWideUpMaxNT = 4;

struct WideUpQ4Args {
    const uint8_t *w_in;
    int64_t row_bytes;
    int d, B, f, n_slots, hs, act;
    const uint16_t *b_up;
    const uint4 *xmf;
    const int32_t *idx, *slot_of;
    uint16_t *hl;                           // the h table (wide_h_store)
    int32_t *status;
    // positions from the predictor's listed-flag words instead of idx/counts (every neuron resident,
    // slot = id): each workgroup counts the set bits of all nwords words, takes its run and writes
    // those positions' ids to idx_out; workgroup 0 writes counts_out {n, n}.  nullptr: idx/counts.
    const uint32_t *bits;
    int nwords;
    int32_t *idx_out, *counts_out;
};
constexpr int kWideUpWordsPerThread = 6;   // bits mode: nwords <= 6 * kWideUpWaves * 64
constexpr int kWideUpRunIds = 512;         // bits mode: a workgroup's run holds at most this many positions

// One pass: tiles t0 .. t0+NT-1 of the run ending at t_hi (n listed positions); run_ids: the ids of
// the run's positions from p_lo on (bits mode), else nullptr (ids from a.idx).
template <int NT>
__device__ __forceinline__ void wide_up_q4_pass(const WideUpQ4Args &a, __amdgpu_buffer_rsrc_t rw, int n, int t0,
                                                int t_hi, f4 (*red)[kWideUpWaves][kWave], const int *run_ids,
                                                int p_lo) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r = lane & 15, g = lane >> 4, d = a.d;
    int sl[NT];
    uint32_t base[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int pu = (t0 + u) * 16 + r;
        sl[u] = (t0 + u < t_hi && pu < n)
                    ? slot_of_id(run_ids != nullptr ? run_ids[pu - p_lo] : a.idx[pu], a.slot_of, a.f, a.n_slots)
                    : -1;
        base[u] = sl[u] >= 0 ? (uint32_t)(sl[u] * a.row_bytes) : kOOB;
    }
    f4 aq[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) aq[u] = f4{0.f, 0.f, 0.f, 0.f};
    for (int blk = wave * kWideUpCols; blk < d; blk += kWideUpWaves * kWideUpCols) {
        uint4 cw[NT][2], xq[2][4];
        uint32_t sc[NT][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t kb = (uint32_t)(blk / 32 + g + 4 * j);
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                cw[u][j] = bld16(rw, base[u] + kb * 16u);
                sc[u][j] = bld2(rw, base[u] + (uint32_t)(d / 2) + kb * 2u);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) xq[j][i] = ld16(a.xmf + ((blk / 128 + j) * 4 + i) * kWave + lane);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 xp = xq[j][q];
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const h2 s2 = __builtin_bit_cast(h2, sc[u][j] | (sc[u][j] << 16));
                    const uint32_t wd = q == 0 ? cw[u][j].x : q == 1 ? cw[u][j].y : q == 2 ? cw[u][j].z : cw[u][j].w;
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        w[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, q4pair(wd, 4 * p)) * s2);
                    aq[u] = mfma16(xp.x, xp.y, w[0], w[1], aq[u]);
                    aq[u] = mfma16(xp.z, xp.w, w[2], w[3], aq[u]);
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) red[u][wave][lane] = aq[u];
    __syncthreads();
    // (tile, v) pairs e = 4 tile + v go round the waves; lane l of the wave takes D element v of lane
    // l of that tile = token 4(l/16) + v, position 16(t0 + tile) + l%16 -- a position whose slot
    // this thread looked up itself (sl[tile])
    for (int e = wave; e < NT * 4; e += kWideUpWaves) {
        const int tile = e >> 2, v = e & 3, l = lane;
        const int b = 4 * (l >> 4) + v;
        float u = 0.f;
#pragma unroll
        for (int w = 0; w < kWideUpWaves; ++w) u += red[tile][w][l][v];
        int st = -1;
#pragma unroll
        for (int k = 0; k < NT; ++k)
            if (k == tile) st = sl[k];
        const float bias = (a.b_up != nullptr && st >= 0) ? half_to_float(a.b_up[st]) : 0.f;
        float hv = fmaxf(u + bias, 0.f);
        if (a.act) hv *= hv;                                     // squared ReLU
        if (st < 0 || b >= a.B) hv = 0.f;
        if (!(fabsf(hv) < 65504.f)) atomicOr(a.status, kStatusHRange);
        if (t0 + tile < t_hi) wide_h_store(a.hl, b, (t0 + tile) * 16 + r, hv);
    }
    __syncthreads();                                             // red is refilled by the next pass
}

__global__ __launch_bounds__(kWideUpWaves * kWave) void k_wide_up_q4(WideUpQ4Args a, const int32_t *__restrict__ counts,
                                                                    int32_t *__restrict__ zero_ptr, int nzero) {
    __shared__ f4 red[kWideUpMaxNT][kWideUpWaves][kWave];
    __shared__ int s_wsum[kWideUpWaves];
    __shared__ int s_ids[kWideUpRunIds];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    if (blockIdx.x == 0)
        for (int t = tid; t < nzero; t += blockDim.x) zero_ptr[t] = 0;
    const int G = gridDim.x;
    int n, T, t_lo, t_hi;
    const int *run_ids = nullptr;
    int p_lo = 0;
    if (a.bits != nullptr) {
        // thread tid counts words [tid*per, tid*per + per); the ascending ranks of the set bits are
        // the positions (exactly the list k_compact_bits would write)
        const int per = (a.nwords + (int)blockDim.x - 1) / (int)blockDim.x;      // <= kWideUpWordsPerThread
        const int w0 = tid * per;
        const __amdgpu_buffer_rsrc_t rb = buf_rsrc(a.bits, (uint32_t)a.nwords * 4u);
        uint32_t wv[kWideUpWordsPerThread];
        int cnt = 0;
#pragma unroll
        for (int v = 0; v < kWideUpWordsPerThread; ++v) {
            wv[v] = bld4(rb, (v < per && w0 + v < a.nwords) ? (uint32_t)(w0 + v) * 4u : kOOB);
            cnt += __popc(wv[v]);
        }
        const int incl = wave_incl_scan(cnt);
        if (lane == kWave - 1) s_wsum[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWideUpWaves; ++w) {
            before += w < wave ? s_wsum[w] : 0;
            total += s_wsum[w];
        }
        n = min(total, a.n_slots);
        T = (n + 15) / 16;
        t_lo = (int)((int64_t)T * blockIdx.x / G);
        t_hi = (int)((int64_t)T * (blockIdx.x + 1) / G);
        p_lo = 16 * t_lo;
        const int p_hi = min(16 * t_hi, n);
        int pos = before + incl - cnt;
#pragma unroll
        for (int v = 0; v < kWideUpWordsPerThread; ++v) {
            const int c = __popc(wv[v]);
            if (pos < p_hi && pos + c > p_lo) {
                for (uint32_t m = wv[v]; m != 0u && pos < p_hi; m &= m - 1u, ++pos) {
                    if (pos >= p_lo) {
                        const int id = (w0 + v) * 32 + __builtin_ctz(m);
                        s_ids[pos - p_lo] = id;
                        a.idx_out[pos] = id;
                    }
                }
            } else {
                pos += c;
            }
        }
        if (blockIdx.x == 0 && tid == 0) {
            a.counts_out[0] = n;
            a.counts_out[1] = total;
        }
        __syncthreads();
        run_ids = s_ids;
    } else {
        n = min(max(counts[0], 0), a.n_slots);
        T = (n + 15) / 16;
        t_lo = (int)((int64_t)T * blockIdx.x / G);
        t_hi = (int)((int64_t)T * (blockIdx.x + 1) / G);
    }
    const int len = t_hi - t_lo;
    if (len <= 0) return;                                        // workgroup-uniform
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(a.w_in, (uint32_t)(a.n_slots * a.row_bytes));
    const int passes = (len + kWideUpMaxNT - 1) / kWideUpMaxNT;
    const int per = (len + passes - 1) / passes;                 // tiles per pass, <= 4
    for (int t0 = t_lo; t0 < t_hi; t0 += per) {
        if (per <= 3) wide_up_q4_pass<3>(a, rw, n, t0, min(t0 + per, t_hi), red, run_ids, p_lo);
        else wide_up_q4_pass<4>(a, rw, n, t0, min(t0 + per, t_hi), red, run_ids, p_lo);
    }
}

// ------------------------------------------------------------------------------ predictor on MFMA

typedef f16 h8 __attribute__((ext_vector_type(8)));

// gfx950's v_mfma_f32_16x16x32_f16: lane l supplies 8 k-values of row l%16 of A and of column l%16
// of B (lane group l/16 holds k-slots 8(l/16) .. +8) and receives D[4(l/16) + v][l%16], v < 4.
__device__ __forceinline__ f4 mfma32(const uint4 &a, const uint4 &b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

// Partial z for up to 16 tokens on MFMA (the first predictor matrix, split over d): workgroup
// (t, ks) covers rows 64t .. 64t+63 of P1 (wave w: 16 rows, the MFMA's n) over columns
// [ks*cw, min(d, (ks+1)*cw)); per 32-column step lane group g reads columns 32j + 8g .. +8 of its row
// and of its token's x (the A operand: fp16 as given, so every product is exact) and issues one MFMA.
// zpart[ks][b][row] receives the chunk's sums (tokens >= B read x as zero and are not stored);
// k_zsum adds the chunks in order and applies the ReLU.
template <int KC>
__global__ __launch_bounds__(256) void k_pred_l1_mfma(const uint16_t *__restrict__ p1, const uint16_t *__restrict__ x,
                                                      int B, int d, int r, int cw, float *__restrict__ zpart) {
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n16 = lane & 15, g = lane >> 4;
    const int row = blockIdx.x * 64 + wave * 16 + n16;
    const int ks = blockIdx.y;
    const int c0 = ks * cw, c1 = min(d, c0 + cw);
    const __amdgpu_buffer_rsrc_t rp = buf_rsrc(p1, (uint32_t)((size_t)r * d * 2));
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x, (uint32_t)B * (uint32_t)d * 2u);
    const uint32_t prow = row < r ? (uint32_t)row * (uint32_t)d * 2u : kOOB;
    const uint32_t xrow = n16 < B ? (uint32_t)n16 * (uint32_t)d * 2u : kOOB;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = c0; k0 < c1; k0 += 32 * KC) {
        uint4 w[KC], xv[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int col = k0 + 32 * j + 8 * g;
            const bool ok = col < c1;                                  // d and cw are multiples of 8
            w[j] = bld16(rp, ok ? prow + (uint32_t)col * 2u : kOOB);
            xv[j] = bld16(rx, ok ? xrow + (uint32_t)col * 2u : kOOB);
        }
#pragma unroll
        for (int j = 0; j < KC; ++j) acc = mfma32(xv[j], w[j], acc);
    }
    // D[m = 4g + v][n = n16]: tokens 4g .. 4g+3 of this lane's row
    if (row < r) {
        const float av[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int b = 4 * g + v;
            if (b < B) zpart[((size_t)ks * B + b) * r + row] = av[v];
        }
    }
}

// z[o] = max(0, sum over ks, in order, of zpart[ks][o]), o < n = B * r.
static __global__ __launch_bounds__(256) void k_zsum(const float *__restrict__ zpart, int KS, int n,
                                                     float *__restrict__ z) {
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= n) return;
    float s = 0.f;
    for (int k0 = 0; k0 < KS; k0 += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = k0 + k < KS ? zpart[(size_t)(k0 + k) * n + o] : 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) s += v[k];
    }
    z[o] = fmaxf(s, 0.f);
}

// fp32 -> fp16 pair (hi = fp16(v), lo = fp16(v - hi)) of 8 consecutive values, so that v = hi + lo
// to ~2^-22 relative and an f16 MFMA over both parts loses nothing against fp32 z.
__device__ __forceinline__ void split8(const float4 &p, const float4 &q, uint4 &hi, uint4 &lo) {
    const float v[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16 a0 = (f16)v[2 * i], a1 = (f16)v[2 * i + 1];
        const f16 b0 = (f16)(v[2 * i] - (float)a0), b1 = (f16)(v[2 * i + 1] - (float)a1);
        h[i] = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
        l[i] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// l[b][i] = P2[i] . z_b + c[i], mask[i] = OR_{b < B} [l > 0] for up to 16 tokens, on MFMA: wave w of
// workgroup t owns neurons 64t + 16w .. +16 (the MFMA's n = l%16) and all 16 token slots (m; tokens
// >= B read z as zero and are never counted).  Per 32-column step lane group g reads columns
// 32j + 8g .. +8 of its neuron's P2 row (16 bytes) and of its token's z (fp32, split into an fp16
// hi + lo pair in registers), and issues two MFMAs.  P2 and z go through buffer resources, so a
// column past r or a row past f reads zero without a branch.  Optional outputs as in k_pred_l2:
// logits, and the placement-restricted listed flags as 32-bit words (bits[2t + w/2]).
template <int KC>
__global__ __launch_bounds__(256) void k_pred_l2_mfma(const uint16_t *__restrict__ p2, const uint16_t *__restrict__ c,
                                                      const float *__restrict__ z, int B, int r, int f,
                                                      float *__restrict__ logits, uint8_t *__restrict__ mask,
                                                      uint32_t *__restrict__ bits, const int32_t *__restrict__ slot_of,
                                                      int n_slots) {
    __shared__ uint32_t s_half[4];
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n16 = lane & 15, g = lane >> 4;
    const int nrow = blockIdx.x * 64 + wave * 16 + n16;               // this lane's neuron (B operand)
    const __amdgpu_buffer_rsrc_t rp = buf_rsrc(p2, (uint32_t)((size_t)f * r * 2));
    const __amdgpu_buffer_rsrc_t rz = buf_rsrc(z, (uint32_t)B * (uint32_t)r * 4u);
    const uint32_t prow = nrow < f ? (uint32_t)nrow * (uint32_t)r * 2u : kOOB;
    const uint32_t zrow = n16 < B ? (uint32_t)n16 * (uint32_t)r * 4u : kOOB;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < r; k0 += 32 * KC) {
        uint4 w[KC];
        float4 za[KC], zb[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int col = k0 + 32 * j + 8 * g;
            const bool ok = col < r;                                   // r % 8 == 0
            w[j] = bld16(rp, ok ? prow + (uint32_t)col * 2u : kOOB);
            za[j] = __builtin_bit_cast(float4, bld16(rz, ok ? zrow + (uint32_t)col * 4u : kOOB));
            zb[j] = __builtin_bit_cast(float4, bld16(rz, ok ? zrow + (uint32_t)col * 4u + 16u : kOOB));
        }
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            uint4 hi, lo;
            split8(za[j], zb[j], hi, lo);
            acc = mfma32(hi, w[j], acc);
            acc = mfma32(lo, w[j], acc);
        }
    }
    // D[m = 4g + v][n = n16]: logits of tokens 4g .. 4g+3 for this lane's neuron
    const float cn = nrow < f ? half_to_float(c[nrow]) : 0.f;
    const float lv[4] = {acc.x + cn, acc.y + cn, acc.z + cn, acc.w + cn};
    bool fired = false;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int b = 4 * g + v;
        if (b < B) {
            fired |= lv[v] > 0.f;
            if (logits != nullptr && nrow < f) logits[(size_t)b * f + nrow] = lv[v];
        }
    }
    const uint64_t bal = __ballot(fired);
    const uint32_t m16 = (uint32_t)((bal | (bal >> 16) | (bal >> 32) | (bal >> 48)) & 0xFFFFu);
    const bool mine = g == 0 && nrow < f;
    if (mine) mask[nrow] = (uint8_t)((m16 >> n16) & 1u);
    if (bits != nullptr) {
        bool resident = false;
        if (mine) {
            const int sl = slot_of != nullptr ? slot_of[nrow] : 0;
            resident = sl >= 0 && sl < n_slots;
        }
        const uint32_t res16 = (uint32_t)(__ballot(resident) & 0xFFFFu);
        if (lane == 0) s_half[wave] = m16 & res16;
        __syncthreads();
        if (threadIdx.x < 2) {
            const int w2 = 2 * threadIdx.x;
            const int word = blockIdx.x * 2 + threadIdx.x;
            if (word * 32 < f) bits[word] = s_half[w2] | (s_half[w2 + 1] << 16);
        }
    }
}

// y over (slab, neuron chunk) tiles (xmap: the XCD-grouped 1-D grid described below, else a 2-D grid
// of S x C); a slab is 16 lanes x CPL columns (fp16: 8 columns, one 16-byte
// load per row; Q4_0: 16 columns, 8 code bytes and a scale per row, so 16 lanes read a whole 128-byte
// line of a row's codes).  The chunk's 16-position steps are split into W contiguous runs, one per
// wave.  In a step, lane l reads its CPL columns of the rows of positions 4(l/16) + v (v < 4)
// and h of token l%16 at the same four positions; MFMA e then takes half e of each of the four
// rows' decoded vectors as its B operand.  Slots are looked up 64 positions at a time, one lane per
// position, and handed to the lanes that need them by ds_bpermute.  The waves' tiles meet in LDS
// (eight MFMA outputs at a time, summed in wave order), each chunk's partial goes to `part`
// ([C][B][d] fp32; C is the launch's chunk count, at most the workspace's), and the last
// workgroup to finish a slab (slab ticket) sums the partials in chunk order and adds b_down, each
// thread issuing the loads of four outputs before the first add.  Tickets must be zero on entry
// (k_wide_up clears them) and are left zero.
template <int WT, int W = kWideDownWaves>
__global__ __launch_bounds__(W * kWave) void k_wide_down(const uint8_t *__restrict__ w_dn, int64_t row_bytes,
                                                            int d, int B, const int32_t *__restrict__ idx,
                                                            const int32_t *__restrict__ counts,
                                                            const int32_t *__restrict__ slot_of, int f, int n_slots,
                                                            const uint16_t *__restrict__ hl, int hs,
                                                            float *__restrict__ part, int C,
                                                            int32_t *__restrict__ tickets,
                                                            const uint16_t *__restrict__ b_down,
                                                            float *__restrict__ y, int xmap, int S) {
    constexpr int CPL = wide_down_cpl(WT), NW = CPL / 2, SC = 16 * CPL;
    __shared__ f4 red[4][8][kWave];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    int slab = blockIdx.x, ck = blockIdx.y;
    if (xmap) {
        // Q4_0: the scales of 8 consecutive slabs share one 128-byte line, so those 8 workgroups go to
        // one XCD (workgroups are dealt to the 8 XCDs round robin) and meet in its L2 instead of each
        // XCD fetching the line.  1-D grid of 64*ceil(ceil(S/8)*C/8) workgroups: XCD x takes the
        // (slab group, chunk) pairs x, x + 8, ..., each as 8 consecutive workgroups of its share.
        const int L = blockIdx.x, x = L & 7, q = L >> 3;
        const int j = q & 7, pp = (q >> 3) * 8 + x;
        const int ng = (S + 7) / 8;
        slab = (pp % ng) * 8 + j;
        ck = pp / ng;
        if (slab >= S || ck >= C) return;                        // padding: the last group, the last pairs
    }
    const int n = min(max(counts[0], 0), n_slots);
    const int T = (n + 15) / 16;                                 // 16-position steps
    const int c_lo = (int)((int64_t)T * ck / C), c_hi = (int)((int64_t)T * (ck + 1) / C);
    const int w_lo = c_lo + (c_hi - c_lo) * wave / W, w_hi = c_lo + (c_hi - c_lo) * (wave + 1) / W;
    const int r = lane & 15, g = lane >> 4;
    const int col = slab * SC + CPL * r;
    const bool colok = col < d;                                  // d % 8 (fp16) or % 256 (Q4_0): all or none
    const int cq = colok ? col : 0;
    f4 acc[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] = f4{0.f, 0.f, 0.f, 0.f};

    const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hl, (uint32_t)hs * 64u);          // the h table
    // slots are looked up 64 positions (four steps) at a time, one lane per position; the lookup of
    // the next four steps goes out right after this step's row loads
    auto lookup = [&](int s0) {
        const int p = s0 * 16 + lane;
        return (p < w_hi * 16 && p < n) ? slot_of_id(idx[p], slot_of, f, n_slots) : -1;
    };
    int sl_next = lookup(w_lo);
    for (int st0 = w_lo; st0 < w_hi; st0 += 4) {
        const int sl = sl_next;
        // every load of the four steps goes out before the first MFMA; a step past the wave's run
        // (its positions looked up as -1) reads slot 0 and the last valid step's h, and is zeroed
        uint32_t okm = 0u;                                       // bit 4q + v: row (q, v) listed and resident
        uint4 wv[4][4];                                          // fp16: 8 columns
        uint2 qc[4][4];                                          // Q4_0: 16 columns of codes
        uint32_t qs[4][4];                                       // Q4_0: their block scale
        uint2 ahi[4], alo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int sq = min(st0 + q, w_hi - 1);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int sqv = __shfl(sl, q * 16 + 4 * g + v);
                okm |= (sqv >= 0 ? 1u : 0u) << (4 * q + v);
                const uint8_t *rw = w_dn + (int64_t)(sqv >= 0 ? sqv : 0) * row_bytes;
                if (WT == WT_F16) {
                    wv[q][v] = ld16(rw + (int64_t)cq * 2);
                } else {
                    qc[q][v] = *reinterpret_cast<const uint2 *>(rw + cq / 2);
                    qs[q][v] = *reinterpret_cast<const uint16_t *>(rw + d / 2 + (cq / 32) * 2);
                }
            }
            const uint4 hv = bld16(rh, ((uint32_t)(sq * 4 + g) * 16u + (uint32_t)r) * 16u);  // positions 4g..+3, token r
            ahi[q] = make_uint2(hv.x, hv.y);
            alo[q] = make_uint2(hv.z, hv.w);
        }
        sl_next = lookup(st0 + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (st0 + q >= w_hi) {                               // wave-uniform
                ahi[q] = make_uint2(0u, 0u);
                alo[q] = make_uint2(0u, 0u);
            }
            uint32_t wq[4][NW];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool okv = ((okm >> (4 * q + v)) & 1u) && colok;
                if (WT == WT_F16) {
                    const uint4 u = okv ? wv[q][v] : zero4();
                    wq[v][0] = u.x; wq[v][1] = u.y; wq[v][2] = u.z; wq[v][3] = u.w;
                } else {
                    // exact (code - 8) pairs times the row's block scale; code word k gives the
                    // halves (w8k, w8k+4, w8k+1, w8k+5, w8k+2, w8k+6, w8k+3, w8k+7) of its 8 columns
                    const h2 s2 = __builtin_bit_cast(h2, okv ? (qs[q][v] | (qs[q][v] << 16)) : 0u);
                    const uint32_t words[2] = {qc[q][v].x, qc[q][v].y};
#pragma unroll
                    for (int k = 0; k < 2; ++k)
#pragma unroll
                        for (int pp = 0; pp < 4; ++pp)
                            wq[v][4 * k + pp] = __builtin_bit_cast(
                                uint32_t, __builtin_bit_cast(h2, q4pair(words[k], 4 * pp)) * s2);
                }
            }
#pragma unroll
            for (int c = 0; c < NW; ++c) {
                // halves 2c (low) and 2c+1 (high) of the four rows, packed as k = 0..3
                const uint32_t e0 = (wq[0][c] & 0xffffu) | (wq[1][c] << 16);
                const uint32_t e1 = (wq[2][c] & 0xffffu) | (wq[3][c] << 16);
                const uint32_t o0 = (wq[0][c] >> 16) | (wq[1][c] & 0xffff0000u);
                const uint32_t o1 = (wq[2][c] >> 16) | (wq[3][c] & 0xffff0000u);
                acc[2 * c] = mfma16(ahi[q].x, ahi[q].y, e0, e1, acc[2 * c]);
                acc[2 * c] = mfma16(alo[q].x, alo[q].y, e0, e1, acc[2 * c]);
                acc[2 * c + 1] = mfma16(ahi[q].x, ahi[q].y, o0, o1, acc[2 * c + 1]);
                acc[2 * c + 1] = mfma16(alo[q].x, alo[q].y, o0, o1, acc[2 * c + 1]);
            }
        }
    }
    const int Bd = B * d;
#pragma unroll
    for (int hh = 0; hh < CPL / 8; ++hh) {                       // MFMA outputs 8hh .. 8hh+7
        if (hh > 0) __syncthreads();                             // the previous half has been read
        // waves 0..3 store their tiles, then waves 4k..4k+3 (k = 1, 2, ...) add theirs in turn:
        // red[w] = tile of wave w + tile of wave w+4 + ...
        if (wave < 4) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wave][e][lane] = acc[8 * hh + e];
        }
#pragma unroll
        for (int k = 1; k < W / 4; ++k) {
            __syncthreads();
            if (wave >= 4 * k && wave < 4 * k + 4) {
#pragma unroll
                for (int e = 0; e < 8; ++e) red[wave - 4 * k][e][lane] += acc[8 * hh + e];
            }
        }
        __syncthreads();
        // output (token b, lane column lc, column c8 of the half): lane 16(b/4) + lc, element b%4
        // of MFMA e, where e = c8 for fp16 rows and the position of column c8 in the Q4_0 half order
        for (int o = tid; o < B * 128; o += blockDim.x) {
            const int b = o >> 7, lc = (o >> 3) & 15, c8 = o & 7;
            const int e = WT == WT_F16 ? c8 : (((c8 & 3) << 1) | (c8 >> 2));
            const int ln = 16 * (b >> 2) + lc, v = b & 3;
            const int gcol = slab * SC + lc * CPL + 8 * hh + c8;
            if (gcol < d)
                store_coherent(part + (size_t)ck * Bd + (size_t)b * d + gcol,
                               red[0][e][ln][v] + red[1][e][ln][v] + red[2][e][ln][v] + red[3][e][ln][v]);
        }
    }
    wait_stores_done();                                          // this thread's partials are out
    __syncthreads();                                             // ... and so are everyone's
    if (tid == 0) s_last = (atomicAdd(&tickets[slab], 1) == C - 1);
    __syncthreads();
    if (!s_last) return;
    constexpr int OPT = kWideB * SC / (W * kWave);               // outputs per thread (2 to 8)
#pragma unroll
    for (int k0 = 0; k0 < OPT; k0 += 4) {
        float pv[4][kWideMaxChunks];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int o = tid + (k0 + k) * (W * kWave);
            const int b = o / SC, cc = o - b * SC;
            const int gcol = slab * SC + cc;
            const bool ok = b < B && gcol < d;
            const size_t off = ok ? (size_t)b * d + gcol : 0;
#pragma unroll
            for (int c = 0; c < kWideMaxChunks; ++c)
                pv[k][c] = (ok && c < C) ? load_coherent(part + (size_t)c * Bd + off) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int o = tid + (k0 + k) * (W * kWave);
            const int b = o / SC, cc = o - b * SC;
            const int gcol = slab * SC + cc;
            if (b >= B || gcol >= d) continue;
            float sum = b_down ? half_to_float(b_down[gcol]) : 0.f;
#pragma unroll
            for (int c = 0; c < kWideMaxChunks; ++c) sum += pv[k][c];
            y[(size_t)b * d + gcol] = sum;
        }
    }
    if (tid == 0) tickets[slab] = 0;
}

// The same logits and flags with z staged once per workgroup in LDS, already split into fp16 hi +
// lo parts and laid out in the MFMA's A-operand order (entry (s, part, L) = 8 values of token L%16
// at columns 32s + 8(L/16) .. +8; tokens >= B are zeros), so each wave reads one 16-byte LDS vector
// per part and step instead of loading and splitting 32 bytes of fp32 z from L2 for every 16
// neurons.  Workgroups of kPredL2Waves waves own 16 * kPredL2Waves neurons; the P2 loads of two
// 32*KC-column steps are in flight per wave (the first go out before the staging).  LDS: 64 r bytes
// (r <= kPredL2StagedMaxRank).  With xmf != nullptr the grid also writes x [B][d] in the operand
// order of the up step (the Q4_0 layout if xq4, else the fp16 one: k_wide_xmf's work, spread over
// the grid, so the layer needs no launch of its own for it).
constexpr int kPredL2Waves = 8;
constexpr int kPredL2StagedMaxRank = 1024;
template <int KC>
__global__ __launch_bounds__(kPredL2Waves * kWave) void k_pred_l2_mfma_s(
    const uint16_t *__restrict__ p2, const uint16_t *__restrict__ c, const float *__restrict__ z, int B, int r, int f,
    float *__restrict__ logits, uint8_t *__restrict__ mask, uint32_t *__restrict__ bits,
    const int32_t *__restrict__ slot_of, int n_slots, const uint16_t *__restrict__ x, int d, int xq4,
    uint4 *__restrict__ xmf) {
    extern __shared__ __align__(16) uint4 zmf[];                       // [r/32][2][kWave]
    __shared__ uint32_t s_half[kPredL2Waves];
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n16 = lane & 15, g = lane >> 4;
    const int nrow = blockIdx.x * (16 * kPredL2Waves) + wave * 16 + n16;   // this lane's neuron (B operand)
    const __amdgpu_buffer_rsrc_t rp = buf_rsrc(p2, (uint32_t)((size_t)f * r * 2));
    const uint32_t prow = nrow < f ? (uint32_t)nrow * (uint32_t)r * 2u : kOOB;
    auto issue = [&](uint4 (&w)[KC], int k0) {
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int col = k0 + 32 * j + 8 * g;
            w[j] = bld16(rp, col < r ? prow + (uint32_t)col * 2u : kOOB);   // r % 8 == 0
        }
    };
    uint4 wa[KC], wb[KC];
    issue(wa, 0);
    if (xmf != nullptr) {
        const int nv = wide_xmf_vectors(d, xq4 != 0);
        for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < nv; v += gridDim.x * blockDim.x) {
            if (xq4) wide_xmf_vec(x, B, d, xmf, v);
            else wide_xf16_vec(x, B, d, xmf, v);
        }
    }
    // staging: item (s, L) -> hi at zmf[2s*64 + L], lo at zmf[(2s+1)*64 + L]
    const __amdgpu_buffer_rsrc_t rz = buf_rsrc(z, (uint32_t)B * (uint32_t)r * 4u);
    const int steps = (r + 31) / 32;
    for (int e = threadIdx.x; e < steps * kWave; e += blockDim.x) {
        const int st = e / kWave, L = e - st * kWave, m = L & 15, col = 32 * st + 8 * (L >> 4);
        const bool ok = m < B && col < r;
        const uint32_t off = ok ? ((uint32_t)m * (uint32_t)r + (uint32_t)col) * 4u : kOOB;
        uint4 hi, lo;
        split8(__builtin_bit_cast(float4, bld16(rz, off)), __builtin_bit_cast(float4, bld16(rz, ok ? off + 16u : kOOB)),
               hi, lo);
        zmf[(2 * st) * kWave + L] = hi;
        zmf[(2 * st + 1) * kWave + L] = lo;
    }
    __syncthreads();
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    auto step = [&](const uint4 (&w)[KC], int k0) {
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int st = k0 / 32 + j;
            if (st < steps) {                                          // wave-uniform
                acc = mfma32(zmf[(2 * st) * kWave + lane], w[j], acc);
                acc = mfma32(zmf[(2 * st + 1) * kWave + lane], w[j], acc);
            }
        }
    };
    for (int k0 = 0; k0 < r; k0 += 64 * KC) {
        issue(wb, k0 + 32 * KC);
        step(wa, k0);
        issue(wa, k0 + 64 * KC);
        step(wb, k0 + 32 * KC);
    }
    // D[m = 4g + v][n = n16]: logits of tokens 4g .. 4g+3 for this lane's neuron
    const float cn = nrow < f ? half_to_float(c[nrow]) : 0.f;
    const float lv[4] = {acc.x + cn, acc.y + cn, acc.z + cn, acc.w + cn};
    bool fired = false;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int b = 4 * g + v;
        if (b < B) {
            fired |= lv[v] > 0.f;
            if (logits != nullptr && nrow < f) logits[(size_t)b * f + nrow] = lv[v];
        }
    }
    const uint64_t bal = __ballot(fired);
    const uint32_t m16 = (uint32_t)((bal | (bal >> 16) | (bal >> 32) | (bal >> 48)) & 0xFFFFu);
    const bool mine = g == 0 && nrow < f;
    if (mine) mask[nrow] = (uint8_t)((m16 >> n16) & 1u);
    if (bits != nullptr) {
        bool resident = false;
        if (mine) {
            const int sl = slot_of != nullptr ? slot_of[nrow] : 0;
            resident = sl >= 0 && sl < n_slots;
        }
        const uint32_t res16 = (uint32_t)(__ballot(resident) & 0xFFFFu);
        if (lane == 0) s_half[wave] = m16 & res16;
        __syncthreads();
        if (threadIdx.x < kPredL2Waves / 2) {
            const int w2 = 2 * threadIdx.x;
            const int word = blockIdx.x * (kPredL2Waves / 2) + threadIdx.x;
            if (word * 32 < f) bits[word] = s_half[w2] | (s_half[w2 + 1] << 16);
        }
    }
}

}  // namespace pik
