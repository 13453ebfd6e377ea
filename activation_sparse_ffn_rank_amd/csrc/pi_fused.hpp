// pi_fused.hpp -- the whole layer (predictor, mask, compaction, sparse FFN) in one persistent kernel.
//
// Each step of the layer is small (a few MB to ~100 MB of weights), so separate kernels pay a fixed
// launch-and-flush cost per kernel that is as large as the work.  Here one launch runs every step:
// a grid of co-resident workgroups walks an ordered list of tasks round-robin (workgroup p takes
// tasks p, p+P, p+2P, ...), and every task waits only on tasks earlier in the list:
//
//   A  4 rows of P1 per task          z = max(0, P1 x); the task completing the count raises the
//                                     "z complete" word (in kGoCopies copies on separate lines)
//   B  32 rows of P2 per task (tile)  mask bits of the tile (its P2 rows are loaded before it waits
//                                     for z, so the second predictor matrix streams during the first)
//   D  TPD tiles per task             h of the tile group's listed neurons -> entries (slot, h)
//   E  (512-column slab, chunk)       partial y of the chunk's entries with nonzero h; the last
//                                     chunk of a slab to finish sums the partials in chunk order -> y
//   X  one task (optional)            ascending idx_out and counts_out
//
// Hand-offs between workgroups carry the launch's stamp in the upper half of 64-bit words written
// with agent-coherent stores (single-copy atomic, no L2-wide flush); a consumer polls the data
// words themselves and re-reads only those that are still stale, so no producer waits for its
// stores to be acknowledged and no separate ready flag is needed.  Stamps are epoch + 1, so
// nothing has to be cleared between launches; the few counters (z count, slab tickets, exit) are
// reset by the last workgroup to leave, which also advances the epoch.  Every wait is bounded
// (kSpinTicks of the constant 100 MHz clock); a wait that runs out raises an abort flag that
// releases every other wait, so the grid always drains, and sets a sticky status word for the
// host.  The workspace must be zero-filled before its first use.
#pragma once

#include "pi_kernels.hpp"

namespace pik {

constexpr int kTile = 32;                      // predictor rows per B task
constexpr int kGoCopies = 64;                  // copies of the "z is complete" word (spread)
constexpr int kFusedMaxChunks = 16;            // chunk partials per slab in the fused kernel
constexpr uint64_t kSpinTicks = 2000000;       // 20 ms of the 100 MHz real-time clock

// Control block: int32 words, each on its own 128-byte line.
enum : int {
    CTL_EPOCH = 0,
    CTL_EXIT = 32,
    CTL_ABORT = 64,
    CTL_STATUS = 96,
    CTL_GO0 = 128,                             // + 32 * copy
    CTL_LAYER0 = CTL_GO0 + 32 * kGoCopies,
    CTL_DONE_A = 0,                            // per-layer offsets
    CTL_TICKET0 = 32,                          // + 32 * slab
};

__host__ __device__ inline int ctl_layer_stride(int slabs) { return CTL_TICKET0 + 32 * slabs; }

struct FusedArgs {
    // shapes (cap = entries per D group)
    int d, f, r, n_slots, slabs, C, TPD, NA, NB, ND, NE, tasks, P, want_x, cap;
    int act;                                       // 1: squared ReLU (non-gated)
    int64_t row_bytes;
    // tensors
    const uint16_t *p1, *p2, *c;
    const uint8_t *w_in, *w_dn;
    const uint16_t *b_up, *b_down;
    const int32_t *slot_of;
    const uint16_t *x;
    float *y;
    uint8_t *mask_out;
    int32_t *idx_out, *counts_out;
    // scratch (workspace); every uint64_t word is (value | stamp << 32)
    int32_t *ctl;        // control block
    uint64_t *z;         // [B][r]     z values
    uint64_t *tword;     // [NB]       listed bits of each tile
    uint64_t *pword;     // [NB]       predicted bits of each tile
    uint64_t *ghead;     // [ND]       listed count of each D group
    uint64_t *ent;       // [ND][cap][1+B]  entry: slot, then h per token
    uint64_t *part;      // [C][B][d]  chunk partials of y
#ifdef PIK_TRACE
    uint64_t *trace;     // [tasks][4]: workgroup, start, dependency met, end (100 MHz clock)
#endif
};

#ifdef PIK_TRACE
#define PIK_TRACE_AT(g, slot)                                                              \
    do {                                                                                   \
        if (a.trace != nullptr && threadIdx.x == 0) {                                      \
            a.trace[(size_t)(g) * 4 + (slot)] = (slot) == 0 ? blockIdx.x : wall_clock64(); \
        }                                                                                  \
    } while (0)
#else
#define PIK_TRACE_AT(g, slot) ((void)0)
#endif

__device__ __forceinline__ int32_t load_coherent_i(const int32_t *p) {
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent_u(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_i(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_c64(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_c64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t stamped(uint32_t v, uint32_t stamp) { return ((uint64_t)stamp << 32) | v; }
__device__ __forceinline__ uint64_t stamped_f(float v, uint32_t stamp) {
    return stamped(__builtin_bit_cast(uint32_t, v), stamp);
}
__device__ __forceinline__ bool fresh(uint64_t w, uint32_t stamp) { return (uint32_t)(w >> 32) == stamp; }
__device__ __forceinline__ float word_f(uint64_t w) { return __builtin_bit_cast(float, (uint32_t)w); }

// Called by every lane of a wave between two polls: true when the wave must stop waiting (the
// abort flag is up, or this wait ran past kSpinTicks, which raises it and records `code`).
__device__ bool poll_give_up(uint64_t t0, int32_t *ctl, int lane, int code) {
    int ab = 0;
    if (lane == 0) ab = load_coherent_i(ctl + CTL_ABORT);
    if (__shfl(ab, 0, kWave)) return true;
    if (wall_clock64() - t0 > kSpinTicks) {
        if (lane == 0) {
            store_coherent_i(ctl + CTL_ABORT, 1);
            atomicOr(ctl + CTL_STATUS, code);
        }
        return true;
    }
    __builtin_amdgcn_s_sleep(4);
    return false;
}

// The same decision for a poll loop that has just re-issued its loads: `ab` is the abort word
// loaded together with them (so a poll costs one round trip, not two).
__device__ __forceinline__ bool poll_stop(int ab, uint64_t t0, int32_t *ctl, int lane, int code) {
    if (__shfl(ab, 0, kWave)) return true;
    if (wall_clock64() - t0 > kSpinTicks) {
        if (lane == 0) {
            store_coherent_i(ctl + CTL_ABORT, 1);
            atomicOr(ctl + CTL_STATUS, code);
        }
        return true;
    }
    return false;
}

// Bounded wait by one thread until *p == stamp.  false = aborted.
__device__ bool wait_stamp(const uint32_t *p, uint32_t stamp, int32_t *ctl) {
    const uint64_t t0 = wall_clock64();
    for (;;) {
        if (load_coherent_u(p) == stamp) return true;
        if (load_coherent_i(ctl + CTL_ABORT)) return false;
        if (wall_clock64() - t0 > kSpinTicks) {
            store_coherent_i(ctl + CTL_ABORT, 1);
            atomicOr(ctl + CTL_STATUS, 1);
            return false;
        }
        __builtin_amdgcn_s_sleep(4);
    }
}

// Wave-wide: load *p (p == nullptr: nothing to load, counts as fresh) and re-read it until its
// stamp is current in every lane (or the wait gives up).
__device__ __forceinline__ uint64_t poll_word(const uint64_t *p, uint32_t stamp, int32_t *ctl, int lane, int code) {
    uint64_t w = p ? load_c64(p) : stamped(0u, stamp);
    const uint64_t t0 = wall_clock64();
    while (__ballot(!fresh(w, stamp)) != 0) {
        const int ab = lane == 0 ? load_coherent_i(ctl + CTL_ABORT) : 0;   // with the re-read
        if (!fresh(w, stamp)) w = load_c64(p);
        if (poll_stop(ab, t0, ctl, lane, code)) break;
    }
    return w;
}

// ------------------------------------------------------------------------------ A: z rows

// One row of P1 per wave.  x comes from the workgroup's LDS copy: natural order for fp16
// layers; for Q4_0 layers it is kept in the q4-paired order, and the P1 words are re-paired the
// same way, which leaves every dot product unchanged.
template <int B, bool XQ4>
__device__ void task_A(const FusedArgs &a, int t, int lane, int wave, const uint16_t *xs, uint32_t stamp) {
    const int j = t * 4 + wave;
    if (j < a.r) {
        const uint16_t *row = a.p1 + (size_t)j * a.d;
        float acc[B];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = 0.f;
        constexpr int V = 16;
        for (int c0 = 0; c0 < a.d; c0 += V * 512) {
            uint4 w[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int col = c0 + lane * 8 + v * 512;
                w[v] = col < a.d ? ld16(row + col) : zero4();
            }
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int col = c0 + lane * 8 + v * 512;
                if (col < a.d) {
                    const uint4 wv = XQ4 ? pair_for_q4(w[v]) : w[v];
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        acc[b] = dot8(wv, *reinterpret_cast<const uint4 *>(xs + (size_t)b * a.d + col), acc[b]);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float s = wave_sum(acc[b]);
            if (lane == 0) store_c64(a.z + (size_t)b * a.r + j, stamped_f(fmaxf(s, 0.f), stamp));
        }
    }
    __syncthreads();
    // The task that completes the count raises the "z complete" word in every copy; B tasks each
    // watch one copy, so no line is polled by every workgroup.  (z words are stamped, so a B task
    // that outruns a z store simply re-reads it.)
    if (threadIdx.x < kWave) {
        int last = 0;
        if (threadIdx.x == 0) last = atomicAdd(a.ctl + CTL_LAYER0 + CTL_DONE_A, 1) == a.NA - 1;
        if (__shfl(last, 0, kWave))
            store_coherent_u(reinterpret_cast<uint32_t *>(a.ctl + CTL_GO0 + 32 * threadIdx.x), stamp);
    }
}

// ------------------------------------------------------------------------------ B: mask tile

template <int B, int NT>
__device__ void task_B(const FusedArgs &a, int t, int lane, int wave, uint32_t stamp, uint32_t *s_words, int g) {
    constexpr int R = 8;
    const int row0 = t * kTile + wave * R;
    uint4 w[R][NT];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const int row = row0 + i, col = lane * 8 + q * 512;
            w[i][q] = (row < a.f && col < a.r) ? ld16(a.p2 + (size_t)row * a.r + col) : zero4();
        }
    constexpr int G = kWave / R;
    const int ri = lane / G;
    const int row = row0 + ri;
    const bool owner = (lane % G) == 0 && row < a.f;
    const float ci = owner ? half_to_float(a.c[row]) : 0.f;
    const bool resident = owner && (a.slot_of == nullptr || a.slot_of[row] >= 0);

    if (threadIdx.x == 0)
        wait_stamp(reinterpret_cast<const uint32_t *>(a.ctl + CTL_GO0 + 32 * (blockIdx.x % kGoCopies)), stamp, a.ctl);
    __syncthreads();
    PIK_TRACE_AT(g, 2);

    uint8_t m = 0;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        // the lane's z words for this token: all loads issued at once, then one re-poll loop for
        // any that are still stale (an A task's store may still be in flight)
        uint64_t zw[NT][8];
        const uint64_t *zb = a.z + (size_t)b * a.r;
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const int col = lane * 8 + q * 512;
#pragma unroll
            for (int e = 0; e < 8; ++e) zw[q][e] = col < a.r ? load_c64(zb + col + e) : stamped(0u, stamp);
        }
        {
            const uint64_t t0 = wall_clock64();
            for (;;) {
                bool stale = false;
#pragma unroll
                for (int q = 0; q < NT; ++q)
#pragma unroll
                    for (int e = 0; e < 8; ++e) stale |= !fresh(zw[q][e], stamp);
                if (__ballot(stale) == 0 || poll_give_up(t0, a.ctl, lane, 8)) break;
#pragma unroll
                for (int q = 0; q < NT; ++q)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (!fresh(zw[q][e], stamp)) zw[q][e] = load_c64(zb + lane * 8 + q * 512 + e);
            }
        }
        float v[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                const uint32_t qq[4] = {w[i][q].x, w[i][q].y, w[i][q].z, w[i][q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const h2 p = __builtin_bit_cast(h2, qq[e]);
                    s = fmaf((float)p.x, word_f(zw[q][2 * e]), s);
                    s = fmaf((float)p.y, word_f(zw[q][2 * e + 1]), s);
                }
            }
            v[i] = s;
        }
        const float l = reduce_scatter<R>(v, lane) + ci;
        if (owner) m |= (uint8_t)(l > 0.f);
    }
    if (owner && a.mask_out) a.mask_out[row] = m;
    // gather the tile's bits: wave w's rows are tile rows 8w .. 8w+7, owned by lanes 0, 8, ..., 56
    const uint64_t lb = __ballot(owner && m && resident);
    const uint64_t pb = __ballot(owner && m);
    uint32_t lbyte = 0, pbyte = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        lbyte |= (uint32_t)((lb >> (i * G)) & 1ull) << i;
        pbyte |= (uint32_t)((pb >> (i * G)) & 1ull) << i;
    }
    if (lane == 0) {
        s_words[wave] = lbyte;
        s_words[4 + wave] = pbyte;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t word = s_words[0] | (s_words[1] << 8) | (s_words[2] << 16) | (s_words[3] << 24);
        const uint32_t pword = s_words[4] | (s_words[5] << 8) | (s_words[6] << 16) | (s_words[7] << 24);
        store_c64(a.tword + t, stamped(word, stamp));
        store_c64(a.pword + t, stamped(pword, stamp));
    }
    __syncthreads();                                  // s_words reused by the next task
}

// ------------------------------------------------------------------------------ D: h of a tile group

// The group's listed neurons go one per wave (wave w takes the w-th, (w+4)-th, ...), each wave
// running the same row passes as the stand-alone up kernel against the LDS copy of x.  Entry j of
// the group (its j-th listed neuron, ascending id) gets its slot and h; the down tasks skip
// entries whose h is zero for every token.
template <int B, bool GATED, int WT>
__device__ void task_D(const FusedArgs &a, int g, int lane, int wave, uint32_t stamp, int *s_misc, int gt,
                       const uint16_t *xs) {
    const int t0 = g * a.TPD, t1 = min(t0 + a.TPD, a.NB);
    int *s_ids = s_misc;                    // [32 * TPD]
    int *s_n = s_misc + 32 * 4;
    if (wave == 0) {
        // one lane per tile polls the tile's word; lane 0 then lists the ids in ascending order
        const uint64_t wd = poll_word(t0 + lane < t1 ? a.tword + t0 + lane : nullptr, stamp, a.ctl, lane, 16);
        const uint32_t mine = (uint32_t)wd;
        int n = 0;
        for (int t = t0; t < t1; ++t) {
            uint32_t bits = (uint32_t)bcast((int)mine, t - t0);
            if (lane == 0)
                for (; bits; bits &= bits - 1) s_ids[n++] = t * kTile + __builtin_ctz(bits);
        }
        if (lane == 0) *s_n = n;
    }
    __syncthreads();
    PIK_TRACE_AT(gt, 2);
    const int n = *s_n;
    const int cap = a.cap;
    const int64_t in_stride = GATED ? 2 * a.row_bytes : a.row_bytes;
    for (int j = wave; j < n; j += 4) {
        const int s = slot_of_id(s_ids[j], a.slot_of, a.f, a.n_slots);
        float ag[B], au[B];
#pragma unroll
        for (int b = 0; b < B; ++b) ag[b] = au[b] = 0.f;
        if (s >= 0) neuron_dots<B, GATED, WT>(a.w_in + (int64_t)s * in_stride, a.row_bytes, a.d, xs, a.d, lane, ag, au);
        const float bias = (!GATED && a.b_up != nullptr && s >= 0) ? half_to_float(a.b_up[s]) : 0.f;
        uint64_t *e = a.ent + ((size_t)g * cap + j) * (1 + B);
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
    __syncthreads();                                  // every entry issued (s_ids reused next task)
    if (threadIdx.x == 0) store_c64(a.ghead + g, stamped((uint32_t)n, stamp));
}

// ------------------------------------------------------------------------------ E: down tile

template <int B, int WT>
__device__ void task_E(const FusedArgs &a, int e, int lane, int wave, uint32_t stamp, float *s_red4, int *s_misc,
                       int *s_last, int gt) {
    constexpr int U = 16;
    const int slab = e % a.slabs, ck = e / a.slabs;
    const int g0 = (int)((int64_t)a.ND * ck / a.C), g1 = (int)((int64_t)a.ND * (ck + 1) / a.C);
    const int col = slab * 512 + lane * 8;
    const bool colok = col < a.d;
    float acc[B][8];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[b][t] = 0.f;
    const int cap = a.cap;
    // wave w takes groups g0 + w, g0 + w + 4, ...; one lane per group polls the group header
    int *s_pref = s_misc + wave * (kWave + 1);
    bool first = true;
    for (int gb = g0 + wave; gb < g1; gb += 4 * kWave) {
        __builtin_amdgcn_wave_barrier();
        const int gi = gb + 4 * lane;
        const uint64_t hw = poll_word(gi < g1 ? a.ghead + gi : nullptr, stamp, a.ctl, lane, 32);
        if (first && wave == 0) PIK_TRACE_AT(gt, 2);
        first = false;
        const int cnt = gi < g1 ? (int)(uint32_t)hw : 0;
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int v = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += v;
        }
        s_pref[lane + 1] = incl;
        if (lane == 0) s_pref[0] = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int total = __shfl(incl, kWave - 1, kWave);
        for (int e0 = 0; e0 < total; e0 += kWave) {
            const int ent = e0 + lane;
            const uint64_t *ep = nullptr;
            if (ent < total) {
                // group of entry `ent`: largest q with s_pref[q] <= ent
                int lo = 0, hi = kWave;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_pref[mid] <= ent) lo = mid; else hi = mid;
                }
                ep = a.ent + ((size_t)(gb + 4 * lo) * cap + (ent - s_pref[lo])) * (1 + B);
            }
            const uint64_t sw = poll_word(ep, stamp, a.ctl, lane, 64);
            int sl = ep ? (int)(uint32_t)sw : -1;
            float hv[B];
            bool any = false;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                hv[b] = word_f(poll_word(ep ? ep + 1 + b : nullptr, stamp, a.ctl, lane, 64));
                any |= hv[b] != 0.f;
            }
            if (!any) sl = -1;                       // h = 0 for every token: an exact zero
            uint64_t live = __ballot(sl >= 0);
            while (live) {
                int js[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    js[u] = live ? __builtin_ctzll(live) : -1;
                    if (live) live &= live - 1;
                }
                if (WT == WT_F16) {
                    uint4 wv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int s = js[u] >= 0 ? bcast(sl, js[u]) : -1;
                        wv[u] = (s >= 0 && colok) ? ld16(a.w_dn + (int64_t)s * a.row_bytes + (int64_t)col * 2) : zero4();
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        if (js[u] < 0) continue;
                        const uint32_t wq[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            const float hb = bcastf(hv[b], js[u]);
#pragma unroll
                            for (int p = 0; p < 4; ++p) {
                                const h2 pr = __builtin_bit_cast(h2, wq[p]);
                                acc[b][2 * p] = fmaf(hb, (float)pr.x, acc[b][2 * p]);
                                acc[b][2 * p + 1] = fmaf(hb, (float)pr.y, acc[b][2 * p + 1]);
                            }
                        }
                    }
                } else {
                    uint32_t cw[U];
                    uint16_t sc[U];
                    bool okv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        // unconditional loads (row 0, column 0 stand in for an absent row or
                        // column), so that all U rows are in flight before the first conversion
                        const int s = js[u] >= 0 ? bcast(sl, js[u]) : -1;
                        okv[u] = s >= 0 && colok;
                        const uint8_t *row = a.w_dn + (int64_t)(okv[u] ? s : 0) * a.row_bytes;
                        const int cc = colok ? col : 0;
                        cw[u] = *reinterpret_cast<const uint32_t *>(row + cc / 2);
                        sc[u] = *reinterpret_cast<const uint16_t *>(row + a.d / 2 + (cc / 32) * 2);
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        if (js[u] < 0) continue;
                        const float scf = okv[u] ? half_to_float(sc[u]) : 0.f;
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const h2 pr = __builtin_bit_cast(h2, q4pair(cw[u], 4 * p));
                            const float lo = (float)pr.x, hi = (float)pr.y;
#pragma unroll
                            for (int b = 0; b < B; ++b) {
                                const float cf = bcastf(hv[b], js[u]) * scf;
                                acc[b][p] = fmaf(cf, lo, acc[b][p]);
                                acc[b][p + 4] = fmaf(cf, hi, acc[b][p + 4]);
                            }
                        }
                    }
                }
            }
        }
    }
    if (first && wave == 0) PIK_TRACE_AT(gt, 2);
    // waves -> LDS -> stamped chunk partial -> slab ticket; the last chunk sums in chunk order
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < 8; ++t) s_red4[((wave * B + b) * 8 + t) * kWave + lane] = acc[b][t];
    __syncthreads();
    const int Bd = B * a.d;
    for (int o = threadIdx.x; o < B * 512; o += blockDim.x) {
        const int b = o / 512, cc = o - b * 512;
        const int ln = cc >> 3, t = cc & 7;
        const int gcol = slab * 512 + cc;
        if (gcol < a.d) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) s += s_red4[((w * B + b) * 8 + t) * kWave + ln];
            store_c64(a.part + (size_t)ck * Bd + (size_t)b * a.d + gcol, stamped_f(s, stamp));
        }
    }
    __syncthreads();
    int32_t *ticket = a.ctl + CTL_LAYER0 + CTL_TICKET0 + 32 * slab;
    if (threadIdx.x == 0) *s_last = (atomicAdd(ticket, 1) == a.C - 1);
    __syncthreads();
    if (*s_last) {
        for (int o = threadIdx.x; o < B * 512; o += blockDim.x) {
            const int b = o / 512, cc = o - b * 512;
            const int gcol = slab * 512 + cc;
            const bool ok = gcol < a.d;
            const size_t off = (size_t)b * a.d + (ok ? gcol : 0);
            uint64_t v[kFusedMaxChunks];
#pragma unroll
            for (int c = 0; c < kFusedMaxChunks; ++c)
                v[c] = (ok && c < a.C) ? load_c64(a.part + (size_t)c * Bd + off) : stamped(0u, stamp);
            // a chunk's partial store may still be in flight: re-read the stale ones
            const uint64_t t0 = wall_clock64();
            for (;;) {
                bool stale = false;
#pragma unroll
                for (int c = 0; c < kFusedMaxChunks; ++c) stale |= !fresh(v[c], stamp);
                if (!stale || load_coherent_i(a.ctl + CTL_ABORT)) break;
                if (wall_clock64() - t0 > kSpinTicks) {
                    store_coherent_i(a.ctl + CTL_ABORT, 1);
                    atomicOr(a.ctl + CTL_STATUS, 128);
                    break;
                }
#pragma unroll
                for (int c = 0; c < kFusedMaxChunks; ++c)
                    if (!fresh(v[c], stamp)) v[c] = load_c64(a.part + (size_t)c * Bd + off);
            }
            float s = (ok && a.b_down) ? half_to_float(a.b_down[gcol]) : 0.f;
#pragma unroll
            for (int c = 0; c < kFusedMaxChunks; ++c) s += word_f(v[c]);
            if (ok) a.y[off] = s;
        }
    }
    __syncthreads();                                  // LDS reused by the next task
}

// ------------------------------------------------------------------------------ X: ascending idx

__device__ void task_X(const FusedArgs &a, int lane, int wave, uint32_t stamp, int *s_misc, int gt) {
    // thread t handles tiles t*per .. ; per-thread counts, block scan, then write ids in order
    const int per = (a.NB + blockDim.x - 1) / blockDim.x;
    const int ta = threadIdx.x * per, tb = min(ta + per, a.NB);
    int cnt = 0, pc = 0;
    for (int t0 = 0; t0 < per; ++t0) {
        const int t = ta + t0;
        const uint64_t w = poll_word(t < tb ? a.tword + t : nullptr, stamp, a.ctl, lane, 256);
        const uint64_t pw = poll_word(t < tb ? a.pword + t : nullptr, stamp, a.ctl, lane, 256);
        if (t < tb) {
            cnt += __popc((uint32_t)w);
            pc += __popc((uint32_t)pw);
        }
    }
    PIK_TRACE_AT(gt, 2);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    int wp = pc;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) wp += __shfl_xor(wp, o, kWave);
    int *s_w = s_misc, *s_p = s_misc + 8;
    if (lane == kWave - 1) s_w[wave] = incl;
    if (lane == 0) s_p[wave] = wp;
    __syncthreads();
    int before = 0, total = 0, tpred = 0;
    for (int w = 0; w < 4; ++w) {
        before += w < wave ? s_w[w] : 0;
        total += s_w[w];
        tpred += s_p[w];
    }
    int pos = before + incl - cnt;
    if (a.idx_out)
        for (int t = ta; t < tb; ++t)
            for (uint32_t wd = (uint32_t)load_c64(a.tword + t); wd; wd &= wd - 1)
                a.idx_out[pos++] = t * kTile + __builtin_ctz(wd);
    if (threadIdx.x == 0 && a.counts_out) {
        a.counts_out[0] = total;
        a.counts_out[1] = tpred;
    }
    __syncthreads();
}

// ------------------------------------------------------------------------------ the kernel

template <int B, bool GATED, int WT, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(B <= 2 ? 3 : 2))) void k_layer_fused(FusedArgs a) {
    extern __shared__ __align__(16) uint16_t xs[];              // x [B][d] (q4-paired for Q4_0)
    __shared__ float s_red4[4 * B * 8 * kWave];                 // E: wave partials
    __shared__ int s_misc[4 * (kWave + 1) + 32 * 4 + 8];        // E prefix / D ids / X scan
    __shared__ uint32_t s_words[8];
    __shared__ int s_last;
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t stamp = (uint32_t)load_coherent_i(a.ctl + CTL_EPOCH) + 1u;
    stage_x<B, WT == WT_Q4_0>(xs, a.x, a.d, 0, a.d, a.d);
    __syncthreads();

    for (int g = blockIdx.x; g < a.tasks; g += a.P) {
        PIK_TRACE_AT(g, 0);
        PIK_TRACE_AT(g, 1);
        PIK_TRACE_AT(g, 2);                           // tasks with a dependency overwrite this
        if (g < a.NA) {
            task_A<B, WT == WT_Q4_0>(a, g, lane, wave, xs, stamp);
        } else if (g < a.NA + a.NB) {
            task_B<B, NT>(a, g - a.NA, lane, wave, stamp, s_words, g);
        } else if (g < a.NA + a.NB + a.ND) {
            task_D<B, GATED, WT>(a, g - a.NA - a.NB, lane, wave, stamp, s_misc, g, xs);
        } else if (g < a.NA + a.NB + a.ND + a.NE) {
            task_E<B, WT>(a, g - a.NA - a.NB - a.ND, lane, wave, stamp, s_red4, s_misc, &s_last, g);
        } else {
            task_X(a, lane, wave, stamp, s_misc, g);
        }
        PIK_TRACE_AT(g, 3);
    }
    // leave: the last workgroup out resets the counters and advances the epoch
    __syncthreads();
    if (threadIdx.x == 0) {
        if (atomicAdd(a.ctl + CTL_EXIT, 1) == a.P - 1) {
            const int ls = ctl_layer_stride(a.slabs);
            for (int i = 0; i < ls; i += 32) store_coherent_i(a.ctl + CTL_LAYER0 + i, 0);
            store_coherent_i(a.ctl + CTL_ABORT, 0);
            store_coherent_i(a.ctl + CTL_EXIT, 0);
            store_coherent_i(a.ctl + CTL_EPOCH, (int32_t)stamp);
        }
    }
}

// Launch of the fused layer kernel for batch width B (one translation unit per B, so the
// variants compile in parallel).  Picks the grid so that every workgroup is resident at once.
// Returns 0 on success, nonzero on a HIP error.
template <int B>
int launch_fused_batch(FusedArgs &a, int wtype, int gated, int NT, hipStream_t st);
template <> int launch_fused_batch<1>(FusedArgs &, int, int, int, hipStream_t);
template <> int launch_fused_batch<2>(FusedArgs &, int, int, int, hipStream_t);
template <> int launch_fused_batch<3>(FusedArgs &, int, int, int, hipStream_t);
template <> int launch_fused_batch<4>(FusedArgs &, int, int, int, hipStream_t);
template <> int launch_fused_batch<5>(FusedArgs &, int, int, int, hipStream_t);
template <> int launch_fused_batch<6>(FusedArgs &, int, int, int, hipStream_t);
template <> int launch_fused_batch<7>(FusedArgs &, int, int, int, hipStream_t);
template <> int launch_fused_batch<8>(FusedArgs &, int, int, int, hipStream_t);


}  // namespace pik
