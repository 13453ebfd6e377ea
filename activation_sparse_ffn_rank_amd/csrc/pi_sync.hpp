// pi_sync.hpp -- hand-offs between the workgroups of one launch (the persistent kernels).
//
// A value handed to another workgroup is a 64-bit word (value | stamp << 32) written with an
// agent-coherent store (single-copy atomic; it does not linger dirty in one XCD's L2) and read with
// agent-coherent loads, which do not return a stale line from the reader's own L2.  The stamp is the
// launch's epoch + 1, so a consumer tells a fresh word from a stale one by its upper half and
// nothing has to be cleared between launches; it re-reads only the words that are still stale, so
// no producer waits for acknowledgements and no separate ready flag is needed.  Agent-scope fences
// are avoided: on gfx950 they compile to whole-L2 writeback/invalidate.
//
// The control block (int32 words, each on its own 128-byte line) holds the epoch, the exit count
// (the last workgroup out advances the epoch), an abort flag and a sticky status word.  Every wait
// is bounded (kSpinTicks of the constant 100 MHz clock); a wait that runs out raises the abort
// flag, which releases every other wait so the grid always drains, and ORs a code into the status
// word for the host.  The control block must be zero-filled before its first use.
#pragma once

#include "pi_kernels.hpp"

namespace pik {

constexpr uint64_t kSpinTicks = 2000000;       // 20 ms of the 100 MHz real-time clock

enum : int {
    CTL_EPOCH = 0,
    CTL_EXIT = 32,
    CTL_ABORT = 64,
    CTL_STATUS = 96,                           // byte offset 384
    CTL_WORDS = 128,
};

__device__ __forceinline__ int32_t load_coherent_i(const int32_t *p) {
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_i(int32_t *p, int32_t v) {
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

// Called by every lane of a wave after a poll that re-issued its loads together with a load of the
// abort word (`ab`, lane 0's copy counts): true when the wave must stop waiting -- the abort flag is
// up, or this wait ran past kSpinTicks, which raises the flag and records `code`.
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

// Workgroup-wide exit of a persistent launch of `grid` workgroups: the last one out clears the
// abort flag and the exit count and advances the epoch (so the next launch's stamp is new).
__device__ __forceinline__ void persistent_exit(int32_t *ctl, uint32_t stamp, int grid) {
    __syncthreads();
    if (threadIdx.x == 0) {
        if (atomicAdd(ctl + CTL_EXIT, 1) == grid - 1) {
            store_coherent_i(ctl + CTL_ABORT, 0);
            store_coherent_i(ctl + CTL_EXIT, 0);
            store_coherent_i(ctl + CTL_EPOCH, (int32_t)stamp);
        }
    }
}

}  // namespace pik
