// pi_kernels.hpp -- gfx950 kernels of the predictor-gated, neuron-aware sparse FFN.
//
// The method (PowerInfer, arXiv 2312.12456: abstract; "method" section of the summary page):
// a low-rank predictor picks the FFN neurons that will fire for the current token(s), and a
// neuron-aware operator reads and computes only those neurons; a GPU index of resident neurons
// restricts the device to the neurons it holds.  At batch <= 8 every step is a GEMV whose weights
// are read exactly once, so the path is HBM-bound and, at these sizes (a few MB to ~100 MB per
// kernel), bound just as much by how many serialized memory round trips a wave makes.  The
// kernels therefore issue every weight load a wave needs before anything else, overlap LDS
// staging of the token vectors with those loads, fetch per-neuron metadata with one lane per
// neuron, and accumulate fp16 products in fp32 with v_dot2.  Their ALU work grows with the batch,
// so from batch 3 (gated or Q4_0 rows) or 6 (plain fp16 rows) the sparse FFN runs on the MFMA
// kernels of pi_wide.hpp instead, and so does the predictor's second matrix from batch 3 (layers of
// 16384 neurons or more) or 6.
//
// Kernels (all stream-ordered; none needs a host sync):
//   k_pred_l1     z = max(0, P1 x)                   one workgroup per row of P1 (4 rows at batch >= 4)
//   k_pred_l2     l = P2 z + c, mask = OR_b [l > 0]  R rows per wave, reduce-scatter sums
//   k_compact     idx = ascending {i : mask_i, slot_of_i >= 0}, counts = {n, n_pred}
//   k_sparse_up   h = ReLU(W_in[s] x + b) or ReLU(W_g x)(W_u x) over the listed neurons
//   k_sparse_down y over (512-column slab, neuron chunk) tiles; waves reduced in LDS, chunks
//                 reduced by the last-arriving workgroup of each slab in fixed order
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pik {

constexpr int kWave = 64;
// Chunk partials per slab that k_sparse_down's last workgroup sums (measured on the 7168 x 28672
// fp16 layer at 3-5 tokens: 24 beats 16, 32 and 55 -- more chunks lengthen that sum, fewer
// lengthen each workgroup's walk over its rows).
constexpr int kDownMaxChunks = 24;

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));

enum { WT_F16 = 1, WT_Q4_0 = 2 };

// ------------------------------------------------------------------------------ helpers

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Loads through a buffer resource (base, size in bytes): the hardware returns zeros for an offset
// at or past the size and touches no memory, so a guarded load needs no branch -- pass kOOB as the
// offset (or as one of two summed parts of it) of a load that must not happen.  Buffers must stay
// below kBufMax bytes, so that a valid part plus kOOB, or kOOB plus kOOB, is still past the end
// and does not wrap around 2^32.
constexpr uint32_t kOOB = 0x40000000u;
constexpr uint64_t kBufMax = 0x40000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint64_t bld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t bld2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

__device__ __forceinline__ float half_to_float(uint16_t b) { return (float)__builtin_bit_cast(f16, b); }

// a.lo*b.lo + a.hi*b.hi + c with fp16 inputs and fp32 accumulation (v_dot2_f32_f16).
__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

__device__ __forceinline__ float dot8(const uint4 &a, const uint4 &b, float c) {
    c = fdot2(a.x, b.x, c);
    c = fdot2(a.y, b.y, c);
    c = fdot2(a.z, b.z, c);
    return fdot2(a.w, b.w, c);
}

// DPP lane permutation of v (gfx9 encodings: quad_perm, row_half_mirror, row_mirror).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, false);
}

// Inclusive prefix sum over the wave: shifts by 1, 2, 3 within each 16-lane row, then by 4 and 8
// (lanes that have them), then row 0's total into row 1 and row 2's into row 3, then rows 0-1's
// total into rows 2-3.  Lanes a move does not reach add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
    int s = x + dpp_i<0x111, 0xF, 0xF>(x);   // row_shr:1
    s += dpp_i<0x112, 0xF, 0xF>(x);           // row_shr:2
    s += dpp_i<0x113, 0xF, 0xF>(x);           // row_shr:3
    s += dpp_i<0x114, 0xF, 0xE>(s);           // row_shr:4, banks 1-3
    s += dpp_i<0x118, 0xF, 0xC>(s);           // row_shr:8, banks 2-3
    s += dpp_i<0x142, 0xA, 0xF>(s);           // row_bcast:15 into rows 1 and 3
    s += dpp_i<0x143, 0xC, 0xF>(s);           // row_bcast:31 into rows 2 and 3
    return s;
}

// Sum over the wave, returned in every lane.  Within each 16-lane row the sum is formed with DPP
// moves (swap neighbours, swap pairs, mirror halves, mirror the row: every lane then holds its
// row's sum), and the four row sums are added from scalar reads -- no LDS round trips, and a
// fixed order, so the result does not depend on timing.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);   // row_half_mirror
    v += dpp_f<0x140>(v);   // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Broadcast lane j's value (j wave-uniform) through a scalar register.
__device__ __forceinline__ int bcast(int v, int j) { return __builtin_amdgcn_readlane(v, j); }
__device__ __forceinline__ float bcastf(float v, int j) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
}

// Sum N per-lane values over the wave, leaving the total of value j in every lane l with
// j = l / (64/N) (so lanes 0, 64/N, 2*64/N, ... hold values 0, 1, 2, ...).  A reduce-scatter:
// each xor step halves the values a lane carries, then the 64/N lanes that share a value
// finish with plain xor steps -- log2(N) + N - 1 + log2(64/N) shuffles instead of 6N.
template <int N>
__device__ __forceinline__ float reduce_scatter(float (&v)[N], int lane) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16, "N");
#pragma unroll
    for (int lvl = 0; (N >> (lvl + 1)) >= 1; ++lvl) {
        const int m = 32 >> lvl, half = N >> (lvl + 1);
        const bool hi = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            // read both values into registers first: a select between two array loads would
            // otherwise become a lane-dependent index into the array, which lives in scratch
            float lo = v[i], up = v[i + half];
            asm volatile("" : "+v"(lo), "+v"(up));
            const float send = hi ? lo : up;
            const float keep = hi ? up : lo;
            v[i] = keep + __shfl_xor(send, m, kWave);
        }
    }
    float t = v[0];
#pragma unroll
    for (int m = 32 / N; m >= 1; m >>= 1) t += __shfl_xor(t, m, kWave);
    return t;
}

// Q4_0 codes: a 32-bit code word holds 8 consecutive weights, weight t in bits [4t, 4t+4).
// q4pair(w, 4i) = fp16 pair (code_i - 8, code_{i+4} - 8), exact: OR-ing a nibble into the
// mantissa of 1024.0 (0x6400) gives 1024 + code, and subtracting 1032 leaves code - 8.
__device__ __forceinline__ uint32_t q4pair(uint32_t w, int shift) {
    h2 p = __builtin_bit_cast(h2, ((w >> shift) & 0x000F000Fu) | 0x64006400u);
    p = p - h2{(f16)1032.0f, (f16)1032.0f};
    return __builtin_bit_cast(uint32_t, p);
}

// Re-pair 8 consecutive fp16 values x0..x7 as (x0,x4),(x1,x5),(x2,x6),(x3,x7): the order in
// which q4pair yields the codes of one code word.
__device__ __forceinline__ uint4 pair_for_q4(const uint4 &v) {
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

// Dot of one Q4_0 block (16 code bytes) with 32 staged x values (q4-paired order), times scale.
__device__ __forceinline__ float q4_block_dot(const uint4 &codes, const uint16_t *xq, float acc, float scale) {
    const uint32_t wd[4] = {codes.x, codes.y, codes.z, codes.w};
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint4 xv = *reinterpret_cast<const uint4 *>(xq + g * 8);
        s = fdot2(q4pair(wd[g], 0), xv.x, s);
        s = fdot2(q4pair(wd[g], 4), xv.y, s);
        s = fdot2(q4pair(wd[g], 8), xv.z, s);
        s = fdot2(q4pair(wd[g], 12), xv.w, s);
    }
    return fmaf(scale, s, acc);
}

// Stage columns [c0, c0+cw) of x [B][d] (fp16) into LDS xs [B][xch]; cw % 8 == 0, B*d*2 <
// kBufMax.  Each thread issues up to 8 loads (through a buffer resource: no branch, so the compiler
// issues them together) before its first LDS store, so staging costs one memory round trip per 8
// vectors a thread copies, not one per vector -- and does not drain the caller's loads in flight
// once per vector.
template <int B, bool Q4ORDER>
__device__ __forceinline__ void stage_x(uint16_t *xs, const uint16_t *__restrict__ x, int d, int c0, int cw,
                                        int xch) {
    constexpr int K = 8;
    const int vecs = cw >> 3, total = B * vecs;
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x, (uint32_t)(B * d) * 2);
    for (int t0 = threadIdx.x; t0 < total; t0 += K * blockDim.x) {
        uint4 v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int t = t0 + k * blockDim.x, b = t / vecs, vv = t - b * vecs;
            v[k] = bld16(rx, t < total ? (uint32_t)(b * d + c0 + vv * 8) * 2 : kOOB);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int t = t0 + k * blockDim.x, b = t / vecs, vv = t - b * vecs;
            if (t < total) *reinterpret_cast<uint4 *>(xs + b * xch + vv * 8) = Q4ORDER ? pair_for_q4(v[k]) : v[k];
        }
    }
}

// Copy n 16-byte vectors from global src to LDS dst (16-byte aligned, n*16 < kBufMax), up to 8
// loads per thread in flight before the first store.
__device__ __forceinline__ void stage_vec16(void *dst, const void *__restrict__ src, int n) {
    constexpr int K = 8;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(src, (uint32_t)n * 16);
    uint4 *d4 = static_cast<uint4 *>(dst);
    for (int t0 = threadIdx.x; t0 < n; t0 += K * blockDim.x) {
        uint4 v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int t = t0 + k * blockDim.x;
            v[k] = bld16(rs, t < n ? (uint32_t)t * 16 : kOOB);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int t = t0 + k * blockDim.x;
            if (t < n) d4[t] = v[k];
        }
    }
}

// Cross-workgroup exchange inside one kernel without L2-wide flushes: values are written with
// agent-coherent stores (global_store ... sc1, which do not linger dirty in one XCD's L2), each
// thread waits until its stores are acknowledged, and readers use agent-coherent loads (sc1),
// which do not return a stale line from their own XCD's L2.  An agent-scope fence would do the
// same with a whole-L2 writeback/invalidate (buffer_wbl2 / buffer_inv), far costlier here.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Slot of neuron id i, or -1 when i or its slot is out of range (then the entry is skipped).
__device__ __forceinline__ int slot_of_id(int i, const int32_t *__restrict__ slot_of, int f, int n_slots) {
    if (i < 0 || i >= f) return -1;
    const int s = slot_of ? slot_of[i] : i;
    return (s >= 0 && s < n_slots) ? s : -1;
}

// ------------------------------------------------------------------------------ predictor

// z[b][j] = max(0, P1[j] . x_b).  One 256-thread workgroup per RW consecutive rows: every
// thread issues its loads of all RW rows and of the matching x vectors of every token before the
// first product (each x vector read through L2 once serves all RW rows), then the four wave sums
// of each (row, token) meet in LDS.  Loads go through buffer resources, so columns past d and rows
// past r read zeros without a branch -- a guarded load would make the compiler wait for each x
// load in turn.  RW > 1 pays at larger batches, where re-reading x for every row would cost more
// L2 traffic than the rows themselves.  Requires B*d*2 < kBufMax.
constexpr int pred_l1_rows(int B) { return B >= 4 ? 4 : 1; }

// U: 16-byte loads per thread per row per pass (a pass covers U*2048 columns), chosen on the host
// so that a pass is not mostly past d.
template <int B, int RW, int U>
__global__ __launch_bounds__(256) void k_pred_l1(const uint16_t *__restrict__ p1, const uint16_t *__restrict__ x,
                                                 float *__restrict__ z, int d, int r) {
    __shared__ float red[4][RW][B];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int j0 = blockIdx.x * RW;
    __amdgpu_buffer_rsrc_t rrow[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i)
        rrow[i] = buf_rsrc(p1 + (size_t)min(j0 + i, r - 1) * d, j0 + i < r ? (uint32_t)d * 2 : 0u);
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x, (uint32_t)(B * d) * 2);
    float acc[RW][B];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = 0.f;
    for (int c0 = 0; c0 < d; c0 += U * 2048) {
        uint4 w[RW][U], xv[B][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int col = c0 + tid * 8 + u * 2048;
            const uint32_t off = col < d ? (uint32_t)col * 2 : kOOB;
#pragma unroll
            for (int i = 0; i < RW; ++i) w[i][u] = bld16(rrow[i], off);
        }
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int col = c0 + tid * 8 + u * 2048;
                xv[b][u] = bld16(rx, col < d ? (uint32_t)(b * d + col) * 2 : kOOB);
            }
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < RW; ++i) acc[i][b] = dot8(w[i][u], xv[b][u], acc[i][b]);
    }
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float s = wave_sum(acc[i][b]);
            if (lane == 0) red[wave][i][b] = s;
        }
    __syncthreads();
    if (tid < RW * B) {
        const int i = tid / B, b = tid - i * B;
        if (j0 + i < r) z[b * r + j0 + i] = fmaxf(red[0][i][b] + red[1][i][b] + red[2][i][b] + red[3][i][b], 0.f);
    }
}

// l[b][i] = P2[i] . z_b + c[i];  mask[i] = OR_b [l > 0].  Each wave owns R consecutive rows and
// issues all R*NT row loads at once; lane L covers columns L*8 + 512t (t < NT, r <= 512*NT), whose
// z values it reads from the workgroup's LDS copy of z once per token and reuses for all R rows;
// the R sums are finished with one reduce-scatter, after which lane (64/R)*i owns row i.
//
// When `bits` is given, the workgroup's 32 rows (R = 8) also leave one 32-bit word of listed flags:
// bit e of bits[blockIdx] is set when neuron 32*blockIdx + e fired for some token AND is resident
// (slot_of == nullptr, or 0 <= slot_of[i] < n_slots) -- the placement-restricted set the sparse FFN
// computes, which it can then read without a compaction pass.
template <int B, int NT, int R>
__global__ __launch_bounds__(256) void k_pred_l2(const uint16_t *__restrict__ p2, const uint16_t *__restrict__ c,
                                                 const float *__restrict__ z, int r, int f,
                                                 float *__restrict__ logits, uint8_t *__restrict__ mask,
                                                 uint32_t *__restrict__ bits, const int32_t *__restrict__ slot_of,
                                                 int n_slots) {
    __shared__ uint32_t s_bits[4];
    extern __shared__ __align__(16) float zs[];                // z [B][r], staged once per workgroup
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int row0 = min((blockIdx.x * 4 + wave) * R, f);        // f: this wave has no rows
    // the wave's rows (fewer at the end of P2) through a buffer resource: columns past r and rows
    // past f read zeros without a branch, so every load is issued before the first product
    const __amdgpu_buffer_rsrc_t rp = buf_rsrc(p2 + (size_t)row0 * r, (uint32_t)(min(R, f - row0) * r) * 2);
    uint4 w[R][NT];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int col = lane * 8 + t * 512;
            w[i][t] = bld16(rp, col < r ? (uint32_t)(i * r + col) * 2 : kOOB);
        }
    // z goes to LDS in one round trip (the rows' loads are already in flight), so no token waits
    // on a load of its own
    stage_vec16(zs, z, B * r / 4);
    __syncthreads();
    if (row0 >= f) {
        if (bits != nullptr) {
            if (lane == 0) s_bits[wave] = 0u;
            __syncthreads();
        }
        return;
    }
    const float c_lane = (lane < R && row0 + lane < f) ? half_to_float(c[row0 + lane]) : 0.f;
    constexpr int G = kWave / R;
    const int ri = lane / G;                                  // row owned after the reduce-scatter
    const bool owner = (lane % G) == 0 && row0 + ri < f;
    const float ci = __shfl(c_lane, ri, kWave);
    uint8_t m = 0;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float zr[NT][8];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // a lane past r reads column 0 (its weights are zero)
            const int col = lane * 8 + t * 512 < r ? lane * 8 + t * 512 : 0;
            const float4 za = *reinterpret_cast<const float4 *>(zs + b * r + col);
            const float4 zb = *reinterpret_cast<const float4 *>(zs + b * r + col + 4);
            zr[t][0] = za.x; zr[t][1] = za.y; zr[t][2] = za.z; zr[t][3] = za.w;
            zr[t][4] = zb.x; zr[t][5] = zb.y; zr[t][6] = zb.z; zr[t][7] = zb.w;
        }
        float v[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float s = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t q[4] = {w[i][t].x, w[i][t].y, w[i][t].z, w[i][t].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const h2 p = __builtin_bit_cast(h2, q[e]);
                    s = fmaf((float)p.x, zr[t][2 * e], s);
                    s = fmaf((float)p.y, zr[t][2 * e + 1], s);
                }
            }
            v[i] = s;
        }
        const float l = reduce_scatter<R>(v, lane) + ci;
        if (owner) {
            m |= (uint8_t)(l > 0.f);
            if (logits != nullptr) logits[(size_t)b * f + row0 + ri] = l;
        }
    }
    if (owner) mask[row0 + ri] = m;
    if (bits != nullptr) {
        static_assert(R == 8, "a workgroup's four waves cover one 32-row word");
        bool listed = false;
        if (owner && m) {
            const int sl = slot_of != nullptr ? slot_of[row0 + ri] : 0;
            listed = sl >= 0 && sl < n_slots;
        }
        const uint64_t bal = __ballot(listed);                 // owners sit at lanes 8*i
        uint32_t piece = 0;
#pragma unroll
        for (int i = 0; i < R; ++i) piece |= (uint32_t)((bal >> (i * G)) & 1u) << i;
        if (lane == 0) s_bits[wave] = piece;
        __syncthreads();
        if (threadIdx.x == 0) bits[blockIdx.x] = s_bits[0] | (s_bits[1] << 8) | (s_bits[2] << 16) | (s_bits[3] << 24);
    }
}

// ------------------------------------------------------------------------------ compaction

// One workgroup of 1024 threads.  Thread t owns the contiguous mask segment [t*seg, (t+1)*seg)
// (seg a multiple of 16), reads it with 16-byte loads, keeps the flags of its first 64 entries in
// a register (re-reading only beyond that), and a single block prefix sum over the per-thread
// counts gives every listed neuron its position -- so idx is ascending.  counts = {listed,
// predicted}.
static __global__ __launch_bounds__(1024) void k_compact(const uint8_t *__restrict__ mask, int f,
                                                  const int32_t *__restrict__ slot_of, int32_t *__restrict__ idx,
                                                  int32_t *__restrict__ counts) {
    __shared__ int wsum[16], wpred[16];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int seg = (((f + 1023) / 1024) + 15) & ~15;
    const int i0 = tid * seg;
    const int i1 = min(i0 + seg, f);
    const bool vec_ok = (reinterpret_cast<uintptr_t>(mask) & 15u) == 0;

    // flags of 64 entries starting at base (bit e = entry base+e predicted), before placement
    auto load_flags = [&](int base) -> uint64_t {
        uint64_t fl = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = base + v * 16;
            if (i >= i1) break;
            if (vec_ok && i + 16 <= i1) {
                const uint4 q = ld16(mask + i);
                const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    fl |= (uint64_t)(((wd[e >> 2] >> (8 * (e & 3))) & 0xFFu) != 0) << (v * 16 + e);
            } else {
                for (int e = 0; e < 16 && i + e < i1; ++e) fl |= (uint64_t)(mask[i + e] != 0) << (v * 16 + e);
            }
        }
        return fl;
    };
    const bool so_vec = (reinterpret_cast<uintptr_t>(slot_of) & 15u) == 0;
    // drop predicted entries that are not resident; the slot loads of a window are all issued
    // before any of them is tested
    auto restrict_flags = [&](uint64_t fl, int base) -> uint64_t {
        if (slot_of == nullptr || fl == 0) return fl;
        uint64_t keep = 0;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = base + v * 4;
            const bool need = ((fl >> (v * 4)) & 0xFull) != 0 && i < i1;
            int s0 = -1, s1 = -1, s2 = -1, s3 = -1;
            if (need) {
                if (so_vec && i + 4 <= i1) {
                    const int4 q = *reinterpret_cast<const int4 *>(slot_of + i);
                    s0 = q.x; s1 = q.y; s2 = q.z; s3 = q.w;
                } else {
                    s0 = slot_of[i];
                    if (i + 1 < i1) s1 = slot_of[i + 1];
                    if (i + 2 < i1) s2 = slot_of[i + 2];
                    if (i + 3 < i1) s3 = slot_of[i + 3];
                }
            }
            keep |= ((uint64_t)(s0 >= 0) | ((uint64_t)(s1 >= 0) << 1) | ((uint64_t)(s2 >= 0) << 2) |
                     ((uint64_t)(s3 >= 0) << 3)) << (v * 4);
        }
        return fl & keep;
    };

    int cnt = 0, npred = 0;
    uint64_t first_act = 0;
    for (int base = i0; base < i1; base += 64) {
        const uint64_t fl = load_flags(base);
        const uint64_t act = restrict_flags(fl, base);
        if (base == i0) first_act = act;
        npred += __popcll(fl);
        cnt += __popcll(act);
    }
    // block exclusive scan of cnt
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    int wp = npred;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) wp += __shfl_xor(wp, o, kWave);
    if (lane == kWave - 1) wsum[wave] = incl;
    if (lane == 0) wpred[wave] = wp;
    __syncthreads();
    int before = 0, total = 0, tpred = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        before += (w < wave) ? wsum[w] : 0;
        total += wsum[w];
        tpred += wpred[w];
    }
    int pos = before + incl - cnt;
    for (int base = i0; base < i1; base += 64) {
        uint64_t act = (base == i0) ? first_act : restrict_flags(load_flags(base), base);
        for (; act; act &= act - 1) idx[pos++] = base + __builtin_ctzll(act);
    }
    if (tid == 0) {
        counts[0] = total;
        counts[1] = tpred;
    }
}

// The same list from the predictor's flag words instead of the mask bytes (one workgroup; at most
// 4 words per thread, so d_ffn <= 131072): bit e of bits[w] = neuron 32w + e predicted.  A 32-fold
// smaller read than the mask; slot_of (or NULL) is looked up only for the predicted neurons.
static __global__ __launch_bounds__(1024) void k_compact_bits(const uint32_t *__restrict__ bits, int nwords,
                                                       const int32_t *__restrict__ slot_of, int n_slots,
                                                       int32_t *__restrict__ idx, int32_t *__restrict__ counts) {
    __shared__ int wsum[16], wpred[16];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int per = (nwords + 1023) / 1024;                  // <= 4
    const int w0 = tid * per;
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(bits, (uint32_t)nwords * 4u);
    uint32_t wv[4], act[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) wv[v] = bld4(rw, (v < per && w0 + v < nwords) ? (uint32_t)(w0 + v) * 4u : kOOB);
    int cnt = 0, npred = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        act[v] = wv[v];
        if (slot_of != nullptr) {
            act[v] = 0u;
            for (uint32_t m = wv[v]; m != 0u; m &= m - 1u) {
                const int b = __builtin_ctz(m), sl = slot_of[(w0 + v) * 32 + b];
                if (sl >= 0 && sl < n_slots) act[v] |= 1u << b;
            }
        }
        npred += __popc(wv[v]);
        cnt += __popc(act[v]);
    }
    const int incl = wave_incl_scan(cnt);
    int wp = npred;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) wp += __shfl_xor(wp, o, kWave);
    if (lane == kWave - 1) wsum[wave] = incl;
    if (lane == 0) wpred[wave] = wp;
    __syncthreads();
    int before = 0, total = 0, tpred = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        before += (w < wave) ? wsum[w] : 0;
        total += wsum[w];
        tpred += wpred[w];
    }
    int pos = before + incl - cnt;
#pragma unroll
    for (int v = 0; v < 4; ++v)
        for (uint32_t m = act[v]; m != 0u; m &= m - 1u) idx[pos++] = (w0 + v) * 32 + __builtin_ctz(m);
    if (tid == 0) {
        counts[0] = total;
        counts[1] = tpred;
    }
}

// ------------------------------------------------------------------------------ sparse FFN

// One pass of a neuron's row dot products, split into "issue the loads" and "consume them" so
// that callers can overlap the loads with other work (x staging, the next lookup).
//   fp16: lane L covers columns c0 + L*8 + 512v, v < V (16 vectors of one row, or 8 of each of the
//         gate and up rows so that both are in flight together).
//   Q4_0: lane L covers 32-weight blocks q0 + L + 64v, v < V (16 code bytes + one scale each).
template <int B, bool GATED, int WT>
struct RowPass {
    static constexpr int V = (WT == WT_F16) ? (GATED ? 8 : 16) : 8;
    static constexpr int STEP = (WT == WT_F16) ? V * 512 : V * kWave;   // columns (fp16) or blocks (Q4_0) per pass
    uint4 wu[V];
    uint4 wg[GATED ? V : 1];
    uint16_t sc[WT == WT_Q4_0 ? V : 1];

    __device__ __forceinline__ static int extent(int d) { return WT == WT_F16 ? d : d / 32; }

    __device__ __forceinline__ void issue(const uint8_t *__restrict__ row, int64_t row_bytes, int d, int p0,
                                          int lane) {
        if (WT == WT_F16) {
            const uint16_t *gr = reinterpret_cast<const uint16_t *>(row);
            const uint16_t *ur = reinterpret_cast<const uint16_t *>(row + (GATED ? row_bytes : 0));
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int col = p0 + lane * 8 + v * 512;
                wu[v] = col < d ? ld16(ur + col) : zero4();
                if (GATED) wg[GATED ? v : 0] = col < d ? ld16(gr + col) : zero4();
            }
        } else {
            // Unconditional loads from a clamped block (consume() skips blocks past the row):
            // a guarded load would let the compiler pull the scale conversion into the guard and
            // wait for each block's load before issuing the next.
            const uint16_t *scales = reinterpret_cast<const uint16_t *>(row + d / 2);
            const int nq = d / 32;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int q = min(p0 + lane + v * kWave, nq - 1);
                wu[v] = ld16(row + (size_t)q * 16);
                sc[WT == WT_Q4_0 ? v : 0] = scales[q];
            }
        }
    }

    // The same loads through a buffer resource over the rows, the neuron's row(s) starting at byte
    // `base`; no branches (columns past d read zeros).
    __device__ __forceinline__ void issue_buf(__amdgpu_buffer_rsrc_t r, uint32_t base, int64_t row_bytes, int d,
                                              int p0, int lane) {
        if (WT == WT_F16) {
            const uint32_t gb = base, ub = base + (GATED ? (uint32_t)row_bytes : 0u);
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int col = p0 + lane * 8 + v * 512;
                wu[v] = bld16(r, col < d ? ub + (uint32_t)col * 2 : kOOB);
                if (GATED) wg[GATED ? v : 0] = bld16(r, col < d ? gb + (uint32_t)col * 2 : kOOB);
            }
        } else {
            const int nq = d / 32;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int q = p0 + lane + v * kWave;
                wu[v] = bld16(r, q < nq ? base + (uint32_t)q * 16 : kOOB);
                sc[WT == WT_Q4_0 ? v : 0] = bld2(r, q < nq ? base + (uint32_t)(d / 2) + (uint32_t)q * 2 : kOOB);
            }
        }
    }

    __device__ __forceinline__ void consume(const uint16_t *xs, int xstride, int d, int p0, int lane, float (&ag)[B],
                                            float (&au)[B]) const {
        if (WT == WT_F16) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int col = p0 + lane * 8 + v * 512;
                if (col < d) {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const uint4 xv = *reinterpret_cast<const uint4 *>(xs + b * xstride + col);
                        au[b] = dot8(wu[v], xv, au[b]);
                        if (GATED) ag[b] = dot8(wg[GATED ? v : 0], xv, ag[b]);
                    }
                }
            }
        } else {
            const int nq = d / 32;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int q = p0 + lane + v * kWave;
                if (q < nq) {
                    const float s = half_to_float(sc[WT == WT_Q4_0 ? v : 0]);
#pragma unroll
                    for (int b = 0; b < B; ++b) au[b] = q4_block_dot(wu[v], xs + b * xstride + q * 32, au[b], s);
                }
            }
        }
    }
};

// All passes of one neuron's row dots against x staged in LDS (row: the neuron's w_in row).
template <int B, bool GATED, int WT>
__device__ __forceinline__ void neuron_dots(const uint8_t *__restrict__ row, int64_t row_bytes, int d,
                                            const uint16_t *xs, int xstride, int lane, float (&ag)[B],
                                            float (&au)[B]) {
    using P = RowPass<B, GATED, WT>;
    for (int p0 = 0; p0 < P::extent(d); p0 += P::STEP) {
        P pass;
        pass.issue(row, row_bytes, d, p0, lane);
        pass.consume(xs, xstride, d, p0, lane, ag, au);
    }
}

// Epilogue of one neuron: finish the wave sums and apply bias + ReLU (or the ReGLU product).
template <int B, bool GATED>
__device__ __forceinline__ void neuron_store(float (&ag)[B], float (&au)[B], int s, int k, const uint16_t *b_up,
                                             float *__restrict__ h, int h_stride, int lane, int act) {
    const float bias = (!GATED && b_up != nullptr && s >= 0) ? half_to_float(b_up[s]) : 0.f;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float u = wave_sum(au[b]);
        float hv;
        if (GATED) {
            const float g = wave_sum(ag[b]);
            hv = fmaxf(g, 0.f) * u;
        } else {
            hv = fmaxf(u + bias, 0.f);
            if (act) hv *= hv;                          // squared ReLU
        }
        if (lane == 0) h[(size_t)b * h_stride + k] = (s >= 0) ? hv : 0.f;
    }
}

// Shape of one step of k_sparse_up: each lane holds U vectors of each of the wave's R neurons
// (fp16: 8 columns per 16-byte vector; Q4_0: one 32-weight block), so a step covers STEP columns.
template <bool GATED, int WT>
struct UpStep {
    static constexpr int R = 4;                                        // neurons per wave at once
    static constexpr int U = WT == WT_F16 ? (GATED ? 2 : 4) : 2;       // vectors per lane per neuron
    static constexpr int VC = WT == WT_F16 ? 8 : 32;                   // columns per vector
    static constexpr int STEP = U * kWave * VC;
};

// h[b][k] for the listed neurons, R neurons per wave at a time.  In pass p, wave w of workgroup g
// holds positions p*R*4G + j*4G + w*G + g (j < R), which spreads the listed neurons over every
// workgroup (and so every CU) first.  x is staged in LDS in column chunks of xch columns (all of
// it when B*d fp16 fit the LDS budget).  For each step of a chunk the loads of all R neurons' row
// pieces go out first (for the chunk's first step, before the chunk is staged, so the two
// latencies overlap), and every x vector read from LDS serves all R neurons.  Each neuron's row
// is read through a buffer resource of its own: a position past n, or a neuron without a slot,
// reads zeros and touches no memory, so no load needs a branch.  Workgroup 0 also clears
// `zero_ptr[0..nzero)` (the down kernel's slab tickets) -- the down kernel always runs after this
// one on the same stream.
template <int B, bool GATED, int WT>
__global__ __launch_bounds__(256) void k_sparse_up(const uint8_t *__restrict__ w_in, int64_t row_bytes, int d,
                                                   const uint16_t *__restrict__ b_up, const uint16_t *__restrict__ x,
                                                   const int32_t *__restrict__ idx, const int32_t *__restrict__ counts,
                                                   const int32_t *__restrict__ slot_of, int f, int n_slots,
                                                   float *__restrict__ h, int h_stride, int xch,
                                                   int32_t *__restrict__ zero_ptr, int nzero, int act) {
    using S = UpStep<GATED, WT>;
    constexpr int R = S::R, U = S::U, VC = S::VC, STEP = S::STEP;
    constexpr int RG = GATED ? R : 1;
    extern __shared__ __align__(16) uint16_t xs[];
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (blockIdx.x == 0)
        for (int t = threadIdx.x; t < nzero; t += blockDim.x) zero_ptr[t] = 0;
    const int G = gridDim.x;
    const int n = min(max(counts[0], 0), n_slots);
    const int64_t in_stride = GATED ? 2 * row_bytes : row_bytes;
    const uint32_t up_off = GATED ? (uint32_t)row_bytes : 0u;           // the up row follows the gate row
    const int nchunks = (d + xch - 1) / xch;

    for (int p0 = 0; p0 < n; p0 += R * 4 * G) {
        if (p0 + (int)blockIdx.x >= n) break;                           // workgroup-uniform
        int kj[R], sj[R];
        __amdgpu_buffer_rsrc_t rs[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            kj[j] = p0 + j * 4 * G + wave * G + (int)blockIdx.x;
            const int s = kj[j] < n ? slot_of_id(idx[kj[j]], slot_of, f, n_slots) : -1;
            sj[j] = __builtin_amdgcn_readfirstlane(s);
            rs[j] = buf_rsrc(w_in + (int64_t)(sj[j] >= 0 ? sj[j] : 0) * in_stride, sj[j] >= 0 ? (uint32_t)in_stride : 0u);
        }
        float au[R][B], ag[RG][B];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                au[j][b] = 0.f;
                if (GATED) ag[GATED ? j : 0][b] = 0.f;
            }
        for (int ch = 0; ch < nchunks; ++ch) {
            const int c0 = ch * xch, cw = min(xch, d - c0);
            for (int st = 0; st < cw; st += STEP) {
                uint4 wu[R][U], wg[RG][U];
                uint16_t sc[R][WT == WT_Q4_0 ? U : 1];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int lc = st + (u * kWave + lane) * VC;            // column inside the chunk
                    const bool ok = lc < cw;
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        if (WT == WT_F16) {
                            const uint32_t off = ok ? (uint32_t)(c0 + lc) * 2 : kOOB;
                            wu[j][u] = bld16(rs[j], off + up_off);
                            if (GATED) wg[GATED ? j : 0][u] = bld16(rs[j], off);
                        } else {
                            const uint32_t q = (uint32_t)(c0 + lc) / 32;
                            wu[j][u] = bld16(rs[j], ok ? q * 16 : kOOB);
                            sc[j][WT == WT_Q4_0 ? u : 0] = bld2(rs[j], ok ? (uint32_t)(d / 2) + q * 2 : kOOB);
                        }
                    }
                }
                if (st == 0) {
                    __syncthreads();                                    // the previous chunk is consumed
                    stage_x<B, WT == WT_Q4_0>(xs, x, d, c0, cw, xch);
                    __syncthreads();
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    // a lane past the chunk reads x at column 0 of it; its weights (and, for Q4_0,
                    // its scales) were read as zeros, so it adds nothing, and no LDS read waits on
                    // a branch
                    const int lc = st + (u * kWave + lane) * VC < cw ? st + (u * kWave + lane) * VC : 0;
                    if (WT == WT_F16) {
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            const uint4 xv = *reinterpret_cast<const uint4 *>(xs + b * xch + lc);
#pragma unroll
                            for (int j = 0; j < R; ++j) {
                                au[j][b] = dot8(wu[j][u], xv, au[j][b]);
                                if (GATED) ag[GATED ? j : 0][b] = dot8(wg[GATED ? j : 0][u], xv, ag[GATED ? j : 0][b]);
                            }
                        }
                    } else {
                        float t[R][B];
#pragma unroll
                        for (int j = 0; j < R; ++j)
#pragma unroll
                            for (int b = 0; b < B; ++b) t[j][b] = 0.f;
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            uint32_t pr[R][4];
#pragma unroll
                            for (int j = 0; j < R; ++j) {
                                const uint32_t cwd = g == 0 ? wu[j][u].x : g == 1 ? wu[j][u].y : g == 2 ? wu[j][u].z : wu[j][u].w;
#pragma unroll
                                for (int e = 0; e < 4; ++e) pr[j][e] = q4pair(cwd, 4 * e);
                            }
#pragma unroll
                            for (int b = 0; b < B; ++b) {
                                const uint4 xv = *reinterpret_cast<const uint4 *>(xs + b * xch + lc + g * 8);
#pragma unroll
                                for (int j = 0; j < R; ++j) {
                                    float s = t[j][b];
                                    s = fdot2(pr[j][0], xv.x, s);
                                    s = fdot2(pr[j][1], xv.y, s);
                                    s = fdot2(pr[j][2], xv.z, s);
                                    s = fdot2(pr[j][3], xv.w, s);
                                    t[j][b] = s;
                                }
                            }
                        }
#pragma unroll
                        for (int j = 0; j < R; ++j) {
                            const float scf = half_to_float(sc[j][WT == WT_Q4_0 ? u : 0]);
#pragma unroll
                            for (int b = 0; b < B; ++b) au[j][b] = fmaf(scf, t[j][b], au[j][b]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (kj[j] >= n) continue;                                   // wave-uniform
            float gj[B], uj[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                uj[b] = au[j][b];
                gj[b] = GATED ? ag[GATED ? j : 0][b] : 0.f;
            }
            neuron_store<B, GATED>(gj, uj, sj[j], kj[j], b_up, h, h_stride, lane, act);
        }
    }
}

// y over (512-column slab, neuron chunk) tiles.  Lane L owns columns slab*512 + 8L .. +8.  The
// chunk's neurons are dealt round-robin to the 4 waves; a wave fetches the metadata (index, h,
// slot) of up to 64 of its neurons at once, one lane per neuron, drops neurons whose h is zero
// for every token (an exact zero contribution), and walks the rest U at a time (16 fp16 or 32
// Q4_0 rows) with all U row reads in flight.  The waves' partials meet in LDS; each chunk's
// partial goes to `part`, and the last workgroup to finish a slab (slab ticket) sums the chunk
// partials in chunk order and adds b_down, so y is deterministic.  Tickets must be zero on entry (k_sparse_up clears them)
// and are left zero.
template <int B, int WT>
__global__ __launch_bounds__(256) void k_sparse_down(const uint8_t *__restrict__ w_dn, int64_t row_bytes, int d,
                                                     const int32_t *__restrict__ idx, const int32_t *__restrict__ counts,
                                                     const int32_t *__restrict__ slot_of, int f, int n_slots,
                                                     const float *__restrict__ h, int h_stride,
                                                     float *__restrict__ part, int C, int32_t *__restrict__ tickets,
                                                     const uint16_t *__restrict__ b_down, float *__restrict__ y) {
    constexpr int U = WT == WT_F16 ? 16 : 32;                    // rows in flight per wave
    constexpr int HB = (B + 3) / 4 * 4;
    __shared__ float red[4][B][8][kWave];
    __shared__ __align__(16) float s_h[4][kWave][HB];           // h of the wave's 64 positions
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int slab = blockIdx.x, ck = blockIdx.y;
    const int n = min(max(counts[0], 0), n_slots);
    const int k0 = (int)((int64_t)n * ck / C), k1 = (int)((int64_t)n * (ck + 1) / C);
    const int col = slab * 512 + lane * 8;
    const bool colok = col < d;
    float acc[B][8];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[b][t] = 0.f;

    for (int base = k0 + wave; base < k1; base += 4 * kWave) {
        const int kk = base + 4 * lane;
        const bool in = kk < k1;
        const int id = in ? idx[kk] : -1;
        float hv[B];
        bool any = false;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            hv[b] = in ? h[(size_t)b * h_stride + kk] : 0.f;
            any |= hv[b] != 0.f;
        }
        const int sl = (in && any) ? slot_of_id(id, slot_of, f, n_slots) : -1;
        uint64_t live = __ballot(sl >= 0);
        // every lane's h goes to the wave's LDS rows, so that a row's B values are read back with
        // B/4 broadcast loads instead of B cross-lane reads (no other wave touches these rows)
#pragma unroll
        for (int b = 0; b < B; ++b) s_h[wave][lane][b] = hv[b];
        auto h_of = [&](int j, float (&hb)[B]) {
#pragma unroll
            for (int q = 0; q < HB / 4; ++q) {
                const float4 v = *reinterpret_cast<const float4 *>(&s_h[wave][j][4 * q]);
                const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (4 * q + k < B) hb[4 * q + k] = e[k];
            }
        };
        while (live) {                                           // wave-uniform
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
                    wv[u] = (s >= 0 && colok) ? ld16(w_dn + (int64_t)s * row_bytes + (int64_t)col * 2) : zero4();
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (js[u] < 0) continue;                     // wave-uniform
                    const uint32_t wq[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
                    float hb[B];
                    h_of(js[u], hb);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const h2 pr = __builtin_bit_cast(h2, wq[p]);
                            acc[b][2 * p] = fmaf(hb[b], (float)pr.x, acc[b][2 * p]);
                            acc[b][2 * p + 1] = fmaf(hb[b], (float)pr.y, acc[b][2 * p + 1]);
                        }
                    }
                }
            } else {
                uint32_t cw[U];
                uint16_t sc[U];
                bool okv[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    // unconditional loads (row 0, column 0 stand in for an absent row or column),
                    // so that all U rows are in flight before the first scale is converted
                    const int s = js[u] >= 0 ? bcast(sl, js[u]) : -1;
                    okv[u] = s >= 0 && colok;
                    const uint8_t *row = w_dn + (int64_t)(okv[u] ? s : 0) * row_bytes;
                    const int cc = colok ? col : 0;
                    cw[u] = *reinterpret_cast<const uint32_t *>(row + cc / 2);
                    sc[u] = *reinterpret_cast<const uint16_t *>(row + d / 2 + (cc / 32) * 2);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (js[u] < 0) continue;
                    const float scf = okv[u] ? half_to_float(sc[u]) : 0.f;
                    float cf[B];
                    h_of(js[u], cf);
#pragma unroll
                    for (int b = 0; b < B; ++b) cf[b] *= scf;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        // q4pair(w, 4p) = (code_p - 8, code_{p+4} - 8): columns p and p+4.
                        const h2 pr = __builtin_bit_cast(h2, q4pair(cw[u], 4 * p));
                        const float lo = (float)pr.x, hi = (float)pr.y;
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            acc[b][p] = fmaf(cf[b], lo, acc[b][p]);
                            acc[b][p + 4] = fmaf(cf[b], hi, acc[b][p + 4]);
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int t = 0; t < 8; ++t) red[wave][b][t][lane] = acc[b][t];
    __syncthreads();
    const int Bd = B * d;
    for (int o = tid; o < B * 512; o += blockDim.x) {
        const int b = o / 512, cc = o - b * 512;
        const int ln = cc >> 3, t = cc & 7;
        const int gcol = slab * 512 + cc;
        if (gcol < d)
            store_coherent(part + (size_t)ck * Bd + (size_t)b * d + gcol,
                           red[0][b][t][ln] + red[1][b][t][ln] + red[2][b][t][ln] + red[3][b][t][ln]);
    }
    wait_stores_done();                                          // this thread's partials are out
    __syncthreads();                                             // ... and so are everyone's
    if (tid == 0) s_last = (atomicAdd(&tickets[slab], 1) == C - 1);
    __syncthreads();
    if (!s_last) return;
    // Sum the chunk partials of this slab in chunk order.  All C loads of an output are issued
    // before the first add (a load-add loop would wait out one memory round trip per chunk).
    for (int o = tid; o < B * 512; o += blockDim.x) {
        const int b = o / 512, cc = o - b * 512;
        const int gcol = slab * 512 + cc;
        const bool ok = gcol < d;
        const size_t off = (size_t)b * d + (ok ? gcol : 0);
        float v[kDownMaxChunks];
#pragma unroll
        for (int c = 0; c < kDownMaxChunks; ++c) v[c] = (ok && c < C) ? load_coherent(part + (size_t)c * Bd + off) : 0.f;
        float s = (ok && b_down) ? half_to_float(b_down[gcol]) : 0.f;
#pragma unroll
        for (int c = 0; c < kDownMaxChunks; ++c) s += v[c];
        if (ok) y[off] = s;
    }
    if (tid == 0) tickets[slab] = 0;
}

}  // namespace pik
