// pi_kernels.hpp -- gfx950 kernels of the predictor-gated, neuron-aware sparse FFN.
//
// The method (PowerInfer, arXiv 2312.12456: abstract; "method" section of the summary page):
// a low-rank predictor picks the FFN neurons that will fire for the current token(s), and a
// neuron-aware operator reads and computes only those neurons; a GPU index of resident neurons
// restricts the device to the neurons it holds.  At batch 1 every step is a GEMV whose weights
// are read exactly once, so the whole path is HBM-bound: the kernels are built around wide,
// coalesced 16-byte row reads with many loads in flight per wave, token vectors staged in LDS,
// fp16 products accumulated in fp32 with v_dot2, wavefront reductions, and no MFMA (there is no
// dense contraction to feed it at batch <= 8).
//
// Kernels (one launch each, all stream-ordered, none needs a host sync):
//   k_pred_l1     z = max(0, P1 x)                 one wave per row of P1, x in LDS
//   k_pred_l2     l = P2 z + c, mask = OR_b [l > 0] several rows per wave, z in LDS
//   k_compact     idx = ascending {i : mask_i, slot_of_i >= 0}, counts = {n, n_pred}
//   k_sparse_up   h = ReLU(W_in[s] x + b) or ReLU(W_g x)(W_u x) for the active rows
//   k_sparse_down partial y over (column slab, neuron chunk) tiles, fp32, waves reduced in LDS
//   k_reduce_y    y = b_down + sum of the chunk partials (fixed order: deterministic)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pik {

constexpr int kWave = 64;

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));

enum { WT_F16 = 1, WT_Q4_0 = 2 };

// ------------------------------------------------------------------------------ helpers

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
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

// Stage columns [c0, c0+cw) of x [B][d] (fp16) into LDS xs [B][xch]; cw % 8 == 0.
template <int B, bool Q4ORDER>
__device__ __forceinline__ void stage_x(uint16_t *xs, const uint16_t *__restrict__ x, int d, int c0, int cw,
                                        int xch) {
    const int vecs = cw >> 3;
    for (int t = threadIdx.x; t < B * vecs; t += blockDim.x) {
        const int b = t / vecs, v = t - b * vecs;
        uint4 val = ld16(x + (size_t)b * d + c0 + v * 8);
        if (Q4ORDER) val = pair_for_q4(val);
        *reinterpret_cast<uint4 *>(xs + b * xch + v * 8) = val;
    }
}

// ------------------------------------------------------------------------------ predictor

// z[b][j] = max(0, P1[j] . x_b).  One wave per row j; 4 waves per workgroup; x staged in LDS in
// column chunks of xch (a single chunk whenever B*d fp16 values fit the LDS budget).
template <int B>
__global__ __launch_bounds__(256) void k_pred_l1(const uint16_t *__restrict__ p1, const uint16_t *__restrict__ x,
                                                 float *__restrict__ z, int d, int r, int xch) {
    extern __shared__ __align__(16) uint16_t xs[];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int j = blockIdx.x * 4 + wave;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    for (int c0 = 0; c0 < d; c0 += xch) {
        const int cw = min(xch, d - c0);
        stage_x<B, false>(xs, x, d, c0, cw, xch);
        __syncthreads();
        if (j < r) {
            const uint16_t *row = p1 + (size_t)j * d + c0;
            int col = lane * 8;
            for (; col + 3 * 512 < cw; col += 4 * 512) {       // 4 loads in flight per lane
                uint4 w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) w[u] = ld16(row + col + u * 512);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        acc[b] = dot8(w[u], *reinterpret_cast<const uint4 *>(xs + b * xch + col + u * 512), acc[b]);
            }
            for (; col < cw; col += 512) {
                uint4 w = ld16(row + col);
#pragma unroll
                for (int b = 0; b < B; ++b)
                    acc[b] = dot8(w, *reinterpret_cast<const uint4 *>(xs + b * xch + col), acc[b]);
            }
        }
        __syncthreads();
    }
    if (j < r) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float s = wave_sum(acc[b]);
            if (lane == 0) z[b * r + j] = fmaxf(s, 0.f);
        }
    }
}

// l[b][i] = P2[i] . z_b + c[i];  mask[i] = OR_b [l > 0].  z [B][r] staged in LDS (fp32).
// Each wave handles RPW consecutive rows, NT 16-byte column groups per lane (r <= 512*NT).
template <int B, int NT, int RPW>
__global__ __launch_bounds__(256) void k_pred_l2(const uint16_t *__restrict__ p2, const uint16_t *__restrict__ c,
                                                 const float *__restrict__ z, int r, int f,
                                                 float *__restrict__ logits, uint8_t *__restrict__ mask) {
    extern __shared__ __align__(16) float zs[];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int t = threadIdx.x; t < B * r / 4; t += blockDim.x)
        reinterpret_cast<float4 *>(zs)[t] = reinterpret_cast<const float4 *>(z)[t];
    __syncthreads();
    const int row0 = (blockIdx.x * 4 + wave) * RPW;
    if (row0 >= f) return;
#pragma unroll 1
    for (int rr = 0; rr < RPW; rr += 4) {
        uint4 w[4][NT];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = row0 + rr + u;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int col = lane * 8 + t * 512;
                w[u][t] = (i < f && col < r) ? ld16(p2 + (size_t)i * r + col) : make_uint4(0, 0, 0, 0);
            }
        }
        float acc[4][B];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[u][b] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int col = lane * 8 + t * 512;
            if (col < r) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float4 za = *reinterpret_cast<const float4 *>(zs + b * r + col);
                    const float4 zb = *reinterpret_cast<const float4 *>(zs + b * r + col + 4);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const h2 a0 = __builtin_bit_cast(h2, w[u][t].x), a1 = __builtin_bit_cast(h2, w[u][t].y);
                        const h2 a2 = __builtin_bit_cast(h2, w[u][t].z), a3 = __builtin_bit_cast(h2, w[u][t].w);
                        float s = acc[u][b];
                        s = fmaf((float)a0.x, za.x, s); s = fmaf((float)a0.y, za.y, s);
                        s = fmaf((float)a1.x, za.z, s); s = fmaf((float)a1.y, za.w, s);
                        s = fmaf((float)a2.x, zb.x, s); s = fmaf((float)a2.y, zb.y, s);
                        s = fmaf((float)a3.x, zb.z, s); s = fmaf((float)a3.y, zb.w, s);
                        acc[u][b] = s;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = row0 + rr + u;
            if (i >= f) break;                                   // wave-uniform
            const float ci = half_to_float(c[i]);
            uint8_t m = 0;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float l = wave_sum(acc[u][b]) + ci;
                m |= (uint8_t)(l > 0.f);
                if (logits != nullptr && lane == 0) logits[(size_t)b * f + i] = l;
            }
            if (lane == 0) mask[i] = m;
        }
    }
}

// ------------------------------------------------------------------------------ compaction

// One workgroup of 1024 threads walks the mask in tiles of 4096 entries: each thread flags 4
// entries, a wave prefix sum plus a 16-entry LDS scan give every flagged entry its position,
// so idx comes out in ascending order.  counts = {listed, predicted}.
__global__ __launch_bounds__(1024) void k_compact(const uint8_t *__restrict__ mask, int f,
                                                  const int32_t *__restrict__ slot_of, int32_t *__restrict__ idx,
                                                  int32_t *__restrict__ counts) {
    __shared__ int wsum[16];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    int base = 0, npred = 0;
    for (int t0 = 0; t0 < f; t0 += 4096) {
        const int i0 = t0 + tid * 4;
        int flags = 0, cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const bool m = i < f && mask[i] != 0;
            const bool a = m && (slot_of == nullptr || slot_of[i] >= 0);
            npred += m;
            cnt += a;
            flags |= (int)a << e;
        }
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int v = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += v;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int v = wsum[w];
            before += (w < wave) ? v : 0;
            total += v;
        }
        int pos = base + before + incl - cnt;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (flags >> e & 1) idx[pos++] = i0 + e;
        base += total;
        __syncthreads();
    }
    npred = wave_sum_int(npred);
    if (lane == 0) wsum[wave] = npred;
    __syncthreads();
    if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < 16; ++w) tot += wsum[w];
        counts[0] = base;
        counts[1] = tot;
    }
}

// ------------------------------------------------------------------------------ sparse FFN

// Slot of the k-th listed neuron, or -1 when the entry is out of range (then it is skipped).
__device__ __forceinline__ int slot_for(const int32_t *__restrict__ idx, const int32_t *__restrict__ slot_of, int k,
                                        int f, int n_slots) {
    const int i = idx[k];
    if (i < 0 || i >= f) return -1;
    const int s = slot_of ? slot_of[i] : i;
    return (s >= 0 && s < n_slots) ? s : -1;
}

// Dot products of one resident row (d weights) with the B staged token chunks.
template <int B, int WT>
__device__ __forceinline__ void row_dot(const uint8_t *__restrict__ row, int d, int c0, int cw, const uint16_t *xs,
                                        int xch, int lane, float (&acc)[B]) {
    if (WT == WT_F16) {
        const uint16_t *rw = reinterpret_cast<const uint16_t *>(row) + c0;
        int col = lane * 8;
        for (; col + 3 * 512 < cw; col += 4 * 512) {
            uint4 w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = ld16(rw + col + u * 512);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int b = 0; b < B; ++b)
                    acc[b] = dot8(w[u], *reinterpret_cast<const uint4 *>(xs + b * xch + col + u * 512), acc[b]);
        }
        for (; col < cw; col += 512) {
            const uint4 w = ld16(rw + col);
#pragma unroll
            for (int b = 0; b < B; ++b) acc[b] = dot8(w, *reinterpret_cast<const uint4 *>(xs + b * xch + col), acc[b]);
        }
    } else {
        // Lane handles whole 32-weight blocks q = c0/32 + lane + 64t: 16 code bytes + one scale.
        const uint8_t *codes = row;
        const uint16_t *scales = reinterpret_cast<const uint16_t *>(row + d / 2);
        const int q0 = c0 / 32, nq = cw / 32;
        for (int qq = lane; qq < nq; qq += kWave) {
            const int q = q0 + qq;
            const uint4 cw4 = ld16(codes + (size_t)q * 16);
            const float sc = half_to_float(scales[q]);
            const uint32_t words[4] = {cw4.x, cw4.y, cw4.z, cw4.w};
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float s = 0.f;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint4 xv = *reinterpret_cast<const uint4 *>(xs + b * xch + qq * 32 + g * 8);
                    s = fdot2(q4pair(words[g], 0), xv.x, s);
                    s = fdot2(q4pair(words[g], 4), xv.y, s);
                    s = fdot2(q4pair(words[g], 8), xv.z, s);
                    s = fdot2(q4pair(words[g], 12), xv.w, s);
                }
                acc[b] = fmaf(sc, s, acc[b]);
            }
        }
    }
}

// h[b][k] for the listed neurons.  Neuron k goes to wave (k / G) % 4 of workgroup k % G in round
// k / (4G), which spreads the listed neurons over every workgroup (and so every CU) first.
// x is staged once per workgroup (in chunks of xch columns when B*d does not fit).
template <int B, bool GATED, int WT>
__global__ __launch_bounds__(256) void k_sparse_up(const uint8_t *__restrict__ w_in, int64_t row_bytes, int d,
                                                   const uint16_t *__restrict__ b_up, const uint16_t *__restrict__ x,
                                                   const int32_t *__restrict__ idx, const int32_t *__restrict__ counts,
                                                   const int32_t *__restrict__ slot_of, int f, int n_slots,
                                                   float *__restrict__ h, int h_stride, int xch) {
    extern __shared__ __align__(16) uint16_t xs[];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int G = gridDim.x;
    const int n = min(max(counts[0], 0), n_slots);
    const int per_round = 4 * G;
    const int rounds = (n + per_round - 1) / per_round;
    const int nchunks = (d + xch - 1) / xch;
    if (rounds == 0 || (int)blockIdx.x >= n) return;             // no neuron for this workgroup
    const int64_t in_stride = GATED ? 2 * row_bytes : row_bytes;
    for (int rd = 0; rd < rounds; ++rd) {
        const int k = rd * per_round + wave * G + blockIdx.x;
        if (rd * per_round + blockIdx.x >= n) break;             // workgroup-uniform: nothing left
        const int s = (k < n) ? slot_for(idx, slot_of, k, f, n_slots) : -1;
        float ag[B], au[B];
#pragma unroll
        for (int b = 0; b < B; ++b) ag[b] = au[b] = 0.f;
        for (int ch = 0; ch < nchunks; ++ch) {
            const int c0 = ch * xch, cw = min(xch, d - c0);
            if (nchunks > 1 || rd == 0) {
                if (nchunks > 1 && (rd > 0 || ch > 0)) __syncthreads();
                stage_x<B, WT == WT_Q4_0>(xs, x, d, c0, cw, xch);
                __syncthreads();
            }
            if (s >= 0) {
                const uint8_t *row = w_in + (int64_t)s * in_stride;
                if (GATED) {
                    row_dot<B, WT>(row, d, c0, cw, xs, xch, lane, ag);
                    row_dot<B, WT>(row + row_bytes, d, c0, cw, xs, xch, lane, au);
                } else {
                    row_dot<B, WT>(row, d, c0, cw, xs, xch, lane, au);
                }
            }
        }
        if (k < n) {
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
                }
                if (lane == 0) h[(size_t)b * h_stride + k] = (s >= 0) ? hv : 0.f;
            }
        }
    }
}

// Partial y over a (512-column slab, neuron chunk) tile.  Every lane owns 8 columns of the slab;
// the 4 waves take the chunk's neurons round-robin, 4 at a time so that 4 row reads are in
// flight per lane; rows whose h is zero for every token are skipped (their contribution is an
// exact zero).  The 4 wave partials are summed in LDS and written to part[chunk][b][d].
template <int B, int WT>
__global__ __launch_bounds__(256) void k_sparse_down(const uint8_t *__restrict__ w_dn, int64_t row_bytes, int d,
                                                     const int32_t *__restrict__ idx, const int32_t *__restrict__ counts,
                                                     const int32_t *__restrict__ slot_of, int f, int n_slots,
                                                     const float *__restrict__ h, int h_stride,
                                                     float *__restrict__ part, int C) {
    __shared__ float red[4][B][8][kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
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

    for (int kb = k0 + wave; kb < k1; kb += 16) {
        int sl[4];
        float hv[4][B];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = kb + 4 * u;
            sl[u] = -1;
            bool any = false;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                hv[u][b] = (k < k1) ? h[(size_t)b * h_stride + k] : 0.f;
                any |= hv[u][b] != 0.f;
            }
            if (k < k1 && any) sl[u] = slot_for(idx, slot_of, k, f, n_slots);
        }
        if (WT == WT_F16) {
            uint4 w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                w[u] = (sl[u] >= 0 && colok) ? ld16(w_dn + (int64_t)sl[u] * row_bytes + (int64_t)col * 2)
                                             : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (sl[u] < 0) continue;                                 // wave-uniform
                const uint32_t wv[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const h2 pr = __builtin_bit_cast(h2, wv[p]);
                    const float lo = (float)pr.x, hi = (float)pr.y;
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        acc[b][2 * p] = fmaf(hv[u][b], lo, acc[b][2 * p]);
                        acc[b][2 * p + 1] = fmaf(hv[u][b], hi, acc[b][2 * p + 1]);
                    }
                }
            }
        } else {
            uint32_t cw[4];
            float sc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = sl[u] >= 0 && colok;
                const uint8_t *row = w_dn + (int64_t)sl[u] * row_bytes;
                cw[u] = ok ? *reinterpret_cast<const uint32_t *>(row + col / 2) : 0u;
                sc[u] = ok ? half_to_float(*reinterpret_cast<const uint16_t *>(row + d / 2 + (col / 32) * 2)) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (sl[u] < 0) continue;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    // q4pair(w, 4p) = (code_p - 8, code_{p+4} - 8): columns p and p+4.
                    const h2 pr = __builtin_bit_cast(h2, q4pair(cw[u], 4 * p));
                    const float lo = (float)pr.x, hi = (float)pr.y;
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float cf = hv[u][b] * sc[u];
                        acc[b][p] = fmaf(cf, lo, acc[b][p]);
                        acc[b][p + 4] = fmaf(cf, hi, acc[b][p + 4]);
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
    for (int o = threadIdx.x; o < B * 512; o += blockDim.x) {
        const int b = o / 512, cc = o - b * 512;
        const int ln = cc >> 3, t = cc & 7;
        const int gcol = slab * 512 + cc;
        if (gcol < d) {
            const float v = red[0][b][t][ln] + red[1][b][t][ln] + red[2][b][t][ln] + red[3][b][t][ln];
            part[((size_t)ck * B + b) * d + gcol] = v;
        }
    }
}

// y[b][j] = b_down[j] + sum over chunks c (ascending) of part[c][b][j].
__global__ __launch_bounds__(256) void k_reduce_y(const float *__restrict__ part, int C, int Bd, int d,
                                                  const uint16_t *__restrict__ b_down, float *__restrict__ y) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= Bd) return;
    float s = b_down ? half_to_float(b_down[t % d]) : 0.f;
    for (int c = 0; c < C; ++c) s += part[(size_t)c * Bd + t];
    y[t] = s;
}

}  // namespace pik
