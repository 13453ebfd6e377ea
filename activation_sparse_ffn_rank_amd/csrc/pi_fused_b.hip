// pi_fused_b.hip -- instantiates the persistent kernels (whole layer, sparse FFN) for one batch
// width, PIK_B (set by the build: this file is compiled once per B in 1..8).
#include "pi_tail.hpp"

#ifndef PIK_B
#error "PIK_B (the batch width of this translation unit) must be defined"
#endif

namespace pik {
namespace {

template <bool GATED, int WT, int NT>
int launch_one(FusedArgs &a, hipStream_t st) {
    auto kern = k_layer_fused<PIK_B, GATED, WT, NT>;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
    const size_t lds = (size_t)PIK_B * a.d * sizeof(uint16_t);   // the LDS copy of x
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess || per_cu < 1) return 1;
    // every workgroup must be resident at once: tasks wait on tasks of other workgroups
    a.P = cus * per_cu < a.tasks ? cus * per_cu : a.tasks;
    if (a.P < 1) a.P = 1;
    hipLaunchKernelGGL(kern, dim3(a.P), dim3(256), lds, st, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <bool GATED, int WT>
int launch_nt(FusedArgs &a, int NT, hipStream_t st) {
    if (NT == 1) return launch_one<GATED, WT, 1>(a, st);
    if (NT == 2) return launch_one<GATED, WT, 2>(a, st);
    return launch_one<GATED, WT, 4>(a, st);
}

template <bool GATED, int WT>
int launch_sparse_one(SparseArgs &a, hipStream_t st) {
    auto kern = k_sparse_ffn<PIK_B, GATED, WT>;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
    const size_t lds = (size_t)PIK_B * a.d * sizeof(uint16_t);   // the LDS copy of x
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess || per_cu < 1) return 1;
    // every workgroup must be resident at once (down tiles wait on up workgroups): about half of
    // the resident slots go to down tiles, the rest (at most one per group of 4 slots) to up work
    const int cap = cus * per_cu;
    int C = (cap / 2) / a.slabs;
    C = C < 1 ? 1 : (C > kSparseMaxChunks ? kSparseMaxChunks : C);
    a.C = C;
    a.NE = a.slabs * C;
    const int groups = (a.n_slots + 3) / 4;
    a.PD = cap - a.NE < groups ? cap - a.NE : groups;
    if (a.PD < 1) a.PD = 1;
    if (a.PD + a.NE > cap) return 1;
    hipLaunchKernelGGL(kern, dim3(a.PD + a.NE), dim3(256), lds, st, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <bool GATED, int WT, int NT>
int launch_tail_one(TailArgs &a, hipStream_t st) {
    auto kern = k_layer_tail<PIK_B, GATED, WT, NT>;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
    const size_t lds = tail_dyn_lds(PIK_B, a.d, a.r);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess || per_cu < 1) return 1;
    // every workgroup must be resident at once (down tiles wait on up workgroups): one up
    // workgroup per neuron tile when the slots allow it, the rest (at most half) to down tiles
    const int cap = cus * per_cu;
    int C = (cap - a.NTL) / a.slabs;
    if (C > (cap / 2) / a.slabs) C = (cap / 2) / a.slabs;
    const int one_round = (a.NTL + kTailListMax / 32 - 1) / (kTailListMax / 32);   // chunks listed in one round
    if (C < one_round) C = one_round;
    C = C < 1 ? 1 : (C > kSparseMaxChunks ? kSparseMaxChunks : C);
    a.C = C;
    a.NE = a.slabs * C;
    a.PU = cap - a.NE < a.NTL ? cap - a.NE : a.NTL;
    if (a.PU < 1) a.PU = 1;
    if (a.PU + a.NE > cap) return 1;
    hipLaunchKernelGGL(kern, dim3(a.PU + a.NE), dim3(256), lds, st, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <bool GATED, int WT>
int launch_tail_nt(TailArgs &a, int NT, hipStream_t st) {
    if (NT == 1) return launch_tail_one<GATED, WT, 1>(a, st);
    if (NT == 2) return launch_tail_one<GATED, WT, 2>(a, st);
    return launch_tail_one<GATED, WT, 4>(a, st);
}

}  // namespace

template <>
int launch_tail_batch<PIK_B>(TailArgs &a, int wtype, int gated, int NT, hipStream_t st) {
    if (wtype == WT_Q4_0) return launch_tail_nt<false, WT_Q4_0>(a, NT, st);
    if (gated) return launch_tail_nt<true, WT_F16>(a, NT, st);
    return launch_tail_nt<false, WT_F16>(a, NT, st);
}

template <>
int launch_sparse_batch<PIK_B>(SparseArgs &a, int wtype, int gated, hipStream_t st) {
    if (wtype == WT_Q4_0) return launch_sparse_one<false, WT_Q4_0>(a, st);
    if (gated) return launch_sparse_one<true, WT_F16>(a, st);
    return launch_sparse_one<false, WT_F16>(a, st);
}

template <>
int launch_fused_batch<PIK_B>(FusedArgs &a, int wtype, int gated, int NT, hipStream_t st) {
    if (wtype == WT_Q4_0) return launch_nt<false, WT_Q4_0>(a, NT, st);
    if (gated) return launch_nt<true, WT_F16>(a, NT, st);
    return launch_nt<false, WT_F16>(a, NT, st);
}

}  // namespace pik
