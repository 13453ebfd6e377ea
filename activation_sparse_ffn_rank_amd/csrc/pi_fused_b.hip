// pi_fused_b.hip -- instantiates the fused layer kernel for one batch width, PIK_B (set by the
// build: this file is compiled once per B in 1..8).
#include "pi_fused.hpp"

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
int launch_sparse_one(FusedArgs &a, hipStream_t st) {
    auto kern = k_sparse_fused<PIK_B, GATED, WT>;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
    const size_t lds = (size_t)PIK_B * a.d * sizeof(uint16_t);   // the LDS copy of x
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess || per_cu < 1) return 1;
    // every workgroup must be resident at once: down tiles wait on up tasks of other workgroups
    const int most = a.ND + a.NE;                                 // ND here: groups of the largest list
    a.P = cus * per_cu < most ? cus * per_cu : most;
    if (a.P < 1) a.P = 1;
    hipLaunchKernelGGL(kern, dim3(a.P), dim3(256), lds, st, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

template <>
int launch_sparse_batch<PIK_B>(FusedArgs &a, int wtype, int gated, hipStream_t st) {
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
