// pi_split.hip -- instantiates the (column slab x list chunk) sparse-FFN kernels of pi_split.hpp
// for batch 1 and 2 and every row kind, and launches them.
#include "pi_split.hpp"
#include "pi_occupancy.hpp"

namespace pik {
namespace {

template <int B, bool GATED, int WT>
int launch_one(SplitArgs &a, hipStream_t st) {
    auto up = k_up_split<B, GATED, WT>;
    auto down = k_down_split<B, GATED, WT>;
    const size_t lds_up = split_dyn_lds(B, WT, a.nwords, false), lds_down = split_dyn_lds(B, WT, a.nwords, true);
    int cus = 0, per_cu = 0;
    if (resident_slots(reinterpret_cast<const void *>(down), kSplitThreads, lds_down, &cus, &per_cu)) return 1;
    // about two workgroups per compute unit: every workgroup moves the same bytes, so the grid
    // spreads them evenly; nothing waits on another workgroup, so residency is not required
    int C = (2 * cus) / a.S;
    C = C < 1 ? 1 : (C > kSplitMaxChunks ? kSplitMaxChunks : C);
    a.C = C;
    const int grid = a.S * C, Bd = B * a.d;
    hipLaunchKernelGGL(up, dim3(grid), dim3(kSplitThreads), lds_up, st, a);
    if (hipGetLastError() != hipSuccess) return 1;
    hipLaunchKernelGGL(down, dim3(grid), dim3(kSplitThreads), lds_down, st, a);
    if (hipGetLastError() != hipSuccess) return 1;
    hipLaunchKernelGGL(k_sum_split, dim3((Bd + kSplitThreads - 1) / kSplitThreads), dim3(kSplitThreads), 0, st,
                       a.ypart, C, Bd, a.d, a.b_down, a.y);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int B>
int launch_b(SplitArgs &a, int wtype, int gated, hipStream_t st) {
    if (wtype == WT_Q4_0) return launch_one<B, false, WT_Q4_0>(a, st);
    if (gated) return launch_one<B, true, WT_F16>(a, st);
    return launch_one<B, false, WT_F16>(a, st);
}

}  // namespace

int launch_split(SplitArgs &a, int B, int wtype, int gated, hipStream_t st) {
    if (B == 1) return launch_b<1>(a, wtype, gated, st);
    if (B == 2) return launch_b<2>(a, wtype, gated, st);
    return 1;
}

}  // namespace pik
