// pi_persist_b.hip -- instantiates the persistent tail kernel of a layer (second predictor matrix,
// mask and sparse FFN) for one batch width, PIK_B (set by the build: this file is compiled once per B in 1..8).
#include "pi_tail.hpp"
#include "pi_occupancy.hpp"

#ifndef PIK_B
#error "PIK_B (the batch width of this translation unit) must be defined"
#endif

namespace pik {
namespace {

template <bool GATED, int WT, int NT>
int launch_tail_one(TailArgs &a, hipStream_t st) {
    auto kern = k_layer_tail<PIK_B, GATED, WT, NT>;
    const size_t lds = tail_dyn_lds(PIK_B, a.d, a.r);
    int cus = 0, per_cu = 0;
    if (resident_slots(reinterpret_cast<const void *>(kern), 256, lds, &cus, &per_cu)) return 1;
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

}  // namespace pik
