// pi_split.hip -- instantiates the (column slab x list chunk) sparse-FFN kernels and the fused
// predictor + up kernel of pi_split.hpp for batch 1 and 2 and every row kind, and launches them.
#include "pi_split.hpp"
#include "pi_occupancy.hpp"

namespace pik {
namespace {

// C: about two workgroups per compute unit -- every workgroup moves the same bytes, so the grid
// spreads them evenly; nothing waits on another workgroup, so residency is not required.
template <int B, bool GATED, int WT>
int choose_chunks(SplitArgs &a) {
    int cus = 0, per_cu = 0;
    const size_t lds_down = split_dyn_lds(B, WT, a.nwords, true);
    if (resident_slots(reinterpret_cast<const void *>(k_down_split<B, GATED, WT, false>), kSplitThreads, lds_down, &cus,
                       &per_cu))
        return 1;
    int C = (2 * cus) / a.S;
    // range mode (h by id): a chunk's flag words must fit one word per thread
    if (a.hin != nullptr && a.nwords > 0) C = C > (a.nwords + kRangeMaxWords - 1) / kRangeMaxWords
                                                  ? C : (a.nwords + kRangeMaxWords - 1) / kRangeMaxWords;
    a.C = C < 1 ? 1 : (C > kSplitMaxChunks ? kSplitMaxChunks : C);
    return 0;
}

// Flag words per chunk in range mode, else 0.
inline int range_words(const SplitArgs &a) {
    return (a.hin != nullptr && a.nwords > 0) ? (a.nwords + a.C - 1) / a.C : 0;
}

// k_down_split then k_sum_split (a.C set).
template <int B, bool GATED, int WT>
int launch_down_sum(SplitArgs &a, hipStream_t st) {
    const int Bd = B * a.d;
    const size_t lds = split_dyn_lds(B, WT, a.nwords, true, range_words(a));
    if (a.hin != nullptr && a.nwords > 0)
        hipLaunchKernelGGL((k_down_split<B, GATED, WT, true>), dim3(a.S * a.C), dim3(kSplitThreads), lds, st, a);
    else
        hipLaunchKernelGGL((k_down_split<B, GATED, WT, false>), dim3(a.S * a.C), dim3(kSplitThreads), lds, st, a);
    if (hipGetLastError() != hipSuccess) return 1;
    hipLaunchKernelGGL(k_sum_split, dim3((Bd + kWave - 1) / kWave), dim3(kWave), 0, st,
                       a.ypart, a.C, Bd, a.d, a.b_down, a.y);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int B, bool GATED, int WT>
int launch_one(SplitArgs &a, hipStream_t st) {
    if (choose_chunks<B, GATED, WT>(a)) return 1;
    hipLaunchKernelGGL((k_up_split<B, GATED, WT>), dim3(a.S * a.C), dim3(kSplitThreads),
                       split_dyn_lds(B, WT, a.nwords, false), st, a);
    if (hipGetLastError() != hipSuccess) return 1;
    return launch_down_sum<B, GATED, WT>(a, st);
}

// Grid of k_pred_up: as many workgroups as fit on the chip at once, evened out so that every
// workgroup takes the same number of tiles (or one fewer), at most kPredUpMaxTiles.  (Measured on
// the 49152 x 1024 predictor: one tile per workgroup, or 3 and 4 per workgroup on fewer
// workgroups, were all slower than the 2 per workgroup this gives there.)
template <int B, bool GATED, int WT, int NT>
int launch_pred_up(PredUpArgs &p, hipStream_t st) {
    const void *kern = reinterpret_cast<const void *>(k_pred_up<B, GATED, WT, NT>);
    const size_t lds = pred_up_lds(B, p.d, p.r);
    int cus = 0, per_cu = 0;
    if (resident_slots(kern, 256, lds, &cus, &per_cu)) return 1;
    const int tiles = (p.f + 31) / 32, slots = cus * per_cu;
    int rounds = (tiles + slots - 1) / slots;
    if (rounds > kPredUpMaxTiles) rounds = kPredUpMaxTiles;   // then more workgroups than fit at once
    const int grid = (tiles + rounds - 1) / rounds;
    hipLaunchKernelGGL((k_pred_up<B, GATED, WT, NT>), dim3(grid), dim3(256), lds, st, p);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int B, bool GATED, int WT>
int launch_layer_one(PredUpArgs &p, SplitArgs &a, int NT, hipStream_t st) {
    if (choose_chunks<B, GATED, WT>(a)) return 1;
    int rc;
    if (NT == 1) rc = launch_pred_up<B, GATED, WT, 1>(p, st);
    else if (NT == 2) rc = launch_pred_up<B, GATED, WT, 2>(p, st);
    else rc = launch_pred_up<B, GATED, WT, 4>(p, st);
    if (rc) return 1;
    return launch_down_sum<B, GATED, WT>(a, st);
}

template <int B>
int launch_b(SplitArgs &a, int wtype, int gated, hipStream_t st) {
    if (wtype == WT_Q4_0) return launch_one<B, false, WT_Q4_0>(a, st);
    if (gated) return launch_one<B, true, WT_F16>(a, st);
    return launch_one<B, false, WT_F16>(a, st);
}

template <int B>
int launch_layer_b(PredUpArgs &p, SplitArgs &a, int wtype, int gated, int NT, hipStream_t st) {
    if (wtype == WT_Q4_0) return launch_layer_one<B, false, WT_Q4_0>(p, a, NT, st);
    if (gated) return launch_layer_one<B, true, WT_F16>(p, a, NT, st);
    return launch_layer_one<B, false, WT_F16>(p, a, NT, st);
}

}  // namespace

int launch_split(SplitArgs &a, int B, int wtype, int gated, hipStream_t st) {
    if (B == 1) return launch_b<1>(a, wtype, gated, st);
    if (B == 2) return launch_b<2>(a, wtype, gated, st);
    return 1;
}

int launch_pred_up_split(PredUpArgs &p, SplitArgs &a, int B, int wtype, int gated, int NT, hipStream_t st) {
    if (B == 1) return launch_layer_b<1>(p, a, wtype, gated, NT, st);
    if (B == 2) return launch_layer_b<2>(p, a, wtype, gated, NT, st);
    return 1;
}

}  // namespace pik
