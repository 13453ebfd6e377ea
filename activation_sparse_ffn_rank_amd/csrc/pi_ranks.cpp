// pi_ranks.cpp -- per-layer predictor rank under a predictor-memory budget (PowerInfer, arXiv
// 2312.12456, methodology and core innovations: adaptive predictors, trained per layer, that find
// the neurons which fire while keeping the GPU memory they take small).
//
// Rule (this library's reading; the pages name adaptive predictors without a sizing formula).  A
// layer whose neurons fire independently with frequencies p_i has  H = sum_i h(p_i)  bits of
// firing pattern per token, h the binary entropy.  A sparser layer (most p_i near 0) or a more
// skewed one (a few p_i near 1, the rest near 0) has a smaller H: there is less for its predictor
// to tell apart, so it gets a smaller rank.  Layer l's rank follows its H_l on the grid
// r_min, r_min + step, ..., r_max:
//     r_l(lambda) = the largest grid rank <= max(r_min, lambda * H_l),
// with lambda as large as the budget allows,  sum_l 2 r_l (d_l + f_l) <= budget  (P1 [r][d] and
// P2 [f][r] in fp16; the offsets c do not depend on r).  Step by step: every layer starts at r_min;
// layer l is raised to the grid rank r at lambda = r / H_l; the raises are taken in ascending lambda
// (equal lambdas: lower layer first) until the next one does not fit the budget.  H_l is rounded to
// 1/1024 bit so that the order of the raises does not hang on the order of a floating-point sum,
// and the raises are compared by cross-multiplying integers and those rounded entropies (exact in
// double precision).
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <queue>
#include <vector>

#include "pi_sparse_ffn.h"

namespace {

// Binary entropy in bits; 0 at p = 0 and p = 1.
double h2(double p) {
    if (p <= 0.0 || p >= 1.0) return 0.0;
    return -(p * log2(p) + (1.0 - p) * log2(1.0 - p));
}

struct Raise {
    int32_t rank;     // the grid rank layer l is raised to
    double H;         // layer l's rounded entropy (> 0)
    int l;
};

// a comes after b: a's lambda (rank / H) is larger, or equal with a higher layer index
struct Later {
    bool operator()(const Raise &a, const Raise &b) const {
        const double la = (double)a.rank * b.H, lb = (double)b.rank * a.H;   // a.rank / a.H vs b.rank / b.H
        if (la != lb) return la > lb;
        return a.l > b.l;
    }
};

}  // namespace

extern "C" {

int pi_predictor_ranks(int32_t n_layers, const int32_t *d_model, const int32_t *d_ffn, const float *freq,
                       int64_t budget_bytes, int32_t r_min, int32_t r_max, int32_t r_step, int32_t *rank,
                       double *entropy_bits) {
    if (n_layers < 1 || !d_model || !d_ffn || !freq || !rank) return PI_ERR_NULL;
    if (r_min < 8 || r_min % 8 != 0 || r_max < r_min || r_max > PI_MAX_RANK || r_step < 8 || r_step % 8 != 0 ||
        (r_max - r_min) % r_step != 0)
        return PI_ERR_SHAPE;
    int64_t total_f = 0, base = 0;
    for (int l = 0; l < n_layers; ++l) {
        if (d_model[l] < 1 || d_model[l] > PI_MAX_D_MODEL || d_ffn[l] < 1 || d_ffn[l] > PI_MAX_D_FFN)
            return PI_ERR_SHAPE;
        total_f += d_ffn[l];
        base += 2 * (int64_t)r_min * ((int64_t)d_model[l] + d_ffn[l]);
    }
    if (budget_bytes < base) return PI_ERR_SHAPE;                         // not even r_min everywhere
    for (int64_t k = 0; k < total_f; ++k)
        if (!(freq[k] >= 0.f && freq[k] <= 1.f)) return PI_ERR_SHAPE;   // also rejects NaN

    std::vector<double> H(n_layers);
    std::priority_queue<Raise, std::vector<Raise>, Later> q;
    int64_t off = 0;
    for (int l = 0; l < n_layers; ++l) {
        double s = 0.0;
        for (int i = 0; i < d_ffn[l]; ++i) s += h2((double)freq[off + i]);
        off += d_ffn[l];
        H[l] = nearbyint(s * 1024.0) / 1024.0;
        rank[l] = r_min;
        if (H[l] > 0.0 && r_min < r_max) q.push({r_min + r_step, H[l], l});
    }
    int64_t left = budget_bytes - base;
    while (!q.empty()) {
        const Raise it = q.top();
        q.pop();
        const int64_t cost = 2 * (int64_t)r_step * ((int64_t)d_model[it.l] + d_ffn[it.l]);
        if (cost > left) break;                    // the next raise in lambda order does not fit
        left -= cost;
        rank[it.l] = it.rank;
        if (it.rank < r_max) q.push({it.rank + r_step, it.H, it.l});
    }
    if (entropy_bits)
        for (int l = 0; l < n_layers; ++l) entropy_bits[l] = H[l];
    return PI_OK;
}

}  // extern "C"
