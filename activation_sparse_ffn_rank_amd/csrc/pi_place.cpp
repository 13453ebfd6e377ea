// pi_place.cpp -- offline neuron placement under a device-memory budget (PowerInfer, arXiv
// 2312.12456, method section: an offline policy, solved as an integer linear program over the
// neurons' activation frequencies and the hardware's bandwidths, decides which neurons are
// preloaded on the GPU; README: the result is the GPU index, sized by a VRAM budget).
//
// Model (this library's reading; the pages give no formulation).  Layer l has f_l neurons of
// c_l bytes each (all of a neuron's rows) and firing frequencies p_{l,i}.  With the GPU holding
// the set H_l, a token streams  G_l = c_l * sum_{i in H_l} p_{l,i}  bytes on the GPU and
// C_l = c_l * sum_{i not in H_l} p_{l,i}  bytes on the host, in parallel, so the layer takes
// T_l = max(G_l / bw_gpu, C_l / bw_host).  Minimize sum_l T_l subject to sum_l c_l |H_l| <= budget.
//
// Solution.  Each layer keeps its n most frequent neurons (they move the most mass off the host;
// this is optimal while the host side dominates -- with a device tens of times faster than the
// host, the regime of any budget that leaves most neurons on the host; once the device side
// dominates, a less frequent set may balance the two sides more finely, by at most one neuron's
// time).  Then T_l depends on n only and its marginal gains fall with n (the host time drops by
// the next frequency until the device time takes over).  The next neuron of every layer sits in a
// priority queue keyed by its gain (T_l before - T_l after) per byte; the best is taken while it
// fits the budget and gains something.  With equal neuron sizes this greedy is exact over such
// placements; with unequal sizes (layers of different weight formats) it is within one neuron's
// gain of it (the knapsack's last item).  Ties in frequency go to the lower id; the placed neurons
// of a layer get slots in ascending id order.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <numeric>
#include <queue>
#include <vector>

#include "pi_sparse_ffn.h"

namespace {

struct LayerState {
    std::vector<int32_t> order;   // neuron ids by descending frequency (ties: lower id first)
    double total = 0.0;           // sum of frequencies
    double placed = 0.0;          // sum of frequencies of the first n
    int n = 0;
};

double layer_time(double c, double placed, double total, double bw_g, double bw_h) {
    const double g = c * placed / bw_g, h = c * (total - placed) / bw_h;
    return g > h ? g : h;
}

}  // namespace

extern "C" {

int pi_place(int32_t n_layers, const int32_t *d_ffn, const int64_t *neuron_bytes, const float *freq,
             int64_t budget_bytes, double gpu_bytes_per_s, double host_bytes_per_s, int32_t *slot_of,
             int32_t *n_placed, double *expected_s) {
    if (n_layers < 1 || !d_ffn || !neuron_bytes || !freq || !slot_of || !n_placed) return PI_ERR_NULL;
    if (budget_bytes < 0 || !(gpu_bytes_per_s > 0.0) || !(host_bytes_per_s > 0.0)) return PI_ERR_SHAPE;
    int64_t total_f = 0;
    for (int l = 0; l < n_layers; ++l) {
        if (d_ffn[l] < 1 || d_ffn[l] > PI_MAX_D_FFN || neuron_bytes[l] < 1) return PI_ERR_SHAPE;
        total_f += d_ffn[l];
    }
    for (int64_t k = 0; k < total_f; ++k)
        if (!(freq[k] >= 0.f && freq[k] <= 1.f)) return PI_ERR_SHAPE;   // also rejects NaN

    std::vector<LayerState> st(n_layers);
    int64_t base = 0;
    for (int l = 0; l < n_layers; ++l) {
        const float *p = freq + base;
        LayerState &s = st[l];
        s.order.resize(d_ffn[l]);
        std::iota(s.order.begin(), s.order.end(), 0);
        std::stable_sort(s.order.begin(), s.order.end(), [p](int32_t a, int32_t b) { return p[a] > p[b]; });
        for (int i = 0; i < d_ffn[l]; ++i) s.total += p[i];
        base += d_ffn[l];
    }
    // gain per byte of placing layer l's next neuron
    std::vector<int64_t> off(n_layers + 1, 0);
    for (int l = 0; l < n_layers; ++l) off[l + 1] = off[l] + d_ffn[l];
    auto gain = [&](int l) -> double {
        const LayerState &s = st[l];
        const double c = (double)neuron_bytes[l];
        const double pn = freq[off[l] + s.order[s.n]];
        return (layer_time(c, s.placed, s.total, gpu_bytes_per_s, host_bytes_per_s) -
                layer_time(c, s.placed + pn, s.total, gpu_bytes_per_s, host_bytes_per_s)) / c;
    };
    using Item = std::pair<double, int>;               // (gain per byte, -layer): ties go to the lower layer
    std::priority_queue<Item> q;
    for (int l = 0; l < n_layers; ++l)
        if (d_ffn[l] > 0) q.push({gain(l), -l});
    int64_t left = budget_bytes;
    while (!q.empty()) {
        const Item it = q.top();
        q.pop();
        const int l = -it.second;
        if (!(it.first > 0.0)) break;                    // nothing left gains anything
        if (neuron_bytes[l] > left) continue;            // this layer's neurons no longer fit
        LayerState &s = st[l];
        s.placed += freq[off[l] + s.order[s.n]];
        ++s.n;
        left -= neuron_bytes[l];
        if (s.n < d_ffn[l]) q.push({gain(l), -l});
    }
    double t = 0.0;
    for (int l = 0; l < n_layers; ++l) {
        LayerState &s = st[l];
        int32_t *so = slot_of + off[l];
        for (int i = 0; i < d_ffn[l]; ++i) so[i] = -1;
        std::vector<int32_t> hot(s.order.begin(), s.order.begin() + s.n);
        std::sort(hot.begin(), hot.end());
        for (int k = 0; k < s.n; ++k) so[hot[k]] = k;
        n_placed[l] = s.n;
        t += layer_time((double)neuron_bytes[l], s.placed, s.total, gpu_bytes_per_s, host_bytes_per_s);
    }
    if (expected_s) *expected_s = t;
    return PI_OK;
}

}  // extern "C"
