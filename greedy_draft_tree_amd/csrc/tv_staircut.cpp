// StairCut on the host ("Drafters and tree verify", StairCut): cut a
// candidate tree to the node count that maximises expected committed tokens
// per millisecond, (1 + min(sum of q, n)) / (verify(rows) + draft + commit).
// Nodes are admitted in the drafter's score order, each with the ancestors it
// needs; a cut ends at 7, 15, 23 or 31 nodes (the longest admission prefix
// within that many) or at the whole candidate.  No GPU work.
#include <cmath>
#include <cstdint>

#include "../../include/treeverify.h"

namespace {
constexpr int kStairNodes[4] = {7, 15, 23, 31};
}

extern "C" int tv_staircut(const int32_t *parents, const float *q, const int32_t *order, int n_nodes,
                           const float *price_tree_ms, const float *price_chain_ms, float draft_ms,
                           float commit_ms, int32_t *keep, int *n_keep, float *score) {
    if (!parents || !price_tree_ms || !price_chain_ms || !keep || !n_keep) return TV_EINVAL;
    if (n_nodes < 1 || n_nodes > TV_MAX_CANDIDATE) return TV_EINVAL;
    if (n_nodes > 1 && (!q || !order)) return TV_EINVAL;   // q and order may be NULL for the root alone
    if (parents[0] != -1) return TV_EINVAL;
    for (int i = 1; i < n_nodes; ++i) {
        if (parents[i] < 0 || parents[i] >= i) return TV_EINVAL;
        if (!(q[i] >= 0.f) || !std::isfinite(q[i])) return TV_EINVAL;
    }
    for (int r = 1; r <= TV_MAX_NODES; ++r)
        if (!std::isfinite(price_tree_ms[r]) || !std::isfinite(price_chain_ms[r])) return TV_EINVAL;
    if (!std::isfinite(draft_ms) || !std::isfinite(commit_ms)) return TV_EINVAL;
    const int K = n_nodes - 1;   // admissions
    bool seen[TV_MAX_CANDIDATE] = {false};
    for (int k = 0; k < K; ++k) {
        const int v = order[k];
        if (v < 1 || v >= n_nodes || seen[v]) return TV_EINVAL;   // a permutation of 1..n_nodes-1
        seen[v] = true;
    }
    // size (nodes, root excluded) of the kept set after each admission prefix
    int size[TV_MAX_CANDIDATE];
    bool in[TV_MAX_CANDIDATE] = {false};
    in[0] = true;
    size[0] = 0;
    for (int k = 0; k < K; ++k) {
        int add = 0;
        for (int j = order[k]; j >= 0 && !in[j]; j = parents[j]) {
            in[j] = true;
            ++add;
        }
        size[k + 1] = size[k] + add;
    }
    // cut ends: per stair, the longest prefix within it; the whole candidate
    int ends[5], n_ends = 0;
    for (int P : kStairNodes) {
        int best = 0;
        for (int k = 0; k <= K; ++k)
            if (size[k] <= P) best = k;
        ends[n_ends++] = best;
    }
    if (size[K] <= kStairNodes[3]) ends[n_ends++] = K;
    // evaluate in increasing size; a strictly better score replaces
    int best_k = -1;
    double best = 0.0;
    for (int pass = 0; pass < n_ends; ++pass) {
        int k = -1;
        for (int e = 0; e < n_ends; ++e) {   // next smallest end not yet visited
            const int c = ends[e];
            if (c < 0) continue;
            if (k < 0 || size[c] < size[k] || (size[c] == size[k] && c < k)) k = c;
        }
        for (int e = 0; e < n_ends; ++e)
            if (ends[e] == k) ends[e] = -1;
        if (k < 0) break;
        bool kept[TV_MAX_CANDIDATE] = {false};
        kept[0] = true;
        for (int a = 0; a < k; ++a)
            for (int j = order[a]; j >= 0 && !kept[j]; j = parents[j]) kept[j] = true;
        double qsum = 0.0;
        int kids[TV_MAX_CANDIDATE] = {0};
        bool chain = true;
        for (int i = 1; i < n_nodes; ++i) {
            if (!kept[i]) continue;
            qsum += q[i];
            if (++kids[parents[i]] > 1) chain = false;
        }
        const int nodes = size[k];
        const double gain = 1.0 + std::fmin(qsum, (double)nodes);
        const double price = (double)(chain ? price_chain_ms : price_tree_ms)[nodes + 1] + draft_ms + commit_ms;
        if (!(price > 0.0)) return TV_EINVAL;
        const double sc = gain / price;
        if (best_k < 0 || sc > best) {
            best = sc;
            best_k = k;
        }
    }
    bool kept[TV_MAX_CANDIDATE] = {false};
    kept[0] = true;
    for (int a = 0; a < best_k; ++a)
        for (int j = order[a]; j >= 0 && !kept[j]; j = parents[j]) kept[j] = true;
    int m = 0;
    for (int i = 0; i < n_nodes; ++i)
        if (kept[i]) keep[m++] = i;
    *n_keep = m;
    if (score) *score = (float)best;
    return TV_OK;
}
