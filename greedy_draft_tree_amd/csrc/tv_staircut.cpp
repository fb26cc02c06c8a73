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

// ------------------------------------------------------------ verify prices
// The verify price by row count for StairCut, from a price file and the
// measured rounds ("Drafters and tree verify", StairCut on Flash-Next, and
// the shared price files): prices by context class and kind (chain or tree);
// a context takes the largest listed class at or below it (the smallest
// listed one when none is); rows between two listed counts interpolate
// linearly, rows past the last add step_ms a row (without step_ms, the last
// two counts' slope); measured round times move a count's live price by an
// exponential moving average, the counts not measured shift by the mean
// offset of the measured ones from the file, and the table is made
// non-decreasing in rows.  With no file every count costs 1 ms.  Host only.
#include <algorithm>
#include <map>
#include <new>
#include <utility>
#include <vector>

struct tv_prices {
    typedef std::vector<std::pair<int, double>> Curve;   // (rows, ms), rows increasing
    std::map<int32_t, Curve> file[2];                    // [kind] class -> curve
    std::vector<int32_t> classes;                        // listed classes, increasing
    bool has_step = false;
    double step_ms = 0.0, ema = 0.1;
    // live prices per (class, kind): (rows, ms) in the order first measured
    std::map<std::pair<int64_t, int>, std::vector<std::pair<int, double>>> live;
};

namespace {
constexpr int64_t kNoClass = INT64_MIN;   // the class key when there is no file

int64_t price_class(const tv_prices *p, int ctx) {
    if (p->classes.empty()) return kNoClass;
    int64_t c = p->classes.front();
    for (int32_t k : p->classes)
        if (k <= ctx) c = k;
    return c;
}

double file_price(const tv_prices *p, int64_t cls, int kind, int rows) {
    if (cls == kNoClass) return 1.0;
    auto it = p->file[kind].find((int32_t)cls);
    if (it == p->file[kind].end() || it->second.empty()) return 1.0;
    const tv_prices::Curve &c = it->second;
    if (rows <= c.front().first) return c.front().second;
    if (rows <= c.back().first) {
        size_t j = 0;
        while (c[j + 1].first < rows) ++j;
        const double slope = (c[j + 1].second - c[j].second) / (double)(c[j + 1].first - c[j].first);
        return slope * (double)(rows - c[j].first) + c[j].second;
    }
    double step = 0.0;
    if (p->has_step) step = p->step_ms;
    else if (c.size() >= 2)
        step = (c.back().second - c[c.size() - 2].second) / (double)(c.back().first - c[c.size() - 2].first);
    return c.back().second + step * (double)(rows - c.back().first);
}

void price_table(const tv_prices *p, int64_t cls, int kind, double *out) {
    double base[TV_MAX_NODES + 1];
    for (int r = 0; r <= TV_MAX_NODES; ++r) base[r] = file_price(p, cls, kind, r);
    double shift = 0.0;
    auto it = p->live.find({cls, kind});
    if (it != p->live.end() && !it->second.empty()) {
        double s = 0.0;
        for (const auto &e : it->second) s += e.second - base[e.first];
        shift = s / (double)it->second.size();
    }
    for (int r = 0; r <= TV_MAX_NODES; ++r) out[r] = base[r] + shift;
    if (it != p->live.end())
        for (const auto &e : it->second) out[e.first] = e.second;
    out[0] = out[1];
    for (int r = 1; r <= TV_MAX_NODES; ++r) out[r] = std::max(out[r], out[r - 1]);
}
} // namespace

extern "C" int tv_prices_create(const int32_t *ctx_class, const int32_t *kind, const int32_t *rows, const double *ms,
                                int n_points, int has_step, double step_ms, double ema, tv_prices **out) {
    if (!out) return TV_EINVAL;
    *out = nullptr;
    if (n_points < 0 || (n_points > 0 && (!ctx_class || !kind || !rows || !ms))) return TV_EINVAL;
    if (!(ema > 0.0 && ema <= 1.0)) return TV_EINVAL;
    if (has_step && !std::isfinite(step_ms)) return TV_EINVAL;
    tv_prices *p = new (std::nothrow) tv_prices;
    if (!p) return TV_EINVAL;   // out of memory
    p->has_step = has_step != 0;
    p->step_ms = step_ms;
    p->ema = ema;
    for (int i = 0; i < n_points; ++i) {
        if ((kind[i] != TV_PRICE_CHAIN && kind[i] != TV_PRICE_TREE) || rows[i] < 1 || !std::isfinite(ms[i])) {
            delete p;
            return TV_EINVAL;
        }
        tv_prices::Curve &c = p->file[kind[i]][ctx_class[i]];
        for (const auto &e : c)
            if (e.first == rows[i]) {   // a count listed twice
                delete p;
                return TV_EINVAL;
            }
        c.emplace_back(rows[i], ms[i]);
        std::sort(c.begin(), c.end());
        if (std::find(p->classes.begin(), p->classes.end(), ctx_class[i]) == p->classes.end())
            p->classes.push_back(ctx_class[i]);
    }
    std::sort(p->classes.begin(), p->classes.end());
    *out = p;
    return TV_OK;
}

extern "C" void tv_prices_destroy(tv_prices *p) { delete p; }

extern "C" int tv_prices_class(const tv_prices *p, int ctx, int32_t *cls, int *has_class) {
    if (!p || !cls || !has_class) return TV_EINVAL;
    const int64_t c = price_class(p, ctx);
    *has_class = c != kNoClass;
    *cls = c == kNoClass ? 0 : (int32_t)c;
    return TV_OK;
}

extern "C" int tv_prices_table(const tv_prices *p, int ctx, int kind, double *out) {
    if (!p || !out || (kind != TV_PRICE_CHAIN && kind != TV_PRICE_TREE)) return TV_EINVAL;
    price_table(p, price_class(p, ctx), kind, out);
    return TV_OK;
}

extern "C" int tv_prices_observe(tv_prices *p, int ctx, int kind, int rows, double ms) {
    if (!p || (kind != TV_PRICE_CHAIN && kind != TV_PRICE_TREE) || rows < 1 || rows > TV_MAX_NODES ||
        !std::isfinite(ms))
        return TV_EINVAL;
    const int64_t cls = price_class(p, ctx);
    std::vector<std::pair<int, double>> &lv = p->live[{cls, kind}];
    for (auto &e : lv)
        if (e.first == rows) {
            e.second = e.second + p->ema * (ms - e.second);
            return TV_OK;
        }
    double table[TV_MAX_NODES + 1];
    price_table(p, cls, kind, table);
    const double cur = table[rows];
    lv.emplace_back(rows, cur + p->ema * (ms - cur));
    return TV_OK;
}
