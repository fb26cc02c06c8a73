// The lookup drafter on the host ("Drafters and tree verify", The lookup
// drafter): copy text instead of predicting it.  The longest match of the
// text's last tokens (orders min..max) among earlier occurrences gives one
// vote per occurrence; the votes' continuations form a tree whose node score
// is its vote share, a path probability, which StairCut takes as q.  No GPU
// work.
//
// One pass over the text measures, for every earlier end position, how many
// of the last tokens it matches (capped at the largest order); the order used
// is the longest match found.  The tree is then grown best first without
// building it whole: a node is expanded (its votes grouped by their next
// token) only when it is admitted, and its children join a priority queue
// ordered by (count descending, depth ascending, path ascending).  A child
// never outranks its parent, so the admitted nodes are exactly the best
// max_nodes nodes of the full tree.
#include <algorithm>
#include <cstdint>
#include <new>
#include <queue>
#include <utility>
#include <vector>

#include "../../include/treeverify.h"

namespace {

struct Node {
    int32_t depth = 0;    // tokens below the root
    int32_t count = 0;    // votes through the node
    int32_t rep = 0;      // a continuation start whose first `depth` tokens are the node's path
    int32_t token = 0;
    int32_t parent = -1;
    int32_t out = -1;     // index in the output
    std::vector<int32_t> votes;   // continuation starts through the node, until it is expanded
    std::vector<int32_t> kids;    // admitted children
};

struct Tree {
    const int32_t *text;
    int len, max_depth;
    std::vector<Node> nodes;

    // a ranks before b: more votes, then shallower, then the smaller path
    bool before(int a, int b) const {
        const Node &x = nodes[a], &y = nodes[b];
        if (x.count != y.count) return x.count > y.count;
        if (x.depth != y.depth) return x.depth < y.depth;
        for (int i = 0; i < x.depth; ++i) {
            const int32_t u = text[x.rep + i], v = text[y.rep + i];
            if (u != v) return u < v;
        }
        return false;
    }

    // children of node id: its votes grouped by the token after its path
    template <class Push>
    void expand(int id, Push push) {
        const int d = nodes[id].depth;
        std::vector<std::pair<int32_t, int32_t>> next;   // (token, start)
        for (int32_t c : nodes[id].votes) {
            const int end = std::min(c + max_depth, len);
            if (c + d < end) next.push_back({text[c + d], c});
        }
        std::vector<int32_t>().swap(nodes[id].votes);
        std::sort(next.begin(), next.end());
        for (size_t i = 0; i < next.size();) {
            size_t j = i;
            while (j < next.size() && next[j].first == next[i].first) ++j;
            Node ch;
            ch.depth = d + 1;
            ch.count = (int32_t)(j - i);
            ch.rep = next[i].second;
            ch.token = next[i].first;
            ch.parent = id;
            ch.votes.reserve(j - i);
            for (size_t k = i; k < j; ++k) ch.votes.push_back(next[k].second);
            nodes.push_back(std::move(ch));
            push((int)nodes.size() - 1);
            i = j;
        }
    }
};

}  // namespace

extern "C" int tv_lookup_draft(const int32_t *text, int len, int min_order, int max_order, int max_depth,
                               int max_nodes, float rho, int32_t *parents, int32_t *tokens, float *q,
                               int32_t *order, int *n_nodes, int *match_order, int *n_votes) {
    if (!text || len < 1 || !parents || !tokens || !q || !n_nodes) return TV_EINVAL;
    if (min_order < 1 || max_order < min_order || max_order > TV_LOOKUP_MAX_ORDER) return TV_EINVAL;
    if (max_depth < 1 || max_depth > TV_MAX_CANDIDATE) return TV_EINVAL;
    if (max_nodes < 0 || max_nodes > TV_MAX_CANDIDATE - 1 || (max_nodes > 0 && !order)) return TV_EINVAL;
    if (!(rho > 0.f && rho <= 1.f)) return TV_EINVAL;
    try {
        // match length of every earlier end position against the text's end
        int o = 0;
        std::vector<int32_t> ell(len > 1 ? len - 1 : 0);
        for (int e = 0; e + 1 < len; ++e) {
            int j = 0;
            while (j < max_order && j <= e && text[e - j] == text[len - 1 - j]) ++j;
            ell[e] = j;
            o = std::max(o, j);
        }
        if (o < min_order) o = 0;
        Tree t{text, len, max_depth, {}};
        t.nodes.reserve(64);
        Node root;
        root.token = text[len - 1];
        if (o > 0)
            for (int e = 0; e + 1 < len; ++e)
                if (ell[e] >= o) root.votes.push_back(e + 1);   // the continuation starts after the match
        const int V = (int)root.votes.size();
        root.count = V;
        t.nodes.push_back(std::move(root));

        auto worse = [&t](int a, int b) { return t.before(b, a); };
        std::priority_queue<int, std::vector<int>, decltype(worse)> frontier(worse);
        std::vector<int32_t> admitted;
        if (V > 0 && max_nodes > 0) {
            t.expand(0, [&](int id) { frontier.push(id); });
            while ((int)admitted.size() < max_nodes && !frontier.empty()) {
                const int id = frontier.top();
                frontier.pop();
                admitted.push_back(id);
                t.nodes[t.nodes[id].parent].kids.push_back(id);
                t.expand(id, [&](int ch) { frontier.push(ch); });
            }
        }
        // depth-first pre-order, siblings by (count descending, token ascending)
        int n = 0;
        std::vector<std::pair<int, int>> stack{{0, -1}};
        while (!stack.empty()) {
            const auto [id, par] = stack.back();
            stack.pop_back();
            Node &x = t.nodes[id];
            x.out = n;
            parents[n] = par;
            tokens[n] = x.token;
            double decay = 1.0;   // rho^depth as depth products, in the oracle's order
            for (int d = 0; d < x.depth; ++d) decay *= (double)rho;
            q[n] = id == 0 ? 1.0f : (float)((double)x.count / (double)V * decay);
            ++n;
            std::sort(x.kids.begin(), x.kids.end(), [&t](int a, int b) {
                const Node &u = t.nodes[a], &v = t.nodes[b];
                return u.count != v.count ? u.count > v.count : u.token < v.token;
            });
            for (auto it = x.kids.rbegin(); it != x.kids.rend(); ++it) stack.push_back({*it, x.out});
        }
        for (size_t k = 0; k < admitted.size(); ++k) order[k] = t.nodes[admitted[k]].out;
        *n_nodes = n;
        if (match_order) *match_order = o;
        if (n_votes) *n_votes = V;
        return TV_OK;
    } catch (const std::bad_alloc &) {
        return TV_EINVAL;
    }
}
