// Host runtime of the tree-verify library: model descriptor, bound buffers,
// per-request state, tree validation and metadata, launch sequence, accept
// walk and commit.  Exposes the C ABI declared in include/treeverify.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/treeverify.h"
#include "tv_internal.h"

using namespace tv;

namespace {

struct Req {
    int ctx_len = 0;
    std::vector<int32_t> history;
    std::vector<uint16_t *> K, V;  // per layer (attention layers)
    std::vector<float *> S;        // per layer (recurrent layers)
    // modifiers
    float rep = 1.f;
    bool mods_on = false;
    std::vector<uint32_t> hist_bits;  // host copy of prior-token bits
    uint32_t *d_hist = nullptr;
    float *d_bias = nullptr;
    uint32_t *d_allow = nullptr;
    bool has_bias = false, has_allow = false;
    // sampling (temp 0: greedy)
    float temp = 0.f;
    uint64_t seed = 0;
    // pending tree of the last verify
    bool pending = false;
    std::vector<int32_t> pparents, ptokens;
    int prow0 = 0;
    // device pointer table {K0, V0, K1, V1, ...} over attention layers
    uint16_t **d_kvtab = nullptr;
    bool kvtab_dirty = true;
    // recurrent layers: bound state table and the last verify's saved k, v, gc
    float **d_stab = nullptr;
    bool stab_dirty = true;
    uint16_t *save_k = nullptr;
    float *save_v = nullptr;   // values, or a delta layer's pseudo-values (fp32)
    float *save_gc = nullptr;
};

struct ProfRec {
    const char *name;
    hipEvent_t a, b;
};

} // namespace

struct tv_ctx {
    tv_model_desc m{};
    std::vector<int> kinds;
    std::vector<int> attn_layers;
    std::vector<int> recur_layers;
    std::vector<int> recur_index;   // layer -> position in recur_layers (or -1)
    hipStream_t stream = nullptr;
    std::string err;
    int G = 1;

    // weights
    const uint16_t *emb = nullptr, *head = nullptr, *final_norm = nullptr;
    std::vector<const uint16_t *> attn_norm, wqkv, wo, wa, ffn_norm, wg, wu, wd;

    std::vector<Req> reqs;

    // scratch (library-owned)
    uint16_t *X = nullptr, *XN = nullptr, *QR = nullptr, *ATT = nullptr, *ACT = nullptr;
    float *logits = nullptr;  // [32, V] when the caller passes none
    void *zeros = nullptr;    // 256 zero bytes
    // dense prefill scratch (allocated on first use, for pf_rows rows)
    int pf_rows = 0;
    uint16_t *pX = nullptr, *pXN = nullptr, *pQKV = nullptr, *pQR = nullptr, *pATT = nullptr, *pACT = nullptr;
    uint16_t *pAB = nullptr;   // recurrent layers: gate (and write-strength) rows
    int32_t *pTok = nullptr, *h_tok = nullptr;
    float *ppo = nullptr, *ppm = nullptr, *ppl = nullptr;
    Top2 *part = nullptr;
    float *po = nullptr, *pm = nullptr, *pl = nullptr;
    float *rope_cos = nullptr, *rope_sin = nullptr;
    PassMeta *d_meta = nullptr;
    float *gemm_partial = nullptr;   // split-K partial tiles
    size_t gemm_partial_floats = 0;
    // pinned host staging
    // pass metadata: written by the host into coherent pinned memory (h_meta;
    // hd_meta the same memory seen from the GPU); the pass's first kernel
    // copies it to d_meta
    PassMeta *h_meta = nullptr, *hd_meta = nullptr;
    // per-row results of a pass (RowResult), written by the top-2 kernel
    // straight into coherent pinned host memory (hd_res: the same memory
    // seen from the GPU)
    RowResult *h_res = nullptr;
    RowResult *hd_res = nullptr;
    // residual tree sampling: per-row uniforms (pinned staging and device copy)
    double *h_resu = nullptr, *d_resu = nullptr;
    void *d_resparts = nullptr;   // per-row chunk maxima and sums of the residual decision
    // device pointer table for the kernel-level calls (pinned staging and device copy)
    void **h_tab = nullptr, **d_tab = nullptr;
    int ns_max = 0;

    // profiling
    bool prof = false;
    std::string prof_only;
    std::vector<ProfRec> recs;
    size_t rec_used = 0;
    std::vector<std::pair<std::string, std::pair<double, int>>> totals;
};

namespace {

int fail(tv_ctx *c, int code, const char *fmt, ...) {
    if (c) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        c->err = buf;
    }
    return code;
}

#define HIPCHECK(c, expr)                                                                   \
    do {                                                                                    \
        hipError_t e_ = (expr);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail((c), TV_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));      \
    } while (0)

size_t vocab_words(const tv_model_desc &m) { return (size_t)(m.vocab + 31) / 32; }

// Record a launch with optional event timing.
struct Launch {
    tv_ctx *c;
    const char *name;
    ProfRec *rec = nullptr;
    Launch(tv_ctx *ctx, const char *nm) : c(ctx), name(nm) {
        if (c->prof && !strncmp(nm, c->prof_only.c_str(), c->prof_only.size())) {
            if (c->rec_used == c->recs.size()) {
                ProfRec r{nm, nullptr, nullptr};
                hipEventCreate(&r.a);
                hipEventCreate(&r.b);
                c->recs.push_back(r);
            }
            rec = &c->recs[c->rec_used++];
            rec->name = nm;
            hipEventRecord(rec->a, c->stream);
        }
    }
    void done() {
        if (rec) hipEventRecord(rec->b, c->stream);
    }
};

void harvest(tv_ctx *c) {
    for (size_t i = 0; i < c->rec_used; ++i) {
        float ms = 0.f;
        hipEventElapsedTime(&ms, c->recs[i].a, c->recs[i].b);
        bool found = false;
        for (auto &t : c->totals)
            if (t.first == c->recs[i].name) {
                t.second.first += ms;
                t.second.second += 1;
                found = true;
                break;
            }
        if (!found) c->totals.push_back({c->recs[i].name, {(double)ms, 1}});
    }
    c->rec_used = 0;
}

// Mark the result records of rows [0, M) empty (before enqueueing a pass).
void clear_results(tv_ctx *c, int M) {
    volatile RowResult *r = c->h_res;
    for (int m = 0; m < M; ++m) {
        r[m].argmax = -1;
        r[m].gap_bits = kGapEmpty;
    }
    std::atomic_thread_fence(std::memory_order_release);
}

// Wait until the kernel that decides the rows has filled every row's record
// (one 8-byte store each, so a gap field other than the empty pattern means
// the whole record has landed; the argmax field may hold any value, -1
// included): spin on the pinned host copy (lower wake-up latency than a
// stream synchronisation),
// polling the stream now and then so that a failed or drained stream ends
// the wait.  With event profiling on, synchronise the stream so the events
// can be read.
int wait_results(tv_ctx *c, int M) {
    if (c->prof) {
        HIPCHECK(c, hipStreamSynchronize(c->stream));
        harvest(c);
    }
    volatile RowResult *r = c->h_res;
    int m = 0;
    for (long it = 1;; ++it) {
        while (m < M && r[m].gap_bits != kGapEmpty) ++m;
        if (m == M) break;
        if ((it & 4095) == 0) {
            const hipError_t q = hipStreamQuery(c->stream);
            if (q == hipSuccess) {
                while (m < M && r[m].gap_bits != kGapEmpty) ++m;
                if (m == M) break;
                return fail(c, TV_EHIP, "pass finished without the result of row %d", m);
            }
            if (q != hipErrorNotReady) return fail(c, TV_EHIP, "stream failed: %s", hipGetErrorString(q));
        }
        __builtin_ia32_pause();
    }
    std::atomic_thread_fence(std::memory_order_acquire);
    return TV_OK;
}

// Copy the records out: argmax[m] and gap[m] (either may be null).
void read_results(tv_ctx *c, int M, int32_t *argmax, float *gap) {
    for (int m = 0; m < M; ++m) {
        if (argmax) argmax[m] = c->h_res[m].argmax;
        if (gap) memcpy(gap + m, &c->h_res[m].gap_bits, 4);
    }
}

// A call that fails after it has enqueued work returns only once that work
// has drained: otherwise a kernel of the failed call could still be reading
// the pinned pass metadata (or scratch) that the next call rewrites.
struct DrainOnError {
    tv_ctx *c;
    bool armed = true;
    explicit DrainOnError(tv_ctx *ctx) : c(ctx) {}
    ~DrainOnError() {
        if (armed) hipStreamSynchronize(c->stream);
    }
    void done() { armed = false; }
};

#define LAUNCH(c, nm, call)                                                                  \
    do {                                                                                     \
        Launch L_(c, nm);                                                                    \
        hipError_t e_ = (call);                                                              \
        L_.done();                                                                           \
        if (e_ != hipSuccess) return fail(c, TV_EHIP, "launch %s: %s", nm, hipGetErrorString(e_)); \
    } while (0)

int check_req(tv_ctx *c, int req) {
    if (!c) return TV_EINVAL;
    if (req < 0 || req >= c->m.max_req) return fail(c, TV_EINVAL, "request %d out of range", req);
    return TV_OK;
}

int check_bound(tv_ctx *c, const std::vector<int> &reqs) {
    const tv_model_desc &m = c->m;
    if (!c->emb || !c->head || !c->final_norm) return fail(c, TV_ESTATE, "emb/head/final_norm not bound");
    for (int l = 0; l < m.n_layer; ++l) {
        if (!c->attn_norm[l] || !c->wqkv[l] || !c->wo[l] || !c->ffn_norm[l] || !c->wg[l] || !c->wu[l] ||
            !c->wd[l])
            return fail(c, TV_ESTATE, "layer %d weights not bound", l);
        if (c->kinds[l] != TV_LAYER_ATTN && !c->wa[l]) return fail(c, TV_ESTATE, "layer %d wa not bound", l);
    }
    for (int r : reqs) {
        const Req &q = c->reqs[r];
        for (int l = 0; l < m.n_layer; ++l) {
            if (c->kinds[l] == TV_LAYER_ATTN && (!q.K[l] || !q.V[l]))
                return fail(c, TV_ESTATE, "request %d layer %d KV cache not bound", r, l);
            if (c->kinds[l] != TV_LAYER_ATTN && !q.S[l])
                return fail(c, TV_ESTATE, "request %d layer %d state not bound", r, l);
        }
    }
    return TV_OK;
}

// Tree rules ("Algorithm and correctness contract", Target position and
// batching): parents before children, distinct sibling tokens.
int validate_tree(tv_ctx *c, const int32_t *parents, const int32_t *tokens, int n) {
    if (!parents || !tokens) return fail(c, TV_EINVAL, "null tree");
    if (n < 1 || n > TV_MAX_NODES) return fail(c, TV_EINVAL, "n_nodes %d not in [1, %d]", n, TV_MAX_NODES);
    if (parents[0] != -1) return fail(c, TV_EINVAL, "parents[0] must be -1");
    for (int i = 0; i < n; ++i) {
        if (tokens[i] < 0 || tokens[i] >= c->m.vocab) return fail(c, TV_EINVAL, "token %d out of range", i);
        if (i > 0 && (parents[i] < 0 || parents[i] >= i))
            return fail(c, TV_EINVAL, "parents[%d] = %d not in [0, %d)", i, parents[i], i);
    }
    for (int i = 1; i < n; ++i)
        for (int j = 1; j < i; ++j)
            if (parents[j] == parents[i] && tokens[j] == tokens[i])
                return fail(c, TV_EINVAL, "sibling nodes %d and %d carry the same token", j, i);
    return TV_OK;
}

int upload_kvtab(tv_ctx *c, Req &q) {
    if (!q.kvtab_dirty) return TV_OK;
    std::vector<uint16_t *> tab;
    for (int l : c->attn_layers) {
        tab.push_back(q.K[l]);
        tab.push_back(q.V[l]);
    }
    if (!tab.empty()) {
        if (!q.d_kvtab) HIPCHECK(c, hipMalloc(&q.d_kvtab, tab.size() * sizeof(void *)));
        HIPCHECK(c, hipMemcpyAsync(q.d_kvtab, tab.data(), tab.size() * sizeof(void *),
                                   hipMemcpyHostToDevice, c->stream));
        HIPCHECK(c, hipStreamSynchronize(c->stream));
    }
    q.kvtab_dirty = false;
    return TV_OK;
}

size_t gemm_partial_need(int N, int K, bool dual, bool always = false) {
    const int S = gemm_splits(N, K);
    if (S <= 1 && !always) return 0;
    const size_t rowblocks = (size_t)((N + 31) / 32 + 3) / 4;
    return rowblocks * S * (dual ? 2 : 1) * 4096;
}

// Rearrange a row-major [N, K] bf16 matrix in place into the packed tile
// order of the GEMM kernel, a chunk of whole tiles at a time.
int pack_inplace(tv_ctx *c, void *ptr, int N, int K) {
    const int ntiles = (N + 31) / 32;
    const size_t tile_bytes = (size_t)32 * K * 2;
    const int per = (int)std::max<size_t>(1, ((size_t)64 << 20) / tile_bytes);
    uint16_t *tmp = nullptr;
    HIPCHECK(c, hipMalloc(&tmp, std::min(per, ntiles) * tile_bytes));
    hipError_t e = hipSuccess;
    for (int t0 = 0; t0 < ntiles && e == hipSuccess; t0 += per) {
        const int nt = std::min(per, ntiles - t0);
        const size_t rows = std::min((size_t)nt * 32, (size_t)N - (size_t)t0 * 32);
        e = hipMemcpyAsync(tmp, (uint16_t *)ptr + (size_t)t0 * 32 * K, rows * K * 2, hipMemcpyDeviceToDevice,
                           c->stream);
        if (e == hipSuccess) e = launch_pack(c->stream, tmp, (uint16_t *)ptr, N, K, t0, nt);
        if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    }
    hipFree(tmp);
    if (e != hipSuccess) return fail(c, TV_EHIP, "packing a weight failed: %s", hipGetErrorString(e));
    return TV_OK;
}

int gemm(tv_ctx *c, const char *name, int epi, GemmArgs g) {
    g.partial = c->gemm_partial;
    g.zeros = c->zeros;
    // the head's top-2 epilogue needs whole sums in the kernel: it never splits
    const int S = epi == EPI_HEAD ? 1 : gemm_splits(g.N, g.K);
    if (S > 1 && gemm_partial_need(g.N, g.K, epi == EPI_SWIGLU) > c->gemm_partial_floats)
        return fail(c, TV_EINVAL, "GEMM N=%d K=%d needs more split-K scratch than allocated", g.N, g.K);
    LAUNCH(c, name, launch_gemm(c->stream, epi, g, S));
    if (S > 1) LAUNCH(c, "splitk_finish", launch_splitk_reduce(c->stream, epi, g, S));
    return TV_OK;
}

// A projection whose consumer finishes the sums: partials only (at float
// offset `off` of the split-K scratch), *S = splits.
int gemm_partial(tv_ctx *c, const char *name, GemmArgs g, int *S, size_t off = 0) {
    g.partial = c->gemm_partial + off;
    g.zeros = c->zeros;
    *S = gemm_splits(g.N, g.K);
    if (off + gemm_partial_need(g.N, g.K, false, true) > c->gemm_partial_floats)
        return fail(c, TV_EINVAL, "GEMM N=%d K=%d needs more split-K scratch than allocated", g.N, g.K);
    LAUNCH(c, name, launch_gemm(c->stream, EPI_PARTIAL, g, *S));
    return TV_OK;
}

#define GEMMP(c, nm, g, S)                          \
    do {                                            \
        int rc_ = gemm_partial((c), (nm), (g), &(S)); \
        if (rc_) return rc_;                        \
    } while (0)

#define GEMM(c, nm, epi, g)                 \
    do {                                    \
        int rc_ = gemm((c), (nm), (epi), (g)); \
        if (rc_) return rc_;                \
    } while (0)

int upload_stab(tv_ctx *c, Req &q) {
    if (!q.stab_dirty || c->recur_layers.empty()) return TV_OK;
    std::vector<float *> tab;
    for (int l : c->recur_layers) tab.push_back(q.S[l]);
    if (!q.d_stab) HIPCHECK(c, hipMalloc(&q.d_stab, tab.size() * sizeof(void *)));
    HIPCHECK(c, hipMemcpyAsync(q.d_stab, tab.data(), tab.size() * sizeof(void *), hipMemcpyHostToDevice,
                               c->stream));
    HIPCHECK(c, hipStreamSynchronize(c->stream));
    q.stab_dirty = false;
    return TV_OK;
}

// One forward pass over `total` rows of up to 32, request after request.
int run_pass(tv_ctx *c, int n_req, const int *reqs, const int32_t *const *parents,
             const int32_t *const *tokens, const int *n_nodes, float *logits_dev, int32_t *argmax,
             float *gap) {
    const tv_model_desc &m = c->m;
    int total = 0;
    for (int r = 0; r < n_req; ++r) {
        int rc = check_req(c, reqs[r]);
        if (rc) return rc;
        for (int s = 0; s < r; ++s)
            if (reqs[s] == reqs[r]) return fail(c, TV_EINVAL, "request %d appears twice", reqs[r]);
        rc = validate_tree(c, parents[r], tokens[r], n_nodes[r]);
        if (rc) return rc;
        if (c->reqs[reqs[r]].ctx_len + n_nodes[r] > m.max_ctx)
            return fail(c, TV_ECAPACITY, "request %d: ctx %d + %d rows > max_ctx %d", reqs[r],
                        c->reqs[reqs[r]].ctx_len, n_nodes[r], m.max_ctx);
        total += n_nodes[r];
    }
    if (total > TV_MAX_NODES) return fail(c, TV_EINVAL, "%d rows in one pass > %d", total, TV_MAX_NODES);
    {
        std::vector<int> rv(reqs, reqs + n_req);
        int rc = check_bound(c, rv);
        if (rc) return rc;
    }
    for (int r = 0; r < n_req; ++r) {
        int rc = upload_kvtab(c, c->reqs[reqs[r]]);
        if (rc) return rc;
        rc = upload_stab(c, c->reqs[reqs[r]]);
        if (rc) return rc;
    }

    // metadata
    PassMeta &pm = *c->h_meta;
    memset(&pm, 0, sizeof pm);
    bool any_mods = false;
    int row0 = 0;
    std::vector<int> row0s(n_req);
    for (int r = 0; r < n_req; ++r) {
        const int n = n_nodes[r];
        Req &q = c->reqs[reqs[r]];
        row0s[r] = row0;
        for (int i = 0; i < n; ++i) {
            const int g = row0 + i;
            const int p = parents[r][i];
            pm.tok[g] = tokens[r][i];
            pm.depth[g] = p < 0 ? 0 : pm.depth[row0 + p] + 1;
            pm.anc[g] = (p < 0 ? 0u : pm.anc[row0 + p]) | (1u << i);
            pm.row_req[g] = r;
            pm.draw_t[g] = q.ctx_len + pm.depth[g] + 1;
            // tokens on root..i
            int L = 0, stack[TV_MAX_NODES];
            for (int j = i; j >= 0; j = parents[r][j]) stack[L++] = tokens[r][j];
            pm.path_len[g] = L;
            for (int d = 0; d < L; ++d) pm.path_tok[g * kMaxRows + d] = stack[L - 1 - d];
        }
        HeadMods &hm = pm.mods[r];
        hm.rep = q.rep;
        hm.hist_bits = (q.mods_on && q.rep != 1.f) ? q.d_hist : nullptr;
        hm.bias = (q.mods_on && q.has_bias) ? q.d_bias : nullptr;
        hm.allow_bits = (q.mods_on && q.has_allow) ? q.d_allow : nullptr;
        if (!q.mods_on) hm.rep = 1.f;
        hm.temp = q.temp;
        hm.seed_lo = (uint32_t)q.seed;
        hm.seed_hi = (uint32_t)(q.seed >> 32);
        any_mods |= q.mods_on || q.temp > 0.f;
        row0 += n;
    }
    const int M = total;
    hipStream_t s = c->stream;
    clear_results(c, M);   // its release fence also publishes the metadata, which the GPU reads where it lies

    const int H = m.hidden, D = m.head_dim, QH = m.n_qhead, KVH = m.n_kvhead;
    // X: residual stream; XN = RMSNorm(X) with the weights of the next
    // projection that reads it (xn_w), written by the kernel that updates X.
    const uint16_t *xn_w = c->attn_norm[0];
    DrainOnError drain(c);
    LAUNCH(c, "embed_norm", launch_embed_norm(s, c->emb, c->hd_meta, c->d_meta, M, H, xn_w, m.eps, c->X, c->XN));
    auto normed = [&](GemmArgs &g, const uint16_t *w) -> int {
        if (xn_w != w) return fail(c, TV_ESTATE, "internal: normalised rows hold another norm");
        g.X = c->XN; g.ldx = H;
        return TV_OK;
    };
#define NORMED(g, w)                 \
    do {                             \
        int rc_ = normed((g), (w));  \
        if (rc_) return rc_;         \
    } while (0)
    for (int l = 0; l < m.n_layer; ++l) {
        if (c->kinds[l] == TV_LAYER_ATTN) {
            GemmArgs g{};
            NORMED(g, c->attn_norm[l]);
            g.W = c->wqkv[l]; g.M = M; g.N = (QH + 2 * KVH) * D; g.K = H;
            int S = 0;
            GEMMP(c, "gemm_qkv", g, S);
            // one launch of each kernel serves every request of the pass
            RopeArgs ra{};
            ra.part = c->gemm_partial; ra.S = S; ra.q_out = c->QR;
            ra.cosT = c->rope_cos; ra.sinT = c->rope_sin; ra.meta = c->d_meta;
            ra.M = M; ra.cap = m.max_ctx; ra.QH = QH; ra.KVH = KVH; ra.D = D; ra.nreq = n_req;
            AttnArgs aa{};
            aa.Q = c->QR; aa.meta = c->d_meta; aa.po = c->po; aa.pm = c->pm; aa.pl = c->pl;
            aa.cap = m.max_ctx; aa.G = c->G; aa.n_qhead = QH;
            aa.scale = (float)(1.0 / std::sqrt((double)D));
            aa.nreq = n_req;
            for (int r = 0; r < n_req; ++r) {
                Req &q = c->reqs[reqs[r]];
                PassReq &p = ra.rq[r];
                p.Kc = q.K[l]; p.Vc = q.V[l];
                p.row0 = row0s[r]; p.n = n_nodes[r]; p.ctx = q.ctx_len;
                p.span = attn_span(q.ctx_len);
                p.nsplit = (q.ctx_len + p.span - 1) / p.span;
                aa.rq[r] = p;
                aa.n = std::max(aa.n, p.n);
                aa.span = std::max(aa.span, p.span);
                aa.ns = std::max(aa.ns, p.nsplit + 1);
            }
            // attention takes the longest contexts first: the grid is dispatched
            // in request order, and a short request's workgroups then fill the
            // CUs the long ones leave rather than holding them back (partials sit
            // at pass rows, so the order changes no result)
            std::stable_sort(aa.rq, aa.rq + n_req, [](const PassReq &x, const PassReq &y) { return x.ctx > y.ctx; });
            LAUNCH(c, "rope_kv", launch_rope_kv(s, ra));
            LAUNCH(c, "attn", launch_attn(s, D, aa));
            LAUNCH(c, "attn_combine", launch_attn_combine(s, D, aa, c->ATT));
        } else {
            const int rl = c->recur_index[l];
            // one projection over the q/k/v rows stacked on the gate rows
            // (and a delta layer's write-strength rows) leaves split-K
            // partials; the read-out kernel finishes them
            const bool delta = c->kinds[l] == TV_LAYER_DELTA;
            GemmArgs g{};
            NORMED(g, c->attn_norm[l]);
            g.W = c->wqkv[l]; g.W2 = c->wa[l]; g.N1 = 3 * QH * D;
            g.M = M; g.N = 3 * QH * D + (delta ? 2 : 1) * QH; g.K = H;
            int Sq = 0;
            GEMMP(c, "gemm_qkv", g, Sq);
            for (int r = 0; r < n_req; ++r) {
                Req &q = c->reqs[reqs[r]];
                RecurArgs ra{};
                ra.qkv_part = c->gemm_partial; ra.qkv_S = Sq;
                ra.a_col = 3 * QH * D; ra.delta = delta;
                ra.S0 = q.S[l]; ra.meta = c->d_meta; ra.out = c->ATT;
                const size_t per = (size_t)kMaxRows * QH * D;
                ra.save_k = q.save_k + rl * per;
                ra.save_v = q.save_v + rl * per;
                ra.save_gc = q.save_gc + (size_t)rl * kMaxRows * QH;
                ra.row0 = row0s[r]; ra.n = n_nodes[r]; ra.QH = QH; ra.eps = m.eps;
                LAUNCH(c, "recur_tree", launch_recur_tree(s, D, ra));
            }
        }
        {
            GemmArgs g{};
            g.X = c->ATT; g.ldx = QH * D; g.W = c->wo[l]; g.M = M; g.N = H; g.K = QH * D;
            int S = 0;
            GEMMP(c, "gemm_o", g, S);
            xn_w = c->ffn_norm[l];
            LAUNCH(c, "resid_norm", launch_resid_norm(s, c->gemm_partial, S, M, H, xn_w, m.eps, c->X, c->XN));
        }
        {
            GemmArgs g{};
            NORMED(g, c->ffn_norm[l]);
            g.W = c->wg[l]; g.W2 = c->wu[l]; g.M = M; g.N = m.ffn; g.K = H;
            g.Y = c->ACT; g.ldy = m.ffn;
            GEMM(c, "gemm_gateup", EPI_SWIGLU, g);
        }
        {
            GemmArgs g{};
            g.X = c->ACT; g.ldx = m.ffn; g.W = c->wd[l]; g.M = M; g.N = H; g.K = m.ffn;
            int S = 0;
            GEMMP(c, "gemm_down", g, S);
            xn_w = l + 1 < m.n_layer ? c->attn_norm[l + 1] : c->final_norm;
            LAUNCH(c, "resid_norm", launch_resid_norm(s, c->gemm_partial, S, M, H, xn_w, m.eps, c->X, c->XN));
        }
    }
    float *out = logits_dev ? logits_dev : c->logits;
    {
        GemmArgs g{};
        NORMED(g, c->final_norm);
        g.W = c->head; g.M = M; g.N = m.vocab; g.K = H;
        g.Yf = out; g.ldyf = m.vocab; g.part = c->part; g.meta = c->d_meta; g.mods_on = any_mods;
        GEMM(c, "gemm_head", EPI_HEAD, g);
    }
    LAUNCH(c, "top2", launch_top2_reduce(s, c->part, ((m.vocab + 31) / 32 + 3) / 4, M, c->hd_res));
    {
        const int rc = wait_results(c, M);
        if (rc) return rc;
    }
    drain.done();
    read_results(c, M, argmax, gap);

    for (int r = 0; r < n_req; ++r) {
        Req &q = c->reqs[reqs[r]];
        q.pending = true;
        q.pparents.assign(parents[r], parents[r] + n_nodes[r]);
        q.ptokens.assign(tokens[r], tokens[r] + n_nodes[r]);
        q.prow0 = row0s[r];
    }
    // a pass overwrites shared scratch: other requests' pending trees stay
    // valid for their KV (held in their own caches) only.
    return TV_OK;
}

void set_bit(std::vector<uint32_t> &b, int v) { b[v >> 5] |= 1u << (v & 31); }



} // namespace

extern "C" {

int tv_create(const tv_model_desc *md, void *stream, tv_ctx **out) {
    if (!md || !out) return TV_EINVAL;
    *out = nullptr;
    const tv_model_desc &m = *md;
    if (m.n_layer < 1 || m.hidden < 64 || m.hidden % 64 || m.n_qhead < 1 || m.n_kvhead < 1 ||
        m.n_qhead % m.n_kvhead || (m.head_dim != 64 && m.head_dim != 128) || m.ffn < 8 || m.ffn % 8 ||
        m.vocab < 2 || m.max_ctx < 1 || m.max_req < 1 || !m.layer_kind || m.eps <= 0.f)
        return TV_EINVAL;
    if (m.n_qhead / m.n_kvhead > 5) return TV_EINVAL;  // attention stages G*32 <= 160 query rows
    if (m.hidden > 8192) return TV_EINVAL;              // a norm workgroup holds one row
    tv_ctx *c = new tv_ctx();
    c->m = m;
    c->kinds.assign(m.layer_kind, m.layer_kind + m.n_layer);
    for (int l = 0; l < m.n_layer; ++l) {
        if (c->kinds[l] != TV_LAYER_ATTN && c->kinds[l] != TV_LAYER_RECUR && c->kinds[l] != TV_LAYER_DELTA) {
            delete c;
            return TV_EINVAL;
        }
        c->recur_index.push_back(-1);
        if (c->kinds[l] == TV_LAYER_ATTN) {
            c->attn_layers.push_back(l);
        } else {
            c->recur_index[l] = (int)c->recur_layers.size();
            c->recur_layers.push_back(l);
        }
    }
    c->m.layer_kind = nullptr;
    c->stream = (hipStream_t)stream;
    c->G = m.n_qhead / m.n_kvhead;
    const int L = m.n_layer;
    c->attn_norm.assign(L, nullptr); c->wqkv.assign(L, nullptr); c->wo.assign(L, nullptr);
    c->wa.assign(L, nullptr); c->ffn_norm.assign(L, nullptr); c->wg.assign(L, nullptr);
    c->wu.assign(L, nullptr); c->wd.assign(L, nullptr);
    c->reqs.resize(m.max_req);
    for (auto &q : c->reqs) {
        q.K.assign(L, nullptr); q.V.assign(L, nullptr); q.S.assign(L, nullptr);
        q.hist_bits.assign(vocab_words(m), 0u);
    }
    auto cleanup = [&](int rc) { tv_destroy(c); return rc; };
    const int R = kMaxRows;
    const int H = m.hidden, D = m.head_dim;
    c->ns_max = 32 + 1;  // at most 32 cache splits (attn_span's 31; a prefill block's 32) plus the tree split
    const size_t RP = (size_t)kMaxRows * kMaxGroup;
    hipError_t e = hipSuccess;
#define ALLOC(p, bytes) if (e == hipSuccess) e = hipMalloc((void **)&(p), (bytes))
    ALLOC(c->X, (size_t)R * H * 2);
    ALLOC(c->XN, (size_t)R * H * 2);
    ALLOC(c->QR, (size_t)R * m.n_qhead * D * 2);
    ALLOC(c->ATT, (size_t)R * m.n_qhead * D * 2);
    ALLOC(c->ACT, (size_t)R * m.ffn * 2);
    ALLOC(c->zeros, 256);
    if (e == hipSuccess) e = hipMemset(c->zeros, 0, 256);
    if (!c->recur_layers.empty()) {
        const size_t nrl = c->recur_layers.size();
        for (auto &q : c->reqs) {
            ALLOC(q.save_k, nrl * R * m.n_qhead * D * 2);
            ALLOC(q.save_v, nrl * R * m.n_qhead * D * 4);
            ALLOC(q.save_gc, nrl * R * m.n_qhead * 4);
        }
    }
    ALLOC(c->logits, (size_t)R * m.vocab * 4);
    ALLOC(c->part, (size_t)((m.vocab + 31) / 32) * 32 * sizeof(Top2));
    ALLOC(c->po, (size_t)m.n_kvhead * c->ns_max * RP * D * 4);
    ALLOC(c->pm, (size_t)m.n_kvhead * c->ns_max * RP * 4);
    ALLOC(c->pl, (size_t)m.n_kvhead * c->ns_max * RP * 4);
    ALLOC(c->rope_cos, (size_t)m.max_ctx * (D / 2) * 4);
    ALLOC(c->rope_sin, (size_t)m.max_ctx * (D / 2) * 4);
    ALLOC(c->d_meta, sizeof(PassMeta));
    {
        const int QD = m.n_qhead * D;
        size_t need = (size_t)8 << 20;  // room for kernel-level calls
        need = std::max(need, gemm_partial_need((m.n_qhead + 2 * m.n_kvhead) * D, H, false, true));
        need = std::max(need, gemm_partial_need(3 * QD + 2 * m.n_qhead, H, false, true));   // recurrent qkv + gate (+ write strength)
        need = std::max(need, gemm_partial_need(H, QD, false, true));
        need = std::max(need, gemm_partial_need(m.ffn, H, true));
        need = std::max(need, gemm_partial_need(H, m.ffn, false, true));
        need = std::max(need, gemm_partial_need(m.vocab, H, false));
        c->gemm_partial_floats = need;
    }
    ALLOC(c->gemm_partial, c->gemm_partial_floats * 4);
#undef ALLOC
    const unsigned res_flags = hipHostMallocCoherent | hipHostMallocMapped;
    if (e == hipSuccess) e = hipHostMalloc((void **)&c->h_meta, sizeof(PassMeta), res_flags);
    if (e == hipSuccess) e = hipHostGetDevicePointer((void **)&c->hd_meta, c->h_meta, 0);
    if (e == hipSuccess) e = hipHostMalloc((void **)&c->h_res, R * sizeof(RowResult), res_flags);
    if (e == hipSuccess) e = hipHostGetDevicePointer((void **)&c->hd_res, c->h_res, 0);
    if (e == hipSuccess) e = hipHostMalloc((void **)&c->h_resu, R * sizeof(double), hipHostMallocDefault);
    if (e == hipSuccess) e = hipMalloc((void **)&c->d_resu, R * sizeof(double));
    if (e == hipSuccess) e = hipMalloc(&c->d_resparts, R * kResidualPartBytes);
    if (e == hipSuccess) e = hipHostMalloc((void **)&c->h_tab, 16 * sizeof(void *), hipHostMallocDefault);
    if (e == hipSuccess) e = hipMalloc((void **)&c->d_tab, 16 * sizeof(void *));
    if (e != hipSuccess) return cleanup(TV_EHIP);
    // RoPE table: angle pos * theta^(-2i/D) in fp64, cos and sin rounded to fp32
    {
        std::vector<float> cs((size_t)m.max_ctx * (D / 2)), sn(cs.size());
        for (int p = 0; p < m.max_ctx; ++p)
            for (int i = 0; i < D / 2; ++i) {
                const double ang = (double)p * std::pow((double)m.rope_theta, -2.0 * i / D);
                cs[(size_t)p * (D / 2) + i] = (float)std::cos(ang);
                sn[(size_t)p * (D / 2) + i] = (float)std::sin(ang);
            }
        e = hipMemcpy(c->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(c->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice);
        if (e != hipSuccess) return cleanup(TV_EHIP);
    }
    *out = c;
    return TV_OK;
}

void tv_destroy(tv_ctx *c) {
    if (!c) return;
    if (c->stream) hipStreamSynchronize(c->stream);
    else hipDeviceSynchronize();
    void *dev[] = {c->X, c->XN, c->QR, c->ATT, c->ACT, c->zeros, c->logits, c->part, c->po, c->pm, c->pl,
                   c->rope_cos, c->rope_sin, c->d_meta, c->gemm_partial, c->pX, c->pXN, c->pQKV, c->pQR,
                   c->pATT, c->pACT, c->pAB, c->pTok, c->ppo, c->ppm, c->ppl, c->d_resu, c->d_resparts,
                   c->d_tab};
    for (void *p : dev)
        if (p) hipFree(p);
    for (auto &q : c->reqs) {
        if (q.d_hist) hipFree(q.d_hist);
        if (q.d_bias) hipFree(q.d_bias);
        if (q.d_allow) hipFree(q.d_allow);
        if (q.d_kvtab) hipFree(q.d_kvtab);
        if (q.d_stab) hipFree(q.d_stab);
        if (q.save_k) hipFree(q.save_k);
        if (q.save_v) hipFree(q.save_v);
        if (q.save_gc) hipFree(q.save_gc);
    }
    void *host[] = {c->h_meta, c->h_res, c->h_tok, c->h_resu, c->h_tab};
    for (void *p : host)
        if (p) hipHostFree(p);
    for (auto &r : c->recs) {
        hipEventDestroy(r.a);
        hipEventDestroy(r.b);
    }
    delete c;
}

const char *tv_last_error(tv_ctx *c) { return c ? c->err.c_str() : noalloc_last_error(); }

int tv_bind(tv_ctx *c, const char *name, void *ptr, size_t bytes) {
    if (!c || !name) return TV_EINVAL;
    if (!ptr) return fail(c, TV_EINVAL, "null pointer for %s", name);
    const tv_model_desc &m = c->m;
    const size_t H = m.hidden, V = m.vocab, F = m.ffn, D = m.head_dim, QH = m.n_qhead, KVH = m.n_kvhead;
    auto want = [&](size_t n) -> int {
        if (bytes != n) return fail(c, TV_EINVAL, "%s: %zu bytes given, %zu expected", name, bytes, n);
        return TV_OK;
    };
    int rc;
    if (!strcmp(name, "emb")) { if ((rc = want(V * H * 2))) return rc; c->emb = (const uint16_t *)ptr; return TV_OK; }
    if (!strcmp(name, "head")) {
        if ((rc = want(V * H * 2))) return rc;
        if (c->head == ptr) return TV_OK;  // re-bound: already packed
        if ((rc = pack_inplace(c, ptr, (int)V, (int)H))) return rc;
        c->head = (const uint16_t *)ptr;
        return TV_OK;
    }
    if (!strcmp(name, "final_norm")) { if ((rc = want(H * 2))) return rc; c->final_norm = (const uint16_t *)ptr; return TV_OK; }
    int l = -1, r = -1, used = 0;
    char field[32] = {0};
    if (sscanf(name, "layers.%d.%31s%n", &l, field, &used) == 2 && name[used] == 0) {
        if (l < 0 || l >= m.n_layer) return fail(c, TV_EINVAL, "%s: layer out of range", name);
        const bool at = c->kinds[l] == TV_LAYER_ATTN;
        const uint16_t *p = (const uint16_t *)ptr;
        if (!strcmp(field, "attn_norm")) { if ((rc = want(H * 2))) return rc; c->attn_norm[l] = p; return TV_OK; }
        if (!strcmp(field, "ffn_norm")) { if ((rc = want(H * 2))) return rc; c->ffn_norm[l] = p; return TV_OK; }
        auto mat = [&](const uint16_t *&slot, size_t n_out, size_t k_in) -> int {
            int r2 = want(n_out * k_in * 2);
            if (r2) return r2;
            if (slot == p) return TV_OK;  // re-bound: already packed
            r2 = pack_inplace(c, ptr, (int)n_out, (int)k_in);
            if (r2) return r2;
            slot = p;
            return TV_OK;
        };
        if (!strcmp(field, "wqkv")) return mat(c->wqkv[l], at ? (QH + 2 * KVH) * D : 3 * QH * D, H);
        if (!strcmp(field, "wa")) {
            if (at) return fail(c, TV_EINVAL, "%s: not a recurrent layer", name);
            return mat(c->wa[l], c->kinds[l] == TV_LAYER_DELTA ? 2 * QH : QH, H);
        }
        if (!strcmp(field, "wo")) return mat(c->wo[l], H, QH * D);
        if (!strcmp(field, "wg")) return mat(c->wg[l], F, H);
        if (!strcmp(field, "wu")) return mat(c->wu[l], F, H);
        if (!strcmp(field, "wd")) return mat(c->wd[l], H, F);
        return fail(c, TV_EINVAL, "unknown tensor %s", name);
    }
    if (sscanf(name, "req.%d.layers.%d.%31s%n", &r, &l, field, &used) == 3 && name[used] == 0) {
        if (r < 0 || r >= m.max_req) return fail(c, TV_EINVAL, "%s: request out of range", name);
        if (l < 0 || l >= m.n_layer) return fail(c, TV_EINVAL, "%s: layer out of range", name);
        Req &q = c->reqs[r];
        const bool at = c->kinds[l] == TV_LAYER_ATTN;
        if (!strcmp(field, "k") || !strcmp(field, "v")) {
            if (!at) return fail(c, TV_EINVAL, "%s: not an attention layer", name);
            if ((rc = want(KVH * (size_t)m.max_ctx * D * 2))) return rc;
            (field[0] == 'k' ? q.K[l] : q.V[l]) = (uint16_t *)ptr;
            q.kvtab_dirty = true;
            return TV_OK;
        }
        if (!strcmp(field, "state")) {
            if (at) return fail(c, TV_EINVAL, "%s: not a recurrent layer", name);
            if ((rc = want(QH * D * D * 4))) return rc;
            q.S[l] = (float *)ptr;
            q.stab_dirty = true;
            return TV_OK;
        }
        return fail(c, TV_EINVAL, "unknown tensor %s", name);
    }
    return fail(c, TV_EINVAL, "unknown tensor %s", name);
}

int tv_set_history(tv_ctx *c, int req, const int32_t *ids, int n_ids, int ctx_len) {
    int rc = check_req(c, req);
    if (rc) return rc;
    if (ctx_len < 0 || ctx_len > c->m.max_ctx) return fail(c, TV_ECAPACITY, "ctx_len %d out of range", ctx_len);
    if (n_ids < 0 || (n_ids > 0 && !ids)) return fail(c, TV_EINVAL, "bad history");
    for (int i = 0; i < n_ids; ++i)
        if (ids[i] < 0 || ids[i] >= c->m.vocab) return fail(c, TV_EINVAL, "history id %d out of range", i);
    Req &q = c->reqs[req];
    q.ctx_len = ctx_len;
    q.history.assign(ids, ids + n_ids);
    std::fill(q.hist_bits.begin(), q.hist_bits.end(), 0u);
    for (int i = 0; i < n_ids; ++i) set_bit(q.hist_bits, ids[i]);
    q.pending = false;
    if (q.d_hist) HIPCHECK(c, hipMemcpy(q.d_hist, q.hist_bits.data(), q.hist_bits.size() * 4, hipMemcpyHostToDevice));
    return TV_OK;
}

int tv_set_modifiers(tv_ctx *c, int req, float rep, const int32_t *bias_ids, const float *bias_vals,
                     int n_bias, const uint32_t *allow_bits) {
    int rc = check_req(c, req);
    if (rc) return rc;
    const tv_model_desc &m = c->m;
    if (!(rep > 0.f) || !std::isfinite(rep)) return fail(c, TV_EINVAL, "repetition penalty must be > 0");
    if (n_bias < 0 || (n_bias > 0 && (!bias_ids || !bias_vals))) return fail(c, TV_EINVAL, "bad bias");
    for (int i = 0; i < n_bias; ++i) {
        if (bias_ids[i] < 0 || bias_ids[i] >= m.vocab) return fail(c, TV_EINVAL, "bias id out of range");
        if (!std::isfinite(bias_vals[i])) return fail(c, TV_EINVAL, "bias value not finite");
    }
    Req &q = c->reqs[req];
    const size_t W = vocab_words(m);
    if (!q.d_hist) HIPCHECK(c, hipMalloc(&q.d_hist, W * 4));
    if (!q.d_bias) HIPCHECK(c, hipMalloc(&q.d_bias, (size_t)m.vocab * 4));
    if (!q.d_allow) HIPCHECK(c, hipMalloc(&q.d_allow, W * 4));
    std::vector<float> bias(m.vocab, 0.f);
    for (int i = 0; i < n_bias; ++i) bias[bias_ids[i]] += bias_vals[i];
    HIPCHECK(c, hipMemcpy(q.d_bias, bias.data(), bias.size() * 4, hipMemcpyHostToDevice));
    if (allow_bits) HIPCHECK(c, hipMemcpy(q.d_allow, allow_bits, W * 4, hipMemcpyHostToDevice));
    HIPCHECK(c, hipMemcpy(q.d_hist, q.hist_bits.data(), W * 4, hipMemcpyHostToDevice));
    q.rep = rep;
    q.has_bias = n_bias > 0;
    q.has_allow = allow_bits != nullptr;
    q.mods_on = rep != 1.f || q.has_bias || q.has_allow;
    return TV_OK;
}

int tv_set_sampling(tv_ctx *c, int req, float temperature, uint64_t seed) {
    int rc = check_req(c, req);
    if (rc) return rc;
    if (!(temperature >= 0.f) || !std::isfinite(temperature))
        return fail(c, TV_EINVAL, "temperature must be finite and >= 0");
    Req &q = c->reqs[req];
    q.temp = temperature;
    q.seed = seed;
    return TV_OK;
}

int tv_verify_tree(tv_ctx *c, int req, const int32_t *parents, const int32_t *tokens, int n_nodes,
                   float *logits_dev, int32_t *argmax, float *gap_ulps) {
    if (!c) return TV_EINVAL;
    if (!argmax) return fail(c, TV_EINVAL, "argmax output is required");
    return run_pass(c, 1, &req, &parents, &tokens, &n_nodes, logits_dev, argmax, gap_ulps);
}

int tv_verify_trees(tv_ctx *c, int n_req, const int *reqs, const int32_t *const *parents,
                    const int32_t *const *tokens, const int *n_nodes, float *logits_dev,
                    int32_t *argmax, float *gap_ulps) {
    if (!c) return TV_EINVAL;
    if (n_req < 1 || n_req > TV_MAX_NODES || !reqs || !parents || !tokens || !n_nodes || !argmax)
        return fail(c, TV_EINVAL, "bad joint verify arguments");
    return run_pass(c, n_req, reqs, parents, tokens, n_nodes, logits_dev, argmax, gap_ulps);
}

int tv_accept_walk(const int32_t *parents, const int32_t *tokens, const int32_t *argmax, int n,
                   int32_t *path, int *path_len, int32_t *emitted, int *n_emitted) {
    if (!parents || !tokens || !argmax || !path || !path_len || !emitted || !n_emitted) return TV_EINVAL;
    if (n < 1 || n > TV_MAX_NODES || parents[0] != -1) return TV_EINVAL;
    for (int i = 1; i < n; ++i)
        if (parents[i] < 0 || parents[i] >= i) return TV_EINVAL;
    int cur = 0, len = 0;
    path[len] = 0;
    for (;;) {
        const int g = argmax[cur];
        emitted[len] = g;
        int next = -1;
        for (int i = cur + 1; i < n; ++i)
            if (parents[i] == cur && tokens[i] == g) { next = i; break; }
        ++len;
        if (next < 0) break;
        path[len] = next;
        cur = next;
    }
    *path_len = len;
    *n_emitted = len;
    return TV_OK;
}

int tv_commit(tv_ctx *c, int req, const int32_t *path, int path_len) {
    int rc = check_req(c, req);
    if (rc) return rc;
    Req &q = c->reqs[req];
    if (!q.pending) return fail(c, TV_ESTATE, "request %d has no pending verify", req);
    const int n = (int)q.pparents.size();
    if (!path || path_len < 1 || path_len > n) return fail(c, TV_EINVAL, "path_len %d not in [1, %d]", path_len, n);
    if (path[0] != 0) return fail(c, TV_EINVAL, "path must start at the root");
    for (int d = 1; d < path_len; ++d)
        if (path[d] <= 0 || path[d] >= n || q.pparents[path[d]] != path[d - 1])
            return fail(c, TV_EINVAL, "path[%d] = %d is not a child of path[%d]", d, path[d], d - 1);
    bool moves = false;
    for (int d = 0; d < path_len; ++d) moves |= path[d] != d;
    hipStream_t s = c->stream;
    PathArg pa{};
    pa.len = path_len;
    for (int d = 0; d < path_len; ++d) pa.node[d] = path[d];
    if (!c->recur_layers.empty()) {
        RecurCommitArgs ra{};
        ra.states = q.d_stab; ra.save_k = q.save_k; ra.save_v = q.save_v; ra.save_gc = q.save_gc;
        ra.path = pa; ra.QH = c->m.n_qhead;
        LAUNCH(c, "commit_state", launch_recur_commit(s, c->m.head_dim, ra, (int)c->recur_layers.size()));
    }
    if (moves && !c->attn_layers.empty()) {
        LAUNCH(c, "commit_kv", launch_commit_kv(s, q.d_kvtab, (int)c->attn_layers.size(), c->m.n_kvhead,
                                                c->m.max_ctx, c->m.head_dim, q.ctx_len, pa));
    }
    q.ctx_len += path_len;
    for (int d = 0; d < path_len; ++d) {
        const int t = q.ptokens[path[d]];
        q.history.push_back(t);
        set_bit(q.hist_bits, t);
    }
    if (q.mods_on && q.d_hist)
        HIPCHECK(c, hipMemcpy(q.d_hist, q.hist_bits.data(), q.hist_bits.size() * 4, hipMemcpyHostToDevice));
    // No synchronisation: the commit is stream-ordered before the next verify,
    // which synchronises (the path travels as a kernel argument).
    q.pending = false;
    return TV_OK;
}

int tv_round(tv_ctx *c, int req, const int32_t *parents, const int32_t *tokens, int n_nodes,
             float *logits_dev, int32_t *argmax, float *gap_ulps, int32_t *path, int *path_len,
             int32_t *emitted, int *n_emitted) {
    if (!c) return TV_EINVAL;
    if (!path || !path_len || !emitted || !n_emitted) return fail(c, TV_EINVAL, "null output");
    int rc = tv_verify_tree(c, req, parents, tokens, n_nodes, logits_dev, argmax, gap_ulps);
    if (rc) return rc;
    rc = tv_accept_walk(parents, tokens, argmax, n_nodes, path, path_len, emitted, n_emitted);
    if (rc) return fail(c, rc, "accept walk rejected the tree");
    return tv_commit(c, req, path, *path_len);
}

int tv_residual_round(tv_ctx *c, int req, const int32_t *parents, const int32_t *tokens, int n_nodes,
                      float *logits_dev, float temperature, const double *uniforms, int32_t *path,
                      int *path_len, int32_t *emitted, int *n_emitted) {
    if (!c) return TV_EINVAL;
    if (!path || !path_len || !emitted || !n_emitted || !uniforms) return fail(c, TV_EINVAL, "null argument");
    if (!(temperature > 0.f) || !std::isfinite(temperature))
        return fail(c, TV_EINVAL, "temperature must be positive and finite");
    if (n_nodes < 1 || n_nodes > TV_MAX_NODES || !parents) return fail(c, TV_EINVAL, "bad tree size");
    int depth[TV_MAX_NODES];
    for (int i = 0; i < n_nodes; ++i) {
        if (i > 0 && (parents[i] < 0 || parents[i] >= i)) return fail(c, TV_EINVAL, "bad parents");
        depth[i] = i == 0 ? 0 : depth[parents[i]] + 1;
        if (!(uniforms[depth[i]] >= 0.0 && uniforms[depth[i]] < 1.0))
            return fail(c, TV_EINVAL, "uniforms must lie in [0, 1)");
    }
    int32_t am[TV_MAX_NODES];
    float gap[TV_MAX_NODES];
    int rc = tv_verify_tree(c, req, parents, tokens, n_nodes, logits_dev, am, gap);
    if (rc) return rc;
    hipStream_t s = c->stream;
    for (int i = 0; i < n_nodes; ++i) c->h_resu[i] = uniforms[depth[i]];
    clear_results(c, n_nodes);
    HIPCHECK(c, hipMemcpyAsync(c->d_resu, c->h_resu, (size_t)n_nodes * sizeof(double), hipMemcpyHostToDevice, s));
    const float *lg = logits_dev ? logits_dev : c->logits;
    DrainOnError drain(c);
    LAUNCH(c, "residual", launch_residual(s, lg, c->m.vocab, c->m.vocab, c->d_meta, n_nodes, temperature, c->d_resu,
                                          c->d_resparts, c->hd_res));
    rc = wait_results(c, n_nodes);
    if (rc) return rc;
    drain.done();
    // the walk: from the root, accept a child or emit and stop
    int cur = 0, pl = 1, ne = 0;
    path[0] = 0;
    while (true) {
        const int32_t d = c->h_res[cur].argmax;
        if (d >= 0) {
            emitted[ne++] = d;
            break;
        }
        const int want = -d - 1;
        int child = -1, k = 0;
        for (int j = cur + 1; j < n_nodes; ++j)
            if (parents[j] == cur && k++ == want) {
                child = j;
                break;
            }
        if (child < 0) return fail(c, TV_EHIP, "internal: residual decision names no child");
        path[pl++] = child;
        emitted[ne++] = tokens[child];
        cur = child;
    }
    *path_len = pl;
    *n_emitted = ne;
    return tv_commit(c, req, path, pl);
}

// ------------------------------------------------------------ dense prefill
namespace {

constexpr int kPrefillMaxChunk = 2048;
constexpr int kPrefillBlock = 32;   // rows of one attention block (a chain)

// Target splits of the cache keys per attention block: about 1024
// workgroups over all blocks and KV heads (at least one split each, at most
// 32 as in a verify, so a combine merges at most 33 partials).
int prefill_splits(int nz, int KVH) { return std::min(32, std::max(1, 1024 / (nz * KVH))); }

int ensure_prefill(tv_ctx *c, int rows) {
    if (c->pf_rows >= rows) return TV_OK;
    const tv_model_desc &m = c->m;
    void *old[] = {c->pX, c->pXN, c->pQKV, c->pQR, c->pATT, c->pACT, c->pAB, c->pTok, c->ppo, c->ppm, c->ppl};
    for (void *p : old)
        if (p) hipFree(p);
    if (c->h_tok) hipHostFree(c->h_tok);
    c->pX = c->pXN = c->pQKV = c->pQR = c->pATT = c->pACT = c->pAB = nullptr;
    c->pTok = c->h_tok = nullptr;
    c->ppo = c->ppm = c->ppl = nullptr;
    c->pf_rows = 0;
    const size_t R = (size_t)rows, H = m.hidden, D = m.head_dim, QH = m.n_qhead, KVH = m.n_kvhead;
    // attention partials: blocks x KV heads x (splits + 1) x query rows
    size_t slots = 0;
    const int nz = (rows + kPrefillBlock - 1) / kPrefillBlock;
    for (int z = 1; z <= nz; ++z) slots = std::max(slots, (size_t)z * KVH * (prefill_splits(z, (int)KVH) + 1));
    const size_t RP = (size_t)kMaxRows * kMaxGroup;
    hipError_t e = hipSuccess;
#define ALLOC(p, bytes) if (e == hipSuccess) e = hipMalloc((void **)&(p), (bytes))
    ALLOC(c->pX, R * H * 2);
    ALLOC(c->pXN, R * H * 2);
    ALLOC(c->pQKV, R * std::max((QH + 2 * KVH) * D, 3 * QH * D) * 2);
    ALLOC(c->pAB, R * 2 * QH * 2);
    ALLOC(c->pQR, R * QH * D * 2);
    ALLOC(c->pATT, R * QH * D * 2);
    ALLOC(c->pACT, R * m.ffn * 2);
    ALLOC(c->pTok, R * 4);
    ALLOC(c->ppo, slots * RP * D * 4);
    ALLOC(c->ppm, slots * RP * 4);
    ALLOC(c->ppl, slots * RP * 4);
    if (e == hipSuccess) e = hipHostMalloc((void **)&c->h_tok, R * 4, hipHostMallocDefault);
#undef ALLOC
    if (e != hipSuccess) return fail(c, TV_EHIP, "prefill scratch for %d rows: %s", rows, hipGetErrorString(e));
    c->pf_rows = rows;
    return TV_OK;
}

// One chunk of m prompt rows at positions pos.. of request q: every layer on
// the dense kernels; the KV rows land in the cache at their slots.
int prefill_chunk(tv_ctx *c, Req &q, const int32_t *tokens, int m, int pos) {
    const tv_model_desc &md = c->m;
    hipStream_t s = c->stream;
    const int H = md.hidden, D = md.head_dim, QH = md.n_qhead, KVH = md.n_kvhead;
    // the staging buffer may still feed the previous chunk's copy
    HIPCHECK(c, hipStreamSynchronize(s));
    memcpy(c->h_tok, tokens, (size_t)m * 4);
    HIPCHECK(c, hipMemcpyAsync(c->pTok, c->h_tok, (size_t)m * 4, hipMemcpyHostToDevice, s));
    LAUNCH(c, "pf_embed_norm", launch_norm_dense(s, c->pTok, c->emb, c->pX, c->attn_norm[0], md.eps, c->pXN, m, H));
    const int nz = (m + kPrefillBlock - 1) / kPrefillBlock;
    const int target = prefill_splits(nz, KVH);
    for (int l = 0; l < md.n_layer; ++l) {
      if (c->kinds[l] != TV_LAYER_ATTN) {
        // a recurrent layer: q/k/v rows and gate rows on the dense GEMM, then
        // the tree read-out on chains of 32 rows in order, each followed by
        // the closed-form state commit of its whole chain
        const bool delta = c->kinds[l] == TV_LAYER_DELTA;
        const int rl = c->recur_index[l], nab = (delta ? 2 : 1) * QH;
        GemmArgs g{};
        g.X = c->pXN; g.ldx = H; g.W = c->wqkv[l]; g.M = m; g.N = 3 * QH * D; g.K = H;
        g.Y = c->pQKV; g.ldy = g.N; g.zeros = c->zeros;
        LAUNCH(c, "pf_gemm_qkv", launch_gemm_dense(s, EPI_BF16, g));
        GemmArgs ga{};
        ga.X = c->pXN; ga.ldx = H; ga.W = c->wa[l]; ga.M = m; ga.N = nab; ga.K = H;
        ga.Y = c->pAB; ga.ldy = nab; ga.zeros = c->zeros;
        LAUNCH(c, "pf_gemm_gate", launch_gemm_dense(s, EPI_BF16, ga));
        const size_t per = (size_t)kMaxRows * QH * D;
        for (int b0 = 0; b0 < m; b0 += kPrefillBlock) {
            const int nb = std::min(kPrefillBlock, m - b0);
            RecurArgs ra{};
            ra.qkv_rows = c->pQKV; ra.ab_rows = c->pAB; ra.ab_ld = nab; ra.a_col = 3 * QH * D; ra.delta = delta;
            ra.S0 = q.S[l]; ra.meta = c->d_meta; ra.out = c->pATT;
            ra.save_k = q.save_k + rl * per; ra.save_v = q.save_v + rl * per;
            ra.save_gc = q.save_gc + (size_t)rl * kMaxRows * QH;
            ra.row0 = b0; ra.n = nb; ra.QH = QH; ra.eps = md.eps;
            LAUNCH(c, "pf_recur", launch_recur_tree(s, D, ra));
            RecurCommitArgs ca{};
            ca.states = q.d_stab + rl; ca.save_k = ra.save_k; ca.save_v = ra.save_v; ca.save_gc = ra.save_gc;
            ca.path.len = nb;
            for (int d = 0; d < nb; ++d) ca.path.node[d] = d;
            ca.QH = QH;
            LAUNCH(c, "pf_commit_state", launch_recur_commit(s, D, ca, 1));
        }
      } else {
        GemmArgs g{};
        g.X = c->pXN; g.ldx = H; g.W = c->wqkv[l]; g.M = m; g.N = (QH + 2 * KVH) * D; g.K = H;
        g.Y = c->pQKV; g.ldy = g.N; g.zeros = c->zeros;
        LAUNCH(c, "pf_gemm_qkv", launch_gemm_dense(s, EPI_BF16, g));
        LAUNCH(c, "pf_rope", launch_rope_dense(s, c->pQKV, g.N, m, pos, QH, KVH, D, c->rope_cos, c->rope_sin,
                                               c->pQR, q.K[l], q.V[l], md.max_ctx));
        AttnArgs aa{};
        aa.Q = c->pQR; aa.Kc = q.K[l]; aa.Vc = q.V[l]; aa.meta = c->d_meta;
        aa.po = c->ppo; aa.pm = c->ppm; aa.pl = c->ppl;
        aa.row0 = 0; aa.n = std::min(m, kPrefillBlock); aa.ctx = pos; aa.cap = md.max_ctx; aa.G = c->G;
        aa.n_qhead = QH; aa.ns = target + 1; aa.ztarget = target;
        // the longest split any block has decides whether loader waves run
        aa.span = attn_span_n(pos + (nz - 1) * kPrefillBlock, target);
        aa.n_ctx_split = 0;
        aa.scale = (float)(1.0 / std::sqrt((double)D));
        aa.zrows = kPrefillBlock; aa.M = m;
        LAUNCH(c, "pf_attn", launch_attn(s, D, aa));
        aa.n = kPrefillBlock;
        LAUNCH(c, "pf_attn_combine", launch_attn_combine(s, D, aa, c->pATT));
      }
        GemmArgs go{};
        go.X = c->pATT; go.ldx = QH * D; go.W = c->wo[l]; go.M = m; go.N = H; go.K = QH * D;
        go.Y = c->pX; go.ldy = H; go.zeros = c->zeros;
        LAUNCH(c, "pf_gemm_o", launch_gemm_dense(s, EPI_RESID, go));
        LAUNCH(c, "pf_norm", launch_norm_dense(s, nullptr, nullptr, c->pX, c->ffn_norm[l], md.eps, c->pXN, m, H));
        GemmArgs gu{};
        gu.X = c->pXN; gu.ldx = H; gu.W = c->wg[l]; gu.W2 = c->wu[l]; gu.M = m; gu.N = md.ffn; gu.K = H;
        gu.Y = c->pACT; gu.ldy = md.ffn; gu.zeros = c->zeros;
        LAUNCH(c, "pf_gemm_gateup", launch_gemm_dense(s, EPI_SWIGLU, gu));
        GemmArgs gd{};
        gd.X = c->pACT; gd.ldx = md.ffn; gd.W = c->wd[l]; gd.M = m; gd.N = H; gd.K = md.ffn;
        gd.Y = c->pX; gd.ldy = H; gd.zeros = c->zeros;
        LAUNCH(c, "pf_gemm_down", launch_gemm_dense(s, EPI_RESID, gd));
        const uint16_t *nw = l + 1 < md.n_layer ? c->attn_norm[l + 1] : c->final_norm;
        LAUNCH(c, "pf_norm", launch_norm_dense(s, nullptr, nullptr, c->pX, nw, md.eps, c->pXN, m, H));
    }
    return TV_OK;
}

} // namespace

int tv_prefill_dense(tv_ctx *c, int req, const int32_t *tokens, int n, int chunk, int32_t *argmax_last) {
    int rc = check_req(c, req);
    if (rc) return rc;
    const tv_model_desc &m = c->m;
    if (n < 1 || !tokens) return fail(c, TV_EINVAL, "empty prompt");
    if (chunk < kPrefillBlock || chunk > kPrefillMaxChunk || chunk % kPrefillBlock)
        return fail(c, TV_EINVAL, "chunk %d must be a multiple of %d in [%d, %d]", chunk, kPrefillBlock,
                    kPrefillBlock, kPrefillMaxChunk);
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m.vocab) return fail(c, TV_EINVAL, "token %d out of range", i);
    Req &q = c->reqs[req];
    if (q.ctx_len + n > m.max_ctx) return fail(c, TV_ECAPACITY, "prompt of %d tokens does not fit", n);
    {
        std::vector<int> rv{req};
        rc = check_bound(c, rv);
        if (rc) return rc;
    }
    rc = upload_stab(c, q);
    if (rc) return rc;
    rc = ensure_prefill(c, chunk);
    if (rc) return rc;
    q.pending = false;
    DrainOnError drain(c);
    int done = 0;
    while (done < n) {
        // the chunk grid: chunks end at multiples of `chunk` positions
        const int pos = q.ctx_len;
        const int k = std::min(n - done, chunk - pos % chunk);
        rc = prefill_chunk(c, q, tokens + done, k, pos);
        if (rc) return rc;
        q.ctx_len += k;
        for (int i = 0; i < k; ++i) {
            q.history.push_back(tokens[done + i]);
            set_bit(q.hist_bits, tokens[done + i]);
        }
        done += k;
        if (done == n && argmax_last) {
            // the last row's token: the head (with the request's modifiers
            // and sampling) on that row only
            if (q.d_hist)
                HIPCHECK(c, hipMemcpy(q.d_hist, q.hist_bits.data(), q.hist_bits.size() * 4, hipMemcpyHostToDevice));
            PassMeta &pm = *c->h_meta;
            memset(&pm, 0, sizeof pm);
            pm.row_req[0] = 0;
            pm.draw_t[0] = q.ctx_len;
            HeadMods &hm = pm.mods[0];
            hm.rep = q.mods_on ? q.rep : 1.f;
            hm.hist_bits = (q.mods_on && q.rep != 1.f) ? q.d_hist : nullptr;
            hm.bias = (q.mods_on && q.has_bias) ? q.d_bias : nullptr;
            hm.allow_bits = (q.mods_on && q.has_allow) ? q.d_allow : nullptr;
            hm.temp = q.temp;
            hm.seed_lo = (uint32_t)q.seed;
            hm.seed_hi = (uint32_t)(q.seed >> 32);
            hipStream_t s = c->stream;
            clear_results(c, 1);
            HIPCHECK(c, hipMemcpyAsync(c->d_meta, c->h_meta, sizeof(PassMeta), hipMemcpyHostToDevice, s));
            GemmArgs g{};
            g.X = c->pXN + (size_t)(k - 1) * m.hidden; g.ldx = m.hidden;
            g.W = c->head; g.M = 1; g.N = m.vocab; g.K = m.hidden;
            g.Yf = c->logits; g.ldyf = m.vocab; g.part = c->part; g.meta = c->d_meta;
            g.mods_on = q.mods_on || q.temp > 0.f; g.zeros = c->zeros;
            GEMM(c, "gemm_head", EPI_HEAD, g);
            LAUNCH(c, "top2", launch_top2_reduce(s, c->part, ((m.vocab + 31) / 32 + 3) / 4, 1, c->hd_res));
            rc = wait_results(c, 1);
            if (rc) return rc;
            float gap;
            read_results(c, 1, argmax_last, &gap);
        }
    }
    if (!argmax_last) HIPCHECK(c, hipStreamSynchronize(c->stream));
    drain.done();
    return TV_OK;
}

int tv_prefill(tv_ctx *c, int req, const int32_t *tokens, int n, int32_t *argmax_last) {
    int rc = check_req(c, req);
    if (rc) return rc;
    if (n < 1 || !tokens) return fail(c, TV_EINVAL, "empty prompt");
    if (c->reqs[req].ctx_len + n > c->m.max_ctx)
        return fail(c, TV_ECAPACITY, "prompt of %d tokens does not fit", n);
    int32_t parents[TV_MAX_NODES], path[TV_MAX_NODES], am[TV_MAX_NODES];
    for (int i = 0; i < TV_MAX_NODES; ++i) {
        parents[i] = i - 1;
        path[i] = i;
    }
    for (int off = 0; off < n; off += TV_MAX_NODES) {
        const int k = std::min(TV_MAX_NODES, n - off);
        rc = tv_verify_tree(c, req, parents, tokens + off, k, nullptr, am, nullptr);
        if (rc) return rc;
        rc = tv_commit(c, req, path, k);
        if (rc) return rc;
        if (argmax_last) *argmax_last = am[k - 1];
    }
    return TV_OK;
}

int tv_linear(tv_ctx *c, const void *x, const void *w, int M, int N, int K, void *y, int y_fp32) {
    if (!c) return TV_EINVAL;
    if (!x || !w || !y) return fail(c, TV_EINVAL, "null operand");
    if (M < 1 || N < 1 || K < 8 || K % 8)
        return fail(c, TV_EINVAL, "shape M=%d N=%d K=%d not supported", M, N, K);
    if (y_fp32 && M <= kMaxRows && N > c->m.vocab) return fail(c, TV_EINVAL, "fp32 output needs N <= vocab");
    GemmArgs g{};
    g.X = (const uint16_t *)x; g.ldx = K; g.W = (const uint16_t *)w; g.M = M; g.N = N; g.K = K;
    g.zeros = c->zeros;
    hipStream_t s = c->stream;
    DrainOnError drain(c);
    if (M > kMaxRows) {   // many rows: the dense (prefill) GEMM
        if (y_fp32) { g.Yf = (float *)y; g.ldyf = N; }
        else { g.Y = (uint16_t *)y; g.ldy = N; }
        LAUNCH(c, "gemm_dense", launch_gemm_dense(s, y_fp32 ? EPI_F32 : EPI_BF16, g));
    } else if (y_fp32) {
        g.Yf = (float *)y; g.ldyf = N; g.part = c->part;
        GEMM(c, "gemm_linear_f32", EPI_HEAD, g);
    } else {
        g.Y = (uint16_t *)y; g.ldy = N;
        GEMM(c, "gemm_linear", EPI_BF16, g);
    }
    HIPCHECK(c, hipStreamSynchronize(s));
    drain.done();
    if (c->prof) harvest(c);
    return TV_OK;
}

int tv_pack_weight(tv_ctx *c, void *w, int N, int K) {
    if (!c) return TV_EINVAL;
    if (!w || N < 1 || K < 8 || K % 8) return fail(c, TV_EINVAL, "bad weight shape N=%d K=%d", N, K);
    return pack_inplace(c, w, N, K);
}

int tv_head_top2(tv_ctx *c, const void *x, int M, float *logits_dev, int32_t *argmax, float *gap) {
    if (!c) return TV_EINVAL;
    if (!x || !logits_dev || !argmax) return fail(c, TV_EINVAL, "null operand");
    if (M < 1 || M > kMaxRows) return fail(c, TV_EINVAL, "M=%d not in [1, 32]", M);
    if (!c->head) return fail(c, TV_ESTATE, "head not bound");
    const tv_model_desc &m = c->m;
    hipStream_t s = c->stream;
    GemmArgs g{};
    g.X = (const uint16_t *)x; g.ldx = m.hidden; g.W = c->head; g.M = M; g.N = m.vocab; g.K = m.hidden;
    g.Yf = logits_dev; g.ldyf = m.vocab; g.part = c->part;
    clear_results(c, M);
    DrainOnError drain(c);
    GEMM(c, "gemm_head", EPI_HEAD, g);
    LAUNCH(c, "top2", launch_top2_reduce(s, c->part, ((m.vocab + 31) / 32 + 3) / 4, M, c->hd_res));
    {
        const int rc2 = wait_results(c, M);
        if (rc2) return rc2;
    }
    drain.done();
    read_results(c, M, argmax, gap);
    return TV_OK;
}

int tv_ctx_len(tv_ctx *c, int req) {
    int rc = check_req(c, req);
    if (rc) return rc;
    return c->reqs[req].ctx_len;
}

int tv_profile_enable(tv_ctx *c, int on, const char *only_prefix) {
    if (!c) return TV_EINVAL;
    c->prof = on != 0;
    c->prof_only = only_prefix ? only_prefix : "";
    return TV_OK;
}

int tv_profile_reset(tv_ctx *c) {
    if (!c) return TV_EINVAL;
    HIPCHECK(c, hipStreamSynchronize(c->stream));
    harvest(c);
    c->totals.clear();
    return TV_OK;
}

int tv_profile_get(tv_ctx *c, const char *prefix, double *total_ms, int *count) {
    if (!c || !prefix || !total_ms || !count) return TV_EINVAL;
    HIPCHECK(c, hipStreamSynchronize(c->stream));
    harvest(c);
    double ms = 0;
    int n = 0;
    const size_t L = strlen(prefix);
    for (auto &t : c->totals)
        if (!strncmp(t.first.c_str(), prefix, L)) {
            ms += t.second.first;
            n += t.second.second;
        }
    *total_ms = ms;
    *count = n;
    return TV_OK;
}

} // extern "C"

// ------------------------------------------------------- kernel-level calls
namespace {

// Tree metadata of one request's n-node tree (validated) for a kernel-level
// call: depth and ancestor-or-self bits, copied to the device copy of the
// pass record that the kernels read.
int upload_tree_meta(tv_ctx *c, const int32_t *parents, int n) {
    if (!parents || n < 1 || n > TV_MAX_NODES || parents[0] != -1)
        return fail(c, TV_EINVAL, "tree of %d nodes: parents[0] must be -1", n);
    for (int i = 1; i < n; ++i)
        if (parents[i] < 0 || parents[i] >= i) return fail(c, TV_EINVAL, "parents[%d] = %d not in [0, %d)", i, parents[i], i);
    PassMeta &pm = *c->h_meta;
    memset(&pm, 0, sizeof pm);
    for (int i = 0; i < n; ++i) {
        const int p = parents[i];
        pm.depth[i] = p < 0 ? 0 : pm.depth[p] + 1;
        pm.anc[i] = (p < 0 ? 0u : pm.anc[p]) | (1u << i);
        pm.row_req[i] = 0;
        pm.path_len[i] = pm.depth[i] + 1;
    }
    HIPCHECK(c, hipMemcpyAsync(c->d_meta, c->h_meta, sizeof(PassMeta), hipMemcpyHostToDevice, c->stream));
    return TV_OK;
}

int finish_call(tv_ctx *c) {
    HIPCHECK(c, hipStreamSynchronize(c->stream));
    if (c->prof) harvest(c);
    return TV_OK;
}

} // namespace

extern "C" {

int tv_attention(tv_ctx *c, const void *q, const void *k_cache, const void *v_cache, int cap, int ctx_len,
                 const int32_t *parents, int n_nodes, void *out) {
    if (!c) return TV_EINVAL;
    const tv_model_desc &m = c->m;
    if (!q || !k_cache || !v_cache || !out) return fail(c, TV_EINVAL, "null operand");
    if (ctx_len < 0 || cap < 1 || n_nodes < 1 || ctx_len + n_nodes > cap)
        return fail(c, TV_ECAPACITY, "ctx_len %d + %d rows does not fit a cache of %d rows", ctx_len, n_nodes, cap);
    const int D = m.head_dim;
    DrainOnError drain(c);
    int rc = upload_tree_meta(c, parents, n_nodes);
    if (rc) return rc;
    AttnArgs aa{};
    aa.Q = (const uint16_t *)q; aa.meta = c->d_meta; aa.po = c->po; aa.pm = c->pm; aa.pl = c->pl;
    aa.cap = cap; aa.G = c->G; aa.n_qhead = m.n_qhead;
    aa.scale = (float)(1.0 / std::sqrt((double)D));
    aa.nreq = 1;
    PassReq &p = aa.rq[0];
    p.Kc = (uint16_t *)k_cache; p.Vc = (uint16_t *)v_cache;
    p.row0 = 0; p.n = n_nodes; p.ctx = ctx_len;
    p.span = attn_span(ctx_len);
    p.nsplit = (ctx_len + p.span - 1) / p.span;
    aa.n = p.n; aa.span = p.span; aa.ns = p.nsplit + 1;
    LAUNCH(c, "attn", launch_attn(c->stream, D, aa));
    LAUNCH(c, "attn_combine", launch_attn_combine(c->stream, D, aa, (uint16_t *)out));
    rc = finish_call(c);
    if (rc) return rc;
    drain.done();
    return TV_OK;
}

int tv_rope_kv(tv_ctx *c, const float *qkv_part, int splits, int n_rows, const int32_t *depth, int ctx_len,
               void *q_out, void *k_cache, void *v_cache, int cap) {
    if (!c) return TV_EINVAL;
    const tv_model_desc &m = c->m;
    if (!qkv_part || !depth || !q_out || !k_cache || !v_cache) return fail(c, TV_EINVAL, "null operand");
    if (n_rows < 1 || n_rows > kMaxRows) return fail(c, TV_EINVAL, "n_rows %d not in [1, %d]", n_rows, kMaxRows);
    if (splits < 1 || splits > 4096) return fail(c, TV_EINVAL, "splits %d out of range", splits);
    if (ctx_len < 0 || ctx_len + n_rows > cap) return fail(c, TV_ECAPACITY, "rows do not fit the cache");
    for (int i = 0; i < n_rows; ++i)
        if (depth[i] < 0 || ctx_len + depth[i] >= m.max_ctx)
            return fail(c, TV_EINVAL, "row %d: position %d outside the rotation table", i, ctx_len + depth[i]);
    DrainOnError drain(c);
    PassMeta &pm = *c->h_meta;
    memset(&pm, 0, sizeof pm);
    for (int i = 0; i < n_rows; ++i) pm.depth[i] = depth[i];
    HIPCHECK(c, hipMemcpyAsync(c->d_meta, c->h_meta, sizeof(PassMeta), hipMemcpyHostToDevice, c->stream));
    RopeArgs ra{};
    ra.part = qkv_part; ra.S = splits; ra.q_out = (uint16_t *)q_out;
    ra.cosT = c->rope_cos; ra.sinT = c->rope_sin; ra.meta = c->d_meta;
    ra.M = n_rows; ra.cap = cap; ra.QH = m.n_qhead; ra.KVH = m.n_kvhead; ra.D = m.head_dim; ra.nreq = 1;
    ra.rq[0].Kc = (uint16_t *)k_cache; ra.rq[0].Vc = (uint16_t *)v_cache;
    ra.rq[0].row0 = 0; ra.rq[0].n = n_rows; ra.rq[0].ctx = ctx_len;
    LAUNCH(c, "rope_kv", launch_rope_kv(c->stream, ra));
    int rc = finish_call(c);
    if (rc) return rc;
    drain.done();
    return TV_OK;
}

int tv_resid_norm(tv_ctx *c, const float *part, int splits, int n_rows, void *x, const void *w, void *y) {
    if (!c) return TV_EINVAL;
    if (!part || !x || !w || !y) return fail(c, TV_EINVAL, "null operand");
    if (n_rows < 1 || n_rows > kMaxRows) return fail(c, TV_EINVAL, "n_rows %d not in [1, %d]", n_rows, kMaxRows);
    if (splits < 1 || splits > 4096) return fail(c, TV_EINVAL, "splits %d out of range", splits);
    DrainOnError drain(c);
    LAUNCH(c, "resid_norm", launch_resid_norm(c->stream, part, splits, n_rows, c->m.hidden, (const uint16_t *)w,
                                              c->m.eps, (uint16_t *)x, (uint16_t *)y));
    int rc = finish_call(c);
    if (rc) return rc;
    drain.done();
    return TV_OK;
}

int tv_recur_tree(tv_ctx *c, int kind, const float *part, int splits, const int32_t *parents, int n_nodes,
                  const float *state, void *out, void *save_k, float *save_v, float *save_gc) {
    if (!c) return TV_EINVAL;
    const tv_model_desc &m = c->m;
    if (kind != TV_LAYER_RECUR && kind != TV_LAYER_DELTA) return fail(c, TV_EINVAL, "kind %d is not recurrent", kind);
    if (!part || !state || !out || !save_k || !save_v || !save_gc) return fail(c, TV_EINVAL, "null operand");
    if (splits < 1 || splits > 4096) return fail(c, TV_EINVAL, "splits %d out of range", splits);
    DrainOnError drain(c);
    int rc = upload_tree_meta(c, parents, n_nodes);
    if (rc) return rc;
    RecurArgs ra{};
    ra.qkv_part = part; ra.qkv_S = splits;
    ra.a_col = 3 * m.n_qhead * m.head_dim; ra.delta = kind == TV_LAYER_DELTA;
    ra.S0 = state; ra.meta = c->d_meta; ra.out = (uint16_t *)out;
    ra.save_k = (uint16_t *)save_k; ra.save_v = save_v; ra.save_gc = save_gc;
    ra.row0 = 0; ra.n = n_nodes; ra.QH = m.n_qhead; ra.eps = m.eps;
    LAUNCH(c, "recur_tree", launch_recur_tree(c->stream, m.head_dim, ra));
    rc = finish_call(c);
    if (rc) return rc;
    drain.done();
    return TV_OK;
}

int tv_recur_commit(tv_ctx *c, float *state, const void *save_k, const float *save_v, const float *save_gc,
                    const int32_t *path, int path_len) {
    if (!c) return TV_EINVAL;
    if (!state || !save_k || !save_v || !save_gc || !path) return fail(c, TV_EINVAL, "null operand");
    if (path_len < 1 || path_len > kMaxRows) return fail(c, TV_EINVAL, "path_len %d not in [1, %d]", path_len, kMaxRows);
    for (int d = 0; d < path_len; ++d)
        if (path[d] < 0 || path[d] >= kMaxRows) return fail(c, TV_EINVAL, "path[%d] = %d out of range", d, path[d]);
    DrainOnError drain(c);
    c->h_tab[0] = state;
    HIPCHECK(c, hipMemcpyAsync(c->d_tab, c->h_tab, sizeof(void *), hipMemcpyHostToDevice, c->stream));
    RecurCommitArgs ra{};
    ra.states = (float *const *)c->d_tab;
    ra.save_k = (const uint16_t *)save_k; ra.save_v = save_v; ra.save_gc = save_gc;
    ra.path.len = path_len;
    for (int d = 0; d < path_len; ++d) ra.path.node[d] = path[d];
    ra.QH = c->m.n_qhead;
    LAUNCH(c, "commit_state", launch_recur_commit(c->stream, c->m.head_dim, ra, 1));
    int rc = finish_call(c);
    if (rc) return rc;
    drain.done();
    return TV_OK;
}

int tv_gather_kv(tv_ctx *c, void *k_cache, void *v_cache, int cap, int ctx_len, const int32_t *path, int path_len) {
    if (!c) return TV_EINVAL;
    if (!k_cache || !v_cache || !path) return fail(c, TV_EINVAL, "null operand");
    if (path_len < 1 || path_len > kMaxRows) return fail(c, TV_EINVAL, "path_len %d not in [1, %d]", path_len, kMaxRows);
    for (int d = 0; d < path_len; ++d)
        if (path[d] < d || path[d] >= kMaxRows || (d > 0 && path[d] <= path[d - 1]))
            return fail(c, TV_EINVAL, "path[%d] = %d: a path's nodes increase and path[d] >= d", d, path[d]);
    if (ctx_len < 0 || ctx_len + path[path_len - 1] >= cap) return fail(c, TV_ECAPACITY, "path rows outside the cache");
    DrainOnError drain(c);
    c->h_tab[0] = k_cache;
    c->h_tab[1] = v_cache;
    HIPCHECK(c, hipMemcpyAsync(c->d_tab, c->h_tab, 2 * sizeof(void *), hipMemcpyHostToDevice, c->stream));
    PathArg pa{};
    pa.len = path_len;
    for (int d = 0; d < path_len; ++d) pa.node[d] = path[d];
    LAUNCH(c, "commit_kv", launch_commit_kv(c->stream, (uint16_t *const *)c->d_tab, 1, c->m.n_kvhead, cap,
                                            c->m.head_dim, ctx_len, pa));
    int rc = finish_call(c);
    if (rc) return rc;
    drain.done();
    return TV_OK;
}

} // extern "C"
