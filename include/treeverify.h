/*
 * treeverify: the tree-verify pass of greedy speculative decoding on one
 * MI355X (gfx950), behind a C ABI.
 *
 * One round ("Drafters and tree verify", The round):
 *   tv_verify_tree  one target-model forward over a draft tree of at most 32
 *                   nodes against the request's KV cache and recurrent state;
 *                   fp32 logits, the argmax token and the top-1/top-2 gap at
 *                   every node (step 2, Verify);
 *   tv_accept_walk  the walk down the tree (step 3, Accept), over the argmax
 *                   of greedy rows or the draw of sampled ones
 *                   (tv_set_sampling);
 *   tv_commit       keep the KV rows and recurrent state of the accepted path
 *                   and drop the rest (step 4, Commit);
 *   tv_round        the three in one call.
 *
 * Around it: prompts (tv_prefill through the verify path, tv_prefill_dense
 * on the MFMA prefill kernels and the chunk grid), sampled requests
 * (tv_set_sampling: seeded Gumbel-max draws; tv_residual_round:
 * deterministic-candidate residual sampling), drafting on the host (the
 * lookup drafter's tree from the request's own text, tv_lookup_draft, and
 * StairCut's cut of a candidate tree, tv_staircut), and kernel-level calls
 * for tests and measurement (tv_linear, tv_head_top2, tv_pack_weight,
 * tv_attention, tv_rope_kv, tv_resid_norm, tv_recur_tree, tv_recur_commit,
 * tv_gather_kv, tv_profile_*).
 *
 * Conventions shared by every call:
 *   - Every call returns TV_OK (0) or a negative TV_E* code and never throws.
 *     A failed call changes no state: validation happens before any work is
 *     enqueued.  tv_last_error() gives a message for the last failure.
 *   - Device memory for weights, KV caches, recurrent states and logits is
 *     allocated by the caller and BORROWED (tv_bind); the library never frees
 *     it.  The library allocates its own small activation scratch in
 *     tv_create and frees it in tv_destroy.
 *   - All device work is enqueued on the stream given to tv_create.  A call
 *     that returns host results (argmax, gaps) returns once its last kernel
 *     has finished, so all work enqueued on the stream before it is complete
 *     (the results reach pinned host memory directly from the GPU);
 *     tv_commit only enqueues (its effects are ordered before later work on
 *     the stream).
 *   - Token ids are int32 in [0, vocab).  A tree is given by parents[] and
 *     tokens[] of n_nodes entries, root included: parents[0] == -1 and
 *     0 <= parents[i] < i (any topological order; depth-first pre-order as
 *     the pages store it is the usual case).  tokens[0] is the root: the last
 *     token emitted, whose KV is not cached yet.  Sibling tokens must differ
 *     ("Algorithm and correctness contract", Target position and batching).
 *   - Row i of a verify is the model's scores after consuming the path
 *     root..i, at position ctx_len + depth(i) ("Drafters and tree verify",
 *     Tree verify through recurrent layers: attention sees its ancestors
 *     and a position equal to its depth).
 *   - A verify writes the tree's KV rows at cache slots ctx_len + i but does
 *     not move ctx_len; only tv_commit does.  Verifying again without a commit
 *     discards the previous tree.
 *   - A context is used by one thread at a time: calls on the same tv_ctx
 *     must not overlap (it owns activation scratch, pinned staging and the
 *     last error message).  Separate contexts may run on separate threads,
 *     each on its own stream.  tv_accept_walk, tv_staircut and
 *     tv_lookup_draft keep no state and may be called from any thread.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_OK 0
#define TV_EINVAL (-1)    /* bad argument, tree, path, name or size */
#define TV_ECAPACITY (-2) /* ctx_len + rows would exceed max_ctx */
#define TV_ESTATE (-3)    /* commit with no pending verify; unbound tensors */
#define TV_EHIP (-4)      /* a HIP runtime call failed (message in tv_last_error) */

#define TV_MAX_NODES 32   /* rows of one pass, all requests together */

#define TV_LAYER_ATTN 0   /* grouped-query attention layer with RoPE */
#define TV_LAYER_RECUR 1  /* gated linear recurrence layer */
#define TV_LAYER_DELTA 2  /* gated delta-rule layer (Gated DeltaNet, "Drafters and
                             tree verify", Tree verify through recurrent layers) */

/* Shapes of the target model.  Every weight matrix is [N_out, K_in]
 * row-major bf16.  An attention layer's wqkv stacks n_qhead, then n_kvhead,
 * then n_kvhead heads of head_dim rows; a recurrent layer's wqkv stacks q, k
 * and v with n_qhead heads each.  wa of a TV_LAYER_RECUR layer is
 * [n_qhead, hidden]: the log-gate g = log sigmoid(x wa^T) of each head, the
 * state S = e^g S_parent + k v^T.  wa of a TV_LAYER_DELTA layer is
 * [2 n_qhead, hidden]: the gate rows, then the write-strength rows
 * b = sigmoid(x wb^T); its state follows the gated delta rule
 * S = e^g (I - b k k^T) S_parent + b k v^T (key index first).  Both read
 * out o = S^T q with q and k L2-normalised per head. */
typedef struct tv_model_desc {
    int n_layer;
    int hidden;
    int n_qhead;
    int n_kvhead;
    int head_dim;       /* 64 or 128 */
    int ffn;
    int vocab;
    const int *layer_kind; /* [n_layer], TV_LAYER_* (copied) */
    float eps;          /* RMSNorm and L2-norm epsilon */
    float rope_theta;
    int max_ctx;        /* KV cache rows per request, tree rows included */
    int max_req;        /* requests (independent caches) */
} tv_model_desc;

typedef struct tv_ctx tv_ctx;

/* Create a context; `stream` is a hipStream_t (NULL = the null stream). */
int tv_create(const tv_model_desc *m, void *stream, tv_ctx **out);
void tv_destroy(tv_ctx *ctx);
/* The message of the last failed call on `ctx`; with ctx == NULL, of the
 * last failed context-free call on the calling thread. */
const char *tv_last_error(tv_ctx *ctx);

/* Bind a caller-owned device buffer by name.  `bytes` must equal the
 * tensor's size.  Names and layouts:
 *   "emb" [vocab, hidden] bf16        "head" [vocab, hidden] bf16
 *   "final_norm" [hidden] bf16
 *   "layers.L.attn_norm", "layers.L.ffn_norm" [hidden] bf16
 *   "layers.L.wqkv", "layers.L.wo", "layers.L.wa" (recurrent and delta only),
 *   "layers.L.wg", "layers.L.wu" [ffn, hidden], "layers.L.wd" [hidden, ffn]
 *   "req.R.layers.L.k", "req.R.layers.L.v"  [n_kvhead, max_ctx, head_dim] bf16
 *   "req.R.layers.L.state"                  [n_qhead, head_dim, head_dim] fp32
 *     (state[h][i][j]: key index i, value index j)
 * Weight matrices (head, wqkv, wo, wa, wg, wu, wd) are given row-major and
 * REARRANGED IN PLACE into the library's packed tile order (see
 * tv_pack_weight): after tv_bind their bytes are no longer row-major.
 * Re-binding a name to the buffer it already holds does not pack it again;
 * binding an already packed buffer under another name does.                */
int tv_bind(tv_ctx *ctx, const char *name, void *dev_ptr, size_t bytes);

/* Declare request `req`'s committed context: ctx_len cache rows already
 * hold its keys (already rotated) and values, and its recurrent states are
 * the bound ones.  `ids` (n_ids tokens, may be NULL) is the text those rows
 * stand for, used only by the repetition penalty.  Drops any pending tree. */
int tv_set_history(tv_ctx *ctx, int req, const int32_t *ids, int n_ids, int ctx_len);

/* Score modifiers of request `req`, applied to every verified row as plain
 * decoding applies them to its one row ("Exactness", The promise): first a
 * repetition penalty theta over the row's prior tokens (history, committed
 * tokens and the row's own path; l > 0 -> l/theta, else l*theta), then
 * logit_bias, then the allow-mask (bit v of allow_bits[v/32]; disallowed ids
 * never win).  rep_penalty == 1, n_bias == 0 and allow_bits == NULL turn
 * each off.  The returned logits stay the raw fp32 values; argmax and gap
 * use the modified scores. */
int tv_set_modifiers(tv_ctx *ctx, int req, float rep_penalty, const int32_t *bias_ids,
                     const float *bias_vals, int n_bias, const uint32_t *allow_bits);

/* Make request `req` a sampled request ("Exactness", Sampling; "Drafters and
 * tree verify", Sampling), or greedy again with temperature == 0 (the state
 * at tv_create).  A sampled row's "argmax" is then the target's own draw: the
 * argmax of fp32(fp32(score / temperature) + G), score the row's modified
 * score and G standard Gumbel noise keyed by (seed, t), t the sequence index
 * of the drawn token (indices count from 0 at the first prompt token; row i
 * draws index ctx_len + depth(i) + 1).  That is an exact draw from
 * softmax(score / temperature), and the accept walk keeps a drafted token
 * exactly while the draw lands on it, so a seed gives the same text for any
 * drafter.  The noise: Philox4x32-10 (Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011), vocabulary id v taking word v % 4
 * of the block at counter (v / 4, t, 0, 0) under key (seed & 0xffffffff,
 * seed >> 32); a word x gives u = (x + 1/2) / 2^32 and G = -log(-log u) in
 * fp64, rounded to fp32.  gap_ulps then measures the two best noisy scores.
 * The setting stays with the request slot until changed.  Errors: TV_EINVAL
 * for a negative, NaN or infinite temperature or a bad request slot. */
int tv_set_sampling(tv_ctx *ctx, int req, float temperature, uint64_t seed);

/* Prefill: forward `n` prompt tokens as chains of at most 32 through the
 * verify path, committing each chain whole (the prefill chunk grid,
 * "Exactness", Caches).  *argmax_last (may be NULL) gets the argmax after
 * the last token: the first token to emit. */
int tv_prefill(tv_ctx *ctx, int req, const int32_t *tokens, int n, int32_t *argmax_last);

/* Dense prefill: the prompt's rows in chunks of up to `chunk` rows through
 * the MFMA-bound prefill kernels (one GEMM over all of a chunk's rows per
 * projection, attention in blocks of 32 rows).  The chunk grid is fixed by
 * absolute position: chunks end at multiples of `chunk` ("Exactness",
 * Caches: snapshots are taken at chunk-grid boundaries and a restored
 * request continues on those boundaries), so a request resumed at a grid
 * point from the cache rows a cold prefill left there computes the same
 * arithmetic, bit for bit.  `chunk` is a multiple of 32 in [32, 2048].
 * Recurrent layers take the chunk's rows as chains of 32 in order (the tree
 * read-out on each, then the closed-form state commit of the chain).  Rows
 * are committed as they go: ctx_len grows by n and the tokens join the
 * history.  *argmax_last (may be NULL) gets the last row's
 * token (with the request's modifiers and sampling), as tv_prefill. */
int tv_prefill_dense(tv_ctx *ctx, int req, const int32_t *tokens, int n, int chunk, int32_t *argmax_last);

/* Verify one tree for request `req`.  logits_dev: device fp32 [n_nodes,
 * vocab] (may be NULL: then logits go to library scratch).  argmax (int32)
 * and gap_ulps (float, may be NULL) are host arrays of n_nodes.  gap_ulps[i]
 * = (top1 - top2) / ulp_bf16(top1) with ulp_bf16(x) = 2^(floor(log2|x|)-7)
 * ("Exactness", The one exception: near ties); +inf when only one id is
 * allowed. */
int tv_verify_tree(tv_ctx *ctx, int req, const int32_t *parents, const int32_t *tokens,
                   int n_nodes, float *logits_dev, int32_t *argmax, float *gap_ulps);

/* Verify n_req trees of distinct requests in one pass ("Exactness",
 * Parallel requests); the sum of n_nodes must be <= 32.  Rows are laid out
 * request after request in the order given.  Each request's rows equal what
 * its own tv_verify_tree gives, bit for bit. */
int tv_verify_trees(tv_ctx *ctx, int n_req, const int *reqs, const int32_t *const *parents,
                    const int32_t *const *tokens, const int *n_nodes, float *logits_dev,
                    int32_t *argmax, float *gap_ulps);

/* The greedy accept walk, host only, integers only: from the root take the
 * model's token argmax[cur] and move to the child carrying it; stop where
 * none does, keeping the model's token there ("Drafters and tree verify",
 * The round, step 3).  path (node ids, root first) and emitted (tokens) are
 * host arrays of at least n_nodes; *path_len == *n_emitted >= 1. */
int tv_accept_walk(const int32_t *parents, const int32_t *tokens, const int32_t *argmax,
                   int n_nodes, int32_t *path, int *path_len, int32_t *emitted, int *n_emitted);

/* Commit the accepted path of request `req`'s pending tree: path[0] == 0
 * and each path[d] a child of path[d-1].  KV rows move from slot
 * ctx_len+path[d] to ctx_len+d ("Drafters and tree verify", Tree verify
 * through recurrent layers: the cache holds every node at its depth-first
 * slot and the commit gathers the accepted rows into place); each recurrent
 * state becomes the state after the path, from the quantities the verify
 * computed (same section, the closed form of S_path).  ctx_len grows by
 * path_len; the path's tokens join the history. */
int tv_commit(tv_ctx *ctx, int req, const int32_t *path, int path_len);

/* One whole round for request `req` ("Drafters and tree verify", The round:
 * verify, accept, commit): tv_verify_tree, then tv_accept_walk on its
 * argmax, then tv_commit of the accepted path, in one call.  Arguments as
 * for those calls; path and emitted are host arrays of at least n_nodes
 * (argmax and gap_ulps too; gap_ulps may be NULL).  On a verify error nothing
 * is committed; the results equal those of the three calls made in turn. */
int tv_round(tv_ctx *ctx, int req, const int32_t *parents, const int32_t *tokens, int n_nodes,
             float *logits_dev, int32_t *argmax, float *gap_ulps, int32_t *path, int *path_len,
             int32_t *emitted, int *n_emitted);

/* StairCut ("Drafters and tree verify", StairCut), host only: cut a
 * candidate tree to the node count that maximises expected committed tokens
 * per millisecond, (1 + min(sum of q over the kept nodes, their number)) /
 * (verify price of the rows + draft_ms + commit_ms).
 *   parents, q: n_nodes entries (1 <= n_nodes <= TV_MAX_CANDIDATE), node 0
 *     the root (the last emitted token, parents[0] == -1, q[0] unused),
 *     0 <= parents[i] < i; q[i] >= 0 is node i's path probability, capped
 *     at 1 by the caller.
 *   order: the n_nodes-1 drafted nodes in the drafter's score order (a
 *     permutation of 1..n_nodes-1); each is admitted with the ancestors it
 *     needs.  q and order may be NULL when n_nodes == 1 (the root alone).
 *   price_tree_ms, price_chain_ms: verify price in ms by row count, index
 *     1..TV_MAX_NODES (index 0 unused); the chain table prices a cut whose
 *     nodes form one path.
 * A cut ends at 7, 15, 23 or 31 nodes (8, 16, 24 or 32 rows: the longest
 * admission prefix within that many nodes) or at the whole candidate when it
 * has at most 31; among equal scores the smaller cut wins.  keep (host, at
 * least 32 entries) receives the kept node ids in increasing order, root
 * first; *n_keep their number (the rows of the verify); *score (may be
 * NULL) the cut's tokens per ms.  TV_EINVAL on a malformed candidate, a
 * non-finite price or cost, or a non-positive total price. */
#define TV_MAX_CANDIDATE 256
int tv_staircut(const int32_t *parents, const float *q, const int32_t *order, int n_nodes,
                const float *price_tree_ms, const float *price_chain_ms, float draft_ms, float commit_ms,
                int32_t *keep, int *n_keep, float *score);

/* StairCut's verify prices by row count ("Drafters and tree verify",
 * StairCut on Flash-Next, and the shared price files), host only: a model
 * built from a price file's points and updated online with measured round
 * times, whose table feeds tv_staircut's price arguments.
 *   tv_prices_create: n_points points (ctx_class[i], kind[i], rows[i],
 *     ms[i]) of a price file, kind TV_PRICE_CHAIN or TV_PRICE_TREE, rows
 *     >= 1, each (class, kind, rows) at most once (n_points may be 0: no
 *     file); has_step says whether the file gives step_ms; ema in (0, 1] is
 *     the weight of a measured round.  *out receives the model (free it with
 *     tv_prices_destroy).
 *   tv_prices_class: the context class of ctx: the largest listed class
 *     <= ctx, else the smallest listed one; *has_class = 0 when there is no
 *     file.
 *   tv_prices_table: out[0..TV_MAX_NODES] (host doubles) = the prices in ms
 *     for the class of ctx and the kind: the file's price of each count (the
 *     first listed price below the first listed count; linear between two
 *     listed counts; past the last, step_ms a row, else the last two counts'
 *     slope, else flat; 1 ms for every count with no file or no entry for
 *     the kind), shifted by the mean offset of the measured counts from the
 *     file, each measured count at its live price, out[0] = out[1], then
 *     made non-decreasing in rows.
 *   tv_prices_observe: a measured round of `rows` rows (1..TV_MAX_NODES)
 *     at ctx took ms: that count's live price (started at its current table
 *     price) moves by ema * (ms - live).
 * Errors: TV_EINVAL for a null pointer, a bad kind, count, weight or
 * non-finite value, a count listed twice, or when memory runs out. */
#define TV_PRICE_CHAIN 0
#define TV_PRICE_TREE 1
typedef struct tv_prices tv_prices;
int tv_prices_create(const int32_t *ctx_class, const int32_t *kind, const int32_t *rows, const double *ms,
                     int n_points, int has_step, double step_ms, double ema, tv_prices **out);
void tv_prices_destroy(tv_prices *p);
int tv_prices_class(const tv_prices *p, int ctx, int32_t *cls, int *has_class);
int tv_prices_table(const tv_prices *p, int ctx, int kind, double *out);
int tv_prices_observe(tv_prices *p, int ctx, int kind, int rows, double ms);

/* The lookup drafter over the request's own text ("Drafters and tree
 * verify", The lookup drafter), host only: it copies text instead of
 * predicting it.  An occurrence of order o is a start p with
 * text[p .. p+o) equal to the last o tokens and p + o <= len - 1 (it is
 * followed by at least one token).  The order used is the largest o in
 * [min_order, max_order] with an occurrence; each of its occurrences is one
 * vote, continuing with text[p+o .. p+o+max_depth) (shorter where the text
 * ends).  A tree node is a token sequence that begins at least one
 * continuation; q = (its votes) / (all votes) * rho^depth, computed in
 * double (rho^depth as depth products) and rounded once to float: its vote
 * share times StairCut's continuation rate a level ("Drafters and tree
 * verify", StairCut: a fixed decay of 1/1.6 a level, or a learned rate;
 * 0 < rho <= 1, rho = 1 for the plain vote shares).
 *   text, len: the request's text (prompt and output so far, len >= 1); its
 *     last token is the tree's root (the next verify's root).
 *   1 <= min_order <= max_order <= TV_LOOKUP_MAX_ORDER (the pages use 2..8);
 *   1 <= max_depth <= TV_MAX_CANDIDATE; 0 <= max_nodes < TV_MAX_CANDIDATE.
 * At most max_nodes nodes are kept (the root excluded), best first by
 * (votes descending, depth ascending, path ascending as a token sequence),
 * an order in which ancestors come first.  Output (host arrays of at least
 * max_nodes + 1 entries): parents, tokens, q of the kept tree in depth-first
 * pre-order with siblings by (votes descending, token ascending), node 0 the
 * root (q 1); order (at least max_nodes entries, may be NULL when max_nodes
 * is 0): the kept nodes by admission, as output indices (StairCut's order);
 * *n_nodes the nodes written, root included; *match_order the order used (0
 * when nothing matched: the root alone) and *n_votes the vote count (either
 * may be NULL).  TV_EINVAL for a bad argument or when memory runs out. */
#define TV_LOOKUP_MAX_ORDER 64
int tv_lookup_draft(const int32_t *text, int len, int min_order, int max_order, int max_depth, int max_nodes,
                    float rho, int32_t *parents, int32_t *tokens, float *q, int32_t *order, int *n_nodes,
                    int *match_order, int *n_votes);

/* One round of deterministic-candidate residual tree sampling ("Algorithm
 * and correctness contract", Deterministic tree candidates and residual
 * verification): tv_verify_tree, then at each visited node the children are
 * tried in index order against the target p = softmax(modified scores /
 * temperature): a candidate x is accepted with probability r(x), r starting
 * at p; a rejected candidate's mass is removed and r renormalised; when every
 * candidate fails (or at a leaf) a replacement is drawn from the residual and
 * the round ends; then tv_commit of the accepted path.  Each visited node
 * consumes one uniform, uniforms[its depth] in [0, 1) (host, at least
 * n_nodes entries): the decision is the first position, over (candidates in
 * index order, then every other id ascending), where the running sum of
 * p exceeds u (fp64 sums).  emitted = the accepted nodes' tokens and the
 * final draw (the next round's root); path, as tv_round.  Errors: TV_EINVAL
 * for a non-positive temperature or a uniform outside [0, 1), else as
 * tv_round. */
int tv_residual_round(tv_ctx *ctx, int req, const int32_t *parents, const int32_t *tokens, int n_nodes,
                      float *logits_dev, float temperature, const double *uniforms, int32_t *path,
                      int *path_len, int32_t *emitted, int *n_emitted);

/* Committed context length of request `req` (negative TV_E* on error). */
int tv_ctx_len(tv_ctx *ctx, int req);

/* Kernel-level calls: the pass's projection and head kernels on caller-given
 * device operands, for per-kernel tests and bandwidth measurement.
 * tv_linear: x [M, K] bf16 (row-major), w [N, K] bf16 packed (tv_pack_weight), M >= 1, K a
 * multiple of 8; y_fp32 == 0 writes bf16(x w^T) to y [M, N] bf16, y_fp32 != 0
 * writes the fp32 sums to y [M, N] fp32 (N <= vocab when M <= 32).  M <= 32
 * runs the verify pass's skinny kernel: the k order of every output is fixed
 * by (N, K) and the output kind alone, never by M.  M > 32 runs the dense
 * (prefill) kernel, whose k order is fixed by K alone.
 * tv_head_top2: the bound "head" on x [M, hidden] bf16: fp32 logits [M,
 * vocab] to logits_dev, argmax and gap (host, M entries) as tv_verify_tree
 * returns them, with no score modifiers.  Both synchronise the stream. */
int tv_linear(tv_ctx *ctx, const void *x, const void *w, int M, int N, int K, void *y, int y_fp32);

/* Rearrange a row-major [N, K] bf16 device matrix in place into the packed
 * order the projection kernels read (tv_bind does this for weights; a
 * tv_linear operand must be packed first).  Rows are cut into tiles of 32,
 * k into steps of 64; a full step of a full tile is 4 KB in which bytes
 * [1024q + 16l, +16) hold row l%32, k = 32*(l/32) + 8q .. +8 of the step
 * (q = 0..3, l = 0..63): the operand layout of one 32x32x16 bf16 matrix
 * instruction per q.  Partial tiles and steps keep the present pieces in
 * the same order.  Each tile stays in its row-major byte range.  Every call
 * packs (packing twice scrambles the matrix).  Synchronises the stream. */
int tv_pack_weight(tv_ctx *ctx, void *w, int N, int K);
int tv_head_top2(tv_ctx *ctx, const void *x, int M, float *logits_dev, int32_t *argmax, float *gap_ulps);

/* Kernel-level calls of the pass's other kernels, on caller-given device
 * operands, for per-kernel parity tests and measurement.  Shapes come from
 * the context's model; each call validates its arguments, runs its kernels
 * on the context's stream and synchronises it.  None reads bound weights.
 *
 * Split-K partial layout (the projections' output that the consumers
 * finish): for `splits` k-ranges S, column n of row m (m < 32) of k-range s
 * is the float at index ((n / 128) * S + s) * 4096 + m * 128 + n % 128.
 * A consumer adds the S partials of an element in k-range order in fp32 and
 * rounds the sum to bf16 (the projection's rounding point).
 *
 * tv_attention ("Drafters and tree verify", Tree verify through recurrent
 *   layers: each node attends to the cached context and to its ancestors
 *   and itself): grouped-query attention of the n_nodes rows of a tree.
 *   q: [n_nodes, n_qhead * head_dim] bf16, already rotated; k_cache,
 *   v_cache: [n_kvhead, cap, head_dim] bf16 whose slots [0, ctx_len) hold
 *   the context and slot ctx_len + i node i's key and value; parents: host
 *   [n_nodes], tree rules as tv_verify_tree.  Query head h uses KV head
 *   h / (n_qhead / n_kvhead); scores are scaled by 1/sqrt(head_dim) and
 *   normalised by an fp32 softmax.  out: [n_nodes, n_qhead * head_dim] bf16.
 *   TV_ECAPACITY when ctx_len + n_nodes > cap.
 * tv_rope_kv (same section: a node sits at position ctx_len + its depth and
 *   in cache slot ctx_len + its index): finishes the QKV projection's
 *   partials (columns: n_qhead, then n_kvhead, then n_kvhead heads of
 *   head_dim) for n_rows <= 32 rows, rotates q and k of row i by position
 *   ctx_len + depth[i] (host array; rotate-half pairs (j, j + head_dim/2),
 *   angle pos * rope_theta^(-2j/head_dim)), writes the rotated q to q_out
 *   [n_rows, n_qhead * head_dim] bf16 and k, v to cache slot ctx_len + i of
 *   k_cache, v_cache [n_kvhead, cap, head_dim] bf16.  Positions must lie
 *   below the model's max_ctx.
 * tv_resid_norm: for n_rows <= 32 rows of x [n_rows, hidden] bf16 (in
 *   place), x = bf16(x + bf16(sum of the `splits` partials)), then
 *   y = bf16(x / sqrt(mean(x^2) + eps) * w) with w [hidden] bf16, y
 *   [n_rows, hidden] bf16: the residual add and the next RMSNorm.
 * tv_recur_tree (same section: the state along each root-to-node path,
 *   never overwriting a parent's): the read-out of a recurrent layer of
 *   `kind` TV_LAYER_RECUR or TV_LAYER_DELTA for an n_nodes tree.  part: the
 *   stacked projection's partials, columns q, k and v (n_qhead heads of
 *   head_dim each), then the n_qhead gate pre-activations, then for a delta
 *   layer the n_qhead write-strength pre-activations; state: [n_qhead,
 *   head_dim, head_dim] fp32, the state before the tree (key index first).
 *   out: [n_nodes, n_qhead * head_dim] bf16 read-outs.  save_k [32, n_qhead,
 *   head_dim] bf16, save_v [32, n_qhead, head_dim] fp32 and save_gc [32,
 *   n_qhead] fp32 receive, per node, the normalised key, the value (a delta
 *   layer: the pseudo-value) and the cumulative log-gate that
 *   tv_recur_commit takes.
 * tv_recur_commit (same section: the closed form of the state after the
 *   accepted path): state = e^{gc_last} state + sum over the path of
 *   e^{gc_last - gc_t} k_t u_t^T, in place, from tv_recur_tree's saves;
 *   path: host node ids (path_len <= 32, each < 32), root first.
 * tv_gather_kv (same section: the commit gathers the accepted rows): slot
 *   ctx_len + path[d] -> ctx_len + d of k_cache and v_cache [n_kvhead, cap,
 *   head_dim], in place; path: host, strictly increasing, path[d] >= d.
 * Errors: TV_EINVAL for a null operand or a bad size, tree or path. */
int tv_attention(tv_ctx *ctx, const void *q, const void *k_cache, const void *v_cache, int cap, int ctx_len,
                 const int32_t *parents, int n_nodes, void *out);
int tv_rope_kv(tv_ctx *ctx, const float *qkv_part, int splits, int n_rows, const int32_t *depth, int ctx_len,
               void *q_out, void *k_cache, void *v_cache, int cap);
int tv_resid_norm(tv_ctx *ctx, const float *part, int splits, int n_rows, void *x, const void *w, void *y);
int tv_recur_tree(tv_ctx *ctx, int kind, const float *part, int splits, const int32_t *parents, int n_nodes,
                  const float *state, void *out, void *save_k, float *save_v, float *save_gc);
int tv_recur_commit(tv_ctx *ctx, float *state, const void *save_k, const float *save_v, const float *save_gc,
                    const int32_t *path, int path_len);
int tv_gather_kv(tv_ctx *ctx, void *k_cache, void *v_cache, int cap, int ctx_len, const int32_t *path,
                 int path_len);

/* tv_linear_noalloc: tv_linear for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same operands, kernels and results as tv_linear (bit
 * for bit), but it takes no context and allocates nothing: its scratch (a
 * zero block, split-K partials and top-2 candidates) is one static device
 * array of 12 MiB + 256 B per GPU, which the library holds until the
 * process ends.  It only enqueues work on `stream` (a hipStream_t, NULL =
 * the null stream) and does not synchronise it.  Every call on one GPU
 * shares that GPU's array, so calls that overlap on a GPU (other streams,
 * other threads) race; calls on one stream are ordered.  TV_EINVAL for a
 * shape whose scratch exceeds the array (fp32 output with M * ceil(N/128)
 * * 16 bytes above 4 MiB); the message is tv_last_error(NULL) on the
 * calling thread. */
int tv_linear_noalloc(const void *x, const void *w, int M, int N, int K, void *y, int y_fp32, void *stream);

/* Kernel timing: with `on` != 0, launches whose kernel name starts with
 * `only_prefix` (all launches when it is NULL or "") are bracketed by HIP
 * events on the context's stream.  tv_profile_get returns the total
 * milliseconds and the launch count recorded for names starting with
 * `prefix` since the last reset (it synchronises the stream). */
int tv_profile_enable(tv_ctx *ctx, int on, const char *only_prefix);
int tv_profile_reset(tv_ctx *ctx);
int tv_profile_get(tv_ctx *ctx, const char *prefix, double *total_ms, int *count);

#ifdef __cplusplus
}
#endif
#endif
