// Internal interface between the host runtime (tv_runtime.cpp) and the gfx950
// kernels (tv_kernels.hip).  Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

constexpr int kMaxRows = 32;   // rows of one pass
constexpr int kMaxGroup = 8;   // query heads per KV head
constexpr int kAttnChunk = 64;  // keys staged in LDS at a time
constexpr int kAttnLoadTasks = 3;  // staging tasks (64 bytes of K and of V) a loader thread holds per chunk
constexpr int kAttnComputeWaves = 5;  // query rows G*n <= 160: one wave per 32
constexpr int kAttnWaves = 8;         // waves of an attention workgroup that stages chunks: the register file
                                       // holds 2 waves a SIMD, and every wave beyond the compute waves loads
constexpr int kRecurSlices = 4; // value-column slices per head in the recurrent read-out

// Candidate pair of a top-2 search: best (v1, i1) and runner-up (v2, i2),
// ordered by value, then by lower token id.
struct Top2 {
    float v1;
    int i1;
    float v2;
    int i2;
};

// Score modifiers of one request of the pass (device arrays or null).
struct HeadMods {
    const uint32_t *hist_bits;  // [ceil(V/32)] prior tokens (history + committed)
    const float *bias;          // [V] dense logit_bias (0 where none)
    const uint32_t *allow_bits; // [ceil(V/32)] allowed ids
    float rep;                  // repetition penalty (1 = off)
    float temp;                 // sampling temperature (0 = greedy)
    uint32_t seed_lo, seed_hi;  // sampling seed: the Philox key
};

// Per-pass metadata, copied to the device once per verify.
struct PassMeta {
    int tok[kMaxRows];
    int depth[kMaxRows];
    uint32_t anc[kMaxRows];      // ancestor-or-self bits, request-local indices
    int row_req[kMaxRows];       // request slot of each row
    int path_len[kMaxRows];      // tokens on root..row
    int path_tok[kMaxRows * kMaxRows];
    int draw_t[kMaxRows];        // sequence index of the token each row draws
    HeadMods mods[kMaxRows];     // per request slot
};

// EPI_PARTIAL: write the fp32 partial sums only (a consumer kernel finishes them)
// EPI_F32 (dense GEMM only): the fp32 sums
enum Epi { EPI_BF16 = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_HEAD = 3, EPI_PARTIAL = 4, EPI_F32 = 5 };

struct GemmArgs {
    const uint16_t *X;  // [M, K] bf16 activations, row stride ldx
    int ldx;
    const uint16_t *W;  // [N, K] bf16 weights
    const uint16_t *W2; // [N, K] second weights (SwiGLU up); for partials: rows N1.. (see N1)
    int N1;             // partials only: rows [0, N1) come from W and [N1, N) from W2
                        // (N1 a multiple of 32; 0 = all rows from W)
    int M, N, K;
    uint16_t *Y;        // bf16 out (or residual in/out), row stride ldy
    int ldy;
    float *Yf;          // fp32 out (head), row stride ldyf
    int ldyf;
    Top2 *part;         // head: [ceil(N/32)][32] per-tile candidates
    const PassMeta *meta; // head modifiers and sampling (null: none)
    int mods_on;          // some request of the pass has modifiers or samples
    float *partial;     // split-K partial tiles (splits > 1)
    const void *zeros;  // >= 16 zero bytes (activation staging beyond M or K)
};

// k-range splits of a GEMM: a function of the weight shape only.  The most
// splits that keep the grid within 512 workgroups (two per CU of the 256, so
// no CU holds a third while others idle), at least 4 k steps each.
inline int gemm_splits(int N, int K) {
    const int rowblocks = ((N + 31) / 32 + 3) / 4;
    const int nsteps = (K + 63) / 64;
    int s = 512 / rowblocks;
    const int most = nsteps / 4 > 1 ? nsteps / 4 : 1;   // at least 4 k steps per split
    if (s > most) s = most;
    return s < 1 ? 1 : s;
}

// One request of a verify pass: its rows [row0, row0 + n) of the pass, this
// layer's cache, its committed context and its attention cache splits.
struct PassReq {
    uint16_t *Kc, *Vc;  // cache [n_kvhead][cap][D]
    int row0, n, ctx;
    int span, nsplit;   // cache keys per split and cache splits (the tree's own split follows them)
};

struct AttnArgs {
    const uint16_t *Q;  // rotated queries, rows row0.., [rows, n_qhead*D]
    const uint16_t *Kc; // cache [n_kvhead][cap][D] (prefill)
    const uint16_t *Vc;
    const PassMeta *meta;
    float *po;          // partials [n_kvhead][ns][kMaxRows*kMaxGroup][D] (prefill: one such block per z)
    float *pm;          // [n_kvhead][ns][kMaxRows*kMaxGroup]
    float *pl;
    int row0, n, ctx, cap, G, n_qhead, ns, n_ctx_split;
    int span;           // cache keys per split (a multiple of kAttnChunk)
    float scale;
    // prefill (zrows > 0): grid.z blocks of zrows consecutive rows of one
    // chain; block z covers rows [z*zrows, min(M, (z+1)*zrows)) at cache
    // slots ctx + row, sees ctx + z*zrows cache keys before it, and sizes its
    // own splits from that; ns is then the partial stride (the most splits
    // any block has, plus one)
    int zrows, M;
    int ztarget;        // prefill: splits of the cache keys per block (about)
    // verify (nreq > 0): grid.z runs over the pass's requests, each with its
    // own cache, context and splits; n, span and ns are the largest of any
    // request (they size the launch), and the partials of a query row sit at
    // its pass row, so requests never share a slot
    int nreq;
    PassReq rq[kMaxRows];
};

// Cache keys per attention split for at most `splits` splits, in whole LDS
// chunks.  A verify takes at most 31 cache splits (a function of the
// context length only): with the tree's own split that is 32 workgroups a KV
// head, 256 for 8 KV heads, one per CU (a workgroup fills its CU's register
// file), so no workgroup waits for a second round.
constexpr int kVerifyCacheSplits = 31;
constexpr int kAttnMaxSplits = 33;   // partial splits of a query row: 32 cache splits at most (a prefill block's) + the tree's
__host__ __device__ inline int attn_span_n(int ctx, int splits) {
    const int chunks = (ctx + kAttnChunk - 1) / kAttnChunk;
    const int per = (chunks + splits - 1) / splits;
    return (per < 1 ? 1 : per) * kAttnChunk;
}
__host__ __device__ inline int attn_span(int ctx) { return attn_span_n(ctx, kVerifyCacheSplits); }

struct RopeArgs {
    const float *part;   // QKV projection partial sums (row-contiguous split-K layout)
    int S;               // its k-range splits
    uint16_t *q_out;     // [rows, QH*D]
    const float *cosT, *sinT; // [max_pos][D/2]
    const PassMeta *meta;
    int M, cap, QH, KVH, D;   // M: rows of the pass
    int nreq;            // requests of the pass, in row order
    PassReq rq[kMaxRows];
};

struct RecurArgs {
    const float *qkv_part; // split-K partials of the stacked projection: q heads, k heads, v heads
                           // (3*QH*D columns), then from column a_col the gate pre-activations
                           // [QH] and, for a delta layer, the write-strength pre-activations [QH]
    int qkv_S;             // its k-range splits
    const float *S0;      // [QH][D][D] state before the round (key index, value index)
    const PassMeta *meta;
    uint16_t *out;        // [rows, QH*D] read-out (bf16)
    uint16_t *save_k;     // [kMaxRows][QH][D] normalised keys of this layer (request-local node order)
    float *save_v;        // [kMaxRows][QH][D] values (a delta layer: pseudo-values u)
    float *save_gc;       // [kMaxRows][QH] cumulative log-gates
    int a_col;             // column of head 0's gate (its write strength: a_col + QH)
    int delta;             // gated delta rule instead of the plain gated recurrence
    int row0, n, QH;
    float eps;
    // prefill blocks: the projection as bf16 rows instead of partials (columns
    // below a_col from qkv_rows [rows][a_col], the rest from ab_rows [rows][ab_ld]),
    // and the rows form a chain (node t's ancestors are 0..t-1)
    const uint16_t *qkv_rows;
    const uint16_t *ab_rows;
    int ab_ld;
};

// An accepted path, passed to the commit kernels by value.
struct PathArg {
    int len;
    int node[kMaxRows];
};

struct RecurCommitArgs {
    float *const *states;   // [n_layers] bound states, [QH][D][D] each
    const uint16_t *save_k; // [n_layers][kMaxRows][QH][D]
    const float *save_v;    // [n_layers][kMaxRows][QH][D] values or pseudo-values
    const float *save_gc;   // [n_layers][kMaxRows][QH]
    PathArg path;
    int QH;
};

// launch wrappers (tv_kernels.hip); each returns hipGetLastError()
// X = embedding rows of the pass's tokens, Y = RMSNorm(X) with weights w
hipError_t launch_embed_norm(hipStream_t s, const uint16_t *emb, const PassMeta *meta, PassMeta *meta_out, int M,
                             int H, const uint16_t *w, float eps, uint16_t *X, uint16_t *Y);
// X = bf16(X + bf16(sum of the S split-K partials P)), Y = RMSNorm(X) with weights w
hipError_t launch_resid_norm(hipStream_t s, const float *P, int S, int M, int H, const uint16_t *w, float eps,
                             uint16_t *X, uint16_t *Y);
hipError_t launch_gemm(hipStream_t s, int epi, const GemmArgs &a, int splits);
hipError_t launch_splitk_reduce(hipStream_t s, int epi, const GemmArgs &a, int splits);
// many activation rows (M > 32): X [M, K] row stride ldx, epilogues BF16, RESID, SWIGLU, F32
hipError_t launch_gemm_dense(hipStream_t s, int epi, const GemmArgs &a);
hipError_t launch_pack(hipStream_t s, const uint16_t *src, uint16_t *dst, int N, int K, int t0, int nt);
hipError_t launch_rope_kv(hipStream_t s, const RopeArgs &a);
hipError_t launch_attn(hipStream_t s, int D, const AttnArgs &a);
hipError_t launch_attn_combine(hipStream_t s, int D, const AttnArgs &a, uint16_t *out);
// prefill row kernels on M rows: X = emb[tok] (when tok is given), Y = RMSNorm(X) with weights w
hipError_t launch_norm_dense(hipStream_t s, const int32_t *tok, const uint16_t *emb, uint16_t *X, const uint16_t *w,
                             float eps, uint16_t *Y, int M, int H);
// prefill RoPE on the dense QKV output qkv [M, ldq] bf16: rows at positions and cache slots pos0 + i
hipError_t launch_rope_dense(hipStream_t s, const uint16_t *qkv, int ldq, int M, int pos0, int QH, int KVH, int D,
                             const float *cosT, const float *sinT, uint16_t *q_out, uint16_t *Kc, uint16_t *Vc,
                             int cap);
// Per-row result of a pass: argmax and the gap's bits, written by one 8-byte
// store into device-visible host memory.  The host fills the records with
// kResultEmpty before a pass and waits until every row's record has changed.
struct RowResult {
    int32_t argmax;
    uint32_t gap_bits;
};
constexpr uint32_t kGapEmpty = 0x7fc0deadu;   // a NaN pattern no gap takes
hipError_t launch_top2_reduce(hipStream_t s, const Top2 *part, int ntiles, int M, RowResult *res);
// residual tree sampling decisions of the pass's n rows (logits [n][ldl]
// fp32, the pass's metadata, u_row[n] device doubles, parts device scratch
// of kResidualPartBytes per row): res[i].argmax = -(j+1) to accept candidate
// j of row i, else the emitted token; gap bits 0
constexpr size_t kResidualPartBytes = 64 * 16;   // per row: at most 64 chunks of (max, sum) doubles
hipError_t launch_residual(hipStream_t s, const float *logits, int ldl, int V, const PassMeta *meta, int n, float T,
                           const double *u_row, void *parts, RowResult *res);
hipError_t launch_recur_tree(hipStream_t s, int D, const RecurArgs &a);
hipError_t launch_recur_commit(hipStream_t s, int D, const RecurCommitArgs &a, int n_layers);
hipError_t launch_commit_kv(hipStream_t s, uint16_t *const *kv_ptrs, int n_layers, int KVH,
                            int cap, int D, int ctx, const PathArg &path);

// message of the last failed context-free call on this thread (tv_noalloc.hip)
const char *noalloc_last_error();

} // namespace tv
