// gfx950 kernels of the tree-verify pass.
//
// Numerics of the target model (the same readings the CPU oracle takes, in
// its own code): bf16 storage of weights, activations and KV; fp32
// accumulation; bf16 round-to-nearest-even after every projection but the
// head, after each residual add, after RMSNorm, after RoPE and after SwiGLU;
// the head accumulates and returns fp32 ("Exactness", The one exception:
// near ties: the head returns fp32 logits and every matrix-product kernel
// fixes its reduction order by the weight's shape, never by the row count).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <type_traits>

#include "tv_internal.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32, which equals the textbook rounding (add 0x7fff plus the
// lowest kept bit, truncate) on every non-NaN input.
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two values at once: a in the low half, b in the high half
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ float bfround(float f) { return bf2f(f2bf(f)); }

__device__ __forceinline__ bf16x8 as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Weight streams are read once per pass: nontemporal loads keep them from
// displacing the activations every workgroup re-reads from the caches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const uint16_t *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return uint4{v.x, v.y, v.z, v.w};
}

// Row index inside a 32x32 MFMA output tile held by accumulator r of a lane
// in half `hf` (lanes 0-31: hf 0, lanes 32-63: hf 1); the column is lane%32.
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// Strict order of top-2 candidates: higher value, then lower id.
__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
    return a > b || (a == b && ia < ib);
}

// Both written as selects: with branches the compiler keeps (v1, i1, v2,
// i2) in a private array and updates it by a computed index (scratch memory).
__device__ __forceinline__ void top2_insert(float &v1, int &i1, float &v2, int &i2, float s, int id) {
    const bool b1 = better(s, id, v1, i1), b2 = better(s, id, v2, i2);
    const float n2 = b1 ? v1 : (b2 ? s : v2);
    const int m2 = b1 ? i1 : (b2 ? id : i2);
    v1 = b1 ? s : v1;
    i1 = b1 ? id : i1;
    v2 = n2;
    i2 = m2;
}

__device__ __forceinline__ void top2_merge(float &v1, int &i1, float &v2, int &i2, float w1, int j1,
                                           float w2, int j2) {
    const bool a1 = better(w1, j1, v1, i1);
    // a1: the new runner-up is the better of (v1, w2); else the better of (w1, v2)
    const bool x = a1 ? better(v1, i1, w2, j2) : better(w1, j1, v2, i2);
    const float n2 = a1 ? (x ? v1 : w2) : (x ? w1 : v2);
    const int m2 = a1 ? (x ? i1 : j2) : (x ? j1 : i2);
    v1 = a1 ? w1 : v1;
    i1 = a1 ? j1 : i1;
    v2 = n2;
    i2 = m2;
}

// ------------------------------------------------------------ sampling
// A sampled row draws the argmax of fp32(fp32(score / T) + G), G standard
// Gumbel noise keyed by (seed, t), t the sequence index of the drawn token:
// the Gumbel-max trick ("Exactness", Sampling; "Drafters and tree verify",
// Sampling).  The noise generator is Philox4x32-10 (Salmon, Moraes, Dror and
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011): vocabulary
// id v takes word v % 4 of the block at counter (v / 4, t, 0, 0) under key
// (seed low word, seed high word), so an aligned quad of ids is one block.

struct U32x4 {
    uint32_t w[4];
};

__device__ __forceinline__ U32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;   // round multipliers of the definition
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;   // key schedule increments of the definition
        k1 += 0xBB67AE85u;
    }
    return U32x4{{c0, c1, c2, c3}};
}

// G = -log(-log(u)) with u = (x + 1/2) / 2^32, exact in fp64 and strictly
// inside (0, 1); the logs run in fp64 and G is rounded once to fp32.
__device__ __forceinline__ float gumbel_of(uint32_t x) {
    const double u = ((double)x + 0.5) * 0x1p-32;
    return (float)(-log(-log(u)));
}

// Modified score of the aligned quad n0..n0+3 (n0 < N) of row m, in place:
// repetition penalty over the prior tokens (history bits, and `pathq`, the
// row's path tokens among the quad in its low 4 bits), logit_bias, the
// allow-mask, then for a sampled request score / T + G.
__device__ __forceinline__ void score_quad(const PassMeta *meta, int m, int n0, int N, uint32_t pathq,
                                           float s[4]) {
    const HeadMods &md = meta->mods[meta->row_req[m]];
    const int w = n0 >> 5, b = n0 & 31;   // the quad lies inside vocabulary word w
    if (md.rep != 1.0f) {
        const uint32_t prior = ((md.hist_bits ? md.hist_bits[w] : 0u) >> b) | pathq;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((prior >> j) & 1u) s[j] = s[j] > 0.f ? s[j] / md.rep : s[j] * md.rep;
    }
    if (md.bias) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (n0 + j < N) s[j] = s[j] + md.bias[n0 + j];
    }
    if (md.allow_bits) {
        const uint32_t allow = md.allow_bits[w] >> b;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (!((allow >> j) & 1u)) s[j] = -INFINITY;
    }
    if (md.temp > 0.f) {
        const U32x4 x = philox4x32_10((uint32_t)(n0 >> 2), (uint32_t)meta->draw_t[m], 0u, 0u, md.seed_lo,
                                      md.seed_hi);
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] = s[j] / md.temp + gumbel_of(x.w[j]);
    }
}

// ------------------------------------------------------- split-K partials
// Projections write fp32 partial sums row-contiguously: for 128-row block
// rb, k-range s and accumulator j (gate/up use two), element (m, n) sits at
// partial[((rb*S + s)*NACC + j)*4096 + m*128 + n%128].  A consumer adds the S
// partials of an element in k-range order, so every element's sum order is
// fixed by the weight shape.


// Split-K sums of U elements (element u's partials start at p[u], one split
// every st floats), with the loads of 16 splits of every element issued
// before any add: one round trip to memory for up to 16 splits.  Each
// element's adds stay in k-range order.
template <int U>
__device__ __forceinline__ void psum_multi(const float *const (&p)[U], size_t st, int S, float (&out)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) out[u] = 0.f;
    for (int k0 = 0; k0 < S; k0 += 16) {
        float l[U][16];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) l[u][j] = k0 + j < S ? p[u][(size_t)(k0 + j) * st] : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (k0 + j < S) out[u] += l[u][j];
    }
}
__device__ __forceinline__ const float *pptr(const float *P, int S, int nacc, int j, int m, int n) {
    return P + ((size_t)(n >> 7) * S * nacc + j) * 4096 + (size_t)m * 128 + (n & 127);
}

// --------------------------------------------- residual stream + RMSNorm
// RMSNorm is y = bf16(x / sqrt(mean(x^2) + eps) * w).  One workgroup owns one
// row, one thread 8 consecutive columns (hidden <= 8192): it forms the row's
// new residual stream x (the embedding row, or x + bf16(sum of a
// projection's split-K partials)), writes it, reduces the sum of squares in
// a fixed order and writes the normalised row y for the next projection.

constexpr int kRowThreads = 1024;
constexpr int kRowSplits = 12;   // split-K partials in flight per thread
enum RowMode { ROW_EMBED = 0, ROW_RESID = 1 };

__device__ __forceinline__ float4 ld_f4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// ROW_EMBED reads the pass metadata where the host wrote it (coherent pinned
// memory, read over the bus): each row takes its token, and workgroup 0 also
// copies the whole record to meta_out in device memory for the later kernels
// of the pass, which replaces a separate copy before the pass.
template <int MODE>
__global__ __launch_bounds__(kRowThreads) void k_row_norm(const uint16_t *__restrict__ emb,
                                                          const PassMeta *__restrict__ meta,
                                                          PassMeta *__restrict__ meta_out,
                                                          const float *__restrict__ P, int S, int H,
                                                          const uint16_t *__restrict__ w, float eps,
                                                          uint16_t *__restrict__ X, uint16_t *__restrict__ Y) {
    __shared__ float red[kRowThreads / 64];
    const int m = blockIdx.x, t = threadIdx.x;
    if constexpr (MODE == ROW_EMBED) {
        if (m == 0 && meta_out) {
            // 16-byte pieces: one load per thread, one trip over the bus
            static_assert(sizeof(PassMeta) % 16 == 0, "the metadata record is copied in 16-byte pieces");
            const uint4 *src = reinterpret_cast<const uint4 *>(meta);
            uint4 *dst = reinterpret_cast<uint4 *>(meta_out);
            for (int i = t; i < (int)(sizeof(PassMeta) / 16); i += blockDim.x) dst[i] = src[i];
        }
    }
    const int n0 = 8 * t;
    const bool ok = n0 < H;
    const uint4 z = {0u, 0u, 0u, 0u};
    uint16_t *xr = X + (size_t)m * H;
    const uint4 wv = ok ? ld16(w + n0) : z;
    float x[8];
    if constexpr (MODE == ROW_EMBED) {
        const uint4 v = ok ? ld16(emb + (size_t)meta->tok[m] * H + n0) : z;
        if (ok) *reinterpret_cast<uint4 *>(xr + n0) = v;
        const uint16_t *ve = reinterpret_cast<const uint16_t *>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf2f(ve[e]);
    } else {
        const uint4 ov = ok ? ld16(xr + n0) : z;
        // partial (s, m, n) sits at ((n/128)*S + s)*4096 + m*128 + n%128; a
        // thread's 8 columns share one 128-column block
        const float *pp = P + (size_t)(ok ? n0 >> 7 : 0) * S * 4096 + (size_t)m * 128 + (n0 & 127);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        for (int s0 = 0; s0 < S; s0 += kRowSplits) {   // loads of kRowSplits splits in flight, adds in split order
            float4 v[kRowSplits][2];
#pragma unroll
            for (int i = 0; i < kRowSplits; ++i) {
                const bool in = ok && s0 + i < S;
                v[i][0] = in ? ld_f4(pp + (size_t)(s0 + i) * 4096) : float4{0.f, 0.f, 0.f, 0.f};
                v[i][1] = in ? ld_f4(pp + (size_t)(s0 + i) * 4096 + 4) : float4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int i = 0; i < kRowSplits; ++i) {
                if (s0 + i < S) {
                    acc[0] += v[i][0].x; acc[1] += v[i][0].y; acc[2] += v[i][0].z; acc[3] += v[i][0].w;
                    acc[4] += v[i][1].x; acc[5] += v[i][1].y; acc[6] += v[i][1].z; acc[7] += v[i][1].w;
                }
            }
        }
        const uint16_t *oe = reinterpret_cast<const uint16_t *>(&ov);
        uint32_t nw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint16_t lo = f2bf(bf2f(oe[2 * e]) + bfround(acc[2 * e]));
            const uint16_t hi = f2bf(bf2f(oe[2 * e + 1]) + bfround(acc[2 * e + 1]));
            x[2 * e] = bf2f(lo);
            x[2 * e + 1] = bf2f(hi);
            nw[e] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        if (ok) *reinterpret_cast<uint4 *>(xr + n0) = uint4{nw[0], nw[1], nw[2], nw[3]};
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    // fixed-order reduction: within each wave by xor shuffles, then the
    // waves' sums in wave order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    const int nw_ = blockDim.x >> 6;
    for (int i = 0; i < nw_; ++i) tot += red[i];
    const float scale = 1.0f / sqrtf(tot / (float)H + eps);
    if (!ok) return;
    const uint16_t *we = reinterpret_cast<const uint16_t *>(&wv);
    uint32_t yw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint16_t lo = f2bf(x[2 * e] * scale * bf2f(we[2 * e]));
        const uint16_t hi = f2bf(x[2 * e + 1] * scale * bf2f(we[2 * e + 1]));
        yw[e] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    *reinterpret_cast<uint4 *>(Y + (size_t)m * H + n0) = uint4{yw[0], yw[1], yw[2], yw[3]};
}

// XOR swizzle of the 16-byte chunks of a staged activation row (128 bytes
// of k): row r keeps chunk x in slot x ^ bswz(r).  A B-operand read takes
// chunk ch of rows c = lane % 32; the LDS serves a 16-byte read for 16
// lanes at a time over its 64 banks, and with bswz(c) = (c / 2) % 8 those
// 16 lanes (8 even rows on one half of the banks, 8 odd rows on the other)
// hit 16 distinct groups of 4 banks.
__device__ __forceinline__ int bswz(int row) { return (row >> 1) & 7; }

// ------------------------------------------------------------ skinny GEMM
// Y[m, n] = sum_k X[m, k] W[n, k] for M <= 32 activation rows.
//
// Weights are stored packed (see k_pack): a tile of 32 rows is cut into
// 64-wide k steps, and a full step is 4 KB laid out so that load q of lane l
// reads bytes [1024q + 16l, +16): the 8 k values [32*(l/32) + 8q, +8) of row
// l%32, exactly v_mfma_f32_32x32x16_bf16's A operand (row = lane%32).  Every
// weight load is then one contiguous 1 KB per wave.
//
// A workgroup of 4 waves owns 4 consecutive tiles (128 rows) and one of S
// k-ranges; the activations of each step (32 x 64 bf16, zero beyond M) are
// staged once in LDS by direct global-to-LDS loads (XOR-swizzled 16-byte
// chunks, conflict-free reads) and shared by the 4 waves as the B operand
// (column = lane%32).  With S > 1 (or for partial-only launches) each
// workgroup writes its fp32 partial tile; a consumer (k_splitk_reduce, the
// RoPE kernel, the row-norm kernel or the recurrent read-out) adds the S
// partials in k-range order.  S is the most splits that keep the grid within
// 512 workgroups, a function of the weight shape only, and the k order of
// every output is fixed by K: M only decides which B columns are zero, so a
// row's result is the same for any row count and any row slot.  A partial
// launch may read two stacked matrices (rows [0, N1) from W, the rest from
// W2), which lets one launch serve the recurrent layer's q/k/v and gate.

// Element offset, inside a packed tile, of the 8-element piece (q, hf) of
// row c at step s; -1 when the piece lies beyond K or the row beyond N.
__device__ __forceinline__ long packed_piece(int s, int q, int hf, int c, int nr, int K) {
    const int kr = min(64, K - 64 * s);
    if (c >= nr || 32 * hf + 8 * q >= kr) return -1;
    const int pi = 2 * q + hf;
    int rank = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p)
        rank += (p < pi && 32 * (p & 1) + 8 * (p >> 1) < kr) ? 1 : 0;
    return (long)64 * s * nr + (long)rank * nr * 8 + c * 8;
}

// Epilogue of one 32x32 output tile held in MFMA accumulator layout (all
// epilogues but the head's).
template <int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &g, int tile, int lane, const f32x16 &acc,
                                              const f32x16 &acc2) {
    const int hf = lane >> 5, c = lane & 31;
    const int m = c, N = g.N;
    if (c >= g.M) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int n = tile * 32 + acc_row(r, hf);
        if (n >= N) continue;
        uint16_t *y = g.Y + (size_t)m * g.ldy + n;
        if constexpr (EPI == EPI_BF16) {
            *y = f2bf(acc[r]);
        } else if constexpr (EPI == EPI_RESID) {
            *y = f2bf(bf2f(*y) + bfround(acc[r]));
        } else {
            const float gt = bfround(acc[r]), up = bfround(acc2[r]);
            *y = f2bf(gt / (1.0f + expf(-gt)) * up);
        }
    }
}

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    constexpr int U = (DUAL || EPI == EPI_HEAD) ? 2 : 4;   // k steps per LDS stage
    constexpr int NACC = DUAL ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][U][32 * 64];
    __shared__ uint32_t pbits[EPI == EPI_HEAD ? kMaxRows * 4 : 1];   // head: path tokens per row

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, c = lane & 31;
    const int N = g.N, K = g.K;
    const int ntiles = (N + 31) >> 5;
    const int tile = blockIdx.x * 4 + wave;
    const bool tok = tile < ntiles;
    const int nr = tok ? min(32, N - tile * 32) : 0;
    const int nsteps = (K + 63) >> 6;
    const int S = gridDim.y, ks = blockIdx.y;
    const int s0 = (nsteps * ks) / S, s1 = (nsteps * (ks + 1)) / S;
    // partials of two stacked matrices: tiles from N1/32 on read W2
    const int t1 = (EPI == EPI_PARTIAL && g.N1 > 0) ? (g.N1 >> 5) : ntiles;
    const uint16_t *tb = tile < t1 ? g.W + (size_t)(tok ? tile : 0) * 32 * K
                                   : g.W2 + (size_t)(tile - t1) * 32 * K;
    const uint16_t *tb2 = DUAL ? g.W2 + (size_t)(tok ? tile : 0) * 32 * K : nullptr;
    const uint4 z = {0u, 0u, 0u, 0u};

    // Activation staging with direct global->LDS loads: thread t fills bytes
    // [16t, 16t+16) of a step's 4 KB block, i.e. row br = t/8, slot sw = t%8,
    // with the row's 16-byte chunk sw ^ bswz(br) (the XOR swizzle that makes
    // the B-operand reads conflict-free); rows beyond M and k beyond K read a
    // zero block.  The next group's loads are issued first in each group (the
    // buffer they fill was released by the previous group's barrier), ahead
    // of the weight loads, and waited for at the group's barrier.
    const int br = tid >> 3, bsw = (tid & 7) ^ bswz(br);
    const uint16_t *xrow = g.X + (size_t)(br < g.M ? br : 0) * g.ldx;
    typedef __attribute__((address_space(3))) uint8_t lds_byte;
    auto bissue = [&](int buf, int sf) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = sf + u, k = s * 64 + bsw * 8;
            const bool ok = s < s1 && br < g.M && k < K;
            const void *src = ok ? static_cast<const void *>(xrow + k) : static_cast<const void *>(g.zeros);
            lds_byte *dst = (lds_byte *)(&Bs[buf][u][0]) + wave * 1024;
            __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
        }
    };

    f32x16 acc = {}, acc2 = {};
    if (EPI == EPI_HEAD && tid < kMaxRows * 4) pbits[tid] = 0u;
    if (s0 < s1) bissue(0, s0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int buf = 0;
    for (int sg = s0; sg < s1; sg += U, buf ^= 1) {
        if (sg + U < s1) bissue(buf ^ 1, sg + U);
        uint4 a[U][4], a2[DUAL ? U : 1][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = sg + u;
            const bool full = (nr == 32) && (s * 64 + 64 <= K);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                long off;
                if (s >= s1 || !tok) off = -1;
                else if (full) off = (long)s * 2048 + q * 512 + lane * 8;
                else off = packed_piece(s, q, hf, c, nr, K);
                a[u][q] = off >= 0 ? ld16_stream(tb + off) : z;
                if constexpr (DUAL) a2[u][q] = off >= 0 ? ld16_stream(tb2 + off) : z;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ch = 4 * hf + q;
                const uint4 b = *reinterpret_cast<const uint4 *>(&Bs[buf][u][c * 64 + ((ch ^ bswz(c)) << 3)]);
                acc = mfma32(a[u][q], b, acc);
                if constexpr (DUAL) acc2 = mfma32(a2[u][q], b, acc2);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads into buf^1 have landed
        __syncthreads();
    }

    if (S > 1 || EPI == EPI_PARTIAL) {
        // partial sums, row-contiguous (see psum); columns beyond M stay unwritten
        if (c < g.M) {
            float *mine = g.partial + ((size_t)blockIdx.x * S + ks) * NACC * 4096 + (size_t)c * 128 + wave * 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) mine[acc_row(r, hf)] = acc[r];
            if constexpr (DUAL) {
#pragma unroll
                for (int r = 0; r < 16; ++r) mine[4096 + acc_row(r, hf)] = acc2[r];
            }
        }
        return;
    }
    if constexpr (EPI == EPI_HEAD) {
        // fp32 logits leave through LDS so each row's 128 values are stored as
        // one contiguous 512-byte run (the loop's last barrier freed Bs)
        float *lt = reinterpret_cast<float *>(&Bs[0][0][0]);   // [32 rows][128]
#pragma unroll
        for (int r = 0; r < 16; ++r) lt[c * 128 + wave * 32 + acc_row(r, hf)] = acc[r];
        if (g.mods_on) {
            // each row's path tokens among this workgroup's 128 columns, for
            // the repetition penalty (pbits was cleared before the k loop)
            for (int i = tid; i < g.M * kMaxRows; i += 256) {
                const int mm = i / kMaxRows, j = i % kMaxRows;
                if (j < g.meta->path_len[mm]) {
                    const unsigned col = (unsigned)(g.meta->path_tok[mm * kMaxRows + j] - (int)blockIdx.x * 128);
                    if (col < 128u) atomicOr(&pbits[mm * 4 + (col >> 5)], 1u << (col & 31));
                }
            }
        }
        __syncthreads();
        // one aligned quad of columns per thread and step: store the logits,
        // score them, and reduce row mm's top-2 over the 32 lanes (half a
        // wave) that hold its 128 columns; the lowest lane writes the
        // workgroup's candidates part[mm * rowblocks + rowblock]
        for (int idx = tid; idx < g.M * 32; idx += 256) {
            const int mm = idx >> 5, q4 = idx & 31;
            const int n0 = blockIdx.x * 128 + q4 * 4;
            const float4 v = *reinterpret_cast<const float4 *>(lt + mm * 128 + q4 * 4);
            float *dst = g.Yf + (size_t)mm * g.ldyf + n0;
            if (n0 + 3 < N && (g.ldyf & 3) == 0) {
                // streaming store: the logits are not read again by this pass
                __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4 *>(dst));
            } else {
                if (n0 < N) dst[0] = v.x;
                if (n0 + 1 < N) dst[1] = v.y;
                if (n0 + 2 < N) dst[2] = v.z;
                if (n0 + 3 < N) dst[3] = v.w;
            }
            float sc[4] = {v.x, v.y, v.z, v.w};
            if (g.mods_on && n0 < N)
                score_quad(g.meta, mm, n0, N, (pbits[mm * 4 + (q4 >> 3)] >> ((q4 & 7) * 4)) & 15u, sc);
            float v1 = -INFINITY, v2 = -INFINITY;
            int i1 = 0x7fffffff, i2 = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n0 + j < N) top2_insert(v1, i1, v2, i2, sc[j], n0 + j);
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) {
                const float w1 = __shfl_xor(v1, o), w2 = __shfl_xor(v2, o);
                const int j1 = __shfl_xor(i1, o), j2 = __shfl_xor(i2, o);
                top2_merge(v1, i1, v2, i2, w1, j1, w2, j2);
            }
            if (q4 == 0) g.part[(size_t)mm * gridDim.x + blockIdx.x] = Top2{v1, i1, v2, i2};
        }
    } else {
        if (tok) gemm_epilogue<EPI>(g, tile, lane, acc, acc2);
    }
}

// ------------------------------------------------------------ dense GEMM
// Y[m, n] = sum_k X[m, k] W[n, k] for many activation rows (prefill
// chunks).  The same packed weights and LDS staging as k_gemm, but a
// workgroup covers MG groups of 32 activation rows and each wave reuses its
// weight tile across all of them: each k step carries MG MFMAs per weight
// load.  The grid is one-dimensional and XCD-aware: workgroups are dealt to
// the 8 XCDs in turn, so consecutive ids are renumbered to keep every
// row-tile of a weight block on one XCD, where the block's later reads hit
// that XCD's L2 instead of going back to memory.  No split-K: the grid has
// enough workgroups.
template <int EPI, int MG, int U = 2>   // U: k steps per LDS stage
__global__ __launch_bounds__(256) void k_gemm_dense(GemmArgs g) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][U][MG][32 * 64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, c = lane & 31;
    const int N = g.N, K = g.K;
    const int ntiles = (N + 31) >> 5;
    const int mt = (g.M + 32 * MG - 1) / (32 * MG);       // row tiles
    const int total = gridDim.x, full = total & ~7;
    int w = blockIdx.x;
    if (w < full) w = (w & 7) * (full >> 3) + (w >> 3);   // XCD w%8 takes a contiguous range
    const int wblock = w / mt, mtile = w % mt;
    const int tile = wblock * 4 + wave;
    const bool tok = tile < ntiles;
    const int nr = tok ? min(32, N - tile * 32) : 0;
    const int nsteps = (K + 63) >> 6;
    const int m0 = mtile * 32 * MG;
    const uint16_t *tb = g.W + (size_t)(tok ? tile : 0) * 32 * K;
    const uint16_t *tb2 = DUAL ? g.W2 + (size_t)(tok ? tile : 0) * 32 * K : nullptr;
    const uint4 z = {0u, 0u, 0u, 0u};

    const int br = tid >> 3, bsw = (tid & 7) ^ bswz(br);
    typedef __attribute__((address_space(3))) uint8_t lds_byte;
    auto bissue = [&](int buf, int sf) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int gi = 0; gi < MG; ++gi) {
                const int s = sf + u, k = s * 64 + bsw * 8, row = m0 + gi * 32 + br;
                const bool ok = s < nsteps && row < g.M && k < K;
                const void *src = ok ? static_cast<const void *>(g.X + (size_t)row * g.ldx + k)
                                     : static_cast<const void *>(g.zeros);
                lds_byte *dst = (lds_byte *)(&Bs[buf][u][gi][0]) + wave * 1024;
                __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
            }
        }
    };

    f32x16 acc[MG], acc2[DUAL ? MG : 1];
#pragma unroll
    for (int gi = 0; gi < MG; ++gi) acc[gi] = f32x16{};
    if constexpr (DUAL) {
#pragma unroll
        for (int gi = 0; gi < MG; ++gi) acc2[gi] = f32x16{};
    }
    bissue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int buf = 0;
    for (int sg = 0; sg < nsteps; sg += U, buf ^= 1) {
        if (sg + U < nsteps) bissue(buf ^ 1, sg + U);
        uint4 a[U][4], a2[DUAL ? U : 1][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = sg + u;
            const bool full = (nr == 32) && (s * 64 + 64 <= K);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                long off;
                if (s >= nsteps || !tok) off = -1;
                else if (full) off = (long)s * 2048 + q * 512 + lane * 8;
                else off = packed_piece(s, q, hf, c, nr, K);
                a[u][q] = off >= 0 ? ld16(tb + off) : z;
                if constexpr (DUAL) a2[u][q] = off >= 0 ? ld16(tb2 + off) : z;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ch = 4 * hf + q;
#pragma unroll
                for (int gi = 0; gi < MG; ++gi) {
                    const uint4 b = *reinterpret_cast<const uint4 *>(&Bs[buf][u][gi][c * 64 + ((ch ^ bswz(c)) << 3)]);
                    acc[gi] = mfma32(a[u][q], b, acc[gi]);
                    if constexpr (DUAL) acc2[gi] = mfma32(a2[u][q], b, acc2[gi]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    if (!tok) return;
    // epilogue: accumulators r = 4j..4j+3 hold 4 consecutive output columns;
    // a residual epilogue reads the row group's old values before its first
    // store (else each load waits for the store before it)
#pragma unroll
    for (int gi = 0; gi < MG; ++gi) {
        const int m = m0 + gi * 32 + c;
        if (m >= g.M) continue;
        uint16_t yold[EPI == EPI_RESID ? 4 : 1][4];
        if constexpr (EPI == EPI_RESID) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n0 = tile * 32 + 8 * j + 4 * hf;
#pragma unroll
                for (int e = 0; e < 4; ++e) yold[j][e] = n0 + e < N ? g.Y[(size_t)m * g.ldy + n0 + e] : (uint16_t)0;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n0 = tile * 32 + 8 * j + 4 * hf;
            float v[4], v2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = acc[gi][4 * j + e];
                if constexpr (DUAL) v2[e] = acc2[gi][4 * j + e];
            }
            if constexpr (EPI == EPI_F32) {
                float *y = g.Yf + (size_t)m * g.ldyf + n0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n0 + e < N) y[e] = v[e];
            } else {
                uint16_t *y = g.Y + (size_t)m * g.ldy + n0;
                uint16_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (n0 + e >= N) continue;
                    if constexpr (EPI == EPI_BF16) {
                        o[e] = f2bf(v[e]);
                    } else if constexpr (EPI == EPI_RESID) {
                        o[e] = f2bf(bf2f(yold[j][e]) + bfround(v[e]));
                    } else {
                        const float gt = bfround(v[e]), up = bfround(v2[e]);
                        o[e] = f2bf(gt / (1.0f + expf(-gt)) * up);
                    }
                }
                if (n0 + 3 < N && (g.ldy & 3) == 0) {
                    *reinterpret_cast<uint2 *>(y) = uint2{(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                          (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n0 + e < N) y[e] = o[e];
                }
            }
        }
    }
}

// ------------------------------------------------ dense GEMM, 256 x 256 tiles
// For prefill chunks with enough rows that 256 x 256 tiles give every CU a
// workgroup: a workgroup of 8 waves (two a SIMD) computes a 256 x 256 tile
// (256 activation rows by 256 weight rows; with SwiGLU 128 gate and 128 up
// rows of the same 128 output columns), each wave 128 rows by two weight
// tiles in 8 accumulator tiles, so every weight fragment a wave reads from
// LDS feeds 4 MFMAs and every activation fragment 2 (the 32-row-group
// kernel above re-reads each weight tile from the caches for every 64
// rows).  Both operands reach LDS by direct global-to-LDS loads in stages
// of 32 k (half of a packed 64-k step: its 1 KB q-blocks 0-1, then 2-3),
// three stages in flight ahead of the one in use, each stage in its own LDS
// array so that the compiler can tell a load into one stage from a read of
// another and holds no read back for loads it does not depend on.  Each
// wave waits for its own loads of the next stage before the barrier that
// publishes it.  Every output takes its MFMAs in the same order as in the
// kernel above (steps in order, q-blocks 0..3 within a step, the same
// operand layout), so the two kernels give the same bits.
constexpr int kBigTile = 256;

template <int EPI, int TR>   // TR: activation rows of a workgroup tile (256, 128 or 64)
__device__ __forceinline__ void gemm_big(const GemmArgs &g) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    static_assert(TR == 256 || TR == 128 || TR == 64, "row tile");
    constexpr int RG = TR / 64;           // row groups of 32 a wave
    constexpr int XB = TR / 128 > 0 ? TR / 128 : 1;   // activation loads a wave issues a stage (some fill nothing)
    constexpr int WAIT = 2 * (2 + XB);    // loads of two stages in flight
    // a stage: weight blocks [8 tiles][2 q-blocks], then activation blocks
    // [8 groups of 32 rows][2 q-blocks], 1 KB (64 x 16 bytes) each
    __shared__ __attribute__((aligned(16))) uint4 L0[2048];
    __shared__ __attribute__((aligned(16))) uint4 L1[2048];
    __shared__ __attribute__((aligned(16))) uint4 L2[2048];
    __shared__ __attribute__((aligned(16))) uint4 L3[2048];
    typedef __attribute__((address_space(3))) uint8_t lds_byte;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, c = lane & 31;
    const int K = g.K, M = g.M;
    const int nst = K >> 5;                       // stages of 32 k
    const int mt = (M + TR - 1) / TR;
    const int total = gridDim.x, full = total & ~7;
    int w = blockIdx.x;
    if (w < full) w = (w & 7) * (full >> 3) + (w >> 3);   // XCD w%8 takes a contiguous range
    const int nb = w / mt, m0 = (w % mt) * TR;
    // 8 waves, two a SIMD: wave (wm, wn) takes TR/2 activation rows (row
    // groups RG wm .. RG wm + RG - 1) and two weight tiles: single weights
    // tiles 2wn and 2wn+1; SwiGLU the gate and the up tile of output
    // columns 32wn..+31
    const int wm = wave & 1, wn = wave >> 1;

    // This wave's loads: weight blocks wave + 8i (i < 2) of tile
    // (wave + 8i) / 2, and activation blocks wave + 8i (i < XB) of row group
    // (wave + 8i) / 2 (with TR = 64 the waves past its 4 blocks load zeros
    // into the unused rest of the stage, so every wave issues the same
    // count); q-block half wave % 2.  Stage st reads bytes
    // 2 KB * st on of a weight tile's packed rows, and k = 64 (st / 2) +
    // 16 (st % 2) on of an activation row (lanes 32-63 four 16-byte chunks
    // further).
    const int qh = wave & 1;
    const uint16_t *wsrc[2];
    const uint16_t *xsrc[XB];
    bool xok[XB];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = (wave + 8 * i) >> 1;
        const uint16_t *tb;
        if constexpr (DUAL) tb = t < 4 ? g.W + (size_t)(4 * nb + t) * 32 * K : g.W2 + (size_t)(4 * nb + t - 4) * 32 * K;
        else tb = g.W + (size_t)(8 * nb + t) * 32 * K;
        wsrc[i] = tb + qh * 512 + lane * 8;
    }
#pragma unroll
    for (int i = 0; i < XB; ++i) {
        const int grp = (wave + 8 * i) >> 1;
        const int row = m0 + grp * 32 + c;
        xok[i] = grp < TR / 32 && row < M;
        xsrc[i] = g.X + (size_t)(xok[i] ? row : 0) * g.ldx + hf * 32 + qh * 8;
    }
    auto issue = [&](int st, uint4 *buf) {
        const bool live = st < nst;   // past the end: zeros into a free stage, so every wait count holds
        const size_t wo = (size_t)st * 1024;   // step st/2, q-blocks 2(st%2) + half: st KB of the tile
        const int xo = (st >> 1) * 64 + (st & 1) * 16;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds(live ? static_cast<const void *>(wsrc[i] + wo) : g.zeros,
                                             (lds_byte *)buf + (wave + 8 * i) * 1024, 16, 0, 0);
#pragma unroll
        for (int i = 0; i < XB; ++i)
            __builtin_amdgcn_global_load_lds(live && xok[i] ? static_cast<const void *>(xsrc[i] + xo) : g.zeros,
                                             (lds_byte *)buf + 16384 + (wave + 8 * i) * 1024, 16, 0, 0);
    };

    f32x16 acc[2][RG];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < RG; ++r) acc[j][r] = f32x16{};
    // the wave's two weight tiles among the 8 staged
    auto wtile = [&](int j) { return DUAL ? 4 * j + wn : 2 * wn + j; };
    auto compute = [&](const uint4 *buf) {
        // every operand of the stage is read first (12 reads in flight), so
        // the products start as soon as the first ones land
        uint4 a[2][2], b[2][RG];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int j = 0; j < 2; ++j) a[q][j] = buf[(wtile(j) * 2 + q) * 64 + lane];
#pragma unroll
            for (int r = 0; r < RG; ++r) b[q][r] = buf[1024 + ((RG * wm + r) * 2 + q) * 64 + lane];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < RG; ++r) acc[j][r] = mfma32(a[q][j], b[q][r], acc[j][r]);
    };
    // wait until at most n of this wave's loads are in flight (vmcnt only)
    auto wait_loads = [&](auto n) {
        constexpr int v = decltype(n)::value;
        __builtin_amdgcn_s_waitcnt((v & 15) | ((v >> 4) << 14) | (0x7 << 4) | (0xf << 8));
    };
    auto publish = [&]() {
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto body = [&](int st, const uint4 *cur, uint4 *nxt) {
        issue(st + 3, nxt);
        compute(cur);
        wait_loads(std::integral_constant<int, WAIT>{});   // stage st+1 landed; st+2, st+3 in flight
        publish();
    };
    issue(0, L0);
    issue(1, L1);
    issue(2, L2);
    wait_loads(std::integral_constant<int, WAIT>{});
    publish();
    for (int st = 0; st < nst; st += 4) {   // nst is a multiple of 4
        body(st, L0, L3);
        body(st + 1, L1, L0);
        body(st + 2, L2, L1);
        body(st + 3, L3, L2);
    }
    wait_loads(std::integral_constant<int, 0>{});

    // epilogue: accumulators r = 4jj..4jj+3 of tile (j, rg) hold 4
    // consecutive output columns of activation row m.  A residual epilogue
    // reads the row group's old values before its first store (in program
    // order a store could alias the next load, so the compiler would wait
    // out each load in turn)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int m = m0 + (RG * wm + rg) * 32 + c;
        if (m >= M) continue;
        uint2 oldv[DUAL ? 1 : 2][4];
        if constexpr (EPI == EPI_RESID) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tile = 8 * nb + 2 * wn + j;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    oldv[j][jj] = *reinterpret_cast<const uint2 *>(g.Y + (size_t)m * g.ldy + tile * 32 + 8 * jj + 4 * hf);
            }
        }
#pragma unroll
        for (int j = 0; j < (DUAL ? 1 : 2); ++j) {
            const int tile = DUAL ? 4 * nb + wn : 8 * nb + 2 * wn + j;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int n0 = tile * 32 + 8 * jj + 4 * hf;
                float v[4], v2[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[j][rg][4 * jj + e];
                    v2[e] = DUAL ? acc[1][rg][4 * jj + e] : 0.f;
                }
                if constexpr (EPI == EPI_F32) {
                    *reinterpret_cast<float4 *>(g.Yf + (size_t)m * g.ldyf + n0) = float4{v[0], v[1], v[2], v[3]};
                } else {
                    uint16_t *y = g.Y + (size_t)m * g.ldy + n0;
                    uint16_t o[4];
                    if constexpr (EPI == EPI_RESID) {
                        const uint2 old = oldv[DUAL ? 0 : j][jj];
                        const uint16_t yo[4] = {(uint16_t)(old.x & 0xffffu), (uint16_t)(old.x >> 16),
                                                (uint16_t)(old.y & 0xffffu), (uint16_t)(old.y >> 16)};
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[e] = f2bf(bf2f(yo[e]) + bfround(v[e]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if constexpr (EPI == EPI_BF16) {
                                o[e] = f2bf(v[e]);
                            } else {
                                const float gt = bfround(v[e]), up = bfround(v2[e]);
                                o[e] = f2bf(gt / (1.0f + expf(-gt)) * up);
                            }
                        }
                    }
                    *reinterpret_cast<uint2 *>(y) = uint2{(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                          (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
                }
            }
        }
    }
}

// One kernel per row-tile height (the body above, instantiated three ways).
template <int EPI>
__global__ __launch_bounds__(512) void k_gemm_big256(GemmArgs g) { gemm_big<EPI, 256>(g); }
template <int EPI>
__global__ __launch_bounds__(512) void k_gemm_big128(GemmArgs g) { gemm_big<EPI, 128>(g); }
template <int EPI>
__global__ __launch_bounds__(512) void k_gemm_big64(GemmArgs g) { gemm_big<EPI, 64>(g); }

// Split-K finish: one thread per output element adds its S partials in
// k-range order and applies the element's epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_reduce(GemmArgs g, int S) {
    constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;   // (rb*32 + m)*128 + nl
    const int nl = (int)(idx & 127), m = (int)((idx >> 7) & 31);
    const int n = (int)((idx >> 12) * 128) + nl;
    if (m >= g.M || n >= g.N) return;
    float sums[NACC];
    if constexpr (NACC == 2) {
        const float *const pp[2] = {pptr(g.partial, S, 2, 0, m, n), pptr(g.partial, S, 2, 1, m, n)};
        psum_multi<2>(pp, 2 * 4096, S, sums);
    } else {
        const float *const pp[1] = {pptr(g.partial, S, 1, 0, m, n)};
        psum_multi<1>(pp, 4096, S, sums);
    }
    const float acc = sums[0];
    uint16_t *y = g.Y + (size_t)m * g.ldy + n;
    if constexpr (EPI == EPI_BF16) {
        *y = f2bf(acc);
    } else if constexpr (EPI == EPI_RESID) {
        *y = f2bf(bf2f(*y) + bfround(acc));
    } else if constexpr (EPI == EPI_SWIGLU) {
        const float gt = bfround(acc), up = bfround(sums[NACC - 1]);
        *y = f2bf(gt / (1.0f + expf(-gt)) * up);
    }
}

// In-place repack of a row-major [N, K] bf16 matrix into the packed tile
// order read by k_gemm.  `src` holds a row-major copy of tiles [t0, t0+nt).
__global__ __launch_bounds__(256) void k_pack(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst,
                                              int N, int K, int t0, int nt) {
    const int nsteps = (K + 63) >> 6;
    const long pieces = (long)nt * nsteps * 8 * 32;
    for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < pieces; i += (long)gridDim.x * blockDim.x) {
        const int c = (int)(i & 31);
        const long j = i >> 5;
        const int pi = (int)(j & 7);
        const long j2 = j >> 3;
        const int s = (int)(j2 % nsteps);
        const int tl = (int)(j2 / nsteps);
        const int tile = t0 + tl;
        const int nr = min(32, N - tile * 32);
        const int q = pi >> 1, hf = pi & 1;
        const long off = packed_piece(s, q, hf, c, nr, K);
        if (off < 0) continue;
        const uint4 v = ld16(src + ((size_t)tl * 32 + c) * K + s * 64 + 32 * hf + 8 * q);
        *reinterpret_cast<uint4 *>(dst + (size_t)tile * 32 * K + off) = v;
    }
}

// ------------------------------------------------------------- top-2 reduce
// One workgroup per row merges the per-tile candidates; the result is a
// selection under a strict order, so it does not depend on the merge order.

__global__ __launch_bounds__(256) void k_top2_reduce(const Top2 *__restrict__ part, int ntiles,
                                                     RowResult *__restrict__ res) {
    // top-2 selection is order-free (ties go to the lower id), so the
    // candidates may be merged in any grouping
    __shared__ Top2 sh[4];
    const int m = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float v1 = -INFINITY, v2 = -INFINITY;
    int i1 = 0x7fffffff, i2 = 0x7fffffff;
    const Top2 *row = part + (size_t)m * ntiles;
    for (int base = 0; base < ntiles; base += 8 * 256) {   // eight loads in flight per thread
        float4 p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = base + i * 256 + t;
            p[i] = idx < ntiles ? *reinterpret_cast<const float4 *>(row + idx)
                                : float4{-INFINITY, __int_as_float(0x7fffffff), -INFINITY, __int_as_float(0x7fffffff)};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            top2_merge(v1, i1, v2, i2, p[i].x, __float_as_int(p[i].y), p[i].z, __float_as_int(p[i].w));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float w1 = __shfl_xor(v1, o), w2 = __shfl_xor(v2, o);
        const int j1 = __shfl_xor(i1, o), j2 = __shfl_xor(i2, o);
        top2_merge(v1, i1, v2, i2, w1, j1, w2, j2);
    }
    if (lane == 0) sh[wave] = Top2{v1, i1, v2, i2};
    __syncthreads();
    if (t == 0) {
        Top2 r = sh[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) top2_merge(r.v1, r.i1, r.v2, r.i2, sh[w].v1, sh[w].i1, sh[w].v2, sh[w].i2);
        // gap in bf16 ulps of top-1: ulp(x) = 2^(floor(log2|x|) - 7), or
        // 2^-133 below the normal range; the difference of two fp32 values
        // is exact in fp64.
        float g;
        if (r.v2 == -INFINITY) {
            g = INFINITY;
        } else {
            const uint32_t e = (__float_as_uint(r.v1) >> 23) & 0xffu;
            const int ex = (e == 0) ? -126 : (int)e - 127;
            g = (float)(((double)r.v1 - (double)r.v2) / ldexp(1.0, ex - 7));
        }
        // argmax and gap leave together in one 8-byte store
        *reinterpret_cast<volatile uint64_t *>(res + m) =
            ((uint64_t)__float_as_uint(g) << 32) | (uint64_t)(uint32_t)r.i1;
    }
}

// ------------------------------------------------- residual tree sampling
// Per verified row: the decision of deterministic-candidate residual
// sampling ("Algorithm and correctness contract", Deterministic tree
// candidates and residual verification) with the row's uniform u.  Its
// candidates are the row's children in index order; the target is the
// softmax of the row's modified scores over T.  One uniform per node: the
// first position, over (candidates, then every other id ascending), where
// the running sum of the weights w = exp(s/T - max) exceeds u times their
// total; fp64 weights and sums.  The result is written to pinned host memory
// as the argmax field of the row's record: -(j+1) to accept candidate j,
// else the emitted token.
//
// Two kernels.  k_residual_chunks spreads each row over chunks of
// kResChunk ids (one workgroup each, 16 consecutive ids a thread): the
// chunk's maximum m_c and the sum s_c of exp(x - m_c) over its non-candidate
// ids.  k_residual_decide (one workgroup a row) takes the row's maximum M,
// weighs the chunks by s_c exp(m_c - M), walks the candidates, then the
// chunks, then the crossing chunk's per-thread sums and ids.

constexpr int kResChunk = 4096, kResThreads = 256, kResPer = kResChunk / kResThreads;
constexpr int kResMaxChunks = 64;   // V <= 2^18

struct ResPart {
    double m, s;
};

// The chunk's path tokens (the repetition penalty's prior ids besides the
// history) and the row's candidate tokens as bit masks over the chunk's ids.
__device__ __forceinline__ void res_masks(const PassMeta *meta, int i, int n, int c0, uint32_t *pmask,
                                          uint32_t *cmask) {
    const int t = threadIdx.x;
    if (t < kResChunk / 32) pmask[t] = cmask[t] = 0u;
    __syncthreads();
    const HeadMods &md = meta->mods[meta->row_req[i]];
    if (md.rep != 1.0f && t < meta->path_len[i]) {
        const unsigned v = (unsigned)(meta->path_tok[i * kMaxRows + t] - c0);
        if (v < (unsigned)kResChunk) atomicOr(&pmask[v >> 5], 1u << (v & 31));
    }
    if (t > i && t < n && meta->depth[t] == meta->depth[i] + 1 && ((meta->anc[t] >> i) & 1u)) {
        const unsigned v = (unsigned)(meta->tok[t] - c0);
        if (v < (unsigned)kResChunk) atomicOr(&cmask[v >> 5], 1u << (v & 31));
    }
    __syncthreads();
}

// modified score over T (fp64: times 1/T, within an ulp of the quotient) of
// id v with its raw logit s; -inf if masked
__device__ __forceinline__ double res_score(float s, int v, const HeadMods &md, bool in_path, double invT) {
    if (md.rep != 1.0f) {
        const bool prior = in_path || (md.hist_bits && ((md.hist_bits[v >> 5] >> (v & 31)) & 1u));
        if (prior) s = s > 0.f ? s / md.rep : s * md.rep;
    }
    if (md.bias) s = s + md.bias[v];
    if (md.allow_bits && !((md.allow_bits[v >> 5] >> (v & 31)) & 1u)) s = -INFINITY;
    return (double)s * invT;
}

__global__ __launch_bounds__(kResThreads) void k_residual_chunks(const float *__restrict__ logits, int ldl, int V,
                                                                 const PassMeta *__restrict__ meta, int n, float T,
                                                                 ResPart *__restrict__ parts) {
    __shared__ uint32_t pmask[kResChunk / 32], cmask[kResChunk / 32];
    __shared__ double red[kResThreads / 64];
    const int c = blockIdx.x, i = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int c0 = c * kResChunk;
    const double invT = 1.0 / (double)T;
    res_masks(meta, i, n, c0, pmask, cmask);
    const HeadMods &md = meta->mods[meta->row_req[i]];
    const float *row = logits + (size_t)i * ldl;
    double x[kResPer];
    double mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kResPer; ++k) {
        const int o = t * kResPer + k, v = c0 + o;
        x[k] = v < V ? res_score(row[v], v, md, (pmask[o >> 5] >> (o & 31)) & 1u, invT) : -INFINITY;
        mx = fmax(mx, x[k]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < kResThreads / 64; ++w) mx = fmax(mx, red[w]);
    __syncthreads();
    double sum = 0.0;   // ascending ids, candidates apart
#pragma unroll
    for (int k = 0; k < kResPer; ++k) {
        const int o = t * kResPer + k;
        if (x[k] != -INFINITY && !((cmask[o >> 5] >> (o & 31)) & 1u)) sum += exp(x[k] - mx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    if (t == 0) {
        double tot = 0.0;
        for (int w = 0; w < kResThreads / 64; ++w) tot += red[w];
        parts[(size_t)i * gridDim.x + c] = ResPart{mx, tot};
    }
}

// inclusive prefix sum over the 64 lanes of a wave (a fixed order of adds)
__device__ __forceinline__ double wave_prefix(double x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

__global__ __launch_bounds__(kResThreads) void k_residual_decide(const float *__restrict__ logits, int ldl, int V,
                                                                 const PassMeta *__restrict__ meta, int n, float T,
                                                                 const double *__restrict__ u_row,
                                                                 const ResPart *__restrict__ parts, int nchunks,
                                                                 RowResult *res) {
    __shared__ uint32_t pmask[kResChunk / 32], cmask[kResChunk / 32];
    __shared__ double seg[kResThreads];
    __shared__ int lastv[kResThreads];
    __shared__ double wts[kResChunk];   // the crossing chunk's weights (0 for candidates and masked ids)
    __shared__ double W[kResMaxChunks], mc[kResMaxChunks], candw[kMaxRows];   // chunk and candidate weights
    __shared__ double sh_M, sh_r;
    __shared__ int sh_chunk, sh_out;
    const int i = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const HeadMods &md = meta->mods[meta->row_req[i]];
    const float *row = logits + (size_t)i * ldl;
    const ResPart *pr = parts + (size_t)i * nchunks;
    const double invT = 1.0 / (double)T;
    // candidates: node t is a child of row i (children in index order)
    const bool is_cand = t > i && t < n && meta->depth[t] == meta->depth[i] + 1 && ((meta->anc[t] >> i) & 1u);
    if (wave == 0) {   // the row's maximum over its chunks
        double m = lane < nchunks ? pr[lane].m : -INFINITY;
        if (lane < nchunks) mc[lane] = m;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
        if (lane == 0) sh_M = m;
    }
    __syncthreads();
    const double M = sh_M;
    if (t < nchunks) W[t] = mc[t] == -INFINITY ? 0.0 : pr[t].s * exp(mc[t] - M);
    if (t < kMaxRows) candw[t] = 0.0;
    if (is_cand) {
        const int v = meta->tok[t];
        bool in_path = false;
        if (md.rep != 1.0f)
            for (int q = 0; q < meta->path_len[i]; ++q) in_path |= meta->path_tok[i * kMaxRows + q] == v;
        const double xv = res_score(row[v], v, md, in_path, invT);
        candw[t] = xv == -INFINITY ? 0.0 : exp(xv - M);
    }
    __syncthreads();
    if (wave == 0) {
        // running sums over the candidates (lane j: node j) and the chunks (lane c)
        const uint64_t cmaskl = __ballot(is_cand);   // wave 0 holds nodes 0..63: every candidate
        const double pc = wave_prefix(lane < kMaxRows ? candw[lane] : 0.0, lane);
        const double pw = wave_prefix(lane < nchunks ? W[lane] : 0.0, lane);
        const double csum = __shfl(pc, 63), rest = __shfl(pw, 63);
        const double thr = u_row[i] * (csum + rest);
        int out = INT_MIN, chunk = -1;
        double r = 0.0;
        const uint64_t hitc = __ballot(pc > thr);   // the first crossing lane is a candidate's
        if (hitc) {
            const int j = __ffsll((unsigned long long)hitc) - 1;
            out = -(__popcll(cmaskl & ((1ull << j) - 1ull)) + 1);
        } else {
            r = thr - csum;
            const uint64_t hitw = __ballot(lane < nchunks && pw > r);
            if (hitw) {
                chunk = __ffsll((unsigned long long)hitw) - 1;
                const double before = __shfl(pw, chunk > 0 ? chunk - 1 : 0);
                r -= chunk > 0 ? before : 0.0;
            } else {   // rounding at the very end: the last chunk with weight, past its end
                const uint64_t pos = __ballot(lane < nchunks && W[lane] > 0.0);
                chunk = pos ? 63 - __clzll((unsigned long long)pos) : -1;
                r = INFINITY;
            }
        }
        if (lane == 0) {
            sh_r = r;
            sh_chunk = chunk;
            sh_out = out;
        }
    }
    __syncthreads();
    const int chunk = sh_chunk;
    if (sh_out == INT_MIN && chunk >= 0) {
        const int c0 = chunk * kResChunk;
        res_masks(meta, i, n, c0, pmask, cmask);
        double sum = 0.0;
        int last = -1;
#pragma unroll
        for (int k = 0; k < kResPer; ++k) {
            const int o = t * kResPer + k, v = c0 + o;
            double w = 0.0;
            if (v < V && !((cmask[o >> 5] >> (o & 31)) & 1u)) {
                const double xv = res_score(row[v], v, md, (pmask[o >> 5] >> (o & 31)) & 1u, invT);
                if (xv != -INFINITY) w = exp(xv - M);
            }
            wts[o] = w;
            sum += w;
            if (w > 0.0) last = v;
        }
        seg[t] = sum;
        lastv[t] = last;
        __syncthreads();
        if (wave == 0) {
            // lane l takes the sums of threads 4l..4l+3 (in order); the first
            // lane whose running sum exceeds r holds the crossing thread
            const double r = sh_r;
            double a[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) a[k] = seg[4 * lane + k];
            const double loc = ((a[0] + a[1]) + a[2]) + a[3];
            const double pre = wave_prefix(loc, lane);
            const double up = __shfl_up(pre, 1);   // every lane takes part in the shuffle
            const double excl = lane > 0 ? up : 0.0;
            const uint64_t hit = __ballot(pre > r);
            int out = -1;
            if (hit) {
                const int L = __ffsll((unsigned long long)hit) - 1;
                if (lane == L) {
                    double rr = r - excl;
                    for (int k = 0; k < 4 && out < 0; ++k) {
                        if (a[k] > rr) {
                            const int tt = 4 * lane + k;   // the crossing thread: walk its ids
                            for (int q = 0; q < kResPer && out < 0; ++q) {
                                const double w = wts[tt * kResPer + q];
                                if (w == 0.0) continue;   // candidates, masked ids, ids past V
                                if (w > rr) out = c0 + tt * kResPer + q;
                                else rr -= w;
                            }
                            if (out < 0) out = lastv[tt];   // rounding inside the thread's ids
                        } else {
                            rr -= a[k];
                        }
                    }
                }
                out = __shfl(out, L);
            }
            if (out < 0) {   // rounding: the chunk's last id with weight
                int lv = -1;
#pragma unroll
                for (int k = 0; k < 4; ++k) lv = lastv[4 * lane + k] >= 0 ? lastv[4 * lane + k] : lv;
                const uint64_t has = __ballot(lv >= 0);
                out = has ? __shfl(lv, 63 - __clzll((unsigned long long)has)) : -1;
            }
            if (lane == 0) sh_out = out;
        }
        __syncthreads();
    }
    if (t == 0) {
        int out = sh_out;
        if (out == INT_MIN) out = -1;   // nothing carries weight (every id masked): the first candidate's slot
        // one 8-byte store: the decision, and gap bits 0 (not the empty pattern) to mark the record done
        *reinterpret_cast<volatile uint64_t *>(res + i) = (uint64_t)(uint32_t)out;
    }
}

// ------------------------------------------------------------- RoPE + KV
// Rotate q and k of each tree node at position ctx + depth (rotate-half
// pairs (i, i + D/2)); k and v go to cache slot ctx + node index ("Drafters
// and tree verify", Tree verify through recurrent layers: position = depth,
// every node at its depth-first slot).

// Grid (row of the pass, slice): thread u of a row handles one q pair, one
// k pair or one v element: units [0, QH*D/2) q, then KVH*D/2 k, then KVH*D
// v.  Every request of the pass is served by the one launch: a row finds its
// request (rows are in request order) and writes that request's cache.
__global__ __launch_bounds__(256) void k_rope_kv(RopeArgs a) {
    const int m = blockIdx.x;
    int r = 0;
    while (r + 1 < a.nreq && m >= a.rq[r + 1].row0) ++r;
    const PassReq &rq = a.rq[r];
    const int i = m - rq.row0;   // node index within its request
    const int D = a.D, half = D / 2;
    const int u = blockIdx.y * 256 + threadIdx.x;
    const int nq = a.QH * half, nk = a.KVH * half, nv = a.KVH * D;
    if (u >= nq + nk + nv) return;
    const int pos = rq.ctx + a.meta->depth[m];
    // projection outputs: bf16 of the partial sums (the QKV projection's rounding point)
    const size_t slot = (size_t)(rq.ctx + i);
    if (u < nq + nk) {
        const bool isq = u < nq;
        const int uu = isq ? u : u - nq;
        const int h = uu / half, p = uu % half;
        const int col = (isq ? 0 : a.QH * D) + h * D + p;
        const float *const pp[2] = {pptr(a.part, a.S, 1, 0, m, col), pptr(a.part, a.S, 1, 0, m, col + half)};
        float xs[2];
        psum_multi<2>(pp, 4096, a.S, xs);
        const float x0 = bfround(xs[0]), x1 = bfround(xs[1]);
        const float c = a.cosT[(size_t)pos * half + p], s = a.sinT[(size_t)pos * half + p];
        uint16_t *o = isq ? a.q_out + (size_t)m * a.QH * D + h * D : rq.Kc + ((size_t)h * a.cap + slot) * D;
        o[p] = f2bf(x0 * c - x1 * s);
        o[p + half] = f2bf(x1 * c + x0 * s);
    } else {
        const int uu = u - nq - nk, h = uu / D, d = uu % D;
        const float *const pp[1] = {pptr(a.part, a.S, 1, 0, m, (a.QH + a.KVH) * D + h * D + d)};
        float xs[1];
        psum_multi<1>(pp, 4096, a.S, xs);
        rq.Vc[((size_t)h * a.cap + slot) * D + d] = f2bf(bfround(xs[0]));
    }
}

// Prefill RoPE: the same rotation on the dense QKV projection's bf16
// output; row i of the chunk is at position and cache slot pos0 + i.
__global__ __launch_bounds__(256) void k_rope_dense(const uint16_t *__restrict__ qkv, int ldq, int pos0, int QH,
                                                    int KVH, int D, const float *__restrict__ cosT,
                                                    const float *__restrict__ sinT, uint16_t *__restrict__ q_out,
                                                    uint16_t *__restrict__ Kc, uint16_t *__restrict__ Vc, int cap) {
    const int i = blockIdx.x, half = D / 2;
    const int u = blockIdx.y * 256 + threadIdx.x;
    const int nq = QH * half, nk = KVH * half, nv = KVH * D;
    if (u >= nq + nk + nv) return;
    const int pos = pos0 + i;
    const uint16_t *x = qkv + (size_t)i * ldq;
    if (u < nq + nk) {
        const bool isq = u < nq;
        const int uu = isq ? u : u - nq;
        const int h = uu / half, p = uu % half;
        const int col = (isq ? 0 : QH * D) + h * D + p;
        const float x0 = bf2f(x[col]), x1 = bf2f(x[col + half]);
        const float c = cosT[(size_t)pos * half + p], s = sinT[(size_t)pos * half + p];
        uint16_t *o = isq ? q_out + (size_t)i * QH * D + h * D : Kc + ((size_t)h * cap + pos) * D;
        o[p] = f2bf(x0 * c - x1 * s);
        o[p + half] = f2bf(x1 * c + x0 * s);
    } else {
        const int uu = u - nq - nk, h = uu / D, d = uu % D;
        Vc[((size_t)h * cap + pos) * D + d] = x[(QH + KVH) * D + h * D + d];
    }
}

// Prefill RMSNorm of M rows (one workgroup per row, one thread per 8
// columns, the same fixed reduction order as k_row_norm); with `tok` the
// rows are first gathered from the embedding into X.
__global__ __launch_bounds__(1024) void k_norm_dense(const int32_t *__restrict__ tok, const uint16_t *__restrict__ emb,
                                                     uint16_t *X, const uint16_t *__restrict__ w, float eps,
                                                     uint16_t *__restrict__ Y, int H) {
    __shared__ float red[16];
    const int m = blockIdx.x, t = threadIdx.x, n0 = 8 * t;
    const bool ok = n0 < H;
    const uint4 zz = {0u, 0u, 0u, 0u};
    uint4 v;
    if (tok) {
        v = ok ? ld16(emb + (size_t)tok[m] * H + n0) : zz;
        if (ok) *reinterpret_cast<uint4 *>(X + (size_t)m * H + n0) = v;
    } else {
        v = ok ? ld16(X + (size_t)m * H + n0) : zz;
    }
    const uint4 wv = ok ? ld16(w + n0) : zz;
    const uint16_t *ve = reinterpret_cast<const uint16_t *>(&v);
    float x[8], ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = bf2f(ve[e]);
        ss += x[e] * x[e];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += red[i];
    const float scale = 1.0f / sqrtf(tot / (float)H + eps);
    if (!ok) return;
    const uint16_t *we = reinterpret_cast<const uint16_t *>(&wv);
    uint32_t yw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) yw[e] = f2bf2(x[2 * e] * scale * bf2f(we[2 * e]), x[2 * e + 1] * scale * bf2f(we[2 * e + 1]));
    *reinterpret_cast<uint4 *>(Y + (size_t)m * H + n0) = uint4{yw[0], yw[1], yw[2], yw[3]};
}

// ---------------------------------------------------------- tree attention
// Workgroup barrier that orders LDS only: global loads a wave has in flight
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Grid (split, kv head); one wave per block of 32 query rows, where row
// r = node*G + head-in-group.  Splits 0..n_ctx_split-1 each take `span`
// cache keys (visible to every row); the last split takes the tree's own
// keys at slots ctx..ctx+n-1, key j visible to node t iff j is t or an
// ancestor of t ("Drafters and tree verify", Tree verify through recurrent
// layers: attention gets a mask of the node's ancestors).
//
// Scores are computed transposed, S^T = K Q^T, on MFMA (A = 32 keys from
// LDS, B = the wave's 32 query rows kept in registers), so every lane owns
// one query row: the online-softmax max, sum and rescale stay in the lane
// (plus its partner lane^32).  P^T then feeds O^T = V^T P^T directly from
// registers: the k slots of each 16-key step are permuted to the keys the
// lane already holds, and V^T is staged in LDS with the same order.  P is
// split into bf16 high and low parts (two MFMAs) so P.V keeps ~16 bits of P.
// The softmax runs in base 2 (scores times scale * log2 e, exp2).  When a
// split spans several 64-key chunks, the workgroup's other waves (up to 8 in
// all) stage the next chunk into the second LDS buffer while the compute
// waves use the first.
// With DS = 2 two waves share a block of 32 rows, each forming the scores
// and probabilities of all the block's keys but only half of the output
// dims (the products of P with V are the largest share of a chunk's work);
// every output value takes the same operations in the same order either way.
// Each workgroup writes its unnormalised partial (max in base-2 units, sum,
// output); the combine kernel merges splits in index order.  Split
// boundaries depend only on ctx, so a row's result does not depend on the
// other rows.

template <int D, int DS>
__global__ __launch_bounds__(64 * kAttnWaves) void k_attn(AttnArgs a) {
    constexpr int CH = kAttnChunk;     // keys per LDS stage
    constexpr int KC = D / 8;          // 16-byte chunks per key row
    constexpr int VSTR = CH + 4;       // bf16 stride of a transposed V row
    constexpr int NDB = D / 32 / DS;   // output dim blocks of one wave
    static_assert(DS == 1 || DS == 2, "one or two waves per block of rows");
    constexpr int NKK = D / 16;        // dim steps of the score MFMA
    // two LDS stages: while the compute waves use one, the loader waves fill
    // the other with the next chunk of keys
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][CH * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VSTR];

    const int split = blockIdx.x, kvh = blockIdx.y, z = blockIdx.z;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, c = lane & 31;
    const int G = a.G;
    // this block's rows, context, splits and cache (a prefill block of a
    // chain, or one request's tree in a verify pass)
    int n = a.n, row0 = a.row0, ctx = a.ctx, span = a.span, nsplit = a.n_ctx_split;
    const uint16_t *Kc = a.Kc, *Vc = a.Vc;
    if (a.nreq > 0) {
        const PassReq &rq = a.rq[z];
        n = rq.n;
        row0 = rq.row0;
        ctx = rq.ctx;
        span = rq.span;
        nsplit = rq.nsplit;
        Kc = rq.Kc;
        Vc = rq.Vc;
        if (split > nsplit) return;            // a request with fewer splits: the whole workgroup leaves
    } else if (a.zrows > 0) {
        row0 = z * a.zrows;
        n = min(a.zrows, a.M - row0);
        ctx = a.ctx + row0;
        span = attn_span_n(ctx, a.ztarget);
        nsplit = (ctx + span - 1) / span;
        if (split > nsplit) return;            // a block with fewer splits: the whole workgroup leaves
    }
    const int R = G * n;
    const int cw = ((R + 31) >> 5) * DS;       // compute waves; any further waves only load
    const int rbi = wave / DS;                 // the wave's block of 32 rows
    const int db0 = (wave % DS) * NDB;         // and its first output dim block
    const bool loaders = nthr > cw * 64;
    const bool tree = split >= nsplit;
    const int key0 = tree ? ctx : split * span;
    const int nkeys = tree ? n : min(span, ctx - key0);
    const int nch = (nkeys + CH - 1) / CH;
    const int row = rbi * 32 + c;              // this lane's query row (compute waves)
    const bool rowok = wave < cw && row < R;
    const int t = rowok ? row / G : 0, hh = rowok ? row % G : 0;
    // keys of the block's own rows visible to row t: its ancestors and itself
    // (a prefill chain: rows 0..t)
    const uint32_t anc = a.zrows > 0 ? (t >= 31 ? 0xffffffffu : ((2u << t) - 1u)) : a.meta->anc[row0 + t];

    const uint16_t *Kb = Kc + (size_t)kvh * a.cap * D;
    const uint16_t *Vb = Vc + (size_t)kvh * a.cap * D;
    // stage the chunk of keys starting at c0 into buffer buf, by threads
    // [0, nt) of a group (tg = this thread's index in it).  Task j loads
    // pieces 2j and 2j+1 of K (consecutive tasks read consecutive 32 bytes)
    // and piece j / NPAIR of the key pair j % NPAIR of V: the key pair runs
    // fastest, so each transposed V store is one dword holding two keys of
    // one dimension and a half-wave's stores fall in distinct banks.  Every
    // load of a pass (TB tasks per thread) is issued before any store.
    constexpr int NPAIR = CH / 2;
    constexpr int NTASK = NPAIR * KC;
    constexpr int TB = 2;
    // A pass is split in two: the loads of up to T tasks per thread (tasks
    // base + i * nt + tg) into registers, then their stores.  The loads are
    // unconditional (a task or key past the end reads the last valid one)
    // so that the compiler's count of loads in flight stays exact; the
    // stores write zeros for keys past the end.
    auto load_pass = [&](int c0, int base, int tg, int nt, auto &kv, auto &vv) {
        constexpr int T = sizeof(kv) / sizeof(kv[0]);
        // a chunk past the split's end (a loader's idle slot) reads the
        // split's first key over and over: cache hits, and the same count
        // of loads in flight on every path
        const bool live = c0 < nkeys;
        const int cn = live ? min(CH, nkeys - c0) : 1;
        if (!live) c0 = 0;
        const uint16_t *kb = Kb + (size_t)(key0 + c0) * D, *vb = Vb + (size_t)(key0 + c0) * D;
#pragma unroll
        for (int i = 0; i < T; ++i) {
            const int j = min(base + i * nt + tg, NTASK - 1);
            const int kk = min((2 * j) / KC, cn - 1), p = (2 * j) % KC;
            const int kp = j % NPAIR, pv = j / NPAIR;
            kv[i][0] = ld16(kb + (size_t)kk * D + p * 8);
            kv[i][1] = ld16(kb + (size_t)kk * D + p * 8 + 8);
            vv[i][0] = ld16(vb + (size_t)min(2 * kp, cn - 1) * D + pv * 8);
            vv[i][1] = ld16(vb + (size_t)min(2 * kp + 1, cn - 1) * D + pv * 8);
        }
    };
    auto store_pass = [&](int c0, int buf, int base, int tg, int nt, const auto &kv, const auto &vv) {
        constexpr int T = sizeof(kv) / sizeof(kv[0]);
        const int cn = min(CH, nkeys - c0);
#pragma unroll
        for (int i = 0; i < T; ++i) {
            const int j = base + i * nt + tg;
            if (j < NTASK) {
                const int kk = (2 * j) / KC, p = (2 * j) % KC;
                const int kp = j % NPAIR, pv = j / NPAIR;
                // keys past the end are stored as zeros (masks on the values)
                const uint32_t mk = kk < cn ? ~0u : 0u, m0 = 2 * kp < cn ? ~0u : 0u, m1 = 2 * kp + 1 < cn ? ~0u : 0u;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint4 k4 = kv[i][h];
                    *reinterpret_cast<uint4 *>(Ks[buf] + kk * D + (((p + h) ^ (kk & (KC - 1))) << 3)) =
                        uint4{k4.x & mk, k4.y & mk, k4.z & mk, k4.w & mk};
                }
                // dim pv*8 + e of keys 2kp and 2kp+1 as one dword
                const uint4 w0 = vv[i][0], w1 = vv[i][1];
                const uint32_t a0[4] = {w0.x & m0, w0.y & m0, w0.z & m0, w0.w & m0},
                               a1[4] = {w1.x & m1, w1.y & m1, w1.z & m1, w1.w & m1};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    *reinterpret_cast<uint32_t *>(Vt[buf] + (pv * 8 + 2 * e) * VSTR + 2 * kp) =
                        (a0[e] & 0xffffu) | (a1[e] << 16);
                    *reinterpret_cast<uint32_t *>(Vt[buf] + (pv * 8 + 2 * e + 1) * VSTR + 2 * kp) =
                        (a0[e] >> 16) | (a1[e] & 0xffff0000u);
                }
            }
        }
    };
    auto stage = [&](int c0, int buf, int tg, int nt) {
        for (int base = 0; base < NTASK; base += TB * nt) {
            uint4 kv[TB][2], vv[TB][2];
            load_pass(c0, base, tg, nt, kv, vv);
            store_pass(c0, buf, base, tg, nt, kv, vv);
        }
    };

    // the wave's 32 query rows, dims 16kk + 8hf .. +8 for each kk
    uint4 q[NKK];
    {
        const uint16_t *qr = a.Q + (size_t)(row0 + t) * a.n_qhead * D + (size_t)(kvh * G + hh) * D;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            q[kk] = rowok ? ld16(qr + kk * 16 + hf * 8) : uint4{0u, 0u, 0u, 0u};
    }
    f32x16 o[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] = (f32x16){};
    float mrun = -INFINITY, lrun = 0.f;   // running max (base-2 units) and sum
    const float scale2 = a.scale * 1.4426950408889634f;

    // the first chunk: every thread
    if (nch > 0) stage(0, 0, tid, nthr);
    if (wave >= cw) {
        // loader waves: the loads of chunk c+2 are issued during chunk c and
        // stay in flight across the barrier that ends it; their stores fill
        // the free buffer at the start of chunk c+1 (at most kAttnLoadTasks
        // tasks a thread: one pass)
        const int tg = tid - cw * 64, nt = nthr - cw * 64;
        uint4 lk[kAttnLoadTasks][2], lv[kAttnLoadTasks][2];
        __builtin_amdgcn_sched_barrier(0);   // after the first chunk's stores, not before them
        load_pass(CH, 0, tg, nt, lk, lv);
        lds_barrier();
        for (int ci = 0; ci < nch; ++ci) {
            if (ci + 1 < nch) store_pass((ci + 1) * CH, (ci & 1) ^ 1, 0, tg, nt, lk, lv);
            load_pass((ci + 2) * CH, 0, tg, nt, lk, lv);
            lds_barrier();
        }
        return;
    }
    lds_barrier();
    for (int ci = 0; ci < nch; ++ci) {
        const int buf = ci & 1, c0 = ci * CH;
        {
            const int cn = min(CH, nkeys - c0);
            const uint16_t *Kl = Ks[buf];
            const uint16_t *Vl = Vt[buf];
            // S^T for 2 blocks of 32 keys: lane (c, hf) holds rows=c, keys kb*32 + acc_row(r, hf)
            f32x16 s[CH / 32];
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb) {
                s[kb] = (f32x16){};
                const int key = kb * 32 + c;
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const uint4 ka = *reinterpret_cast<const uint4 *>(Kl + key * D + (((2 * kk + hf) ^ (key & (KC - 1))) << 3));
                    s[kb] = mfma32(ka, q[kk], s[kb]);
                }
            }
            // scores in base-2 units: softmax(x * scale) = 2^(x * scale * log2 e - max).
            // The maximum is taken over the raw scores and scaled once (a
            // product by a positive constant, correctly rounded, keeps the
            // order); a full chunk of cache keys needs no mask, otherwise
            // keys outside the range, and for the tree's own keys those not
            // an ancestor-or-self of this row, become -inf
            float mx = -INFINITY;
            if (cn >= CH && !tree) {
#pragma unroll
                for (int kb = 0; kb < CH / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            } else {
                uint64_t vis = cn >= 64 ? ~0ull : ((1ull << cn) - 1ull);
                if (tree) vis &= (uint64_t)anc;   // the tree's keys are one chunk (c0 = 0)
                if (!rowok) vis = 0ull;
#pragma unroll
                for (int kb = 0; kb < CH / 32; ++kb) {
                    const uint32_t vb = (uint32_t)(vis >> (32 * kb));
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float v = ((vb >> acc_row(r, hf)) & 1u) ? s[kb][r] : -INFINITY;
                        s[kb][r] = v;
                        mx = fmaxf(mx, v);
                    }
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale2;
            const float mnew = fmaxf(mrun, mx);
            // with no visible key yet every score here is -inf: subtract 0
            const float msub = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = mrun == -INFINITY ? (mnew == -INFINITY ? 1.f : 0.f) : exp2f(mrun - mnew);
            // p = 2^(round(score * scale2) - max): the product and the
            // difference each rounded (no fused multiply-add, so every
            // probability has the bits of the plain two-step form), then
            // the exponential instruction (a probability below 2^-126, which
            // it flushes, moves no sum or product it enters); a masked score
            // gives 2^-inf = 0
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
#pragma clang fp contract(off)
                    const float p = __builtin_amdgcn_exp2f(s[kb][r] * scale2 - msub);
                    s[kb][r] = p;
                    ls += p;
                }
            ls += __shfl_xor(ls, 32);
            lrun = lrun * alpha + ls;
            mrun = mnew;
#pragma unroll
            for (int d = 0; d < NDB; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[d][r] *= alpha;

            // O^T += V^T P^T over 16-key steps (kb, h): lane hf supplies keys
            // kb*32 + 16h + {4hf..4hf+3, 8+4hf..8+4hf+3} = its accumulators r = 8h..8h+7
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p0 = s[kb][8 * h + 2 * e], p1 = s[kb][8 * h + 2 * e + 1];
                        hw[e] = f2bf2(p0, p1);
                        lw[e] = f2bf2(p0 - __uint_as_float(hw[e] << 16), p1 - __uint_as_float(hw[e] & 0xffff0000u));
                    }
                    const uint4 phi = {hw[0], hw[1], hw[2], hw[3]}, plo = {lw[0], lw[1], lw[2], lw[3]};
                    const int k0 = kb * 32 + 16 * h + 4 * hf;
#pragma unroll
                    for (int d = 0; d < NDB; ++d) {
                        const uint16_t *vr = Vl + ((db0 + d) * 32 + c) * VSTR;
                        const uint2 v0 = *reinterpret_cast<const uint2 *>(vr + k0);
                        const uint2 v1 = *reinterpret_cast<const uint2 *>(vr + k0 + 8);
                        const uint4 va = {v0.x, v0.y, v1.x, v1.y};
                        o[d] = mfma32(va, phi, o[d]);
                        o[d] = mfma32(va, plo, o[d]);
                    }
                }
        }
        lds_barrier();
        if (!loaders && ci + 1 < nch) {   // no loader waves: stage the next chunk in turn
            stage(c0 + CH, buf ^ 1, tid, nthr);
            lds_barrier();
        }
    }

    if (!rowok || hf > 1) return;
    const int RP = kMaxRows * kMaxGroup;
    // a prefill block's partials at its z; a verify row's at its pass row
    const size_t pb = a.nreq > 0 ? ((size_t)kvh * a.ns + split) * RP + row0 * G + row
                                 : (((size_t)z * gridDim.y + kvh) * a.ns + split) * RP + row;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) a.po[pb * D + (db0 + d) * 32 + acc_row(r, hf)] = o[d][r];
    if (hf == 0 && db0 == 0) {
        a.pm[pb] = mrun;
        a.pl[pb] = lrun;
    }
}

// Merge the splits of every (node, query head) in split order.
template <int D>
__global__ __launch_bounds__(D) void k_attn_combine(AttnArgs a, uint16_t *__restrict__ out) {
    __shared__ float ms[64], wl[64], ws[64];
    const int t = blockIdx.x, h = blockIdx.y, z = blockIdx.z, d = threadIdx.x;
    const int G = a.G, kvh = h / G, row = t * G + (h % G);
    const int RP = kMaxRows * kMaxGroup;
    int ns = a.ns, row0 = a.row0;
    if (a.nreq > 0) {    // request z of a verify pass: its own rows and split count
        const PassReq &rq = a.rq[z];
        if (t >= rq.n) return;
        row0 = rq.row0;
        ns = rq.nsplit + 1;
    } else if (a.zrows > 0) {   // a prefill block: its own split count
        row0 = z * a.zrows;
        if (row0 + t >= a.M) return;
        const int ctx = a.ctx + row0, span = attn_span_n(ctx, a.ztarget);
        ns = (ctx + span - 1) / span + 1;
    }
    const size_t b0 = a.nreq > 0 ? ((size_t)kvh * a.ns) * RP + row0 * G + row
                                 : (((size_t)z * (a.n_qhead / G) + kvh) * a.ns) * RP + row;
    // every split's output of this dim and (thread d) split d's maximum and
    // sum: all loads in flight at once
    float pv[kAttnMaxSplits];
#pragma unroll
    for (int s = 0; s < kAttnMaxSplits; ++s) pv[s] = s < ns ? a.po[(b0 + (size_t)s * RP) * D + d] : 0.f;
    if (d < ns) {
        ms[d] = a.pm[b0 + (size_t)d * RP];
        wl[d] = a.pl[b0 + (size_t)d * RP];
    }
    __syncthreads();
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ms[s]);
    // split maxima are in base-2 units (scores times log2 e)
    if (d < ns) ws[d] = (ms[d] == -INFINITY) ? 0.f : exp2f(ms[d] - M);
    __syncthreads();
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int s = 0; s < kAttnMaxSplits; ++s) {   // adds in split order
        if (s < ns) {
            L += ws[s] * wl[s];
            O += ws[s] * pv[s];
        }
    }
    out[(size_t)(row0 + t) * a.n_qhead * D + h * D + d] = f2bf(O / L);
}

// ------------------------------------------------------- gated recurrence
// Tree verify through a gated linear recurrence layer ("Drafters and tree
// verify", Tree verify through recurrent layers).  Per head, the state after
// node t is e^{g_t} S(parent) + k_t v_t^T; unrolled along the root-to-t path,
//   o_t = S(t)^T q_t = e^{gc_t} S0^T q_t + sum_{s in anc*(t)} e^{gc_t - gc_s} (q_t . k_s) v_s
// with gc the cumulative log-gate along the path, so no node overwrites its
// parent's state.  q and k are L2-normalised per head and rounded to bf16,
// g = log sigmoid(a).  One workgroup per head; it also saves k, v and gc of
// every node for the commit.
//
// Gated delta rule (the pages' Gated DeltaNet layers; Yang, Kautz and
// Hatamizadeh, ICLR 2025): S(t) = e^{g_t} (I - b_t k_t k_t^T) S(parent)
// + b_t k_t v_t^T with write strength b = sigmoid(.).  Written as
// S(t) = e^{g_t} S(parent) + k_t u_t^T it is the same recurrence with the
// pseudo-value u_t in place of v_t, where
//   u_t + sum_{s strict ancestor of t} b_t e^{gc_t - gc_s} (k_t . k_s) u_s
//       = b_t (v_t - e^{gc_t} S0^T k_t):
// a unit lower-triangular system whose off-diagonal part is ancestor-masked
// ("Drafters and tree verify", Tree verify through recurrent layers), solved
// by forward substitution in node order; u replaces v in the read-out and
// in what the commit saves.

__device__ __forceinline__ float log_sigmoid(float a) {
    // -log(1 + e^{-a}) for a >= 0, a - log(1 + e^{a}) below: both take e^{-|a|}
    const float l = log1pf(expf(-fabsf(a)));
    return a >= 0.f ? -l : a - l;
}

// Sum over groups of W consecutive lanes (W = 8 or 16, inside one 16-lane
// DPP row), every lane of a group getting the same total: adds with lanes
// xor 1 and xor 2 (quad permutes), then the mirror inside each half-row and
// inside the row.  A fixed tree: the result depends only on the values.
template <int W>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(W == 8 || W == 16, "one or two half rows");
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // row_half_mirror
    if constexpr (W == 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
    return x;
}

// Eight consecutive fp32 values as bf16 (exact when they are bf16 values).
__device__ __forceinline__ uint4 pack_bf8(const float *x) {
    return uint4{f2bf2(x[0], x[1]), f2bf2(x[2], x[3]), f2bf2(x[4], x[5]), f2bf2(x[6], x[7])};
}

// Lane k's x for every lane of its quad (quad_perm [k, k, k, k]); k is a
// constant once the caller's loop is unrolled.
__device__ __forceinline__ float quad_bcast(float x, int k) {
    const int v = __float_as_int(x);
    switch (k & 3) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false));
    }
}

// Cumulative gate of lane t's node: the sum of g_s over its ancestors-or-self
// s (bits of anc; ancestors have lower indices, so no bit lies above t) in
// index order, root first, each g_s broadcast from lane s of the wave; a
// non-ancestor adds an exact zero.  NN >= n: the slots from n on are
// non-ancestors, and since the sum starts at +0 and is never -0, dropping
// them leaves it unchanged.
template <int NN>
__device__ __forceinline__ float cum_gate(float g, uint32_t anc) {
    float gc = 0.f;
#pragma unroll
    for (int s = 0; s < NN; ++s) {
        const float gs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), s));
        gc += ((anc >> s) & 1u) ? gs : 0.f;
    }
    return gc;
}

// Forward substitution for value column c of the delta rule's unit
// lower-triangular system (n <= NN nodes; ancestors have lower indices, so
// node order is a topological order), by the four lanes of a quad: lane j
// holds in registers the nodes t = j, j + 4, ... of the column.  Once u_s is
// final its owner (lane s % 4) hands it to the quad (a DPP broadcast) and it
// is taken out of every later node's right-hand side, so node t's sum runs
// over s = 0, 1, ..., t - 1 in order.  akq[s][j][i] is the coefficient of
// node 4i + j in row s.  u[t] for t >= n is never stored.
template <int NN, int VW>
__device__ __forceinline__ void delta_solve(float (*vsm)[VW + 1], const float (*akq)[kMaxRows + 4], int n, int c, int j) {
    constexpr int NI = NN / 4;
    constexpr int PD = 4;   // coefficient rows in flight ahead of the step that uses them
    float u[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) u[i] = 4 * i + j < n ? vsm[4 * i + j][c] : 0.f;
    // ring of the next PD rows' coefficients: row s sits in a[s % PD] and is
    // replaced by row s + PD once step s has used it (rows past n are read,
    // never used: akq has kMaxRows rows)
    float a[PD][NI];
#pragma unroll
    for (int q = 0; q < PD; ++q)
#pragma unroll
        for (int i = 0; i < NI; ++i) a[q][i] = akq[q][j * NI + i];
#pragma unroll
    for (int s = 0; s < NN - 1; ++s) {
        if (s + 1 >= n) break;
        const float us = quad_bcast(u[s / 4], s);   // u_s from lane s % 4 of the quad
#pragma unroll
        for (int i = s / 4; i < NI; ++i)
            if (4 * i + j > s) u[i] -= a[s % PD][i] * us;
        if (s + PD < NN - 1) {
#pragma unroll
            for (int i = 0; i < NI; ++i) a[s % PD][i] = akq[s + PD][j * NI + i];
        }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
        if (4 * i + j < n) vsm[4 * i + j][c] = u[i];
}

// Threads of a read-out workgroup: 8 waves at head size 128 (two a SIMD, so
// each wave's loads, norms and sums are half as long and a SIMD has a
// second wave to switch to), 4 at 64 (the state-slice mapping's limit).
constexpr int recur_threads(int D) { return D >= 128 ? 512 : 256; }

template <int D, bool DELTA>
__global__ __launch_bounds__(recur_threads(D)) void k_recur_tree(RecurArgs r) {
    // grid (head, value slice): a workgroup produces value columns
    // [v0, v0 + VW) of its head for every node; the small per-head setup
    // (norms, cumulative gates, the node-node coefficients) is repeated by
    // the head's slices.  The three small products of the read-out run on
    // MFMA (v_mfma_f32_32x32x16_bf16, nodes and value columns padded to 32):
    // Q K^T and K K^T with exact bf16 operands (q and k are bf16 values), and
    // S0^T Q, S0^T K with the fp32 state split into bf16 hi + lo parts
    // (|S0 - hi - lo| <= 2^-17 |S0|).
    constexpr int VS = kRecurSlices;
    constexpr int NT = recur_threads(D);
    constexpr int VW = D / VS;             // value columns per workgroup (<= 32)
    constexpr int BP = D + 8;              // padded bf16 row stride (16-byte rows, spread banks)
    constexpr int KB = D / 16;             // MFMA k blocks
    static_assert(VW <= 32 && D % 16 == 0, "slice shape");
    __shared__ __attribute__((aligned(16))) uint16_t qb[kMaxRows][BP], kb[kMaxRows][BP];   // normalised, bf16
    __shared__ __attribute__((aligned(16))) uint16_t s0h[VW][BP], s0l[VW][BP];  // S0 slice, transposed, hi/lo
    __shared__ float vsm[kMaxRows][VW + 1];   // v, then (delta) the right-hand side and u (odd stride: a
                                              // wave of nodes at one column hits distinct banks)
    __shared__ float accq[kMaxRows][VW + 1];   // e^{gc_t} S0^T q_t
    __shared__ float gcs[kMaxRows];
    __shared__ uint32_t ancs[kMaxRows];    // ancestor-or-self bits of each node
    __shared__ float coef[kMaxRows][kMaxRows + 1];
    // delta rule: write strengths, and the coefficient b_t e^{gc_t - gc_s}
    // (k_t . k_s) of node t in row s, for strict ancestors s of t (zero
    // otherwise), at akq[s][(t % 4) * NI + t / 4] with NI = (n <= 16 ? 4 : 8)
    // (node t's solver lane is t % 4; rows padded to 36 floats)
    __shared__ float bsh[DELTA ? kMaxRows : 1];
    __shared__ __attribute__((aligned(16))) float akq[DELTA ? kMaxRows : 1][kMaxRows + 4];
    const int h = blockIdx.x, v0 = blockIdx.y * VW, tid = threadIdx.x, n = r.n, QH = r.QH;
    const int lane = tid & 63, wave = tid >> 6, hf = lane >> 5, l32 = lane & 31;

    // state slice (every load in flight first), read already transposed: a
    // thread takes KPT consecutive keys of one value column (one 4-byte load
    // per key, a wave's loads coalesced along the columns) and later writes
    // them as bf16 hi + lo runs of its column's row
    constexpr int KPT = D * VW / NT;       // keys per thread
    static_assert(NT % VW == 0 && KPT % 4 == 0, "state slice mapping");
    const int sc = tid % VW, sk0 = (tid / VW) * KPT;
    float st[KPT];
    {
        const float *S0 = r.S0 + (size_t)h * D * D + (size_t)sk0 * D + v0 + sc;
#pragma unroll
        for (int i = 0; i < KPT; ++i) st[i] = S0[(size_t)i * D];
    }
    // Projection outputs: split-K partials summed in k-range order (or, for
    // a prefill block, bf16 rows), rounded to bf16 (the projection's output
    // rounding).  Each thread takes eight consecutive columns of q and of k
    // for rows qr0, qr0 + RPP, ... (TPR threads a row), four of this slice's
    // v columns for row vr, and lane t of the last wave node t's gate (and
    // write strength): every load of every split (four splits a round) is
    // in flight before the first add.
    constexpr int TPR = D / 8;             // threads per q or k row (16 or 8: one DPP row)
    constexpr int RPP = NT / TPR;          // rows per pass
    constexpr int NP = kMaxRows / RPP;     // passes cover every row slot (rows >= n are zero)
    constexpr int VT = VW / 4;             // threads per v row
    static_assert(NP * RPP == kMaxRows && (NT / VT) >= kMaxRows, "load mapping");
    const bool rows_in = r.qkv_rows != nullptr;   // a prefill block: bf16 rows, a chain
    if (tid < n) ancs[tid] = rows_in ? (tid >= 31 ? 0xffffffffu : ((2u << tid) - 1u)) : r.meta->anc[r.row0 + tid];
    const int qr0 = tid / TPR, qc = (tid % TPR) * 8;
    const int vr = tid / VT, vc = (tid % VT) * 4;
    // gates: lane t of the last wave takes node t (its rows of q and k are
    // padding up to 28 nodes at head size 128, 24 at 64)
    const int gl = tid - (NT - 64);
    const bool vok = vr < n, gok = gl >= 0 && gl < n;
    const uint32_t ganc = !gok ? 0u : rows_in ? (gl >= 31 ? 0xffffffffu : ((2u << gl) - 1u)) : r.meta->anc[r.row0 + gl];
    float qx[NP][8], kx[NP][8], ga = 0.f, gb = 0.f;
    float4 vx = {0.f, 0.f, 0.f, 0.f};
    if (rows_in) {
        auto row4 = [&](bool ok, int m, int col) -> uint2 {   // four bf16 values of row m
            return ok ? *reinterpret_cast<const uint2 *>(r.qkv_rows + (size_t)m * r.a_col + col) : uint2{0u, 0u};
        };
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int m = qr0 + i * RPP;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint2 wq = row4(m < n, r.row0 + m, h * D + qc + 4 * hh);
                const uint2 wk = row4(m < n, r.row0 + m, (QH + h) * D + qc + 4 * hh);
                qx[i][4 * hh + 0] = __uint_as_float(wq.x << 16); qx[i][4 * hh + 1] = __uint_as_float(wq.x & 0xffff0000u);
                qx[i][4 * hh + 2] = __uint_as_float(wq.y << 16); qx[i][4 * hh + 3] = __uint_as_float(wq.y & 0xffff0000u);
                kx[i][4 * hh + 0] = __uint_as_float(wk.x << 16); kx[i][4 * hh + 1] = __uint_as_float(wk.x & 0xffff0000u);
                kx[i][4 * hh + 2] = __uint_as_float(wk.y << 16); kx[i][4 * hh + 3] = __uint_as_float(wk.y & 0xffff0000u);
            }
        }
        const uint2 wv = row4(vok, r.row0 + vr, (2 * QH + h) * D + v0 + vc);
        vx = float4{__uint_as_float(wv.x << 16), __uint_as_float(wv.x & 0xffff0000u),
                    __uint_as_float(wv.y << 16), __uint_as_float(wv.y & 0xffff0000u)};
        if (gok) {
            ga = bf2f(r.ab_rows[(size_t)(r.row0 + gl) * r.ab_ld + h]);
            if (DELTA) gb = bf2f(r.ab_rows[(size_t)(r.row0 + gl) * r.ab_ld + QH + h]);
        }
    } else {
        const float *P = r.qkv_part;
        const int S = r.qkv_S;
        auto pp = [&](int m, int col, int sp) {   // partial of split sp, row m, column col
            return P + ((size_t)(col >> 7) * S + sp) * 4096 + (size_t)m * 128 + (col & 127);
        };
#pragma unroll
        for (int i = 0; i < NP; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) qx[i][e] = kx[i][e] = 0.f;
        for (int k0 = 0; k0 < S; k0 += 4) {
            float4 lq[NP][4][2], lk[NP][4][2], lv[4];
            float4 lga, lgb;   // gate (and write-strength) partials of four splits
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool sj = k0 + j < S;
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    const int m = qr0 + i * RPP;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        lq[i][j][hh] = lk[i][j][hh] = float4{0.f, 0.f, 0.f, 0.f};
                        if (sj && m < n) {
                            lq[i][j][hh] = *reinterpret_cast<const float4 *>(pp(r.row0 + m, h * D + qc + 4 * hh, k0 + j));
                            lk[i][j][hh] = *reinterpret_cast<const float4 *>(pp(r.row0 + m, (QH + h) * D + qc + 4 * hh, k0 + j));
                        }
                    }
                }
                lv[j] = float4{0.f, 0.f, 0.f, 0.f};
                if (sj && vok) lv[j] = *reinterpret_cast<const float4 *>(pp(r.row0 + vr, (2 * QH + h) * D + v0 + vc, k0 + j));
                const float g1 = (sj && gok) ? *pp(r.row0 + gl, r.a_col + h, k0 + j) : 0.f;
                const float g2 = (DELTA && sj && gok) ? *pp(r.row0 + gl, r.a_col + QH + h, k0 + j) : 0.f;
                if (j == 0) { lga.x = g1; lgb.x = g2; }
                else if (j == 1) { lga.y = g1; lgb.y = g2; }
                else if (j == 2) { lga.z = g1; lgb.z = g2; }
                else { lga.w = g1; lgb.w = g2; }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (k0 + j < S) {
#pragma unroll
                    for (int i = 0; i < NP; ++i)
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            qx[i][4 * hh + 0] += lq[i][j][hh].x; qx[i][4 * hh + 1] += lq[i][j][hh].y;
                            qx[i][4 * hh + 2] += lq[i][j][hh].z; qx[i][4 * hh + 3] += lq[i][j][hh].w;
                            kx[i][4 * hh + 0] += lk[i][j][hh].x; kx[i][4 * hh + 1] += lk[i][j][hh].y;
                            kx[i][4 * hh + 2] += lk[i][j][hh].z; kx[i][4 * hh + 3] += lk[i][j][hh].w;
                        }
                    vx.x += lv[j].x; vx.y += lv[j].y; vx.z += lv[j].z; vx.w += lv[j].w;
                    ga += j == 0 ? lga.x : j == 1 ? lga.y : j == 2 ? lga.z : lga.w;
                    gb += j == 0 ? lgb.x : j == 1 ? lgb.y : j == 2 ? lgb.z : lgb.w;
                }
            }
        }
    }
    // the state slice as bf16 hi + lo parts, KPT keys of column sc at a time
#pragma unroll
    for (int i = 0; i < KPT; i += 4) {
        uint32_t wh[2], wl[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float x0 = st[i + 2 * e], x1 = st[i + 2 * e + 1];
            wh[e] = f2bf2(x0, x1);
            wl[e] = f2bf2(x0 - __uint_as_float(wh[e] << 16), x1 - __uint_as_float(wh[e] & 0xffff0000u));
        }
        *reinterpret_cast<uint2 *>(&s0h[sc][sk0 + i]) = uint2{wh[0], wh[1]};
        *reinterpret_cast<uint2 *>(&s0l[sc][sk0 + i]) = uint2{wl[0], wl[1]};
    }
    // q and k: round the sums, then each row's sum of squares over its TPR
    // lanes (consecutive lanes of one DPP row; a fixed tree of DPP
    // exchanges), then the normalised row rounded to bf16 (rows >= n are
    // zero: the matrix-core padding); the first slice also saves the keys
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int m = qr0 + i * RPP;
        if ((wave * 64) / TPR + i * RPP >= n) {   // every row of this wave's pass is padding
            *reinterpret_cast<uint4 *>(&qb[m][qc]) = uint4{0u, 0u, 0u, 0u};
            *reinterpret_cast<uint4 *>(&kb[m][qc]) = uint4{0u, 0u, 0u, 0u};
            continue;
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qx[i][e] = bfround(qx[i][e]);
            kx[i][e] = bfround(kx[i][e]);
            sq += qx[i][e] * qx[i][e];
            sk += kx[i][e] * kx[i][e];
        }
        sq = row_sum<TPR>(sq);
        sk = row_sum<TPR>(sk);
        const float fq = 1.0f / sqrtf(sq + r.eps), fk = 1.0f / sqrtf(sk + r.eps);
        float nq[8], nk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            nq[e] = qx[i][e] * fq;
            nk[e] = kx[i][e] * fk;
        }
        const uint4 wq = pack_bf8(nq), wk = pack_bf8(nk);
        *reinterpret_cast<uint4 *>(&qb[m][qc]) = m < n ? wq : uint4{0u, 0u, 0u, 0u};
        *reinterpret_cast<uint4 *>(&kb[m][qc]) = m < n ? wk : uint4{0u, 0u, 0u, 0u};
        if (blockIdx.y == 0 && m < n) *reinterpret_cast<uint4 *>(r.save_k + ((size_t)m * QH + h) * D + qc) = wk;
    }
    if (vok) {
        vsm[vr][vc] = bfround(vx.x);
        vsm[vr][vc + 1] = bfround(vx.y);
        vsm[vr][vc + 2] = bfround(vx.z);
        vsm[vr][vc + 3] = bfround(vx.w);
    }
    float gate_g = 0.f;   // the gate wave's lane t: g_t, summed over ancestors after the barrier
    if (wave == NT / 64 - 1) {
        // lane t's gate g_t (every lane computes one; lanes >= n are never
        // added) and, for a delta layer, its write strength b_t
        gate_g = log_sigmoid(bfround(ga));
        if constexpr (DELTA)
            if (gok) bsh[gl] = 1.0f / (1.0f + expf(-bfround(gb)));
    }
    __syncthreads();
    // the small products, one wave each: lane (hf, j = lane % 32) supplies k
    // slots 16*kk + 8*hf + 0..7 of A row j and of B column j; accumulator r
    // holds row acc_row(r, hf) of column j.  Their MFMA chains run while the
    // gate wave forms the cumulative gates, which the epilogues read after a
    // barrier.
    const uint4 z = {0u, 0u, 0u, 0u};
    const bool pw_qk = wave == 0 || (DELTA && wave == 1);   // Q K^T (coef) and K K^T (akq)
    const bool pw_s0 = wave == 2 || (DELTA && wave == 3);   // S0^T Q and S0^T K
    if (wave == NT / 64 - 1) {
        // the cumulative gate over the ancestors-or-self in index order, root
        // first (ancestors have lower indices)
        const float gc = n <= 16 ? cum_gate<16>(gate_g, ganc) : cum_gate<kMaxRows>(gate_g, ganc);
        if (gok) gcs[gl] = gc;
    }
    f32x16 acc = {};
    if (pw_qk) {
        const uint16_t(*A)[BP] = wave == 0 ? qb : kb;
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const uint4 a = *reinterpret_cast<const uint4 *>(&A[l32][16 * kk + 8 * hf]);
            const uint4 b = *reinterpret_cast<const uint4 *>(&kb[l32][16 * kk + 8 * hf]);
            acc = mfma32(a, b, acc);
        }
    } else if (pw_s0) {
        // A row = value column (S0 transposed), B column = node
        const uint16_t(*B)[BP] = wave == 2 ? qb : kb;
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const uint4 b = *reinterpret_cast<const uint4 *>(&B[l32][16 * kk + 8 * hf]);
            const uint4 ah = l32 < VW ? *reinterpret_cast<const uint4 *>(&s0h[l32][16 * kk + 8 * hf]) : z;
            const uint4 al = l32 < VW ? *reinterpret_cast<const uint4 *>(&s0l[l32][16 * kk + 8 * hf]) : z;
            acc = mfma32(ah, b, acc);
            acc = mfma32(al, b, acc);
        }
    }
    __syncthreads();
    if (pw_qk) {
        // coef (wave 0): e^{gc_t - gc_s} (q_t . k_s) over ancestors-or-self s;
        // akq (wave 1, by solver lane): b_t e^{gc_t - gc_s} (k_t . k_s) over strict ancestors
        const int s = l32;
        if (s < n) {
            const int rrn = n <= 16 ? 8 : 16;   // accumulators rr >= 8 hold nodes >= 16
            // every node-indexed read issued first (slots past n are read and not used)
            float gt[16], bt[16];
            uint32_t at[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int t = acc_row(rr, hf);
                gt[rr] = gcs[t];
                at[rr] = ancs[t];
                bt[rr] = DELTA ? bsh[DELTA ? t : 0] : 0.f;
            }
            const float gs = gcs[s];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int t = acc_row(rr, hf);
                if (rr >= rrn) break;
                if (t >= n) continue;
                const bool anc = (at[rr] >> s) & 1u;
                const float decay = expf(gt[rr] - gs);
                if (wave == 0) {
                    coef[t][s] = anc ? decay * acc[rr] : 0.f;
                } else if constexpr (DELTA) {
                    akq[s][(t & 3) * (n <= 16 ? 4 : 8) + (t >> 2)] = (anc && s != t) ? bt[rr] * decay * acc[rr] : 0.f;
                }
            }
        }
    } else if (pw_s0) {
        // wave 2 keeps e^{gc_t} S0^T q_t for the read-out; wave 3 (delta)
        // turns v into the right-hand side b_t (v_t - e^{gc_t} S0^T k_t) in
        // place (no other wave touches v in this phase)
        const int t = l32;
        if (t < n) {
            const float eg = expf(gcs[t]), bt = DELTA ? bsh[DELTA ? t : 0] : 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int c = acc_row(rr, hf);
                if (c >= VW) continue;
                if (wave == 2) accq[t][c] = eg * acc[rr];
                else if constexpr (DELTA) vsm[t][c] = bt * (vsm[t][c] - eg * acc[rr]);
            }
        }
    }
    __syncthreads();
    if constexpr (DELTA) {
        // forward substitution, a quad of lanes a value column (the column in registers)
        if (tid < 4 * VW) {
            if (n <= 16) delta_solve<16, VW>(vsm, akq, n, tid >> 2, tid & 3);
            else delta_solve<kMaxRows, VW>(vsm, akq, n, tid >> 2, tid & 3);
        }
        __syncthreads();
    }
    // read-out o_t = e^{gc_t} S0^T q_t + sum over ancestors-or-self s of
    // coef[t][s] u_s (u = v for the plain recurrence)
    for (int idx = tid; idx < n * VW; idx += NT) {
        const int t = idx / VW, c = idx % VW;
        float o = accq[t][c];
        int s = 0;
        for (; s + 3 <= t; s += 4) {   // four terms' reads in flight, then their adds in order
            const float c0 = coef[t][s], c1 = coef[t][s + 1], c2 = coef[t][s + 2], c3 = coef[t][s + 3];
            const float u0 = vsm[s][c], u1 = vsm[s + 1][c], u2 = vsm[s + 2][c], u3 = vsm[s + 3][c];
            o += c0 * u0;
            o += c1 * u1;
            o += c2 * u2;
            o += c3 * u3;
        }
        for (; s <= t; ++s) o += coef[t][s] * vsm[s][c];
        r.out[(size_t)(r.row0 + t) * QH * D + h * D + v0 + c] = f2bf(o);
        r.save_v[((size_t)t * QH + h) * D + v0 + c] = vsm[t][c];
    }
    if (blockIdx.y == 0 && tid < n) r.save_gc[(size_t)tid * QH + h] = gcs[tid];
}

// State commit: the state after the accepted path from the quantities the
// verify saved ("Drafters and tree verify", Tree verify through recurrent
// layers: S_path = e^{gc_last} S0 + sum over the path of e^{gc_last - gc_t}
// k_t (x) u_t, u = v for the plain gated recurrence), in place; one read and
// write of the state, no weights.
template <int D>
__global__ __launch_bounds__(256) void k_recur_commit(RecurCommitArgs a) {
    __shared__ float kk[kMaxRows][D], vv[kMaxRows][D], w[kMaxRows];
    __shared__ float elast;
    const int l = blockIdx.x / a.QH, h = blockIdx.x % a.QH, tid = threadIdx.x, QH = a.QH;
    const int L = a.path.len;
    const uint16_t *sk = a.save_k + (size_t)l * kMaxRows * QH * D;
    const float *sv = a.save_v + (size_t)l * kMaxRows * QH * D;
    const float *sg = a.save_gc + (size_t)l * kMaxRows * QH;
    for (int idx = tid; idx < L * D; idx += 256) {
        const int d = idx / D, e = idx % D, node = a.path.node[d];
        kk[d][e] = bf2f(sk[((size_t)node * QH + h) * D + e]);
        vv[d][e] = sv[((size_t)node * QH + h) * D + e];
    }
    const float gl = sg[(size_t)a.path.node[L - 1] * QH + h];
    if (tid < L) w[tid] = expf(gl - sg[(size_t)a.path.node[tid] * QH + h]);
    if (tid == 0) elast = expf(gl);
    __syncthreads();
    float *S = a.states[l] + (size_t)h * D * D;
    for (int idx = tid; idx < D * D; idx += 256) {
        const int i = idx / D, j = idx % D;
        float s = elast * S[idx];
        for (int d = 0; d < L; ++d) s += (w[d] * kk[d][i]) * vv[d][j];
        S[idx] = s;
    }
}

// ---------------------------------------------------------------- commit
// Gather the accepted path's KV rows: slot ctx+path[d] -> ctx+d.  One
// workgroup per (layer, KV head) reads every moved row before writing any,
// so the in-place move is safe in any order.

__global__ __launch_bounds__(256) void k_commit_kv(uint16_t *const *__restrict__ kv_ptrs, int cap,
                                                   int D, int ctx, PathArg path) {
    const int path_len = path.len;
    __shared__ __attribute__((aligned(16))) uint16_t buf[2 * kMaxRows * 128];
    const int layer = blockIdx.x, h = blockIdx.y;
    uint16_t *Kc = kv_ptrs[2 * layer] + (size_t)h * cap * D;
    uint16_t *Vc = kv_ptrs[2 * layer + 1] + (size_t)h * cap * D;
    const int per = D / 8;
    const int total = path_len * per;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
        const int d = idx / per, p = idx % per;
        const size_t src = (size_t)(ctx + path.node[d]) * D + p * 8;
        *reinterpret_cast<uint4 *>(buf + d * D + p * 8) = ld16(Kc + src);
        *reinterpret_cast<uint4 *>(buf + (kMaxRows + d) * D + p * 8) = ld16(Vc + src);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < total; idx += 256) {
        const int d = idx / per, p = idx % per;
        if (path.node[d] == d) continue;
        const size_t dst = (size_t)(ctx + d) * D + p * 8;
        *reinterpret_cast<uint4 *>(Kc + dst) = *reinterpret_cast<const uint4 *>(buf + d * D + p * 8);
        *reinterpret_cast<uint4 *>(Vc + dst) =
            *reinterpret_cast<const uint4 *>(buf + (kMaxRows + d) * D + p * 8);
    }
}

// ------------------------------------------------------------ launchers

static int row_threads(int H) { return ((H / 8 + 63) / 64) * 64; }

hipError_t launch_embed_norm(hipStream_t s, const uint16_t *emb, const PassMeta *meta, PassMeta *meta_out, int M,
                             int H, const uint16_t *w, float eps, uint16_t *X, uint16_t *Y) {
    if (H % 8 || H > 8 * kRowThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_row_norm<ROW_EMBED>, dim3(M), dim3(row_threads(H)), 0, s, emb, meta, meta_out, nullptr, 0,
                       H, w, eps, X, Y);
    return hipGetLastError();
}

hipError_t launch_resid_norm(hipStream_t s, const float *P, int S, int M, int H, const uint16_t *w, float eps,
                             uint16_t *X, uint16_t *Y) {
    if (H % 8 || H > 8 * kRowThreads || S < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_row_norm<ROW_RESID>, dim3(M), dim3(row_threads(H)), 0, s, nullptr, nullptr, nullptr, P, S,
                       H, w, eps, X, Y);
    return hipGetLastError();
}

hipError_t launch_gemm(hipStream_t s, int epi, const GemmArgs &a, int splits) {
    const int rowblocks = ((a.N + 31) / 32 + 3) / 4;
    const dim3 grid(rowblocks, splits), block(256);
    switch (epi) {
    case EPI_BF16: hipLaunchKernelGGL((k_gemm<EPI_BF16>), grid, block, 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm<EPI_RESID>), grid, block, 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_gemm<EPI_SWIGLU>), grid, block, 0, s, a); break;
    case EPI_HEAD: hipLaunchKernelGGL((k_gemm<EPI_HEAD>), grid, block, 0, s, a); break;
    case EPI_PARTIAL: hipLaunchKernelGGL((k_gemm<EPI_PARTIAL>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The 32-row-group kernel over the whole shape.
static hipError_t launch_gemm_groups(hipStream_t s, int epi, const GemmArgs &a) {
    if (a.M < 1 || a.N < 1 || a.K < 8 || a.K % 8) return hipErrorInvalidValue;
    const int wblocks = ((a.N + 31) / 32 + 3) / 4;
    const dim3 block(256);
    // Row groups per workgroup, from a sweep at 1024 rows: single epilogues
    // take 4 groups (128 rows) when that still gives at least 448 workgroups
    // (about 1.75 per CU), else 2; SwiGLU (two weight tiles per wave) takes 2
    // groups and one k step per LDS stage.  The k order of every output is
    // the same for any choice (whole steps in order).
    // One group (32 rows) when two would leave CUs idle (the last weight
    // blocks of a shape whose bulk ran on the 256 x 256 tiles).
    const int g4 = ((a.M + 127) / 128) * wblocks, g2 = ((a.M + 63) / 64) * wblocks, g1 = ((a.M + 31) / 32) * wblocks;
    const bool four = g4 >= 448, one = g2 < 256;
    switch (epi) {
    case EPI_BF16:
        if (four) hipLaunchKernelGGL((k_gemm_dense<EPI_BF16, 4>), dim3(g4), block, 0, s, a);
        else if (one) hipLaunchKernelGGL((k_gemm_dense<EPI_BF16, 1>), dim3(g1), block, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_dense<EPI_BF16, 2>), dim3(g2), block, 0, s, a);
        break;
    case EPI_RESID:
        if (four) hipLaunchKernelGGL((k_gemm_dense<EPI_RESID, 4>), dim3(g4), block, 0, s, a);
        else if (one) hipLaunchKernelGGL((k_gemm_dense<EPI_RESID, 1>), dim3(g1), block, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_dense<EPI_RESID, 2>), dim3(g2), block, 0, s, a);
        break;
    case EPI_F32:
        if (four) hipLaunchKernelGGL((k_gemm_dense<EPI_F32, 4>), dim3(g4), block, 0, s, a);
        else if (one) hipLaunchKernelGGL((k_gemm_dense<EPI_F32, 1>), dim3(g1), block, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_dense<EPI_F32, 2>), dim3(g2), block, 0, s, a);
        break;
    case EPI_SWIGLU:
        if (one) hipLaunchKernelGGL((k_gemm_dense<EPI_SWIGLU, 1, 1>), dim3(g1), block, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_dense<EPI_SWIGLU, 2, 1>), dim3(g2), block, 0, s, a);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


// k_gemm_big of row tile mt_rows (256, 128 or 64) over nblk weight blocks.
static hipError_t launch_gemm_big(hipStream_t s, int epi, const GemmArgs &a, int nblk, int mt_rows) {
    const dim3 grid(nblk * ((a.M + mt_rows - 1) / mt_rows)), block(512);
#define TV_BIG(K)                                                                                             \
    switch (epi) {                                                                                            \
    case EPI_BF16: hipLaunchKernelGGL(K<EPI_BF16>, grid, block, 0, s, a); break;                              \
    case EPI_RESID: hipLaunchKernelGGL(K<EPI_RESID>, grid, block, 0, s, a); break;                            \
    case EPI_F32: hipLaunchKernelGGL(K<EPI_F32>, grid, block, 0, s, a); break;                                \
    case EPI_SWIGLU: hipLaunchKernelGGL(K<EPI_SWIGLU>, grid, block, 0, s, a); break;                          \
    default: return hipErrorInvalidValue;                                                                     \
    }
    if (mt_rows == 256) { TV_BIG(k_gemm_big256) }
    else if (mt_rows == 128) { TV_BIG(k_gemm_big128) }
    else if (mt_rows == 64) { TV_BIG(k_gemm_big64) }
    else return hipErrorInvalidValue;
#undef TV_BIG
    return hipGetLastError();
}

hipError_t launch_gemm_dense(hipStream_t s, int epi, const GemmArgs &a) {
    if (a.M < 1 || a.N < 1 || a.K < 8 || a.K % 8) return hipErrorInvalidValue;
    // 256 x 256 tiles (same bits) for 256 rows and more when the shape is
    // whole (k a multiple of 128, whole weight blocks, 16-byte aligned rows)
    // and the tiles fill every CU at least once.  Only whole rounds of 256
    // tiles (one workgroup a CU) run on them: the weight blocks of a last,
    // partial round take tiles of 128 or 64 rows in a second launch, which
    // spreads them over more CUs (every tile height gives the same bits, so
    // where the cut falls changes no output).  Measured at 1024 and 2048
    // rows on the 5120-wide layer's shapes.
    const bool dual = epi == EPI_SWIGLU;
    const int bw = dual ? 128 : 256;                 // output columns of a weight block
    const int nblk = a.N / bw, mt = (a.M + kBigTile - 1) / kBigTile;
    const bool whole = a.M >= kBigTile && a.K % 128 == 0 && a.N % bw == 0 && a.ldx % 8 == 0 &&
                       ((uintptr_t)a.X & 15) == 0 &&
                       (epi == EPI_F32 ? a.ldyf % 4 == 0 && ((uintptr_t)a.Yf & 15) == 0
                                       : a.ldy % 4 == 0 && ((uintptr_t)a.Y & 7) == 0);
    const int rem = (nblk * mt) % 256 ? ((nblk * mt) % 256 + mt - 1) / mt : 0;   // blocks of the partial round
    if (!whole) return launch_gemm_groups(s, epi, a);
    if ((nblk - rem) * mt < 256) {
        // too few 256-row tiles for a round: 128-row tiles when they cover
        // at least half the CUs, else 64-row tiles on the same terms (at
        // 512-1024 rows of the 5120-wide layer's QKV, O and down shapes 10-20 %
        // faster than the 32-row-group kernel, which stays below that)
        if (nblk * ((a.M + 127) / 128) >= 128) return launch_gemm_big(s, epi, a, nblk, 128);
        if (nblk * ((a.M + 63) / 64) >= 128) return launch_gemm_big(s, epi, a, nblk, 64);
        return launch_gemm_groups(s, epi, a);
    }
    hipError_t e = launch_gemm_big(s, epi, a, nblk - rem, kBigTile);
    if (e != hipSuccess || rem == 0) return e;
    // the last rem weight blocks: output columns c0.. of the same rows
    const int c0 = (nblk - rem) * bw;
    GemmArgs r = a;
    r.N = rem * bw;
    r.W = a.W + (size_t)c0 * a.K;                    // whole 32-row tiles of the packed weights
    if (dual) r.W2 = a.W2 + (size_t)c0 * a.K;
    if (epi == EPI_F32) r.Yf = a.Yf + c0;
    else r.Y = a.Y + c0;
    return launch_gemm_big(s, epi, r, rem, rem * ((a.M + 127) / 128) >= 256 ? 128 : 64);
}

hipError_t launch_splitk_reduce(hipStream_t s, int epi, const GemmArgs &a, int splits) {
    const int rowblocks = ((a.N + 31) / 32 + 3) / 4;
    const dim3 grid(rowblocks * 16), block(256);   // 4096 elements per row block
    switch (epi) {
    case EPI_BF16: hipLaunchKernelGGL((k_splitk_reduce<EPI_BF16>), grid, block, 0, s, a, splits); break;
    case EPI_RESID: hipLaunchKernelGGL((k_splitk_reduce<EPI_RESID>), grid, block, 0, s, a, splits); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_splitk_reduce<EPI_SWIGLU>), grid, block, 0, s, a, splits); break;
    default: return hipErrorInvalidValue;   // the head runs unsplit
    }
    return hipGetLastError();
}

hipError_t launch_pack(hipStream_t s, const uint16_t *src, uint16_t *dst, int N, int K, int t0, int nt) {
    const long pieces = (long)nt * ((K + 63) / 64) * 8 * 32;
    const int grid = (int)std::min<long>((pieces + 255) / 256, 65536);
    hipLaunchKernelGGL(k_pack, dim3(grid), dim3(256), 0, s, src, dst, N, K, t0, nt);
    return hipGetLastError();
}

hipError_t launch_rope_kv(hipStream_t s, const RopeArgs &a) {
    if (a.nreq < 1 || a.nreq > kMaxRows || a.M < 1 || a.M > kMaxRows || a.rq[0].row0 != 0 ||
        a.rq[a.nreq - 1].row0 + a.rq[a.nreq - 1].n != a.M)
        return hipErrorInvalidValue;
    const int units = a.QH * a.D / 2 + a.KVH * a.D / 2 + a.KVH * a.D;
    hipLaunchKernelGGL(k_rope_kv, dim3(a.M, (units + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_rope_dense(hipStream_t s, const uint16_t *qkv, int ldq, int M, int pos0, int QH, int KVH, int D,
                             const float *cosT, const float *sinT, uint16_t *q_out, uint16_t *Kc, uint16_t *Vc,
                             int cap) {
    if (M < 1 || pos0 + M > cap) return hipErrorInvalidValue;
    const int units = QH * D / 2 + KVH * D / 2 + KVH * D;
    hipLaunchKernelGGL(k_rope_dense, dim3(M, (units + 255) / 256), dim3(256), 0, s, qkv, ldq, pos0, QH, KVH, D, cosT,
                       sinT, q_out, Kc, Vc, cap);
    return hipGetLastError();
}

hipError_t launch_norm_dense(hipStream_t s, const int32_t *tok, const uint16_t *emb, uint16_t *X, const uint16_t *w,
                             float eps, uint16_t *Y, int M, int H) {
    if (M < 1 || H % 8 || H > 8 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_norm_dense, dim3(M), dim3(row_threads(H)), 0, s, tok, emb, X, w, eps, Y, H);
    return hipGetLastError();
}

hipError_t launch_attn(hipStream_t s, int D, const AttnArgs &a) {
    const int rb = (a.G * a.n + 31) / 32;   // compute waves
    if (rb > kAttnComputeWaves) return hipErrorInvalidValue;
    // loader waves only when a split spans more than one chunk of keys: all
    // the waves the CU holds beyond the compute waves, so that a chunk is
    // staged in one pass of loads for up to 24 rows (two passes with two
    // loader waves cost 10 % at 8k context)
    // two waves per block of rows (half the output dims each) when the CU
    // has the waves for them and, with loaders, at least four loader waves
    const bool multi = a.span > kAttnChunk;
    const int ds = 2 * rb + (multi ? 4 : 0) <= kAttnWaves ? 2 : 1;
    const int lw = multi ? kAttnWaves - rb * ds : 0;
    // the loader waves stage a chunk in one pass of kAttnLoadTasks tasks a thread
    if (multi && lw * 64 * kAttnLoadTasks < kAttnChunk / 2 * (D / 8)) return hipErrorInvalidValue;
    const int nz = a.nreq > 0 ? a.nreq : a.zrows > 0 ? (a.M + a.zrows - 1) / a.zrows : 1;
    if (a.zrows > 0 && (a.zrows > kMaxRows || a.M < 1)) return hipErrorInvalidValue;
    if (a.nreq > kMaxRows || (a.nreq > 0 && a.zrows > 0)) return hipErrorInvalidValue;
    for (int r = 0; r < a.nreq; ++r)   // the launch is sized by the largest request
        if (a.rq[r].n > a.n || a.rq[r].nsplit + 1 > a.ns || a.rq[r].span > a.span ||
            (a.rq[r].row0 + a.rq[r].n) * a.G > kMaxRows * kMaxGroup)
            return hipErrorInvalidValue;
    const dim3 grid(a.ns, a.n_qhead / a.G, nz), block(64 * (rb * ds + lw));
    if (D == 128 && ds == 2) hipLaunchKernelGGL((k_attn<128, 2>), grid, block, 0, s, a);
    else if (D == 128) hipLaunchKernelGGL((k_attn<128, 1>), grid, block, 0, s, a);
    else if (D == 64 && ds == 2) hipLaunchKernelGGL((k_attn<64, 2>), grid, block, 0, s, a);
    else if (D == 64) hipLaunchKernelGGL((k_attn<64, 1>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_combine(hipStream_t s, int D, const AttnArgs &a, uint16_t *out) {
    if (a.ns > kAttnMaxSplits || D < kAttnMaxSplits) return hipErrorInvalidValue;
    const dim3 grid(a.n, a.n_qhead, a.nreq > 0 ? a.nreq : a.zrows > 0 ? (a.M + a.zrows - 1) / a.zrows : 1);
    if (D == 128) hipLaunchKernelGGL(k_attn_combine<128>, grid, dim3(128), 0, s, a, out);
    else if (D == 64) hipLaunchKernelGGL(k_attn_combine<64>, grid, dim3(64), 0, s, a, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_residual(hipStream_t s, const float *logits, int ldl, int V, const PassMeta *meta, int n, float T,
                           const double *u_row, void *parts, RowResult *res) {
    const int nchunks = (V + kResChunk - 1) / kResChunk;
    if (n < 1 || n > kMaxRows || V < 1 || nchunks > kResMaxChunks || !(T > 0.f)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_residual_chunks, dim3(nchunks, n), dim3(kResThreads), 0, s, logits, ldl, V, meta, n, T,
                       static_cast<ResPart *>(parts));
    hipLaunchKernelGGL(k_residual_decide, dim3(n), dim3(kResThreads), 0, s, logits, ldl, V, meta, n, T, u_row,
                       static_cast<const ResPart *>(parts), nchunks, res);
    return hipGetLastError();
}

hipError_t launch_top2_reduce(hipStream_t s, const Top2 *part, int ntiles, int M, RowResult *res) {
    hipLaunchKernelGGL(k_top2_reduce, dim3(M), dim3(256), 0, s, part, ntiles, res);
    return hipGetLastError();
}

hipError_t launch_recur_tree(hipStream_t s, int D, const RecurArgs &a) {
    if (a.n < 1 || a.n > kMaxRows) return hipErrorInvalidValue;
    const dim3 grid(a.QH, kRecurSlices), block(recur_threads(D));
    if (D == 128 && a.delta) hipLaunchKernelGGL((k_recur_tree<128, true>), grid, block, 0, s, a);
    else if (D == 128) hipLaunchKernelGGL((k_recur_tree<128, false>), grid, block, 0, s, a);
    else if (D == 64 && a.delta) hipLaunchKernelGGL((k_recur_tree<64, true>), grid, block, 0, s, a);
    else if (D == 64) hipLaunchKernelGGL((k_recur_tree<64, false>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_recur_commit(hipStream_t s, int D, const RecurCommitArgs &a, int n_layers) {
    if (a.path.len < 1 || a.path.len > kMaxRows) return hipErrorInvalidValue;
    const dim3 grid(n_layers * a.QH);
    if (D == 128) hipLaunchKernelGGL(k_recur_commit<128>, grid, dim3(256), 0, s, a);
    else if (D == 64) hipLaunchKernelGGL(k_recur_commit<64>, grid, dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_commit_kv(hipStream_t s, uint16_t *const *kv_ptrs, int n_layers, int KVH, int cap,
                            int D, int ctx, const PathArg &path) {
    if (path.len < 1 || path.len > kMaxRows) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_commit_kv, dim3(n_layers, KVH), dim3(256), 0, s, kv_ptrs, cap, D, ctx, path);
    return hipGetLastError();
}

} // namespace tv
