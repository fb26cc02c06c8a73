// tv_linear_noalloc: the projection kernels of tv_linear for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It needs no context: its scratch
// (the zero block the activation staging reads beyond M and K, the split-K
// partials and the fp32 path's top-2 candidates) lives in one file-scope
// device array per GPU, looked up once per device, and the call only
// enqueues work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "../../include/treeverify.h"
#include "tv_internal.h"

using namespace tv;

namespace {

// Scratch layout: [0, 256) zeros (never written: static device memory starts
// zeroed), then the split-K partials, then the top-2 candidates.
constexpr size_t kZeroBytes = 256;
constexpr size_t kPartialBytes = (size_t)512 * 4096 * 4;   // rowblocks x splits <= 512 tiles of 4096 floats
constexpr size_t kCandBytes = (size_t)4 << 20;             // M x ceil(N/128) top-2 candidates of 16 bytes
constexpr size_t kScratchBytes = kZeroBytes + kPartialBytes + kCandBytes;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// message of the last failed call on this thread (a fixed buffer: no
// allocation on any path)
thread_local char g_last_error[256] = "no error";

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

// The device address of this GPU's scratch array.  The array's name in host
// code is only a stand-in for the symbol, so every host use goes through the
// address hipGetSymbolAddress returns on the device that is current.
int scratch_ptr(unsigned char **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TV_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(TV_EINVAL, "device index %d out of range", dev);
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_err[dev] != hipSuccess || !g_ptr[dev])
        return fail(TV_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(g_err[dev]));
    *out = static_cast<unsigned char *>(g_ptr[dev]);
    return TV_OK;
}

} // namespace

namespace tv {
const char *noalloc_last_error() { return g_last_error; }
}

extern "C" int tv_linear_noalloc(const void *x, const void *w, int M, int N, int K, void *y, int y_fp32,
                                 void *stream) {
    if (!x || !w || !y) return fail(TV_EINVAL, "tv_linear_noalloc: null operand");
    if (M < 1 || N < 1 || K < 8 || K % 8)
        return fail(TV_EINVAL, "tv_linear_noalloc: shape M=%d N=%d K=%d not supported", M, N, K);
    const int rowblocks = ((N + 31) / 32 + 3) / 4;
    const bool skinny = M <= kMaxRows;
    const int S = (skinny && !y_fp32) ? gemm_splits(N, K) : 1;
    const size_t part_need = S > 1 ? (size_t)rowblocks * S * 4096 * 4 : 0;
    const size_t cand_need = (skinny && y_fp32) ? (size_t)M * rowblocks * sizeof(Top2) : 0;
    if (part_need > kPartialBytes || cand_need > kCandBytes)
        return fail(TV_EINVAL,
                    "tv_linear_noalloc: M=%d N=%d K=%d needs %zu bytes of split-K partials and %zu of candidates; "
                    "the static scratch holds %zu and %zu",
                    M, N, K, part_need, cand_need, kPartialBytes, kCandBytes);
    unsigned char *base = nullptr;
    int rc = scratch_ptr(&base);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    GemmArgs g{};
    g.X = static_cast<const uint16_t *>(x); g.ldx = K;
    g.W = static_cast<const uint16_t *>(w);
    g.M = M; g.N = N; g.K = K;
    g.zeros = base;
    g.partial = reinterpret_cast<float *>(base + kZeroBytes);
    g.part = reinterpret_cast<Top2 *>(base + kZeroBytes + kPartialBytes);
    hipError_t e;
    if (!skinny) {
        if (y_fp32) { g.Yf = static_cast<float *>(y); g.ldyf = N; }
        else { g.Y = static_cast<uint16_t *>(y); g.ldy = N; }
        e = launch_gemm_dense(s, y_fp32 ? EPI_F32 : EPI_BF16, g);
    } else if (y_fp32) {
        g.Yf = static_cast<float *>(y); g.ldyf = N;
        e = launch_gemm(s, EPI_HEAD, g, 1);
    } else {
        g.Y = static_cast<uint16_t *>(y); g.ldy = N;
        e = launch_gemm(s, EPI_BF16, g, S);
        if (e == hipSuccess && S > 1) e = launch_splitk_reduce(s, EPI_BF16, g, S);
    }
    if (e != hipSuccess) return fail(TV_EHIP, "tv_linear_noalloc: launch failed: %s", hipGetErrorString(e));
    return TV_OK;
}
