/*
 * CPU oracle primitive: y = W x with bf16 weights and fp64 accumulation.
 *
 * Test infrastructure only (the slow reference the HIP library is checked
 * against).  Nothing in the product library links or calls this file.
 *
 * W is row-major [N, K] bf16 (the upper 16 bits of an IEEE binary32), x and
 * y are fp64.  Each output is one plain left-to-right dot product; OpenMP
 * only splits the outputs between threads, so the result does not depend on
 * the thread count.
 */
#include <stdint.h>
#include <string.h>
#include <omp.h>

static double bf16_to_double(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void orc_matvec_bf16(const uint16_t *W, int64_t N, int64_t K, const double *x, double *y) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        const uint16_t *w = W + n * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) acc += bf16_to_double(w[k]) * x[k];
        y[n] = acc;
    }
}

void orc_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int orc_get_threads(void) { return omp_get_max_threads(); }
