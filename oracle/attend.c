/*
 * ORACLE -- test infrastructure only.  Nothing in the product library links,
 * loads or calls this file; only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do.
 *
 * Masked softmax attention written out from its definition, in fp64.
 *
 * What it follows: the chunk-wise attention of a causal video DiT, in which
 * a query attends a set of keys chosen by a mask ("Infinite Worlds with
 * Versatile Interactions", paragraph on causal pretraining and the MoBA
 * mask; "Mix Forcing: Causal Pre-Training via Mixture Attention for
 * Interactive World Models", Overview and "Mix the training modes").  The
 * mask itself (which keys a row may see) is decided by the Python side of
 * the oracle and handed in as a list of key intervals per query row.
 *
 * For query row i, head h, and the allowed key set A(i):
 *     s_j   = scale * sum_d q[i][h][d] * k[j][h][d]        for j in A(i)
 *     m     = max_j s_j
 *     out   = sum_j exp(s_j - m) * v[j][h][:] / sum_j exp(s_j - m)
 * Two passes (max, then exponentials), every product and sum in double.
 * A row with an empty A(i) gets an all-zero output.
 *
 * Layout: q [nq][H][D], k and v [nk][H][D], all float32 (bf16 inputs are
 * widened exactly before the call); out [nq][H][D] double.  Intervals of row
 * i are [lo[t], hi[t]) for t in [ptr[i], ptr[i+1]); they must be disjoint
 * and inside [0, nk).  probs, when not NULL, receives the dense [nq][H][nk]
 * softmax matrix (zeros outside A(i)); for tiny shapes only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int oracle_attend(const float* q, int64_t nq, const float* k, const float* v, int64_t nk, int32_t H, int32_t D,
                  const int64_t* ptr, const int64_t* lo, const int64_t* hi, double scale, double* out,
                  double* probs) {
    if (nq < 0 || nk < 0 || H <= 0 || D <= 0) return 1;
    for (int64_t i = 0; i < nq; ++i)
        for (int64_t t = ptr[i]; t < ptr[i + 1]; ++t)
            if (lo[t] < 0 || hi[t] > nk || lo[t] > hi[t]) return 2;
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        if (s == NULL || acc == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t ih = 0; ih < nq * (int64_t)H; ++ih) {
            if (s == NULL || acc == NULL) continue;
            int64_t i = ih / H;
            int32_t h = (int32_t)(ih % H);
            const float* qi = q + (i * H + h) * D;
            double m = -INFINITY;
            int64_t count = 0;
            /* pass 1: scores and their maximum */
            for (int64_t t = ptr[i]; t < ptr[i + 1]; ++t) {
                for (int64_t j = lo[t]; j < hi[t]; ++j) {
                    const float* kj = k + (j * H + h) * D;
                    double dot = 0.0;
                    for (int32_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
                    s[j] = scale * dot;
                    if (s[j] > m) m = s[j];
                    ++count;
                }
            }
            double* oi = out + (i * H + h) * D;
            for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
            double l = 0.0;
            /* pass 2: exponentials, their sum and the weighted sum of values */
            for (int64_t t = ptr[i]; t < ptr[i + 1]; ++t) {
                for (int64_t j = lo[t]; j < hi[t]; ++j) {
                    double p = exp(s[j] - m);
                    s[j] = p;
                    l += p;
                    const float* vj = v + (j * H + h) * D;
                    for (int32_t d = 0; d < D; ++d) acc[d] += p * (double)vj[d];
                }
            }
            for (int32_t d = 0; d < D; ++d) oi[d] = count > 0 ? acc[d] / l : 0.0;
            if (probs != NULL) {
                double* pi = probs + (i * H + h) * nk;
                memset(pi, 0, sizeof(double) * (size_t)nk);
                for (int64_t t = ptr[i]; t < ptr[i + 1]; ++t)
                    for (int64_t j = lo[t]; j < hi[t]; ++j) pi[j] = s[j] / l;
            }
        }
        free(s);
        free(acc);
    }
    return failed ? 3 : 0;
}
