/*
 * based_direct.c - the causal Based forward by its definition, in plain C, float64.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests (through oracle/based_direct_c.py) to check the HIP path;
 * nothing on the product path links or calls it. It shares no code with the HIP kernels.
 *
 * Definition (the page "Write a fast Based (Taylor linear attention) forward kernel", field spec_md, with
 * the argument rules of field contract_md): for every batch b, head h and position t,
 *     s_j = sigma * (q_t . k_j),   A_j = 1 + s_j + s_j^2 / 2          for j = 0 .. t (diagonal included)
 *     o_t = ( sum_j A_j v_j ) / ( sum_j A_j + 1e-6 )
 * Inputs are bfloat16 bit patterns (the top 16 bits of a float32), decoded exactly; every product and sum
 * is float64 and every sum runs over its index in increasing order. One output row costs O(t (K + V)).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline double bf16_value(uint16_t bits) {
    const uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Rows of one (b, h) evaluated together: their keys and values are decoded once. */
#define ROW_BLOCK 256

/*
 * q, k: (B, T, H, K) and v: (B, T, H, V) bfloat16 bits, row-major. rows: `nrows` positions t to evaluate
 * (each in [0, T)), the same for every (b, h); NULL means all T positions in order (nrows = T). out:
 * (B, nrows, H, V) float64, row n of (b, h) at ((b * nrows + n) * H + h) * V. Returns 0, -1 for bad
 * arguments, -2 when memory runs out.
 */
int based_direct_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B, int64_t T,
                      int64_t H, int64_t K, int64_t V, double sigma, const int64_t* rows, int64_t nrows,
                      double* out) {
    if (!q || !k || !v || !out || B < 1 || T < 1 || H < 1 || K < 1 || V < 1) return -1;
    if (!rows) nrows = T;
    for (int64_t n = 0; rows && n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= T) return -1;
    const int64_t blocks = (nrows + ROW_BLOCK - 1) / ROW_BLOCK;
    const int64_t units = B * H * blocks;
    int failed = 0;
#pragma omp parallel
    {
        double* qt = malloc(sizeof(double) * (size_t)K);
        double* kd = malloc(sizeof(double) * (size_t)(T * K));  /* k_j of this (b, h), j = 0 .. T-1 */
        double* vd = malloc(sizeof(double) * (size_t)(T * V));  /* v_j of this (b, h) */
        double* num = malloc(sizeof(double) * (size_t)V);
        if (!qt || !kd || !vd || !num) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (failed) continue;
            const int64_t blk = u % blocks, bh = u / blocks, h = bh % H, b = bh / H;
            const int64_t n0 = blk * ROW_BLOCK, n1 = n0 + ROW_BLOCK < nrows ? n0 + ROW_BLOCK : nrows;
            int64_t tmax = 0;  /* the keys and values the block's rows reach */
            for (int64_t n = n0; n < n1; ++n) {
                const int64_t t = rows ? rows[n] : n;
                if (t > tmax) tmax = t;
            }
            for (int64_t j = 0; j <= tmax; ++j) {
                for (int64_t a = 0; a < K; ++a) kd[j * K + a] = bf16_value(k[((b * T + j) * H + h) * K + a]);
                for (int64_t c = 0; c < V; ++c) vd[j * V + c] = bf16_value(v[((b * T + j) * H + h) * V + c]);
            }
            for (int64_t n = n0; n < n1; ++n) {
                const int64_t t = rows ? rows[n] : n;
                for (int64_t a = 0; a < K; ++a) qt[a] = bf16_value(q[((b * T + t) * H + h) * K + a]);
                for (int64_t c = 0; c < V; ++c) num[c] = 0.0;
                double den = 0.0;
                for (int64_t j = 0; j <= t; ++j) {
                    double dot = 0.0;
                    for (int64_t a = 0; a < K; ++a) dot += qt[a] * kd[j * K + a];
                    const double s = sigma * dot;
                    const double A = 1.0 + s + 0.5 * s * s;
                    den += A;
                    for (int64_t c = 0; c < V; ++c) num[c] += A * vd[j * V + c];
                }
                double* o = out + ((b * nrows + n) * H + h) * V;
                for (int64_t c = 0; c < V; ++c) o[c] = num[c] / (den + 1e-6);
            }
        }
        free(qt);
        free(kd);
        free(vd);
        free(num);
    }
    return failed ? -2 : 0;
}
