/* The oracle's entry points on small layers, built with AddressSanitizer and UBSan. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int64_t oracle_count_kept(const float* w, const uint8_t* mask, int64_t n);
void oracle_csr_from_dense(int32_t M, int32_t crs, const float* w, const uint8_t* mask, int32_t* rowptr,
                           int32_t* colidx, float* value);
void oracle_conv_def(int32_t N, int32_t C, int32_t H, int32_t W, int32_t M, int32_t R, int32_t S, int32_t stride,
                     int32_t pad, const float* x, const float* w, const uint8_t* mask, double* y, double* mag);
void oracle_conv_csr(int32_t N, int32_t C, int32_t H, int32_t W, int32_t M, int32_t R, int32_t S, int32_t stride,
                     int32_t pad, const float* x, const int32_t* rowptr, const int32_t* colidx, const float* value,
                     double* y, double* mag, int32_t nthreads);
int64_t oracle_out_size(int64_t in, int64_t pad, int64_t k, int64_t stride);

int main(void) {
    unsigned seed = 7;
    int bad = 0;
    for (int it = 0; it < 60; it++) {
        seed = seed * 1103515245u + 12345u;
        int N = 1 + (int)(seed >> 8) % 3, C = 1 + (int)(seed >> 12) % 5, M = 1 + (int)(seed >> 16) % 6;
        int R = 1 + (int)(seed >> 20) % 4, S = 1 + (int)(seed >> 24) % 4, st = 1 + (int)(seed >> 4) % 3;
        int pad = (int)(seed >> 28) % 3, H = R + (int)(seed >> 6) % 9, W = S + (int)(seed >> 10) % 9;
        int64_t E = oracle_out_size(H, pad, R, st), F = oracle_out_size(W, pad, S, st);
        int64_t nx = (int64_t)N * C * H * W, nw = (int64_t)M * C * R * S, ny = (int64_t)N * M * E * F;
        float* x = malloc(sizeof(float) * nx);
        float* w = malloc(sizeof(float) * nw);
        uint8_t* mask = malloc(nw);
        for (int64_t i = 0; i < nx; i++) x[i] = (float)((i * 37) % 17) - 8.0f;
        for (int64_t i = 0; i < nw; i++) {
            w[i] = (float)((i * 11) % 7) - 3.0f;
            mask[i] = (uint8_t)((i * 13) % 3 == 0);
        }
        int64_t nnz = oracle_count_kept(w, mask, nw);
        int32_t* rowptr = malloc(sizeof(int32_t) * (M + 1));
        int32_t* colidx = malloc(sizeof(int32_t) * (nnz + 1));
        float* value = malloc(sizeof(float) * (nnz + 1));
        oracle_csr_from_dense(M, C * R * S, w, mask, rowptr, colidx, value);
        double* y1 = calloc(ny + 1, sizeof(double));
        double* m1 = calloc(ny + 1, sizeof(double));
        double* y2 = calloc(ny + 1, sizeof(double));
        double* m2 = calloc(ny + 1, sizeof(double));
        oracle_conv_def(N, C, H, W, M, R, S, st, pad, x, w, mask, y1, m1);
        oracle_conv_csr(N, C, H, W, M, R, S, st, pad, x, rowptr, colidx, value, y2, m2, 1);
        for (int64_t i = 0; i < ny; i++)
            if (y1[i] != y2[i] || m1[i] != m2[i]) bad++;  /* small integers: exact in double */
        free(x); free(w); free(mask); free(rowptr); free(colidx); free(value);
        free(y1); free(m1); free(y2); free(m2);
    }
    printf("oracle forms disagree on %d outputs\n", bad);
    return bad != 0;
}
