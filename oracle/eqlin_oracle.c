/*
 * eqlin_oracle.c -- plain fp64 CPU oracle for the cyclic-group equivariant linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU path never calls it, and the two share no code:
 * no kernels, headers, helpers or tables.
 *
 * What it follows: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete
 * Fourier Transform" (explainer page, gist.science/es/paper/2607.21271).
 *   - Section "Declaración del Problema": the usual EQ-Linear unrolls its shared, structured weights
 *     into a dense matrix and hands it to a generic dense product.
 *   - Section "Percepción Central": that dense matrix is group-circulant -- each block row is a cyclic
 *     shift of one learnable parameter set -- so the layer is a circular convolution along the group
 *     axis composed with a linear map along channels.
 *   - Section "Principales Contribuciones": the fast method is exact, i.e. it must reach the same
 *     result as the unrolled product up to floating-point rounding.
 * The oracle therefore does the unrolled product and nothing cleverer: it materialises the
 * (C_out*G) x (C_in*G) matrix E with E[o*G+h][i*G+g] = W[o][i][(h-g) mod G] (the circular
 * convolution read of the group index, h minus g), and forms y = E x + b with b[o] broadcast over h,
 * in fp64, one fixed summation order (c ascending), OpenMP over tokens only.
 *
 * The half-spectrum weight transform (eqlin_oracle_dft_weights) is the textbook DFT definition along
 * the group axis, kept to check the library's spectral weights: section "Enfoque Algorítmico"
 * (transform to the frequency domain; only the non-redundant half of a real signal's spectrum).
 *
 * The gradients of the same layer (the pages' operator has a backward pass: section
 * "Implementación", forward and backward kernels; "Resultados Experimentales", backward speedups)
 * follow from the unrolled product by the chain rule and nothing else: with y = E x + b,
 *   dx = E^T dy,
 *   dE = dy^T x summed over tokens, and since E[o*G+h][i*G+g] = W[o][i][(h-g) mod G] each W entry
 *   collects the dE entries it was copied to: dW[o][i][d] = sum over h of dE[o*G+h][i*G+(h-d) mod G],
 *   db[o] = sum over tokens and h of dy[n][o*G+h].
 *
 * Layouts (all row-major, fp64): x[N][C_in][G], W[C_out][C_in][G], b[C_out] (or NULL),
 * y[N][C_out][G], E[C_out*G][C_in*G]; spectral re/im[C_out][C_in][G/2+1]; dy like y, dx like x,
 * dW like W, db like b.
 * Return value: 0 on success, -1 on a bad argument, -2 when memory runs out.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads for one call: nthreads > 0 asks for that many, else OpenMP's default. Passed as a clause
 * of the call's parallel loop, so one call's request does not change the next call's default. */
static int team_size(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int eqlin_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* E[o*G+h][i*G+g] = W[o][i][(h-g) mod G]: the unrolled block-circulant weight. */
int eqlin_oracle_expand(const double *W, int64_t C_out, int64_t C_in, int64_t G, double *E) {
    if (!W || !E || C_out <= 0 || C_in <= 0 || G <= 0) return -1;
    const int64_t cols = C_in * G;
    for (int64_t o = 0; o < C_out; ++o)
        for (int64_t h = 0; h < G; ++h)
            for (int64_t i = 0; i < C_in; ++i)
                for (int64_t g = 0; g < G; ++g) {
                    int64_t d = ((h - g) % G + G) % G;
                    E[(o * G + h) * cols + i * G + g] = W[(o * C_in + i) * G + d];
                }
    return 0;
}

/* y[n][r] = b[r / G] + sum_{c} E[r][c] * x[n][c], r = o*G+h, c = i*G+g, c ascending. */
int eqlin_oracle_forward(const double *x, const double *W, const double *b, double *y, int64_t N,
                         int64_t C_out, int64_t C_in, int64_t G, int nthreads) {
    if (N < 0 || C_out <= 0 || C_in <= 0 || G <= 0 || !W) return -1;
    if (N == 0) return 0;
    if (!x || !y) return -1;
    const int64_t rows = C_out * G, cols = C_in * G;
    double *E = (double *)malloc((size_t)(rows * cols) * sizeof(double));
    if (!E) return -2;
    eqlin_oracle_expand(W, C_out, C_in, G, E);
    const int nt = team_size(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t n = 0; n < N; ++n) {
        const double *xn = x + n * cols;
        double *yn = y + n * rows;
        for (int64_t r = 0; r < rows; ++r) {
            const double *er = E + r * cols;
            double acc = 0.0;
            for (int64_t c = 0; c < cols; ++c) acc += er[c] * xn[c];
            yn[r] = acc + (b ? b[r / G] : 0.0);
        }
    }
    free(E);
    return 0;
}

/* Textbook DFT along the group axis, non-redundant half k = 0..G/2:
 *   What[o][i][k] = sum_d W[o][i][d] * exp(-2*pi*I*d*k/G).                                       */
int eqlin_oracle_dft_weights(const double *W, int64_t C_out, int64_t C_in, int64_t G, double *re,
                             double *im) {
    if (!W || !re || !im || C_out <= 0 || C_in <= 0 || G <= 0) return -1;
    const int64_t K = G / 2 + 1;
    const double two_pi = 6.283185307179586476925286766559;
    for (int64_t o = 0; o < C_out; ++o)
        for (int64_t i = 0; i < C_in; ++i)
            for (int64_t k = 0; k < K; ++k) {
                double sr = 0.0, si = 0.0;
                for (int64_t d = 0; d < G; ++d) {
                    double w = W[(o * C_in + i) * G + d];
                    double ang = two_pi * (double)((d * k) % G) / (double)G;
                    sr += w * cos(ang);
                    si -= w * sin(ang);
                }
                re[(o * C_in + i) * K + k] = sr;
                im[(o * C_in + i) * K + k] = si;
            }
    return 0;
}

/* dx[n][c] = sum_r E[r][c] * dy[n][r], r = o*G+h, c = i*G+g, r ascending (the transpose of the
 * unrolled product; the bias does not depend on x). */
int eqlin_oracle_backward_data(const double *dy, const double *W, double *dx, int64_t N, int64_t C_out,
                               int64_t C_in, int64_t G, int nthreads) {
    if (N < 0 || C_out <= 0 || C_in <= 0 || G <= 0 || !W) return -1;
    if (N == 0) return 0;
    if (!dy || !dx) return -1;
    const int64_t rows = C_out * G, cols = C_in * G;
    double *E = (double *)malloc((size_t)(rows * cols) * sizeof(double));
    if (!E) return -2;
    eqlin_oracle_expand(W, C_out, C_in, G, E);
    const int nt = team_size(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t n = 0; n < N; ++n) {
        const double *dyn = dy + n * rows;
        double *dxn = dx + n * cols;
        for (int64_t c = 0; c < cols; ++c) {
            double acc = 0.0;
            for (int64_t r = 0; r < rows; ++r) acc += E[r * cols + c] * dyn[r];
            dxn[c] = acc;
        }
    }
    free(E);
    return 0;
}

/* dE[r][c] = sum_n dy[n][r] * x[n][c] (n ascending); dW[o][i][d] = sum_h dE[o*G+h][i*G+(h-d) mod G]
 * (h ascending); db[o] = sum_n sum_h dy[n][o*G+h] (n, then h ascending). db may be NULL. */
int eqlin_oracle_backward_weights(const double *x, const double *dy, double *dW, double *db, int64_t N,
                                  int64_t C_out, int64_t C_in, int64_t G, int nthreads) {
    if (N < 0 || C_out <= 0 || C_in <= 0 || G <= 0 || !dW) return -1;
    if (N > 0 && (!x || !dy)) return -1;
    const int64_t rows = C_out * G, cols = C_in * G;
    int failed = 0;
    const int nt = team_size(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt) reduction(| : failed)
    for (int64_t o = 0; o < C_out; ++o) {
        /* the G rows of dE that belong to output channel o */
        double *dE = (double *)malloc((size_t)(G * cols) * sizeof(double));
        if (!dE) {
            failed = 1;
            continue;
        }
        for (int64_t k = 0; k < G * cols; ++k) dE[k] = 0.0;
        double bsum = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double *xn = x + n * cols;
            for (int64_t h = 0; h < G; ++h) {
                const double d = dy[n * rows + o * G + h];
                bsum += d;
                double *row = dE + h * cols;
                for (int64_t c = 0; c < cols; ++c) row[c] += d * xn[c];
            }
        }
        for (int64_t i = 0; i < C_in; ++i)
            for (int64_t d = 0; d < G; ++d) {
                double acc = 0.0;
                for (int64_t h = 0; h < G; ++h) acc += dE[h * cols + i * G + ((h - d) % G + G) % G];
                dW[(o * C_in + i) * G + d] = acc;
            }
        if (db) db[o] = bsum;
        free(dE);
    }
    return failed ? -2 : 0;
}
