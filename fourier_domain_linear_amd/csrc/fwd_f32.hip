// fwd_f32.hip -- the spectral EQ-Linear forward in fp32 (vector ALU), any G in {1, 2, 4, 8} and any
// channel counts. Same method as the bf16 path ("Flash EQ-Linear" explainer, "Enfoque Algorítmico"
// and "Implementación": fp32 kernels alongside the half-precision ones), with fp32 everywhere:
// group DFT of x into LDS, per-frequency channel products (a complex frequency as four real
// products), inverse DFT + bias in registers, one store. The weights arrive as fp32 planes
// [G][C_out][C_in] with the inverse's 1/G and 2/G factors folded in.
//
// Workgroup tile: 32 tokens x 64 outputs, 256 threads; thread t owns token t/8 and the 8 outputs
// o0 + t%8 + 8j. K steps of 16 channels through LDS (rows padded to 17 floats: no bank conflicts).
#include <stdio.h>

#include "act.h"
#include "device_common.h"
#include "eqlin_internal.h"

namespace eqlin {

constexpr int F_TM = 32, F_TN = 64, F_KC = 16, F_PAD = F_KC + 1;

template <int G, bool GELU, bool D4>
__global__ __launch_bounds__(256) void k_fwd_f32(const float *__restrict__ x,
                                                 const float *__restrict__ planes,
                                                 const float *__restrict__ bias, int bias_shift,
                                                 float *__restrict__ y, int64_t N, int C_in,
                                                 int C_out) {
    __shared__ float Xs[G][F_TM][F_PAD];
    __shared__ float Ws[G][F_TN][F_PAD];
    const int t = threadIdx.x;
    const int tm = t >> 3, tj = t & 7;
    const int64_t n0 = (int64_t)blockIdx.x * F_TM;
    const int o0 = blockIdx.y * F_TN;
    const size_t plane_stride = (size_t)C_out * C_in;

    float acc[8][G];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int p = 0; p < G; ++p) acc[j][p] = 0.f;

    for (int k0 = 0; k0 < C_in; k0 += F_KC) {
        // activations: (token, channel) items -> DFT -> planes in LDS
        for (int it = t; it < F_TM * F_KC; it += 256) {
            const int m = it / F_KC, c = it % F_KC;
            const int64_t n = n0 + m;
            const int i = k0 + c;
            float v[G], P[G];
            const bool live = n < N && i < C_in;
#pragma unroll
            for (int g = 0; g < G; ++g) v[g] = live ? x[(n * C_in + i) * G + g] : 0.f;
            group_forward<G, D4>(v, P);
#pragma unroll
            for (int p = 0; p < G; ++p) Xs[p][m][c] = P[p];
        }
        // weights
        for (int it = t; it < G * F_TN * F_KC; it += 256) {
            const int p = it / (F_TN * F_KC), r = it % (F_TN * F_KC);
            const int ol = r / F_KC, c = r % F_KC;
            const int o = o0 + ol, i = k0 + c;
            Ws[p][ol][c] = (o < C_out && i < C_in) ? planes[p * plane_stride + (size_t)o * C_in + i] : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int c = 0; c < F_KC; ++c) {
            float xv[G];
#pragma unroll
            for (int p = 0; p < G; ++p) xv[p] = Xs[p][tm][c];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int ol = tj + 8 * j;
                float wv[G];
#pragma unroll
                for (int p = 0; p < G; ++p) wv[p] = Ws[p][ol][c];
                if constexpr (D4) {
                    // characters: one product each; 2 x 2 irrep: Y_ab += X_a0 W_0b + X_a1 W_1b
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[j][q] = fmaf(xv[q], wv[q], acc[j][q]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int ra = e >> 1, cb = e & 1;
                        acc[j][4 + e] = fmaf(xv[4 + 2 * ra], wv[4 + cb], acc[j][4 + e]);
                        acc[j][4 + e] = fmaf(xv[5 + 2 * ra], wv[6 + cb], acc[j][4 + e]);
                    }
                    continue;
                }
                acc[j][0] = fmaf(xv[0], wv[0], acc[j][0]);
                if constexpr (G >= 2) acc[j][1] = fmaf(xv[1], wv[1], acc[j][1]);
#pragma unroll
                for (int k = 1; k < G / 2; ++k) {
                    const int re = 2 * k, im = 2 * k + 1;
                    acc[j][re] = fmaf(xv[re], wv[re], acc[j][re]);
                    acc[j][re] = fmaf(-xv[im], wv[im], acc[j][re]);
                    acc[j][im] = fmaf(xv[re], wv[im], acc[j][im]);
                    acc[j][im] = fmaf(xv[im], wv[re], acc[j][im]);
                }
            }
        }
        __syncthreads();
    }

    const int64_t n = n0 + tm;
    if (n >= N) return;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int o = o0 + tj + 8 * j;
        if (o >= C_out) continue;
        const float bo = bias ? bias[o >> bias_shift] : 0.f;
        float out[G];
        group_inverse<G, D4>(acc[j], out);
#pragma unroll
        for (int h = 0; h < G; ++h) out[h] += bo;
        apply_act<GELU>(out);
#pragma unroll
        for (int h = 0; h < G; ++h) y[(n * C_out + o) * G + h] = out[h];
    }
}

template <int G, bool D4>
static hipError_t launch_f32(const Plan *p, const void *x, const void *b, void *y, int64_t N, int act,
                             hipStream_t s) {
    const dim3 grid((unsigned)((N + F_TM - 1) / F_TM), (unsigned)((p->C_out + F_TN - 1) / F_TN));
    auto kern = act == EQLIN_ACT_GELU ? k_fwd_f32<G, true, D4> : k_fwd_f32<G, false, D4>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const float *)x, (const float *)p->planes,
                       (const float *)b, p->bias_shift, (float *)y, N, p->C_in, p->C_out);
    return hipGetLastError();
}

bool select_f32(int G, bool d4, int C_in, int C_out, KernelChoice *out) {
    (void)C_in;
    (void)C_out;
    LaunchFn fn = nullptr;
    switch (G) {
        case 1: fn = launch_f32<1, false>; break;
        case 2: fn = launch_f32<2, false>; break;
        case 4: fn = launch_f32<4, false>; break;
        case 8: fn = d4 ? launch_f32<8, true> : launch_f32<8, false>; break;
        default: return false;
    }
    if (d4 && G != 8) return false;
    out->kind = KIND_F32;
    out->nb_tile = F_TN / 16;
    out->tokens_per_block = F_TM;
    out->block_threads = 256;
    out->lds_bytes = (size_t)G * (F_TM + F_TN) * F_PAD * sizeof(float);
    out->launch = fn;
    snprintf(out->name, sizeof(out->name), "f32 valu %s%d tile=%dx%d", d4 ? "D" : "G=", d4 ? 4 : G, F_TM, F_TN);
    return true;
}

}  // namespace eqlin
