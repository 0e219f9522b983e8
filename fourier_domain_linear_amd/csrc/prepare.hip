// prepare.hip -- weight preparation: W -> spectral planes (once per weight set), W -> unrolled E,
// and the export kernels that read them back in a canonical layout for checking.
//
// Spectral weights ("Flash EQ-Linear" explainer, "Enfoque Algorítmico"): What_k = sum_d W_d
// exp(-2 pi i d k / G) along the group axis for k = 0..G/2, the same DFT as the activations' (a
// convolution, so no conjugate). Computed in fp32 from the given W (bf16 or fp32), with the inverse
// transform's 1/G (real planes) and 2/G (complex planes) folded in -- exact power-of-two scalings --
// then rounded once to bf16 for the matrix-core path.
//
// Unrolled weight ("Declaración del Problema": the naive layer replicates and cyclically shifts the
// shared weights into a dense matrix): E[o*G+h][i*G+g] = W[o][i][(h-g) mod G].
//
// Every kernel here also serves the dihedral group D4 (d4 = true, G = 8; element a + 4b = r^a s^b):
// its Fourier transform (dft.h) with the 1/8 and 2/8 scalings, and the group product g^-1 h in place
// of h - g.
#include "device_common.h"
#include "eqlin_internal.h"

namespace eqlin {

// One weight element as fp32; half = true: 16-bit elements of type E (bf16 or fp16), else fp32.
template <class E>
__device__ __forceinline__ float load_w(const void *W, bool half, size_t idx) {
    return half ? elem_to_float<E>(((const uint16_t *)W)[idx]) : ((const float *)W)[idx];
}

// The group's forward transform and plane scale, cyclic or D4 (D4 only exists at G = 8).
template <int G>
__device__ __forceinline__ void weight_planes(bool d4, const float *v, float *P) {
    if constexpr (G == 8) {
        if (d4) {
            forward_planes_d4(v, P);
            return;
        }
    }
    forward_planes<G>(v, P);
}

// Index of g^-1 h: the cyclic (h - g) mod G, or D4's product (r^a s^b)^-1 r^c s^d, which is
// r^(c - a) s^d when b = 0 and r^(a - c) s^(1 + d) when b = 1 (s r = r^-1 s).
__device__ __forceinline__ int ginv_h(bool d4, int G, int g, int h) {
    if (!d4) return (h - g + G) % G;
    const int a = g & 3, b = g >> 2, c = h & 3, d = h >> 2;
    return b == 0 ? ((c - a) & 3) + 4 * d : ((a - c) & 3) + 4 * (d ^ 1);
}

// Index of v^-1: -v mod G, or for D4 r^-a for a rotation and v itself for a reflection.
__device__ __forceinline__ int ginv(bool d4, int G, int v) {
    if (!d4) return (G - v) % G;
    return v >= 4 ? v : (4 - v) & 3;
}

// Fragment position of What_p[o][i] in the chunked layouts the forward kernels read. Every chunk is
// 1 KB = one matrix-core operand: 64 lanes x 8 bf16 k-slots; chunk index (ob * KS + ks) * G + p.
// kind 1 (stream kernel, 16x16x32 operands): ob = o / 16, ks = i / 32; lane (g*16 + o%16) holds the
//         8 k-slots j of lane group g, and k-slot (g, j) is the channel the stream kernel's x operand
//         holds there: load q = j / (8/G) of lane group g reads 16-byte piece 4q + g of the K-step and
//         a piece holds 8/G whole channels, so channel c = piece * (8/G) + t has g = piece % 4,
//         j = (piece / 4) * (8/G) + t.
// kind 2 (large-channel kernel, 32x32x16 operands): ob = o / 32, ks = i / 16; lane (h*32 + o%32)
//         holds channels 8h + j of the K-step (natural order).
// Returns a bf16 element index.
__device__ __forceinline__ size_t frag_index(int G, int KS, int kind, int o, int i, int p) {
    int ob, ks, lane, j;
    if (kind == 2) {
        ob = o >> 5;
        ks = i >> 4;
        lane = ((i & 15) >> 3) * 32 + (o & 31);
        j = i & 7;
    } else {
        ob = o >> 4;
        ks = i >> 5;
        const int c = i & 31, w = 8 / G, piece = c / w, t = c % w;
        lane = (piece & 3) * 16 + (o & 15);
        j = (piece >> 2) * w + t;
    }
    return ((((size_t)ob * KS + ks) * G + p) * 64 + lane) * 8 + j;
}

// One thread per (o, i) of the padded domain [NB_total * rows] x [KS * kc]; padding gets zeros.
// planes are stored in E (the layer's half type); W is E as well (w_is_half) or fp32
template <int G, class E>
__global__ void k_prep_frag(const void *__restrict__ W, bool w_is_half, bool d4, int C_out, int C_in, int KS,
                            int NB_total, int kind, uint16_t *__restrict__ frag) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int ipad = KS * (kind == 2 ? 16 : 32), rows = kind == 2 ? 32 : 16;
    if (t >= (int64_t)NB_total * rows * ipad) return;
    const int o = (int)(t / ipad), i = (int)(t % ipad);
    float v[G], P[G];
    const bool live = o < C_out && i < C_in;
#pragma unroll
    for (int d = 0; d < G; ++d) v[d] = live ? load_w<E>(W, w_is_half, ((size_t)o * C_in + i) * G + d) : 0.f;
    weight_planes<G>(d4, v, P);
#pragma unroll
    for (int p = 0; p < G; ++p) frag[frag_index(G, KS, kind, o, i, p)] = pack1<E>(P[p] * group_plane_scale(G, d4, p));
}

template <int G, class E>
__global__ void k_export_frag(const uint16_t *__restrict__ frag, bool d4, int C_out, int C_in, int KS, int kind,
                              float *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)C_out * C_in) return;
    const int o = (int)(t / C_in), i = (int)(t % C_in);
#pragma unroll
    for (int p = 0; p < G; ++p) {
        const float s = elem_to_float<E>(frag[frag_index(G, KS, kind, o, i, p)]);
        out[((size_t)p * C_out + o) * C_in + i] = s / group_plane_scale(G, d4, p);
    }
}

template <int G>
__global__ void k_prep_plain_f32(const float *__restrict__ W, bool d4, int C_out, int C_in,
                                 float *__restrict__ planes) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)C_out * C_in) return;
    float v[G], P[G];
#pragma unroll
    for (int d = 0; d < G; ++d) v[d] = W[t * G + d];
    weight_planes<G>(d4, v, P);
#pragma unroll
    for (int p = 0; p < G; ++p) planes[(size_t)p * C_out * C_in + t] = P[p] * group_plane_scale(G, d4, p);
}

template <int G>
__global__ void k_export_plain_f32(const float *__restrict__ planes, bool d4, int C_out, int C_in,
                                   float *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)C_out * C_in) return;
#pragma unroll
    for (int p = 0; p < G; ++p)
        out[(size_t)p * C_out * C_in + t] = planes[(size_t)p * C_out * C_in + t] / group_plane_scale(G, d4, p);
}

// E[o*G+h][i*G+g] = W[o][i][g^-1 h] ((h-g) mod G for the cyclic group); one thread per element of E.
template <typename T>
__global__ void k_expand(const T *__restrict__ W, bool d4, int G, int C_out, int C_in, T *__restrict__ E) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t cols = (int64_t)C_in * G;
    if (t >= (int64_t)C_out * G * cols) return;
    const int64_t r = t / cols, c = t % cols;
    const int o = (int)(r / G), h = (int)(r % G), i = (int)(c / G), g = (int)(c % G);
    E[t] = W[((int64_t)o * C_in + i) * G + ginv_h(d4, G, g, h)];
}

// Wt[i][o][d] = W[o][i][d^-1] ((G - d) mod G for the cyclic group): the weight of the layer whose
// forward is this layer's data gradient (dx[n, i, g] = sum_{o, h} W[o, i, g^-1 h] dy[n, o, h]
// = sum_{o, h} Wt[i, o, h^-1 g] dy[n, o, h]). Pure index permutation: exact in any element type.
template <typename T>
__global__ void k_transpose_reverse(const T *__restrict__ W, bool d4, int G, int C_out, int C_in, T *__restrict__ Wt) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)C_out * C_in * G) return;
    const int d = (int)(t % G);
    const int64_t io = t / G;
    const int o = (int)(io % C_out), i = (int)(io / C_out);
    Wt[t] = W[((int64_t)o * C_in + i) * G + ginv(d4, G, d)];
}

static inline unsigned blocks_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

#define DISPATCH_G(G, CALL)                     \
    switch (G) {                                \
        case 1: { constexpr int GG = 1; CALL; } break; \
        case 2: { constexpr int GG = 2; CALL; } break; \
        case 4: { constexpr int GG = 4; CALL; } break; \
        case 8: { constexpr int GG = 8; CALL; } break; \
        default: return hipErrorInvalidValue;   \
    }

hipError_t launch_prep_frag(const void *W, bool w_is_half, bool f16, bool d4, int G, int C_out, int C_in, int KS,
                            int NB_total, int kind, void *frag, hipStream_t s) {
    const int64_t n = (int64_t)NB_total * KS * 512;
    if (f16)
        DISPATCH_G(G, hipLaunchKernelGGL((k_prep_frag<GG, F16>), dim3(blocks_for(n, 256)), dim3(256), 0, s, W,
                                         w_is_half, d4, C_out, C_in, KS, NB_total, kind, (uint16_t *)frag))
    else
        DISPATCH_G(G, hipLaunchKernelGGL((k_prep_frag<GG, BF16>), dim3(blocks_for(n, 256)), dim3(256), 0, s, W,
                                         w_is_half, d4, C_out, C_in, KS, NB_total, kind, (uint16_t *)frag))
    return hipGetLastError();
}

hipError_t launch_export_frag(const void *frag, bool f16, bool d4, int G, int C_out, int C_in, int KS, int NB_total,
                              int kind, float *out, hipStream_t s) {
    (void)NB_total;
    const int64_t n = (int64_t)C_out * C_in;
    if (f16)
        DISPATCH_G(G, hipLaunchKernelGGL((k_export_frag<GG, F16>), dim3(blocks_for(n, 256)), dim3(256), 0, s,
                                         (const uint16_t *)frag, d4, C_out, C_in, KS, kind, out))
    else
        DISPATCH_G(G, hipLaunchKernelGGL((k_export_frag<GG, BF16>), dim3(blocks_for(n, 256)), dim3(256), 0, s,
                                         (const uint16_t *)frag, d4, C_out, C_in, KS, kind, out))
    return hipGetLastError();
}

hipError_t launch_prep_plain_f32(const float *W, bool d4, int G, int C_out, int C_in, float *planes,
                                 hipStream_t s) {
    const int64_t n = (int64_t)C_out * C_in;
    DISPATCH_G(G, hipLaunchKernelGGL(k_prep_plain_f32<GG>, dim3(blocks_for(n, 256)), dim3(256), 0, s,
                                     W, d4, C_out, C_in, planes));
    return hipGetLastError();
}

hipError_t launch_export_plain_f32(const float *planes, bool d4, int G, int C_out, int C_in, float *out,
                                   hipStream_t s) {
    const int64_t n = (int64_t)C_out * C_in;
    DISPATCH_G(G, hipLaunchKernelGGL(k_export_plain_f32<GG>, dim3(blocks_for(n, 256)), dim3(256), 0,
                                     s, planes, d4, C_out, C_in, out));
    return hipGetLastError();
}

hipError_t launch_transpose_reverse(const void *W, int elem_bytes, bool d4, int G, int C_out, int C_in, void *Wt,
                                   hipStream_t s) {
    const int64_t n = (int64_t)C_out * C_in * G;
    if (elem_bytes == 2)
        hipLaunchKernelGGL(k_transpose_reverse<uint16_t>, dim3(blocks_for(n, 256)), dim3(256), 0, s,
                           (const uint16_t *)W, d4, G, C_out, C_in, (uint16_t *)Wt);
    else
        hipLaunchKernelGGL(k_transpose_reverse<float>, dim3(blocks_for(n, 256)), dim3(256), 0, s,
                           (const float *)W, d4, G, C_out, C_in, (float *)Wt);
    return hipGetLastError();
}

hipError_t launch_expand(const void *W, int elem_bytes, bool d4, int G, int C_out, int C_in, void *E,
                         hipStream_t s) {
    const int64_t n = (int64_t)C_out * G * C_in * G;
    if (elem_bytes == 2)
        hipLaunchKernelGGL(k_expand<uint16_t>, dim3(blocks_for(n, 256)), dim3(256), 0, s,
                           (const uint16_t *)W, d4, G, C_out, C_in, (uint16_t *)E);
    else
        hipLaunchKernelGGL(k_expand<float>, dim3(blocks_for(n, 256)), dim3(256), 0, s,
                           (const float *)W, d4, G, C_out, C_in, (float *)E);
    return hipGetLastError();
}

}  // namespace eqlin
