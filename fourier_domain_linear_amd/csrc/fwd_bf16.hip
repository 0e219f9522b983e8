// fwd_bf16.hip -- the spectral EQ-Linear forward for bf16 activations on gfx950 matrix cores.
//
// Method: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
// Transform" (gist.science explainer). "Enfoque Algorítmico": the group DFT turns the circular
// convolution over the group axis into one channel product per frequency, and only k = 0..G/2 is
// needed. "Especialización para el Grupo de Rotación p4": at G = 4 the transforms are adds/subtracts
// and the per-frequency work is six real matrix products. "Implementación": one fused kernel, the
// Fourier fragments held in registers / on-chip memory, nothing intermediate written to global
// memory.
//
// Per 16-token row block a wave does, entirely on chip:
//   1. load x[n][i0..i0+7][0..G-1] per lane (16*G contiguous bytes; G is innermost in memory),
//   2. G-point DFT per channel in fp32 registers -> G real planes, rounded once to bf16; these ARE
//      the matrix-core A operands (lane l: token l%16, channels 8*(l/16)..+7), no LDS round trip,
//   3. per frequency: Y_k += X_k * What_k^T on v_mfma_f32_16x16x32_bf16, fp32 accumulation; a complex
//      frequency is four real products (Re = XrWr - XiWi, Im = XrWi + XiWr; the minus is a sign flip
//      of the packed bf16 Xi operand),
//   4. inverse DFT + bias in fp32 registers (the 1/G, 2/G factors are pre-folded into What),
//   5. one bf16 (round-to-nearest-even) store per output element, G contiguous.
//
// Weight fragments. The spectral weights are stored as 1 KB chunks, one per (16 outputs, 32 inputs,
// plane): chunk c = (nb * KS + ks) * G + p holds, for lane l, the 8 bf16 What_p[o][i] with
// o = nb*16 + l%16 and i = ks*32 + 8*(l/16) + j (j = 0..7): exactly the B operand of one matrix-core
// instruction, so a wave's read of a chunk is one linear 1 KB access.
//
// Two kernels:
//   k_rowblock  small channel counts (C_in <= 128): each wave owns 16 tokens x the C_out tile; the
//               tile's weight chunks are copied to LDS once per workgroup (global_load_lds, no VGPR
//               staging); x goes straight from global memory into the A operands.
//   k_tiled     any channel count: workgroup tile BM tokens x BN outputs, 32-channel K steps; the
//               workgroup DFTs its x slab once into LDS (A operands) and copies the weight chunks of
//               the step into LDS; each of the 4 waves computes a WM x WN sub-tile for all G planes.
#include <stdio.h>

#include "device_common.h"
#include "eqlin_internal.h"

namespace eqlin {

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// Copy one 1 KB chunk (64 lanes x 16 B) global -> LDS without a register round trip. `dst` must be
// the same for every lane of the wave (each lane lands at dst + 16 * lane).
__device__ __forceinline__ void chunk_to_lds(const uint4 *src_lane, uint4 *dst_wave) {
    __builtin_amdgcn_global_load_lds((gbl_void *)src_lane, (lds_void *)dst_wave, 16, 0, 0);
}

// One lane's share of a 32-channel step: token n, channels i0..i0+7, all G samples (G uint4).
template <int G>
__device__ __forceinline__ void load_x_step(const uint4 *__restrict__ x4, int64_t n, int64_t N,
                                            int C_in, int i0, uint4 (&r)[G]) {
    if (n < N && i0 < C_in) {
        const uint4 *p = x4 + ((n * C_in + i0) >> 3) * G;
#pragma unroll
        for (int q = 0; q < G; ++q) r[q] = p[q];
    } else {
#pragma unroll
        for (int q = 0; q < G; ++q) r[q] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// G samples of 8 channels (channel-major, sample-minor: element j*G+g) -> G planes of 8 bf16.
template <int G>
__device__ __forceinline__ void dft_to_frags(const uint4 (&r)[G], uint4 (&a)[G]) {
    float pl[G][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v[G], P[G];
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] = bf16_at(r[(j * G + g) >> 3], (j * G + g) & 7);
        forward_planes<G>(v, P);
#pragma unroll
        for (int p = 0; p < G; ++p) pl[p][j] = P[p];
    }
#pragma unroll
    for (int p = 0; p < G; ++p) a[p] = pack_bf16x8(pl[p]);
}

// Negated copies of the imaginary planes (p odd, p >= 3) for the Re = XrWr - XiWi products.
template <int G>
__device__ __forceinline__ void negate_imag(const uint4 (&a)[G], uint4 (&an)[G]) {
#pragma unroll
    for (int p = 0; p < G; ++p) an[p] = (p >= 3 && (p & 1)) ? neg_bf16x8(a[p]) : a[p];
}

// All 2G-2 real products of one (16 tokens x 32 channels) x (32 channels x 16 outputs) block.
template <int G>
__device__ __forceinline__ void spectral_mfma(const uint4 (&a)[G], const uint4 (&an)[G],
                                              const uint4 (&b)[G], f32x4 (&acc)[G]) {
    acc[0] = mfma16x16x32(a[0], b[0], acc[0]);
    if constexpr (G >= 2) acc[1] = mfma16x16x32(a[1], b[1], acc[1]);
#pragma unroll
    for (int k = 1; k < G / 2; ++k) {
        const int r = 2 * k, i = 2 * k + 1;
        acc[r] = mfma16x16x32(a[r], b[r], acc[r]);
        acc[r] = mfma16x16x32(an[i], b[i], acc[r]);
        acc[i] = mfma16x16x32(a[r], b[i], acc[i]);
        acc[i] = mfma16x16x32(a[i], b[r], acc[i]);
    }
}

// Inverse DFT + bias of accumulator row v, then one store of G bf16 at y[n][o][0..G-1].
template <int G>
__device__ __forceinline__ void store_row(const f32x4 (&acc)[G], int v, float bias,
                                          uint16_t *__restrict__ y, int64_t n, int C_out, int o) {
    float Y[G], out[G];
#pragma unroll
    for (int p = 0; p < G; ++p) Y[p] = acc[p][v];
    inverse_planes<G>(Y, out);
    uint16_t *dst = y + (n * C_out + o) * G;
    if constexpr (G == 1) {
        *dst = pack_bf16(out[0] + bias);
    } else if constexpr (G == 2) {
        *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(out[0] + bias, out[1] + bias);
    } else if constexpr (G == 4) {
        uint2 w;
        w.x = pack_bf16x2(out[0] + bias, out[1] + bias);
        w.y = pack_bf16x2(out[2] + bias, out[3] + bias);
        *reinterpret_cast<uint2 *>(dst) = w;
    } else {
        float t[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) t[h] = out[h] + bias;
        *reinterpret_cast<uint4 *>(dst) = pack_bf16x8(t);
    }
}

__device__ __forceinline__ float load_bias(const uint16_t *__restrict__ bias, int idx) {
    return bias ? __uint_as_float((uint32_t)bias[idx] << 16) : 0.0f;
}

// ------------------------------------------------------------------------------------------------
// k_rowblock<G, KS, NB, NW>: NW waves x 16 tokens per workgroup, NB output blocks of 16 per wave.
// grid = (ceil(N / (16 NW)), NB_total / NB). Dynamic LDS = NB * KS * G KB (the tile's weights).
template <int G, int KS, int NB, int NW>
__global__ __launch_bounds__(NW * 64) void k_rowblock(const uint4 *__restrict__ x4,
                                                      const uint4 *__restrict__ wfrag,
                                                      const uint16_t *__restrict__ bias,
                                                      int bias_shift, uint16_t *__restrict__ y,
                                                      int64_t N, int C_in, int C_out) {
    extern __shared__ uint4 lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n_base = (int64_t)blockIdx.x * (NW * 16) + wave * 16;
    const int nb0 = blockIdx.y * NB;

    // 1. this wave's activations: all K steps in flight at once
    uint4 xr[KS][G];
    const int64_t n_ld = n_base + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_x_step<G>(x4, n_ld, N, C_in, ks * 32 + (lane >> 4) * 8, xr[ks]);

    // 2. the C_out tile's weight chunks -> LDS (contiguous in global memory for a tile)
    constexpr int CHUNKS = NB * KS * G;
    const uint4 *src = wfrag + (size_t)nb0 * KS * G * 64;
    for (int c = wave; c < CHUNKS; c += NW) chunk_to_lds(src + c * 64 + lane, lds + c * 64);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // 3. DFT -> A operands, then the per-frequency products for every output block
    f32x4 acc[NB][G];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int p = 0; p < G; ++p) acc[nb][p] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 a[G], an[G];
        dft_to_frags<G>(xr[ks], a);
        negate_imag<G>(a, an);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint4 bw[G];
#pragma unroll
            for (int p = 0; p < G; ++p) bw[p] = lds[((nb * KS + ks) * G + p) * 64 + lane];
            spectral_mfma<G>(a, an, bw, acc[nb]);
        }
    }

    // 4./5. inverse DFT + bias, store
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int o = (nb0 + nb) * 16 + (lane & 15);
        if (o >= C_out) continue;
        const float bo = load_bias(bias, o >> bias_shift);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t n = n_base + 4 * (lane >> 4) + v;
            if (n < N) store_row<G>(acc[nb], v, bo, y, n, C_out, o);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// k_tiled<G, BM, BN, WM, WN>: 4 waves, (BM/WM) x (BN/WN) == 4. grid = (ceil(N/BM), NB_total/(BN/16)).
// LDS per K step: A planes [G][BM/16] chunks + B chunks [BN/16][G], 1 KB each.
template <int G, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_tiled(const uint4 *__restrict__ x4,
                                               const uint4 *__restrict__ wfrag,
                                               const uint16_t *__restrict__ bias, int bias_shift,
                                               uint16_t *__restrict__ y, int64_t N, int C_in,
                                               int C_out, int KS) {
    static_assert((BM / WM) * (BN / WN) == 4, "4 waves per workgroup");
    constexpr int MB = BM / 16, WMB = WM / 16, WNB = WN / 16, BNB = BN / 16;
    constexpr int ITEMS = BM * 4 / 256;  // (token, 8-channel group) items per thread per K step
    static_assert(ITEMS >= 1 && BM * 4 % 256 == 0, "BM must be a multiple of 64");
    extern __shared__ uint4 lds[];
    uint4 *ldsA = lds;                  // [G][MB][64]
    uint4 *ldsB = lds + G * MB * 64;    // [BNB][G][64]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / (BN / WN), wn = wave % (BN / WN);
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int nb0 = blockIdx.y * BNB;

    f32x4 acc[WMB][WNB][G];
#pragma unroll
    for (int mi = 0; mi < WMB; ++mi)
#pragma unroll
        for (int ni = 0; ni < WNB; ++ni)
#pragma unroll
            for (int p = 0; p < G; ++p) acc[mi][ni][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int ks = 0; ks < KS; ++ks) {
        // weights of this K step -> LDS
        for (int c = wave; c < BNB * G; c += 4) {
            const int nbl = c / G, p = c % G;
            const uint4 *src = wfrag + ((size_t)((nb0 + nbl) * KS + ks) * G + p) * 64;
            chunk_to_lds(src + lane, ldsB + c * 64);
        }
        // activations of this K step: DFT once per workgroup -> A operand chunks in LDS
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = threadIdx.x + it * 256;
            const int m = item >> 2, kg = item & 3;
            uint4 r[G], a[G];
            load_x_step<G>(x4, m0 + m, N, C_in, ks * 32 + kg * 8, r);
            dft_to_frags<G>(r, a);
#pragma unroll
            for (int p = 0; p < G; ++p) ldsA[(p * MB + (m >> 4)) * 64 + kg * 16 + (m & 15)] = a[p];
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        uint4 a[WMB][G], an[WMB][G];
#pragma unroll
        for (int mi = 0; mi < WMB; ++mi) {
#pragma unroll
            for (int p = 0; p < G; ++p) a[mi][p] = ldsA[(p * MB + wm * WMB + mi) * 64 + lane];
            negate_imag<G>(a[mi], an[mi]);
        }
#pragma unroll
        for (int ni = 0; ni < WNB; ++ni) {
            uint4 bw[G];
#pragma unroll
            for (int p = 0; p < G; ++p) bw[p] = ldsB[((wn * WNB + ni) * G + p) * 64 + lane];
#pragma unroll
            for (int mi = 0; mi < WMB; ++mi) spectral_mfma<G>(a[mi], an[mi], bw, acc[mi][ni]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int ni = 0; ni < WNB; ++ni) {
        const int o = (nb0 + wn * WNB + ni) * 16 + (lane & 15);
        if (o >= C_out) continue;
        const float bo = load_bias(bias, o >> bias_shift);
#pragma unroll
        for (int mi = 0; mi < WMB; ++mi) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t n = m0 + (wm * WMB + mi) * 16 + 4 * (lane >> 4) + v;
                if (n < N) store_row<G>(acc[mi][ni], v, bo, y, n, C_out, o);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Launchers and selection.

// Raise the kernel's dynamic-LDS limit above 64 KB where needed (gfx950 has 160 KB per CU). A
// refusal is not fatal here: the launch itself then reports the error.
static hipError_t set_lds_limit(const void *fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    (void)hipGetLastError();
    return e;
}

template <int G, int KS, int NB>
static hipError_t launch_rowblock(const Plan *p, const void *x, const void *b, void *y, int64_t N,
                                  hipStream_t s) {
    constexpr int NW = 4;
    const auto fn = k_rowblock<G, KS, NB, NW>;
    const size_t lds = (size_t)NB * KS * G * 1024;
    const dim3 grid((unsigned)((N + NW * 16 - 1) / (NW * 16)), (unsigned)(p->NB_total / NB));
    hipLaunchKernelGGL(fn, grid, dim3(NW * 64), lds, s, (const uint4 *)x, (const uint4 *)p->planes,
                       (const uint16_t *)b, p->bias_shift, (uint16_t *)y, N, p->C_in, p->C_out);
    return hipGetLastError();
}

template <int G, int KS, int NB>
static hipError_t init_rowblock() {
    return set_lds_limit((const void *)k_rowblock<G, KS, NB, 4>, (size_t)NB * KS * G * 1024);
}

template <int G, int BM, int BN, int WM, int WN>
static hipError_t launch_tiled(const Plan *p, const void *x, const void *b, void *y, int64_t N,
                               hipStream_t s) {
    const auto fn = k_tiled<G, BM, BN, WM, WN>;
    const size_t lds = (size_t)(G * (BM / 16) + (BN / 16) * G) * 1024;
    const dim3 grid((unsigned)((N + BM - 1) / BM), (unsigned)(p->NB_total / (BN / 16)));
    hipLaunchKernelGGL(fn, grid, dim3(256), lds, s, (const uint4 *)x, (const uint4 *)p->planes,
                       (const uint16_t *)b, p->bias_shift, (uint16_t *)y, N, p->C_in, p->C_out, p->KS);
    return hipGetLastError();
}

template <int G, int BM, int BN, int WM, int WN>
static hipError_t init_tiled() {
    return set_lds_limit((const void *)k_tiled<G, BM, BN, WM, WN>,
                         (size_t)(G * (BM / 16) + (BN / 16) * G) * 1024);
}

struct RowblockEntry {
    int G, KS, NB;
    LaunchFn launch;
    hipError_t (*init)();
};
#define RB(G, KS, NB) {G, KS, NB, launch_rowblock<G, KS, NB>, init_rowblock<G, KS, NB>}
static const RowblockEntry kRowblock[] = {
    RB(1, 1, 8), RB(1, 2, 8), RB(1, 3, 8), RB(1, 4, 8),
    RB(2, 1, 8), RB(2, 2, 8), RB(2, 3, 8), RB(2, 4, 8),
    RB(4, 1, 4), RB(4, 2, 4), RB(4, 3, 4), RB(4, 4, 4),
    RB(4, 1, 6), RB(4, 2, 6), RB(4, 3, 6),
    RB(8, 1, 4), RB(8, 2, 4), RB(8, 3, 2), RB(8, 4, 2),
};
#undef RB

struct TiledEntry {
    int G, BM, BN;
    LaunchFn launch;
    hipError_t (*init)();
};
#define TL(G, BM, BN, WM, WN) {G, BM, BN, launch_tiled<G, BM, BN, WM, WN>, init_tiled<G, BM, BN, WM, WN>}
static const TiledEntry kTiled[] = {
    TL(1, 128, 128, 64, 64),
    TL(2, 128, 128, 64, 64),
    TL(4, 128, 64, 64, 32),
    TL(8, 64, 64, 32, 32),
};
#undef TL

bool select_bf16(int G, int C_in, int C_out, KernelChoice *out) {
    const int KS = (C_in + 31) / 32;
    const int nb_needed = (C_out + 15) / 16;
    // Rowblock when the whole (or half the) output fits one or two tiles and C_in <= 128: the DFT is
    // then done at most twice per token and x streams straight into registers.
    const RowblockEntry *best = nullptr;
    int best_waste = 1 << 30;
    for (const auto &e : kRowblock) {
        if (e.G != G || e.KS != KS) continue;
        const int tiles = (nb_needed + e.NB - 1) / e.NB;
        if (tiles > 2) continue;
        const int waste = tiles * e.NB - nb_needed;
        if (waste < best_waste || (waste == best_waste && best && e.NB > best->NB)) {
            best = &e;
            best_waste = waste;
        }
    }
    if (best) {
        (void)best->init();
        out->kind = KIND_ROWBLOCK;
        out->nb_tile = best->NB;
        out->tokens_per_block = 64;
        out->block_threads = 256;
        out->lds_bytes = (size_t)best->NB * KS * G * 1024;
        out->launch = best->launch;
        snprintf(out->name, sizeof(out->name), "bf16 rowblock G=%d KS=%d NB=%d waves=4", G, KS, best->NB);
        return true;
    }
    for (const auto &e : kTiled) {
        if (e.G != G) continue;
        (void)e.init();
        out->kind = KIND_TILED;
        out->nb_tile = e.BN / 16;
        out->tokens_per_block = e.BM;
        out->block_threads = 256;
        out->lds_bytes = (size_t)(G * (e.BM / 16) + (e.BN / 16) * G) * 1024;
        out->launch = e.launch;
        snprintf(out->name, sizeof(out->name), "bf16 tiled G=%d BM=%d BN=%d KS=%d", G, e.BM, e.BN, KS);
        return true;
    }
    return false;
}

}  // namespace eqlin
