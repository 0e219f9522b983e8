// fwd_big.hip -- the spectral EQ-Linear forward for large channel counts (and the unrolled dense
// comparator at large sizes, run as G = 1), bf16 in/out, on v_mfma_f32_32x32x16_bf16.
//
// Method: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
// Transform" (gist.science explainer), "Enfoque Algorítmico" (group DFT -> per-frequency channel
// products, k = 0..G/2) and "Implementación" (one fused kernel, Fourier fragments on chip).
//
// Workgroup tile: BO outputs x BT tokens, all G planes; OW x TW waves, each owning WA x WB blocks of
// 32 outputs x 32 tokens. The channel (K) loop runs in stages of SC input channels (SC*G*2 bytes per
// token row: whole 128-byte lines):
//   - x: raw rows are loaded into registers one stage ahead, transformed (group DFT, fp32) and
//     written to a three-slot LDS ring as bf16 B operands (32 tokens x 16 channels x 1 plane per
//     1 KB chunk), shared by every wave of the workgroup;
//   - weights: fragment chunks (32 outputs x 16 channels x 1 plane per 1 KB) are copied global ->
//     LDS without VGPR staging, two stages ahead, into the same ring (the VGPR file is needed for
//     operands and the DFT; the 256 accumulator registers hold the tile);
//   - products: weights as the A operand (rows = outputs), x planes as B (columns = tokens); a
//     complex frequency is four real products (Re = WrXr - WiXi via a sign-flipped Xi operand).
// Epilogue: the bias sits in the k = 0 accumulator from the start; inverse DFT in fp32; each wave
// stages its 32 x 32 blocks in LDS (XOR-swizzled) and writes whole lines with non-temporal stores.
#include <stdio.h>

#include <algorithm>

#include "device_common.h"
#include "eqlin_internal.h"

namespace eqlin {

template <int G>
struct BigStage {
    static constexpr int SC = G >= 4 ? 16 : 64 / G;  // input channels per pipeline stage
    static constexpr int KSS = SC / 16;              // 32x32x16 K-steps per stage
    static constexpr int GRP = SC / 8;               // 8-channel groups per token row per stage
    static constexpr int SA = G == 1 ? 2 : 1;        // 32-output blocks per epilogue store unit
};

template <int G>
__device__ __forceinline__ void spectral_mfma32(const uint4 (&w)[G], const uint4 (&a)[G],
                                                const uint4 (&an)[G], f32x16 (&acc)[G]) {
    acc[0] = mfma32x32x16(w[0], a[0], acc[0]);
    if constexpr (G >= 2) acc[1] = mfma32x32x16(w[1], a[1], acc[1]);
#pragma unroll
    for (int k = 1; k < G / 2; ++k) {
        const int r = 2 * k, i = 2 * k + 1;
        acc[r] = mfma32x32x16(w[r], a[r], acc[r]);
        acc[r] = mfma32x32x16(w[i], an[i], acc[r]);
        acc[i] = mfma32x32x16(w[i], a[r], acc[i]);
        acc[i] = mfma32x32x16(w[r], a[i], acc[i]);
    }
}

// G samples of 8 channels (element j*G+g) -> G bf16 planes of 8 channels; same as the stream path.
template <int G>
__device__ __forceinline__ void dft8(const uint4 (&r)[G], uint4 (&a)[G]) {
    float pl[G][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v[G], P[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 &q = r[(j * G + g) >> 3];
            const int e = (j * G + g) & 7;
            const uint32_t wd = (e >> 1) == 0 ? q.x : (e >> 1) == 1 ? q.y : (e >> 1) == 2 ? q.z : q.w;
            v[g] = (e & 1) ? __uint_as_float(wd & 0xffff0000u) : __uint_as_float(wd << 16);
        }
        forward_planes<G>(v, P);
#pragma unroll
        for (int p = 0; p < G; ++p) pl[p][j] = P[p];
    }
#pragma unroll
    for (int p = 0; p < G; ++p) a[p] = pack_bf16x8(pl[p]);
}

// One 1 KB chunk global -> LDS (lane l's 16 bytes land at lds_byte + 16 l). Issued as inline asm on
// purpose: the compiler tracks the builtin form as an LDS write and then waits for *all* outstanding
// vector-memory operations before any later LDS read, which would serialise the prefetch pipeline.
// Untracked, it is covered by the kernel's own counted waits; an untracked load can only make the
// compiler's own vmcnt waits stricter (loads complete in issue order), never looser. No register
// output; M0 is set in the same block (nothing else in these kernels uses M0).
__device__ __forceinline__ void chunk_dma(const uint4 *src_lane, uint32_t lds_byte) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_byte), "v"(src_lane)
                 : "memory");
}

__device__ __forceinline__ void st_nt16(uint4 *p, const uint4 &v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

template <int G, int WA, int WB, int OW, int TW>
struct BigCfg {
    static constexpr int NW = OW * TW, NT = NW * 64;
    static constexpr int BO = 32 * WA * OW, BT = 32 * WB * TW;
    static constexpr int KSS = BigStage<G>::KSS, GRP = BigStage<G>::GRP, SA = BigStage<G>::SA;
    static constexpr int XCH = (BT / 32) * KSS * G;         // x-plane chunks per stage (1 KB each)
    static constexpr int WCH = (BO / 32) * KSS * G;         // weight chunks per stage
    static constexpr int DMA_PER_WAVE = WCH / NW;           // weight chunk copies per wave per stage
    static constexpr int STAGE = (XCH + WCH) * 64;          // uint4 per LDS ring slot
    static constexpr int RING = 3;                          // LDS ring slots: weights two stages ahead
    static constexpr int ITEMS = (BT * GRP + NT - 1) / NT;  // x items (token, 8 channels) per thread
    static constexpr int PR = 4 * SA * G;                   // 16-byte pieces per staged output row
    static constexpr int STG = 32 * PR;                     // uint4 of epilogue staging per wave
    static constexpr int LDS_U4 = RING * STAGE > NW * STG ? RING * STAGE : NW * STG;
    static constexpr size_t LDS = (size_t)LDS_U4 * 16 + BO * 4;
    static_assert(WA % SA == 0, "store unit must divide the wave's output blocks");
    static_assert(WCH % NW == 0, "weight chunks must split evenly over the waves");
};

template <int G, int WA, int WB, int OW, int TW>
__global__ __launch_bounds__(OW * TW * 64) void k_big(const uint4 *__restrict__ x4,
                                                      const uint4 *__restrict__ wfrag,
                                                      const uint16_t *__restrict__ bias, int bias_shift,
                                                      uint16_t *__restrict__ y, int64_t N, int C_in,
                                                      int C_out, int n_stages, int KS16, int tiles_t) {
    using C = BigCfg<G, WA, WB, OW, TW>;
    constexpr int KSS = C::KSS, GRP = C::GRP;
    extern __shared__ uint4 lds[];
    float *lbias = reinterpret_cast<float *>(lds + C::LDS_U4);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wo = wave % OW, wt = wave / OW;
    const int tt = blockIdx.x % tiles_t, ot = blockIdx.x / tiles_t;
    const int64_t t0 = (int64_t)tt * C::BT;
    const int o0 = ot * C::BO, ob0 = o0 / 32;

    // LDS ring slot r: [x planes: XCH chunks][weights: WCH chunks]
    auto slot = [&](int st) { return lds + (st % C::RING) * C::STAGE; };

    // ---- loaders: raw x one stage ahead in registers, weights copied global -> LDS ----
    uint4 xr[C::ITEMS][G];
    auto load_x = [&](int stage) {
#pragma unroll
        for (int k = 0; k < C::ITEMS; ++k) {
            const int item = (tid + k * C::NT) % (C::BT * GRP);  // duplicates re-load a real item
            const int tl = item / GRP, c8 = item % GRP;
            int64_t n = t0 + tl;
            n = n < N ? n : N - 1;
            int i0 = (stage * GRP + c8) * 8;
            i0 = i0 < C_in ? i0 : C_in - 8;  // padded channels meet zero weight columns
            const uint4 *p = x4 + ((n * C_in + i0) >> 3) * G;
#pragma unroll
            for (int q = 0; q < G; ++q) xr[k][q] = p[q];
        }
    };
    auto dma_w = [&](int stage) {
        uint4 *wb = slot(stage) + C::XCH * 64;
#pragma unroll
        for (int k = 0; k < C::DMA_PER_WAVE; ++k) {
            const int c = wave + k * C::NW;
            const int obl = c / (KSS * G), rem = c % (KSS * G);
            const uint4 *src = wfrag + ((size_t)((ob0 + obl) * KS16 + stage * KSS) * G + rem) * 64;
            chunk_dma(src + lane, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(wb + c * 64)));
        }
    };
    auto dft_store = [&](int stage) {
        uint4 *xb = slot(stage);
#pragma unroll
        for (int k = 0; k < C::ITEMS; ++k) {
            const int item = (tid + k * C::NT) % (C::BT * GRP);
            const int tl = item / GRP, c8 = item % GRP;
            uint4 a[G];
            dft8<G>(xr[k], a);
            const int sl = (c8 & 1) * 32 + (tl & 31);
#pragma unroll
            for (int p = 0; p < G; ++p) xb[(((tl >> 5) * KSS + (c8 >> 1)) * G + p) * 64 + sl] = a[p];
        }
    };

    // ---- prologue: bias; weights of stages 0 and 1 in flight; x of stage 0 transformed ----
    if (tid < C::BO) {
        const int o = o0 + tid;
        lbias[tid] = (bias && o < C_out) ? __uint_as_float((uint32_t)bias[o >> bias_shift] << 16) : 0.f;
    }
    dma_w(0);
    load_x(0);
    if (n_stages > 1) dma_w(1);
    dft_store(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 acc[WA][WB][G];
#pragma unroll
    for (int a = 0; a < WA; ++a) {
        f32x16 b0;
#pragma unroll
        for (int v = 0; v < 16; ++v) b0[v] = lbias[(wo * WA + a) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)];
#pragma unroll
        for (int b = 0; b < WB; ++b) {
            acc[a][b][0] = b0;
#pragma unroll
            for (int p = 1; p < G; ++p) acc[a][b][p] = f32x16{};
        }
    }

    // ---- main loop: stage s consumes ring slot s%3 (x planes transformed at the end of stage s-1,
    // weights copied since stage s-2). During stage s: request the weights of stage s+2 and the raw x
    // of stage s+1, run the products, transform x of s+1 into slot (s+1)%3, wait for the weights of
    // stage s+1 only (older than this stage's requests), barrier. ----
    for (int s = 0; s < n_stages; ++s) {
        const bool w_ahead = s + 2 < n_stages, x_ahead = s + 1 < n_stages;
        // x first: the transform below waits for it, and loads complete in issue order, so the
        // weight copies of stage s+2 issued after it stay in flight through that wait
        if (x_ahead) load_x(s + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (w_ahead) dma_w(s + 2);
        __builtin_amdgcn_sched_barrier(0);
        const uint4 *xb = slot(s), *wb = slot(s) + C::XCH * 64;
#pragma unroll
        for (int kk = 0; kk < KSS; ++kk)
#pragma unroll
            for (int b = 0; b < WB; ++b) {
                uint4 xf[G], xn[G];
#pragma unroll
                for (int p = 0; p < G; ++p) xf[p] = xb[(((wt * WB + b) * KSS + kk) * G + p) * 64 + lane];
#pragma unroll
                for (int p = 0; p < G; ++p) xn[p] = (p >= 3 && (p & 1)) ? neg_bf16x8(xf[p]) : xf[p];
#pragma unroll
                for (int a = 0; a < WA; ++a) {
                    uint4 wf[G];
#pragma unroll
                    for (int p = 0; p < G; ++p) wf[p] = wb[(((wo * WA + a) * KSS + kk) * G + p) * 64 + lane];
                    spectral_mfma32<G>(wf, xf, xn, acc[a][b]);
                }
            }
        if (x_ahead) dft_store(s + 1);
        // vector-memory ops younger than the weight copies of stage s+1: only those of stage s+2
        // (the x loads of s+1, issued before them, were consumed by the transform)
        if (w_ahead)
            __builtin_amdgcn_s_waitcnt((C::DMA_PER_WAVE & 15) | ((C::DMA_PER_WAVE >> 4) << 14) | (7 << 4));
        else
            __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: inverse DFT, stage, whole-line non-temporal stores ----
    const bool vec_rows = (C_out * G) % 8 == 0;
    const int yrow_pieces = C_out * G / 8;
    uint4 *stg = lds + wave * C::STG;
    const int h = lane >> 5, rcol = lane & 31;
#pragma unroll
    for (int b = 0; b < WB; ++b) {
        const int64_t nblk = t0 + (wt * WB + b) * 32;
#pragma unroll
        for (int a0 = 0; a0 < WA; a0 += C::SA) {
            if (!vec_rows) {
#pragma unroll
                for (int ai = 0; ai < C::SA; ++ai)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int o = o0 + (wo * WA + a0 + ai) * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                        const int64_t n = nblk + rcol;
                        if (o >= C_out || n >= N) continue;
                        float Y[G], out[G];
#pragma unroll
                        for (int p = 0; p < G; ++p) Y[p] = acc[a0 + ai][b][p][v];
                        inverse_planes<G>(Y, out);
#pragma unroll
                        for (int g = 0; g < G; ++g) y[(n * C_out + o) * G + g] = pack_bf16(out[g]);
                    }
                continue;
            }
#pragma unroll
            for (int ai = 0; ai < C::SA; ++ai)
#pragma unroll
                for (int vq = 0; vq < 4; ++vq) {
                    float out[4 * G];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float Y[G];
#pragma unroll
                        for (int p = 0; p < G; ++p) Y[p] = acc[a0 + ai][b][p][4 * vq + v];
                        inverse_planes<G>(Y, out + v * G);
                    }
                    const int ol = ai * 32 + 8 * vq + 4 * h;  // first of the 4 outputs in the unit row
                    if constexpr (G == 1) {
                        uint2 w;
                        w.x = pack_bf16x2(out[0], out[1]);
                        w.y = pack_bf16x2(out[2], out[3]);
                        const int piece = ol / 8;  // 8 outputs x 2 B per piece
                        reinterpret_cast<uint2 *>(stg + rcol * C::PR + (piece ^ (rcol & 7)))[(ol >> 2) & 1] = w;
                    } else {
#pragma unroll
                        for (int k = 0; k < G / 2; ++k) {
                            const int piece = ol * G / 8 + k;
                            stg[rcol * C::PR + (piece ^ (rcol & 7))] = pack_bf16x8(out + 8 * k);
                        }
                    }
                }
            const int piece0 = (o0 + (wo * WA + a0) * 32) * G / 8;
#pragma unroll
            for (int j = 0; j < C::PR / 2; ++j) {
                const int r = j * (64 / C::PR) + lane / C::PR, pc = lane % C::PR;
                const uint4 v = stg[r * C::PR + (pc ^ (r & 7))];
                const int64_t n = nblk + r;
                if (n < N && piece0 + pc < yrow_pieces)
                    st_nt16(reinterpret_cast<uint4 *>(y) + n * yrow_pieces + piece0 + pc, v);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------

template <int G, int WA, int WB, int OW, int TW>
static hipError_t launch_big(const Plan *p, const void *x, const void *b, void *y, int64_t N, hipStream_t s) {
    using C = BigCfg<G, WA, WB, OW, TW>;
    const int64_t tiles_t = (N + C::BT - 1) / C::BT;
    const int tiles_o = p->NB_total / (C::BO / 32);
    const int n_stages = p->KS / C::KSS;
    if (tiles_t * tiles_o > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_big<G, WA, WB, OW, TW>), dim3((unsigned)(tiles_t * tiles_o)), dim3(C::NT), C::LDS, s,
                       (const uint4 *)x, (const uint4 *)p->planes, (const uint16_t *)b, p->bias_shift,
                       (uint16_t *)y, N, p->C_in, p->C_out, n_stages, p->KS, (int)tiles_t);
    return hipGetLastError();
}

template <int G, int WA, int WB, int OW, int TW>
static hipError_t init_big() {
    using C = BigCfg<G, WA, WB, OW, TW>;
    hipError_t e = hipSuccess;
    if (C::LDS > 65536)
        e = hipFuncSetAttribute((const void *)k_big<G, WA, WB, OW, TW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)C::LDS);
    (void)hipGetLastError();
    return e;
}

struct BigEntry {
    int G, BO, BT, KSS, NT;
    size_t lds;
    LaunchFn launch;
    hipError_t (*init)();
    const char *tile;
};
#define BE(G, WA, WB, OW, TW)                                                                            \
    {G, BigCfg<G, WA, WB, OW, TW>::BO, BigCfg<G, WA, WB, OW, TW>::BT, BigCfg<G, WA, WB, OW, TW>::KSS,      \
     BigCfg<G, WA, WB, OW, TW>::NT, BigCfg<G, WA, WB, OW, TW>::LDS, launch_big<G, WA, WB, OW, TW>,         \
     init_big<G, WA, WB, OW, TW>, #WA "x" #WB " blocks/wave, " #OW "x" #TW " waves"}
static const BigEntry kBig[] = {
    BE(1, 2, 4, 4, 1),
    BE(2, 2, 4, 4, 1),
    BE(4, 2, 2, 4, 1),
    BE(8, 1, 2, 4, 1),
};
#undef BE

bool select_big(int G, int C_in, int C_out, KernelChoice *out) {
    (void)C_in;
    (void)C_out;
    for (const auto &e : kBig) {
        if (e.G != G) continue;
        (void)e.init();
        out->kind = KIND_TILED;
        out->frag_kind = 2;
        out->rows_per_block = 32;
        out->kc = 16;
        out->ks_mult = e.KSS;
        out->nb_tile = e.BO / 32;
        out->tokens_per_block = e.BT;
        out->block_threads = e.NT;
        out->lds_bytes = e.lds;
        out->launch = e.launch;
        snprintf(out->name, sizeof(out->name), "bf16 big G=%d BO=%d BT=%d (%s) mfma32x32x16", G, e.BO, e.BT,
                 e.tile);
        return true;
    }
    return false;
}

}  // namespace eqlin
