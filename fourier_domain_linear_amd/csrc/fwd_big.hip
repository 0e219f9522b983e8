// fwd_big.hip -- the spectral EQ-Linear forward for large channel counts (and the unrolled dense
// comparator at large sizes, run as G = 1), bf16 in/out, on v_mfma_f32_32x32x16_bf16.
//
// Method: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
// Transform" (gist.science explainer), "Enfoque Algorítmico" (group DFT -> per-frequency channel
// products, k = 0..G/2) and "Implementación" (one fused kernel, Fourier fragments on chip).
//
// Workgroup tile: BO outputs x BT tokens, all G planes; OW x TW waves, each owning WA x WB blocks of
// 32 outputs x 32 tokens. The channel (K) loop runs in stages of SC input channels (SC*G*2 bytes per
// token row: whole 128-byte lines), two stages per loop trip so every register slot is fixed:
//   - x: raw rows are loaded into a two-slot register ring two stages ahead (HBM latency spans
//     several stages of products), transformed (group DFT, fp32) one stage ahead and written to one
//     of two LDS buffers as bf16 B operands (32 tokens x 16 channels x 1 plane per 1 KB chunk),
//     shared by every wave of the workgroup; each thread transforms distinct (token, 4 or 8
//     channel) items, so no transform is repeated;
//   - weights: each wave owns distinct output rows, so LDS staging would buy no reuse: fragment
//     chunks (32 outputs x 16 channels x 1 plane per 1 KB, one coalesced load per wave) go straight
//     into a two-slot register ring one stage ahead (they are L2 hits: every token tile of an output
//     tile reads the same ones);
//   - products: weights as the A operand (rows = outputs), x planes as B (columns = tokens); a
//     complex frequency is four real products (Re = WrXr - WiXi via a sign-flipped Xi operand).
// All global loads are plain loads, so the compiler's waits count exactly the ones in flight; the
// per-stage barrier waits for LDS only.
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

// G samples of NCH channels (element j*G+g) -> G planes of NCH bf16 (NCH = 4 or 8).
template <int G, int NCH>
__device__ __forceinline__ void dft_ch(const uint4 (&r)[NCH * G / 8], float (&pl)[G][NCH]) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
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
}

// Workgroup barrier that orders LDS only: outstanding global loads stay in flight across it (the
// fence in __syncthreads would wait for them too).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
    asm volatile("s_barrier" ::: "memory");
}

// Scheduling pattern for one region of a stage: a 32x32x16 product keeps the matrix core busy for
// 32 cycles while the wave goes on issuing independent instructions, so the region's loads and the
// transform's vector ALU work are spread over its NM products: the region's NR LDS reads first,
// then after each product one global load (the first NV products) and up to VPM vector ALU
// instructions.
template <int NR, int NM, int NV, int VPM>
__device__ __forceinline__ void interleave_stage() {
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // LDS reads, as one batch
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // vector ALU
    }
}

__device__ __forceinline__ void st_nt16(uint4 *p, const uint4 &v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

template <int V>
struct IC {
    static constexpr int value = V;
};

template <int G, int WA, int WB, int OW, int TW>
struct BigCfg {
    static constexpr int NW = OW * TW, NT = NW * 64;
    static constexpr int BO = 32 * WA * OW, BT = 32 * WB * TW;
    static constexpr int SC = BigStage<G>::SC, KSS = BigStage<G>::KSS, GRP = BigStage<G>::GRP;
    static constexpr int SA = BigStage<G>::SA;
    // x work items: (token, NCH channels); NCH = 4 where 8-channel items would leave threads idle
    static constexpr int NCH = (G >= 2 && BT * GRP < NT) ? 4 : 8;
    static constexpr int ITEMS = BT * (SC / NCH) / NT;      // x items per thread per stage
    static constexpr int XU4 = NCH * G / 8;                 // uint4 of raw x per item
    static constexpr int XST = (BT / 32) * KSS * G * 64;    // uint4 per x-plane buffer (1 KB chunks)
    static constexpr int WF = WA * KSS * G;                 // weight fragments per wave per stage
    static constexpr int VPM = G == 8 ? 10 : G == 2 ? 5 : G == 4 ? 4 : 3;  // transform ALU ops per product
    static constexpr int PR = 4 * SA * G;                   // 16-byte pieces per staged output row
    static constexpr int STG = 32 * PR;                     // uint4 of epilogue staging per wave
    static constexpr int LDS_U4 = 2 * XST > NW * STG ? 2 * XST : NW * STG;
    static constexpr size_t LDS = (size_t)LDS_U4 * 16 + BO * 4;
    static_assert(WA % SA == 0, "store unit must divide the wave's output blocks");
    static_assert(ITEMS >= 1 && ITEMS * NT == BT * (SC / NCH), "x items must split evenly over the threads");
};

template <int G, int WA, int WB, int OW, int TW>
__global__ __launch_bounds__(OW * TW * 64) void k_big(const uint4 *__restrict__ x4,
                                                      const uint4 *__restrict__ wfrag,
                                                      const uint16_t *__restrict__ bias, int bias_shift,
                                                      uint16_t *__restrict__ y, int64_t N, int C_in,
                                                      int C_out, int n_stages, int KS16, int tiles_t) {
    using C = BigCfg<G, WA, WB, OW, TW>;
    constexpr int KSS = C::KSS, NCH = C::NCH;
    __shared__ uint4 lds[C::LDS_U4];  // two x-plane buffers; the epilogue's staging afterwards
    __shared__ float lbias[C::BO];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wo = wave % OW, wt = wave / OW;
    const int tt = blockIdx.x % tiles_t, ot = blockIdx.x / tiles_t;
    const int64_t t0 = (int64_t)tt * C::BT;
    const int o0 = ot * C::BO, ob0 = o0 / 32;

    // ---- loaders. Stages past the last one re-load the last stage (valid addresses, unused data),
    // so the loop body has no branches around loads. ----
    auto load_x = [&](int stage, uint4 (&dst)[C::ITEMS][C::XU4]) {
        stage = stage < n_stages ? stage : n_stages - 1;
#pragma unroll
        for (int k = 0; k < C::ITEMS; ++k) {
            const int item = tid + k * C::NT;
            const int tl = item / (C::SC / NCH), cq = item % (C::SC / NCH);
            int64_t n = t0 + tl;
            n = n < N ? n : N - 1;
            int i0 = stage * C::SC + cq * NCH;
            i0 = i0 < C_in ? i0 : C_in - NCH;  // padded channels meet zero weight columns
            const uint4 *p = x4 + (n * C_in + i0) * G / 8;
#pragma unroll
            for (int q = 0; q < C::XU4; ++q) dst[k][q] = p[q];
        }
    };
    auto load_w = [&](int stage, uint4 (&dst)[C::WF]) {
        stage = stage < n_stages ? stage : n_stages - 1;
#pragma unroll
        for (int a = 0; a < WA; ++a) {
            const uint4 *src = wfrag + (size_t)((ob0 + wo * WA + a) * KS16 + stage * KSS) * G * 64 + lane;
#pragma unroll
            for (int r = 0; r < KSS * G; ++r) dst[a * KSS * G + r] = src[r * 64];
        }
    };
    auto dft_store = [&](const uint4 (&src)[C::ITEMS][C::XU4], uint4 *xb) {
#pragma unroll
        for (int k = 0; k < C::ITEMS; ++k) {
            const int item = tid + k * C::NT;
            const int tl = item / (C::SC / NCH), cq = item % (C::SC / NCH);
            const int c0 = cq * NCH;  // first channel of the item within the stage
            uint4 *dst = xb + ((tl >> 5) * KSS + (c0 >> 4)) * G * 64 + ((c0 >> 3) & 1) * 32 + (tl & 31);
            float pl[G][NCH];
            dft_ch<G, NCH>(src[k], pl);
#pragma unroll
            for (int p = 0; p < G; ++p) {
                if constexpr (NCH == 8) {
                    dst[p * 64] = pack_bf16x8(pl[p]);
                } else {
                    uint2 w;
                    w.x = pack_bf16x2(pl[p][0], pl[p][1]);
                    w.y = pack_bf16x2(pl[p][2], pl[p][3]);
                    reinterpret_cast<uint2 *>(dst + p * 64)[(c0 >> 2) & 1] = w;
                }
            }
        }
    };

    // ---- prologue: bias; weights of stage 0 and raw x of stages 0 and 1 requested; x of stage 0
    // transformed (n_stages is even, so at least 2) ----
    uint4 xr[2][C::ITEMS][C::XU4];
    uint4 wr[2][C::WF];
    if (tid < C::BO) {
        const int o = o0 + tid;
        lbias[tid] = (bias && o < C_out) ? __uint_as_float((uint32_t)bias[o >> bias_shift] << 16) : 0.f;
    }
    load_w(0, wr[0]);
    load_x(0, xr[0]);
    load_x(1, xr[1]);
    dft_store(xr[0], lds);
    lds_barrier();

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

    // ---- main loop. Stage s: request the weights of s+1 and the raw x of s+2 (each into the
    // register slot its stage-s predecessor vacated), run the products of stage s, transform the raw
    // x of s+1 into the other x-plane buffer, barrier. ----
    // products of (K-step kk, token block b) pairs [lo, hi) of the stage, kk major
    auto products = [&](auto lo, auto hi, const uint4 (&w_cur)[C::WF], const uint4 *planes) {
#pragma unroll
        for (int q = decltype(lo)::value; q < decltype(hi)::value; ++q) {
            const int kk = q / WB, b = q % WB;
            uint4 xf[G], xn[G];
#pragma unroll
            for (int p = 0; p < G; ++p) xf[p] = planes[(((wt * WB + b) * KSS + kk) * G + p) * 64 + lane];
#pragma unroll
            for (int p = 0; p < G; ++p) xn[p] = (p >= 3 && (p & 1)) ? neg_bf16x8(xf[p]) : xf[p];
#pragma unroll
            for (int a = 0; a < WA; ++a) {
                uint4 wf[G];
#pragma unroll
                for (int p = 0; p < G; ++p) wf[p] = w_cur[(a * KSS + kk) * G + p];
                spectral_mfma32<G>(wf, xf, xn, acc[a][b]);
            }
        }
    };
    // One stage in two scheduling regions, so the loads leave in a fixed order: the weights of s+1
    // under the first half of the products, then the raw x of s+2 and the transform of x(s+1) under
    // the second half. The next stage's products then wait for the weights only, with the raw x
    // still in flight (vector-memory operations complete in issue order).
    auto step = [&](int s, uint4 (&x_free)[C::ITEMS][C::XU4], const uint4 (&x_next)[C::ITEMS][C::XU4],
                    const uint4 (&w_cur)[C::WF], uint4 (&w_next)[C::WF], const uint4 *planes,
                    uint4 *planes_next) {
        constexpr int P = KSS * WB, H = P / 2;
        load_w(s + 1, w_next);
        products(IC<0>{}, IC<H>{}, w_cur, planes);
        interleave_stage<H * G, H * WA * real_products(G), C::WF, 1>();
        __builtin_amdgcn_sched_barrier(0);
        load_x(s + 2, x_free);
        products(IC<H>{}, IC<P>{}, w_cur, planes);
        dft_store(x_next, planes_next);  // after the last stage: unused planes, harmless
        interleave_stage<(P - H) * G, (P - H) * WA * real_products(G), C::ITEMS * C::XU4, C::VPM>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);  // each stage is its own scheduling region
    };
    for (int s = 0; s < n_stages; s += 2) {  // n_stages is even (the channel padding sees to it)
        step(s, xr[0], xr[1], wr[0], wr[1], lds, lds + C::XST);
        step(s + 1, xr[1], xr[0], wr[1], wr[0], lds + C::XST, lds);
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
    hipLaunchKernelGGL((k_big<G, WA, WB, OW, TW>), dim3((unsigned)(tiles_t * tiles_o)), dim3(C::NT), 0, s,
                       (const uint4 *)x, (const uint4 *)p->planes, (const uint16_t *)b, p->bias_shift,
                       (uint16_t *)y, N, p->C_in, p->C_out, n_stages, p->KS, (int)tiles_t);
    return hipGetLastError();
}

struct BigEntry {
    int G, BO, BT, KSS, NT;
    size_t lds;
    LaunchFn launch;
    const char *tile;
};
#define BE(G, WA, WB, OW, TW)                                                                            \
    {G, BigCfg<G, WA, WB, OW, TW>::BO, BigCfg<G, WA, WB, OW, TW>::BT, BigCfg<G, WA, WB, OW, TW>::KSS,      \
     BigCfg<G, WA, WB, OW, TW>::NT, BigCfg<G, WA, WB, OW, TW>::LDS, launch_big<G, WA, WB, OW, TW>,         \
     #WA "x" #WB " blocks/wave, " #OW "x" #TW " waves"}
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
        out->kind = KIND_TILED;
        out->frag_kind = 2;
        out->rows_per_block = 32;
        out->kc = 16;
        out->ks_mult = 2 * e.KSS;  // an even number of stages: the main loop runs them in pairs
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
