// bwd.hip -- the gradients of the EQ-Linear layer: dW (and db) from x and dy.
//
// Method: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
// Transform" (gist.science explainer), "Implementación" (the operator has forward and backward
// kernels) and "Enfoque Algorítmico" (group DFT -> independent per-frequency channel products). The
// data gradient dx is a forward pass of the layer whose weight is W transposed over (o, i) and
// reversed along the group axis (built at prepare; eqlin_api.cpp). This file computes the weight
// gradient
//
//     dW[o, i, d] = sum_n sum_h dy[n, o, h] * x[n, i, (h - d) mod G],   db[o] = sum_{n, h} dy[n, o, h],
//
// a circular cross-correlation along the group axis summed over tokens. With the same DFT as the
// forward (X_k = sum_g x_g e^{-2 pi i g k / G}) it becomes one channel product per frequency,
//
//     C_k[o, i] = sum_n DY_k[n, o] * conj(X_k[n, i]),   k = 0..G/2,
//
// and dW[o, i, :] is the inverse DFT of C (Hermitian symmetry fills k > G/2): the forward's inverse
// transform with its 1/G and 2/G plane scalings. In real planes, a complex frequency is four real
// products: Re C = DYr Xr + DYi Xi, Im C = DYi Xr - DYr Xi.
//
// bf16 or fp16, G = 4 or 8 (matrix cores), three passes over a caller-provided workspace:
//   1. k_bw_planes: x and dy -> DFT planes (fp32, rounded once to the half type) in 32x32x16 fragment order
//      with tokens along K: chunk (channel block cb of 32, token step kt of 16, plane p) is 1 KB, lane
//      l holds channel cb*32 + l%32, tokens kt*16 + 8*(l/32) .. +7. Each token's transform is done
//      once (in the product pass every x tile meets many dy tiles). Tokens past N are zeros. The dy
//      pass also sums plane 0 (= sum over h, in fp32) over its 64 tokens: db partials.
//   2. k_bw_gemm: C_k over a split of the tokens for one output tile (128 outputs x 32*WB inputs),
//      written as fp32 partial planes. Two waves per SIMD split the planes (role 0: planes 0..G/2-1,
//      role 1: the rest) and share the tile; the dy fragments go straight to registers (each wave its
//      own), the x fragments through LDS (shared by all waves).
//   3. k_bw_reduce: sum of the splits, inverse DFT (scaled) -> dW fp32; k_bw_dbsum: db from its
//      partials.
// The dihedral group D4 and fp16 take the same matrix-core passes (D4: its irreps' adjoint products and
// inverse); small channel counts take one fused pass per token range instead (k_bw_small). Other cases
// (fp32, G = 1 or 2): k_bw_direct, the definition above in fp32 with LDS token tiles. For D4 (element
// a + 4b = r^a s^b) the definition reads dW[o, i, d] = sum_n sum_h dy[n, o, h] x[n, i, h d^-1] (the g
// with g^-1 h = d).
#include <stdio.h>

#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "eqlin_internal.h"

namespace eqlin {

// ------------------------------------------------------------------------------------------------
// Pass 1: group DFT of a [N][C][G] bf16 / fp16 tensor into K-major fragments.
constexpr int kBwTok = 64;         // tokens per pass-1 workgroup (4 token steps of 16)
constexpr int kBwRow = kBwTok + 8;  // LDS row of one (plane, channel): padded against bank conflicts

template <int G, class E, bool D4>
__global__ __launch_bounds__(256) void k_bw_planes(const uint16_t *__restrict__ src, int64_t N, int C, int KT,
                                                   uint4 *__restrict__ frag, float *__restrict__ db_part) {
    __shared__ __attribute__((aligned(16))) uint16_t sp[G][32][kBwRow];
    __shared__ float red[32][kBwTok + 1];
    const int t = threadIdx.x;
    const int tl = t >> 2, cg = t & 3;            // token within the tile, 8-channel group
    const int64_t n = (int64_t)blockIdx.x * kBwTok + tl;
    const int cb = blockIdx.y, c0 = cb * 32 + cg * 8;
    // 8 channels x G samples of one token (C % 8 == 0: a group is wholly inside or outside)
    uint4 r[G];
    const bool live = n < N && c0 < C;
    const uint4 *p = reinterpret_cast<const uint4 *>(src + (live ? (n * C + c0) * G : 0));
#pragma unroll
    for (int q = 0; q < G; ++q) r[q] = live ? p[q] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v[G], P[G];
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] = elem_at<E>(r[(j * G + g) >> 3], (j * G + g) & 7);
        group_forward<G, D4>(v, P);
#pragma unroll
        for (int pl = 0; pl < G; ++pl) sp[pl][cg * 8 + j][tl] = pack1<E>(P[pl]);
        red[cg * 8 + j][tl] = P[0];  // plane 0 is the sum over the group samples
    }
    __syncthreads();
    if (db_part && t < 32) {
        float s = 0.f;
        for (int k = 0; k < kBwTok; ++k) s += red[t][k];
        db_part[(int64_t)blockIdx.x * gridDim.y * 32 + cb * 32 + t] = s;
    }
    // 4 token steps x G planes, one 1 KB chunk each; a thread writes one 16-byte piece per round
#pragma unroll
    for (int rd = 0; rd < G; ++rd) {
        const int q = rd * 4 + (t >> 6), lane = t & 63;
        const int ktl = q & 3, pl = q >> 2;
        const int c = lane & 31, tok = ktl * 16 + 8 * (lane >> 5);
        const uint4 v = *reinterpret_cast<const uint4 *>(&sp[pl][c][tok]);
        const int kt = blockIdx.x * (kBwTok / 16) + ktl;
        frag[((int64_t)(cb * KT + kt) * G + pl) * 64 + lane] = v;
    }
}

// ------------------------------------------------------------------------------------------------
// Pass 2: per-frequency products over a token split.
template <int V>
struct IC2 {
    static constexpr int value = V;
};

template <int G>
struct BwCfg {
    static constexpr int NW = 8, NT = NW * 64;
    static constexpr int HP = G / 2;              // planes per role
    static constexpr int WB = G == 8 ? 2 : 4;     // 32-input blocks per wave (accumulators: WB * HP * 16)
    static constexpr int BO = 128, BI = 32 * WB;  // output tile: 4 o-blocks (one per SIMD) x WB i-blocks
    static constexpr int XCH = WB * G;            // x chunks per token step (1 KB each)
    static constexpr int XU = XCH * 64 / NT;      // 16-byte pieces per thread per token step
    static constexpr int LDS_U4 = 2 * XCH * 64;
    static_assert(XU * NT == XCH * 64, "x chunks split evenly over the threads");
};

// LDS-only workgroup barrier: outstanding global loads stay in flight across it.
__device__ __forceinline__ void bw_lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
    asm volatile("s_barrier" ::: "memory");
}

template <int G, class E, bool D4>
__global__ __launch_bounds__(512) void k_bw_gemm(const uint4 *__restrict__ xf, const uint4 *__restrict__ dyf,
                                                 float *__restrict__ part, int KT, int tiles_i, int splits,
                                                 int C_in_pad, int C_out_pad) {
    using C = BwCfg<G>;
    constexpr int HP = C::HP, WB = C::WB;
    __shared__ uint4 lds[C::LDS_U4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wo = wave_u & 3, role = wave_u >> 2;
    const int split = blockIdx.x % splits, tile = blockIdx.x / splits;
    const int ti = tile % tiles_i, to = tile / tiles_i;
    const int ob = to * 4 + wo;  // this wave's 32-output block
    const int ib0 = ti * WB;     // the tile's first 32-input block
    const int kt0 = (int)((int64_t)KT * split / splits), kt1 = (int)((int64_t)KT * (split + 1) / splits);
    const int nk = kt1 - kt0;
    const int nst = (nk + 1) & ~1;  // even: the loop runs stages in pairs (the extra one reads zeros)
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    // a position past the split's range reads zeros: its offset lies outside every resource's range
    constexpr int kDead = 0x7fffffff;

    // dy fragments of this wave: (ob, kt, plane role * HP + r), straight to registers
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(dyf + ((int64_t)ob * KT + kt0) * G * 64 + role * HP * 64), (short)0,
        nk * G * 1024 - role * HP * 1024, 0x00020000);
    auto load_a = [&](int s, uint4 (&dst)[HP]) {
        const bool live = s < nk;
#pragma unroll
        for (int r = 0; r < HP; ++r) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(a_rs, live ? lane * 16 + r * 1024 : kDead,
                                                                  live ? s * G * 1024 : 0, 0);
            dst[r] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    // x fragments of the tile (WB blocks x G planes per token step): the thread's XU pieces, which
    // belong to block e / (G * 64); one resource per piece slot
    __amdgpu_buffer_rsrc_t b_rs[C::XU];
#pragma unroll
    for (int u = 0; u < C::XU; ++u) {
        const int blk = (tid + u * C::NT) / (G * 64);
        b_rs[u] = __builtin_amdgcn_make_buffer_rsrc((void *)(xf + ((int64_t)(ib0 + blk) * KT + kt0) * G * 64),
                                                    (short)0, nk * G * 1024, 0x00020000);
    }
    auto load_b = [&](int s, uint4 (&dst)[C::XU]) {
        const bool live = s < nk;
#pragma unroll
        for (int u = 0; u < C::XU; ++u) {
            const int rem = (tid + u * C::NT) % (G * 64);  // (plane, lane) within the block
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(b_rs[u], live ? rem * 16 : kDead,
                                                                  live ? s * G * 1024 : 0, 0);
            dst[u] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    auto store_b = [&](const uint4 (&src)[C::XU], uint4 *buf) {
#pragma unroll
        for (int u = 0; u < C::XU; ++u) buf[tid + u * C::NT] = src[u];  // [block][plane][lane]
    };

    // the whole loop once per role (wave-uniform), so the products are branch-free; both roles run
    // the same barriers
    auto run = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        f32x16 acc[WB][HP];
#pragma unroll
        for (int b = 0; b < WB; ++b)
#pragma unroll
            for (int q = 0; q < HP; ++q) acc[b][q] = f32x16{};
        // one token step: Re C += Ar Br + Ai Bi, Im C += Ai Br + (-Ar) Bi; role 0's planes 0 and 1
        // are the real frequencies 0 and G/2
        auto products = [&](const uint4 (&a)[HP], const uint4 *buf) {
            uint4 an[HP];
#pragma unroll
            for (int r = 0; r < HP; ++r) an[r] = neg_bf16x8(a[r]);
#pragma unroll
            for (int b = 0; b < WB; ++b) {
                uint4 bf[HP];
#pragma unroll
                for (int r = 0; r < HP; ++r) bf[r] = buf[(b * G + R * HP + r) * 64 + lane];
                if constexpr (D4) {
                    // role 0: the characters, G_k = sum DY_k X_k; role 1: the 2 x 2 irrep, entry
                    // (c, b') at local plane 2c + b': G_cb' = sum_a X_ac DY_ab'
                    if constexpr (R == 0) {
#pragma unroll
                        for (int q = 0; q < HP; ++q) acc[b][q] = mma32<E>(a[q], bf[q], acc[b][q]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int c = e >> 1, bb = e & 1;
                            acc[b][e] = mma32<E>(a[bb], bf[c], acc[b][e]);
                            acc[b][e] = mma32<E>(a[2 + bb], bf[2 + c], acc[b][e]);
                        }
                    }
                    continue;
                }
#pragma unroll
                for (int c = 0; c < HP; c += 2) {
                    if constexpr (R == 0) {
                        if (c == 0) {
                            acc[b][0] = mma32<E>(a[0], bf[0], acc[b][0]);
                            acc[b][1] = mma32<E>(a[1], bf[1], acc[b][1]);
                            continue;
                        }
                    }
                    acc[b][c] = mma32<E>(a[c], bf[c], acc[b][c]);
                    acc[b][c] = mma32<E>(a[c + 1], bf[c + 1], acc[b][c]);
                    acc[b][c + 1] = mma32<E>(a[c + 1], bf[c], acc[b][c + 1]);
                    acc[b][c + 1] = mma32<E>(an[c], bf[c + 1], acc[b][c + 1]);
                }
            }
        };

        uint4 ar[2][HP], br[2][C::XU];
        load_a(0, ar[0]);
        load_b(0, br[0]);
        load_b(1, br[1]);
        store_b(br[0], lds);
        bw_lds_barrier();
        for (int s = 0; s < nst; s += 2) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int st = s + h;
                const uint4 *cur = lds + h * C::XCH * 64;
                uint4 *nxt = lds + (1 - h) * C::XCH * 64;
                load_a(st + 1, ar[1 - h]);
                load_b(st + 2, br[h]);  // past the range: zeros, unused
                products(ar[h], cur);
                store_b(br[1 - h], nxt);  // the next step's x (past the range: zeros, unused)
                bw_lds_barrier();
            }
        }

        // fp32 partial planes part[split][plane][o][i]; D lane l: input column l % 32, outputs
        // 8 (v / 4) + 4 (l / 32) + v % 4 of the wave's block
        const int64_t plane_sz = (int64_t)C_out_pad * C_in_pad;
        float *pb = part + (int64_t)split * G * plane_sz;
#pragma unroll
        for (int b = 0; b < WB; ++b)
#pragma unroll
            for (int q = 0; q < HP; ++q) {
                const int pl = R * HP + q;
                const int i = (ib0 + b) * 32 + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int o = ob * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    pb[pl * plane_sz + (int64_t)o * C_in_pad + i] = acc[b][q][v];
                }
            }
    };
    if (role == 0)
        run(IC2<0>{});
    else
        run(IC2<1>{});
}

// ------------------------------------------------------------------------------------------------
// Pass 3: splits summed, inverse DFT with the plane scalings -> dW. A workgroup covers 32 consecutive
// inputs i of one output o (whole 128-byte lines of every partial plane): thread (sub, i) sums the
// splits sub, sub + 8, ... of each plane; the 8 shares are added in a fixed order in LDS, then 32
// threads run the inverse transforms.
template <int G, bool D4>
__global__ __launch_bounds__(256) void k_bw_reduce(const float *__restrict__ part, int splits, int C_out, int C_in,
                                                   int C_out_pad, int C_in_pad, float *__restrict__ dW) {
    __shared__ float red[G][8][33];
    const int t = threadIdx.x, il = t & 31, sub = t >> 5;
    const int ib = C_in_pad / 32;
    const int o = blockIdx.x / ib, i = (blockIdx.x % ib) * 32 + il;
    const int64_t plane_sz = (int64_t)C_out_pad * C_in_pad;
    const float *src = part + (int64_t)o * C_in_pad + i;
#pragma unroll
    for (int p = 0; p < G; ++p) {
        float s = 0.f;
        for (int k = sub; k < splits; k += 8) s += src[((int64_t)k * G + p) * plane_sz];
        red[p][sub][il] = s;
    }
    __syncthreads();
    if (t < 32 && o < C_out && i < C_in) {
        float Y[G], out[G];
#pragma unroll
        for (int p = 0; p < G; ++p) {
            const float a = (red[p][0][il] + red[p][1][il]) + (red[p][2][il] + red[p][3][il]);
            const float b = (red[p][4][il] + red[p][5][il]) + (red[p][6][il] + red[p][7][il]);
            Y[p] = (a + b) * group_plane_scale(G, D4, p);
        }
        group_inverse<G, D4>(Y, out);
#pragma unroll
        for (int d = 0; d < G; ++d) dW[((int64_t)o * C_in + i) * G + d] = out[d];
    }
}

// db[o] from the per-token-tile partials: 64 threads per output, each a strided share, LDS sum.
__global__ __launch_bounds__(256) void k_bw_dbsum(const float *__restrict__ db_part, int n_tiles, int C_out,
                                                  int C_out_pad, float *__restrict__ db) {
    __shared__ float red[4][65];
    const int t = threadIdx.x, ol = t >> 6, sub = t & 63;
    const int o = blockIdx.x * 4 + ol;
    float s = 0.f;
    if (o < C_out)
        for (int k = sub; k < n_tiles; k += 64) s += db_part[(int64_t)k * C_out_pad + o];
    red[ol][sub] = s;
    __syncthreads();
    if (sub == 0 && o < C_out) {
        float acc = 0.f;
        for (int k = 0; k < 64; ++k) acc += red[ol][k];
        db[o] = acc;
    }
}

// ------------------------------------------------------------------------------------------------
// Direct kernel (fp32, bf16 or fp16 inputs, any G): the definition in fp32. Workgroup: 16 x 16 (o, i)
// pairs, 256 threads (one pair each, all G shifts d); token tiles of 32 through LDS.
// Index of h d^-1: (h - d) mod G, or in D4, with h = r^c s^e and d = r^a s^b: d^-1 = r^a' s^b (a' = -a
// for a rotation, a for a reflection) and the product rule r^c s^e r^a' s^b = r^(c + (-1)^e a') s^(e + b).
template <int G, bool D4>
__host__ __device__ constexpr int h_dinv(int h, int d) {
    if constexpr (!D4) {
        return (h - d + G) % G;
    } else {
        const int a = d & 3, b = d >> 2;
        const int ai = b ? a : (4 - a) & 3;  // d^-1 = r^ai s^b
        const int c = h & 3, e = h >> 2;
        return ((e ? c - ai : c + ai) & 3) + 4 * ((e + b) & 1);
    }
}

// One element of a layer tensor as fp32: T is float, or the 16-bit tag BF16 / F16.
template <typename T>
__device__ __forceinline__ float load_elem(const void *p, int64_t k) {
    if constexpr (__is_same(T, float))
        return static_cast<const float *>(p)[k];
    else
        return elem_to_float<T>(static_cast<const uint16_t *>(p)[k]);
}

template <typename T, int G, bool D4>
__global__ __launch_bounds__(256) void k_bw_direct(const void *__restrict__ x, const void *__restrict__ dy, int64_t N,
                                                   int C_in, int C_out, float *__restrict__ dW) {
    constexpr int TK = 32;
    __shared__ float xs[TK][16][G + 1];
    __shared__ float ds[TK][16][G + 1];
    const int t = threadIdx.x, ol = t >> 4, il = t & 15;
    const int o0 = blockIdx.y * 16, i0 = blockIdx.x * 16;
    auto ld = [](const void *p, int64_t k) -> float { return load_elem<T>(p, k); };
    float acc[G];
#pragma unroll
    for (int d = 0; d < G; ++d) acc[d] = 0.f;
    for (int64_t n0 = 0; n0 < N; n0 += TK) {
        for (int e = t; e < TK * 16 * G; e += 256) {
            const int k = e / (16 * G), c = (e / G) % 16, g = e % G;
            const int64_t n = n0 + k;
            const int i = i0 + c, o = o0 + c;
            xs[k][c][g] = (n < N && i < C_in) ? ld(x, (n * C_in + i) * G + g) : 0.f;
            ds[k][c][g] = (n < N && o < C_out) ? ld(dy, (n * C_out + o) * G + g) : 0.f;
        }
        __syncthreads();
        for (int k = 0; k < TK; ++k)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float dv = ds[k][ol][h];
#pragma unroll
                for (int d = 0; d < G; ++d) acc[d] += dv * xs[k][il][h_dinv<G, D4>(h, d)];
            }
        __syncthreads();
    }
    const int o = o0 + ol, i = i0 + il;
    if (o < C_out && i < C_in)
#pragma unroll
        for (int d = 0; d < G; ++d) dW[((int64_t)o * C_in + i) * G + d] = acc[d];
}

// db[o] = sum_{n, h} dy[n, o, h] (fp32): 64 outputs per workgroup, 4 token phases reduced in LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_bw_bias(const void *__restrict__ dy, int64_t N, int C_out, int G,
                                                 float *__restrict__ db) {
    __shared__ float red[4][64];
    const int t = threadIdx.x, ol = t & 63, ph = t >> 6;
    const int o = blockIdx.x * 64 + ol;
    float s = 0.f;
    if (o < C_out)
        for (int64_t n = ph; n < N; n += 4)
            for (int h = 0; h < G; ++h) {
                s += load_elem<T>(dy, (n * C_out + o) * G + h);
            }
    red[ph][ol] = s;
    __syncthreads();
    if (ph == 0 && o < C_out) db[o] = ((red[0][ol] + red[1][ol]) + red[2][ol]) + red[3][ol];
}

// ------------------------------------------------------------------------------------------------
// Small channel counts (bf16 or fp16, G = 4 or 8 cyclic or D4, C_in_pad * C_out_pad * G <= 40960): one fused pass.
// (D4: the character planes give G_k = sum DY_k X_k, the 2 x 2 irrep G_cb = sum_a X_ac DY_ab, the
// adjoint of Y = X W; the inverse transform with the forward's scalings then gives dW.)
// At such sizes the three-pass path spends its time writing and re-reading transformed planes and on
// 128-wide tiles padding 64 or 96 channels; here each workgroup owns a contiguous token range and the
// whole C_out x C_in x G spectrum of it in registers (8 waves, at most 5 32x32 accumulator blocks
// each), so x and dy are read once and only the fp32 partial spectra leave. The range is walked in
// super-chunks of 32 tokens through two LDS fragment buffers: in step s the waves issue the loads of
// super-chunk s + 2 (one item of 8 tokens x 16 bytes per thread), run the products of super-chunk s
// from one buffer and write the group DFT of super-chunk s + 1 (half type, K-major fragments: tokens along
// K, as in pass 1) into the other, so the transform's vector ALU and the products overlap and each
// load has a whole step to arrive. Partials go to part[split][plane][o][i] and db partials to
// db_part[split][o]; k_bw_small_reduce sums them in a fixed order and k_bw_small_inverse applies the
// inverse DFT.
struct SmallBwCfg {
    static constexpr int NT = 512, ST = 32, KT = ST / 16;
    // accumulator blocks per wave: 5 at G = 4 (96 x 96 x 4), 4 at G = 8 (64 x 64 x 8; G = 8's transform
    // needs the registers)
    static constexpr int maxb(int G) { return G == 8 ? 4 : 5; }
};

template <int G, bool D4, class E>
__global__ __launch_bounds__(512) void k_bw_small(const uint16_t *__restrict__ x, const uint16_t *__restrict__ dy,
                                                  int64_t N, int C_in, int C_out, int tok_wg, int CB_in, int CB_out,
                                                  float *__restrict__ part, float *__restrict__ db_part) {
    using C = SmallBwCfg;
    constexpr int CPU = 8 / G;  // channels per 16-byte unit of a token row
    constexpr int MAXB = C::maxb(G);
    extern __shared__ uint4 frag[];  // two buffers of [KT][CB_in][G] x fragments then [KT][CB_out][G] dy fragments
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int C_in_pad = CB_in * 32, C_out_pad = CB_out * 32;
    const int DYB = C::KT * CB_in * G;              // first dy fragment of a buffer
    const int FR = DYB + C::KT * CB_out * G;        // fragments per buffer
    const int64_t n_begin = (int64_t)blockIdx.x * tok_wg;
    const int64_t n_end = N - n_begin < tok_wg ? N : n_begin + tok_wg;
    const int nsc = (int)((n_end - n_begin + C::ST - 1) / C::ST);  // super-chunks of this range
    // this thread's item (16-byte unit u of a token row, 8-token group tg) of every super-chunk: x's
    // items first, then dy's; C_in * G % 128 == 0 puts the boundary between waves (wave-uniform tensor)
    const int ux = C_in / CPU, uy = C_out / CPU;
    const int nx = ux * 4, items = (ux + uy) * 4;
    const bool live = t < items;
    const bool isx = __builtin_amdgcn_readfirstlane(t < nx ? 1 : 0) != 0;
    const int ki = isx ? t : t - nx, uu = isx ? ux : uy;
    const int tg = ki / uu, u = ki % uu;
    const int row = (isx ? C_in : C_out) * G * 2, col = u * 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(isx ? x : dy), (short)0, (int)(N * (isx ? C_in : C_out) * G * 2), 0x00020000);

    for (int k = t; k < 2 * FR * 64; k += C::NT) frag[k] = make_uint4(0u, 0u, 0u, 0u);  // padded channels

    uint4 raw[2][8];
    auto load = [&](int sc, uint4 (&dst)[8]) {  // all 8 tokens of this thread's item in flight at once
        const int64_t nb = n_begin + (int64_t)sc * C::ST + tg * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t n = nb + j;
            const int off = (live && n < n_end) ? (int)(n * row) + col : 0x7fffffff;  // dead: zeros
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
            dst[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    float dbacc[CPU];
#pragma unroll
    for (int c = 0; c < CPU; ++c) dbacc[c] = 0.f;
    auto transform = [&](const uint4 (&src)[8], int buf) {  // DFT -> half-type fragments (+ dy's plane 0)
        if (!live) return;
        const int step = tg >> 1, half = tg & 1;
        // (fp16 at G = 4: one channel at a time; unrolled, the two channels' fp16 conversions were kept
        // live together and 56 registers spilled)
        constexpr int UNR = (__is_same(E, F16) && CPU > 1) ? 1 : CPU;
#pragma unroll UNR
        for (int c = 0; c < CPU; ++c) {
            float pl[G][8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float v[G], P[G];
#pragma unroll
                for (int g = 0; g < G; ++g) v[g] = elem_at<E>(src[j], c * G + g);
                group_forward<G, D4>(v, P);
#pragma unroll
                for (int q = 0; q < G; ++q) pl[q][j] = P[q];
                if (!isx)
#pragma unroll
                    for (int cc = 0; cc < CPU; ++cc)  // (a compile-time index also when c is not)
                        if (cc == c) dbacc[cc] += P[0];
            }
            const int ch = u * CPU + c;
            const int base = buf * FR + (isx ? (step * CB_in + (ch >> 5)) * G : DYB + (step * CB_out + (ch >> 5)) * G);
            const int lf = (ch & 31) + 32 * half;
#pragma unroll
            for (int q = 0; q < G; ++q) frag[(base + q) * 64 + lf] = pack8<E>(pl[q]);
        }
    };

    // accumulator blocks: b = p * tiles + (ob * CB_in + ib), dealt round-robin to the waves (so every
    // wave gets a mix of real and complex planes); plane and fragment offsets decoded once
    const int tiles = CB_in * CB_out, nbk = tiles * G;
    f32x16 acc[MAXB];
    int bp[MAXB], boa[MAXB], bob[MAXB];
#pragma unroll
    for (int q = 0; q < MAXB; ++q) {
        acc[q] = f32x16{};
        const int b = wave + 8 * q, tile = b % tiles;
        bp[q] = b < nbk ? b / tiles : -1;
        boa[q] = (DYB + (tile / CB_in) * G) * 64;
        bob[q] = ((tile % CB_in) * G) * 64;
    }
    auto products = [&](int buf, int steps) {
        for (int k = 0; k < steps; ++k)
#pragma unroll
            for (int q = 0; q < MAXB; ++q) {
                const int pp = bp[q];
                if (pp < 0) continue;  // wave-uniform
                const uint4 *A = frag + buf * FR * 64 + boa[q] + k * CB_out * G * 64 + lane;  // dy: rows = outputs
                const uint4 *B = frag + buf * FR * 64 + bob[q] + k * CB_in * G * 64 + lane;   // x: columns = inputs
                if constexpr (D4) {
                    if (pp < 4) {  // a character: G_k = sum DY_k X_k
                        acc[q] = mma32<E>(A[pp * 64], B[pp * 64], acc[q]);
                    } else {  // the 2 x 2 irrep, entry (c, b): G_cb = sum_a X_ac DY_ab
                        const int c = (pp - 4) >> 1, bb = (pp - 4) & 1;
                        acc[q] = mma32<E>(A[(4 + bb) * 64], B[(4 + c) * 64], acc[q]);
                        acc[q] = mma32<E>(A[(6 + bb) * 64], B[(6 + c) * 64], acc[q]);
                    }
                    continue;
                }
                if (pp < 2) {
                    acc[q] = mma32<E>(A[pp * 64], B[pp * 64], acc[q]);
                } else if ((pp & 1) == 0) {  // Re C_k = DYr Xr + DYi Xi
                    acc[q] = mma32<E>(A[pp * 64], B[pp * 64], acc[q]);
                    acc[q] = mma32<E>(A[(pp + 1) * 64], B[(pp + 1) * 64], acc[q]);
                } else {  // Im C_k = DYi Xr - DYr Xi
                    acc[q] = mma32<E>(A[pp * 64], B[(pp - 1) * 64], acc[q]);
                    acc[q] = mma32<E>(neg_bf16x8(A[(pp - 1) * 64]), B[pp * 64], acc[q]);
                }
            }
    };
    auto steps_of = [&](int sc) {  // 16-token steps holding tokens of this range
        const int64_t left = n_end - n_begin - (int64_t)sc * C::ST;
        return left >= C::ST ? C::KT : (int)((left + 15) / 16);
    };
    // step s: loads of s + 2 into the register set s's data came in, products of s (buffer s % 2),
    // transform of s + 1 (registers (s + 1) % 2 -> buffer (s + 1) % 2)
    auto stage = [&](auto rc, int sc) {
        constexpr int R = decltype(rc)::value;  // sc % 2
        if (sc + 2 < nsc) load(sc + 2, raw[R]);
        products(R, steps_of(sc));
        if (sc + 1 < nsc) transform(raw[1 - R], 1 - R);
        __syncthreads();
    };

    __syncthreads();  // zero fill done
    load(0, raw[0]);
    if (nsc > 1) load(1, raw[1]);
    transform(raw[0], 0);
    __syncthreads();
    for (int sc = 0; sc < nsc; sc += 2) {
        stage(IC2<0>{}, sc);
        if (sc + 1 < nsc) stage(IC2<1>{}, sc + 1);
    }

    // partial spectra of this token range, fp32
    const int64_t plane_sz = (int64_t)C_out_pad * C_in_pad;
#pragma unroll
    for (int q = 0; q < MAXB; ++q) {
        const int b = wave + 8 * q;
        if (b >= nbk) continue;
        const int pp = b / tiles, tile = b % tiles, ob = tile / CB_in, ib = tile % CB_in;
        float *dst = part + ((int64_t)blockIdx.x * G + pp) * plane_sz +
                     (int64_t)(ob * 32 + 4 * (lane >> 5)) * C_in_pad + ib * 32 + (lane & 31);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {  // rows 8 * v4 + 4 * (lane / 32) + 0..3
#pragma unroll
            for (int v = 0; v < 4; ++v) dst[v * C_in_pad] = acc[q][4 * v4 + v];
            dst += 8 * C_in_pad;
        }
    }
    // db: this range's sum over tokens and h, the 4 token groups added in a fixed order (LDS; every wave
    // is past its last products: the loop ends on a barrier)
    float *red = reinterpret_cast<float *>(frag);  // [4][C_out]
    if (live && !isx)
#pragma unroll
        for (int c = 0; c < CPU; ++c) red[tg * C_out + u * CPU + c] = dbacc[c];
    __syncthreads();
    for (int o = t; o < C_out; o += C::NT) {
        float a = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) a += red[g * C_out + o];
        db_part[(int64_t)blockIdx.x * C_out_pad + o] = a;
    }
}

// Sum of the fused pass's partial spectra over its token ranges, in a fixed order: one workgroup per
// (group of 32 consecutive (o, i) positions of the padded [C_out][C_in_pad] grid, plane p), 16
// interleaved shares of the ranges with every load of a share issued before the first add, then the
// shares in turn; the scaled plane sums go to `psum` [G][C_out_pad][C_in_pad]. The trailing
// workgroups sum the db partials. (k_bw_small_inverse then applies the inverse DFT: a second launch,
// because making the plane sums of other workgroups visible inside this one takes device-scope
// fences, and each of those writes back an XCD's L2.)
template <int G, bool D4>
__global__ __launch_bounds__(512) void k_bw_small_reduce(const float *__restrict__ part, const float *__restrict__ db_part,
                                                         int splits, int C_out, int C_out_pad, int C_in_pad, int n_main,
                                                         float *__restrict__ psum, float *__restrict__ db) {
    constexpr int NS = 16, KMAX = 16;  // split shares; splits per share (splits <= NS * KMAX)
    __shared__ float red[NS][33];
    const int t = threadIdx.x, pl = t & 31, sg = t >> 5;
    const int64_t plane_sz = (int64_t)C_out_pad * C_in_pad;
    if ((int)blockIdx.x < n_main) {
        const int pg = (int)blockIdx.x / G, p = (int)blockIdx.x % G;
        const int64_t pos = (int64_t)pg * 32 + pl;  // < C_out * C_in_pad
        const float *src = part + p * plane_sz + pos;
        float v[KMAX];
#pragma unroll
        for (int kk = 0; kk < KMAX; ++kk) {
            const int k = sg + kk * NS;
            v[kk] = k < splits ? src[(int64_t)k * G * plane_sz] : 0.f;
        }
        float a = 0.f;
#pragma unroll
        for (int kk = 0; kk < KMAX; ++kk) a += v[kk];
        red[sg][pl] = a;
        __syncthreads();
        if (sg == 0) {
            float sum = 0.f;
#pragma unroll
            for (int k = 0; k < NS; ++k) sum += red[k][pl];
            psum[p * plane_sz + pos] = sum * group_plane_scale(G, D4, p);
        }
    } else {
        if (!db) return;  // uniform over the workgroup
        const int o = ((int)blockIdx.x - n_main) * 32 + pl;
        float a = 0.f;
        if (o < C_out)
            for (int k = sg; k < splits; k += NS) a += db_part[(int64_t)k * C_out_pad + o];
        red[sg][pl] = a;
        __syncthreads();
        if (sg == 0 && o < C_out) {
            float sum = 0.f;
#pragma unroll
            for (int k = 0; k < NS; ++k) sum += red[k][pl];
            db[o] = sum;
        }
    }
}

// dW[o, i, :] = inverse DFT of the scaled plane sums; one thread per (o, i).
template <int G, bool D4>
__global__ __launch_bounds__(256) void k_bw_small_inverse(const float *__restrict__ psum, int C_out, int C_in,
                                                          int C_out_pad, int C_in_pad, float *__restrict__ dW) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= (int64_t)C_out * C_in) return;
    const int o = (int)(k / C_in), i = (int)(k % C_in);
    const int64_t plane_sz = (int64_t)C_out_pad * C_in_pad;
    float Y[G], out[G];
#pragma unroll
    for (int q = 0; q < G; ++q) Y[q] = psum[q * plane_sz + (int64_t)o * C_in_pad + i];
    group_inverse<G, D4>(Y, out);
#pragma unroll
    for (int d = 0; d < G; ++d) dW[k * G + d] = out[d];
}

// Zero fill (the gradients of an empty batch), a kernel rather than a memset so that a captured HIP
// graph holds only kernel nodes.
__global__ __launch_bounds__(256) void k_zero_f32(float *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Host side: workspace layout and launch.
namespace {

bool mfma_path(const Plan *p) { return p->dtype != EQLIN_F32 && (p->G == 4 || p->G == 8); }

struct BwLayout {
    int KT = 0, CB_in = 0, CB_out = 0, tiles_i = 0, tiles_o = 0, splits = 0, ptiles = 0;
    int C_in_pad = 0, C_out_pad = 0;
    size_t off_x = 0, off_dy = 0, off_part = 0, off_db = 0, total = 0;
};

template <int G>
BwLayout bw_layout(const Plan *p, int64_t N) {
    using C = BwCfg<G>;
    BwLayout L;
    const int64_t n_pad = (N + kBwTok - 1) / kBwTok * kBwTok;
    L.KT = (int)(n_pad / 16);
    L.ptiles = (int)(n_pad / kBwTok);
    L.tiles_i = (p->C_in + C::BI - 1) / C::BI;
    L.tiles_o = (p->C_out + C::BO - 1) / C::BO;
    L.C_in_pad = L.tiles_i * C::BI;
    L.C_out_pad = L.tiles_o * C::BO;
    L.CB_in = L.C_in_pad / 32;
    L.CB_out = L.C_out_pad / 32;
    const int tiles = L.tiles_i * L.tiles_o;
    const int cus = device_num_cus();
    // token splits: enough workgroups to stream the fragments (cus / tiles), at least 8 token steps
    // each, and no more than balances a split's fragment reads (KT / S steps at a CU's ~90 GB/s)
    // against the partial planes all splits write and the reduction reads back (S x the tile's
    // output at ~3 TB/s for the chip): S ~ sqrt(KT * step bytes * 33 / tile bytes) (estimates)
    const double step_bytes = (double)(C::BO + C::BI) * 16 * G * 2, out_bytes = (double)C::BO * C::BI * G * 4;
    const int s_bal = std::max(1, (int)std::sqrt((double)L.KT * step_bytes * 33.0 / out_bytes));
    L.splits = std::max(1, std::min({cus / std::max(1, tiles), L.KT / 8, s_bal}));
    auto al = [](size_t v) { return (v + 255) / 256 * 256; };
    L.off_x = 0;
    L.off_dy = al(L.off_x + (size_t)L.CB_in * L.KT * G * 1024);
    L.off_part = al(L.off_dy + (size_t)L.CB_out * L.KT * G * 1024);
    L.off_db = al(L.off_part + (size_t)L.splits * G * L.C_out_pad * L.C_in_pad * 4);
    L.total = al(L.off_db + (size_t)L.ptiles * L.C_out_pad * 4);
    return L;
}

// The fused small-channel pass (k_bw_small): its conditions and workspace.
struct SmallLayout {
    bool ok = false;
    int CB_in = 0, CB_out = 0, tok_wg = 0, splits = 0;
    size_t lds = 0, off_part = 0, off_db = 0, off_psum = 0, total = 0;
    int n_groups = 0;  // reduction position groups (32 positions of the padded grid)
};

SmallLayout small_layout(const Plan *p, int64_t N) {
    SmallLayout L;
    const int G = p->G;
    if (p->dtype == EQLIN_F32 || (G != 4 && G != 8) || N <= 0) return L;
    L.CB_in = (p->C_in + 31) / 32;
    L.CB_out = (p->C_out + 31) / 32;
    if (L.CB_in * L.CB_out * G > 8 * SmallBwCfg::maxb(G)) return L;  // accumulator blocks per workgroup
    if ((p->C_in + p->C_out) * G / 2 > SmallBwCfg::NT) return L;  // one load item per thread
    if ((p->C_in * G) % 128 != 0 || p->C_out % 8 != 0) return L;  // wave-uniform x/dy items
    if (N * p->C_in * G * 2 > 0x7fffffff || N * p->C_out * G * 2 > 0x7fffffff) return L;  // 32-bit offsets
    L.lds = (size_t)2 * SmallBwCfg::KT * (L.CB_in + L.CB_out) * G * 1024;
    if (L.lds > 160 * 1024) return L;
    // one token range per compute unit (each range costs one full C_out x C_in x G partial spectrum)
    const int ranges = device_num_cus();
    const int64_t per = (N + ranges - 1) / ranges;
    L.tok_wg = (int)((per + SmallBwCfg::ST - 1) / SmallBwCfg::ST * SmallBwCfg::ST);
    L.splits = (int)((N + L.tok_wg - 1) / L.tok_wg);
    if (L.splits > 256) return L;  // the reduction's shares hold at most 256 ranges
    auto al = [](size_t v) { return (v + 255) / 256 * 256; };
    L.off_part = 0;
    L.off_db = al((size_t)L.splits * G * (L.CB_out * 32) * (L.CB_in * 32) * 4);
    L.off_psum = al(L.off_db + (size_t)L.splits * (L.CB_out * 32) * 4);
    L.n_groups = (int)((int64_t)p->C_out * L.CB_in * 32 / 32);
    L.total = al(L.off_psum + (size_t)G * (L.CB_out * 32) * (L.CB_in * 32) * 4);
    L.ok = true;
    return L;
}

// the fused pass's instance for the element type
typedef void (*SmallFn)(const uint16_t *, const uint16_t *, int64_t, int, int, int, int, int, float *, float *);
template <int G, bool D4>
SmallFn kernel_small(eqlin_dtype_t dt) {
    if (dt == EQLIN_F16) return k_bw_small<G, D4, F16>;
    return k_bw_small<G, D4, BF16>;
}

template <int G, bool D4>
hipError_t launch_small(const Plan *p, const SmallLayout &L, const void *x, const void *dy, float *dW, float *db,
                        int64_t N, void *ws, hipStream_t s) {
    char *w = static_cast<char *>(ws);
    float *part = reinterpret_cast<float *>(w + L.off_part), *dbp = reinterpret_cast<float *>(w + L.off_db);
    float *psum = reinterpret_cast<float *>(w + L.off_psum);
    const SmallFn kfn = kernel_small<G, D4>(p->dtype);
    if (L.lds > 65536) {
        const hipError_t e =
            hipFuncSetAttribute((const void *)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kfn, dim3(L.splits), dim3(SmallBwCfg::NT), L.lds, s, (const uint16_t *)x,
                       (const uint16_t *)dy, N, p->C_in, p->C_out, L.tok_wg, L.CB_in, L.CB_out, part, dbp);
    const int n_main = L.n_groups * G;
    const int n_db = db ? (p->C_out + 31) / 32 : 0;
    hipLaunchKernelGGL((k_bw_small_reduce<G, D4>), dim3(n_main + n_db), dim3(512), 0, s, (const float *)part,
                       (const float *)dbp, L.splits, p->C_out, L.CB_out * 32, L.CB_in * 32, n_main, psum, db);
    const int64_t n_inv = ((int64_t)p->C_out * p->C_in + 255) / 256;
    hipLaunchKernelGGL((k_bw_small_inverse<G, D4>), dim3((unsigned)n_inv), dim3(256), 0, s, (const float *)psum, p->C_out,
                       p->C_in, L.CB_out * 32, L.CB_in * 32, dW);
    return hipGetLastError();
}

BwLayout layout_for(const Plan *p, int64_t N) {
    if (p->G == 8) return bw_layout<8>(p, N);
    return bw_layout<4>(p, N);
}

template <int G, class E, bool D4 = false>
hipError_t launch_mfma(const Plan *p, const void *x, const void *dy, float *dW, float *db, int64_t N, void *ws,
                       hipStream_t s) {
    const BwLayout L = bw_layout<G>(p, N);
    char *w = static_cast<char *>(ws);
    uint4 *xf = reinterpret_cast<uint4 *>(w + L.off_x), *dyf = reinterpret_cast<uint4 *>(w + L.off_dy);
    float *part = reinterpret_cast<float *>(w + L.off_part), *dbp = reinterpret_cast<float *>(w + L.off_db);
    if ((int64_t)L.ptiles > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_bw_planes<G, E, D4>), dim3(L.ptiles, L.CB_in), dim3(256), 0, s, (const uint16_t *)x, N, p->C_in,
                       L.KT, xf, (float *)nullptr);
    hipLaunchKernelGGL((k_bw_planes<G, E, D4>), dim3(L.ptiles, L.CB_out), dim3(256), 0, s, (const uint16_t *)dy, N, p->C_out,
                       L.KT, dyf, dbp);
    const int grid = L.tiles_i * L.tiles_o * L.splits;
    hipLaunchKernelGGL((k_bw_gemm<G, E, D4>), dim3(grid), dim3(512), 0, s, (const uint4 *)xf, (const uint4 *)dyf, part,
                       L.KT, L.tiles_i, L.splits, L.C_in_pad, L.C_out_pad);
    const int64_t rgrid = (int64_t)p->C_out * (L.C_in_pad / 32);
    if (rgrid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_bw_reduce<G, D4>), dim3((unsigned)rgrid), dim3(256), 0, s, (const float *)part, L.splits,
                       p->C_out, p->C_in, L.C_out_pad, L.C_in_pad, dW);
    if (db)
        hipLaunchKernelGGL(k_bw_dbsum, dim3((p->C_out + 3) / 4), dim3(256), 0, s, (const float *)dbp, L.ptiles,
                           p->C_out, L.C_out_pad, db);
    return hipGetLastError();
}

template <typename T, int G, bool D4 = false>
hipError_t launch_direct(const Plan *p, const void *x, const void *dy, float *dW, float *db, int64_t N,
                         hipStream_t s) {
    hipLaunchKernelGGL((k_bw_direct<T, G, D4>), dim3((p->C_in + 15) / 16, (p->C_out + 15) / 16), dim3(256), 0, s,
                       x, dy, N, p->C_in, p->C_out, dW);
    if (db) hipLaunchKernelGGL(k_bw_bias<T>, dim3((p->C_out + 63) / 64), dim3(256), 0, s, dy, N, p->C_out, G, db);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_direct_g(const Plan *p, const void *x, const void *dy, float *dW, float *db, int64_t N,
                           hipStream_t s) {
    switch (p->G) {
        case 1: return launch_direct<T, 1>(p, x, dy, dW, db, N, s);
        case 2: return launch_direct<T, 2>(p, x, dy, dW, db, N, s);
        case 4: return launch_direct<T, 4>(p, x, dy, dW, db, N, s);
        case 8: return p->d4 ? launch_direct<T, 8, true>(p, x, dy, dW, db, N, s)
                             : launch_direct<T, 8, false>(p, x, dy, dW, db, N, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t bw_workspace_bytes(const Plan *p, int64_t N) {
    const SmallLayout S = small_layout(p, N);
    if (S.ok) return S.total;
    if (!mfma_path(p) || N <= 0) return 0;
    return layout_for(p, N).total;
}

hipError_t launch_backward_weights(const Plan *p, const void *x, const void *dy, float *dW, float *db, int64_t N,
                                   void *ws, hipStream_t s) {
    const SmallLayout S = small_layout(p, N);
    if (S.ok) return p->G == 8 ? (p->d4 ? launch_small<8, true>(p, S, x, dy, dW, db, N, ws, s)
                                        : launch_small<8, false>(p, S, x, dy, dW, db, N, ws, s))
                               : launch_small<4, false>(p, S, x, dy, dW, db, N, ws, s);
    if (mfma_path(p)) {
        const bool f16 = p->dtype == EQLIN_F16;
        if (p->d4)
            return f16 ? launch_mfma<8, F16, true>(p, x, dy, dW, db, N, ws, s)
                       : launch_mfma<8, BF16, true>(p, x, dy, dW, db, N, ws, s);
        if (f16)
            return p->G == 8 ? launch_mfma<8, F16>(p, x, dy, dW, db, N, ws, s) : launch_mfma<4, F16>(p, x, dy, dW, db, N, ws, s);
        return p->G == 8 ? launch_mfma<8, BF16>(p, x, dy, dW, db, N, ws, s) : launch_mfma<4, BF16>(p, x, dy, dW, db, N, ws, s);
    }
    if (p->dtype == EQLIN_BF16) return launch_direct_g<BF16>(p, x, dy, dW, db, N, s);
    if (p->dtype == EQLIN_F16) return launch_direct_g<F16>(p, x, dy, dW, db, N, s);
    return launch_direct_g<float>(p, x, dy, dW, db, N, s);
}

const char *bw_kernel_name(const Plan *p) {
    // (the fused pass serves every token count at these channel counts up to the 2 GB offset limit)
    if (small_layout(p, 1).ok) return "fused dft + mfma32x32x16 per token range + reduce (small channels)";
    return mfma_path(p) ? "dft planes + plane-split mfma32x32x16 split-K + reduce" : "direct fp32 valu";
}

}  // namespace eqlin
