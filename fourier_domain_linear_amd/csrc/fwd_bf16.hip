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
//   k_stream    small C_in (a row block's x fits in registers): one persistent workgroup per CU
//               keeps the C_out tile's weight chunks in LDS (copied with global_load_lds, no VGPR
//               staging) and streams 16-token row blocks through its waves; x goes straight from
//               global memory into the A operands.
//   (larger channel counts go to k_big in fwd_big.hip)
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>

#include "act.h"
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

// G samples of 8 channels (channel-major, sample-minor: element j*G+g) -> G planes of 8 bf16 (the
// cyclic group's DFT, or D4's Fourier transform when D4).
template <int G, bool D4, class E>
__device__ __forceinline__ void dft_to_frags(const uint4 (&r)[G], uint4 (&a)[G]) {
    float pl[G][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v[G], P[G];
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] = elem_at<E>(r[(j * G + g) >> 3], (j * G + g) & 7);
        group_forward<G, D4>(v, P);
#pragma unroll
        for (int p = 0; p < G; ++p) pl[p][j] = P[p];
    }
#pragma unroll
    for (int p = 0; p < G; ++p) a[p] = pack8<E>(pl[p]);
}

// Negated copies of the imaginary planes (p odd, p >= 3) for the Re = XrWr - XiWi products.
template <int G>
__device__ __forceinline__ void negate_imag(const uint4 (&a)[G], uint4 (&an)[G]) {
#pragma unroll
    for (int p = 0; p < G; ++p) an[p] = (p >= 3 && (p & 1)) ? neg_bf16x8(a[p]) : a[p];
}

// The 2G-2 real products with the weights as the A operand (rows = outputs) and the x planes as
// the B operand (columns = tokens): D lane l holds outputs 4*(l/16)+v of token l%16. D4: the four
// characters' products, then Y(rho) = X(rho) W(rho) entry by entry, Y_ab += W_cb X_ac over c = 0, 1
// (twelve products; no negated operand).
template <int G, bool D4, class E>
__device__ __forceinline__ void spectral_mfma_wx(const uint4 (&w)[G], const uint4 (&a)[G],
                                                 const uint4 (&an)[G], f32x4 (&acc)[G]) {
    if constexpr (D4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = mma16<E>(w[k], a[k], acc[k]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ra = e >> 1, cb = e & 1;
            acc[4 + e] = mma16<E>(w[4 + cb], a[4 + 2 * ra], acc[4 + e]);
            acc[4 + e] = mma16<E>(w[6 + cb], a[5 + 2 * ra], acc[4 + e]);
        }
        return;
    }
    acc[0] = mma16<E>(w[0], a[0], acc[0]);
    if constexpr (G >= 2) acc[1] = mma16<E>(w[1], a[1], acc[1]);
#pragma unroll
    for (int k = 1; k < G / 2; ++k) {
        const int r = 2 * k, i = 2 * k + 1;
        acc[r] = mma16<E>(w[r], a[r], acc[r]);
        acc[r] = mma16<E>(w[i], an[i], acc[r]);
        acc[i] = mma16<E>(w[i], a[r], acc[i]);
        acc[i] = mma16<E>(w[r], a[i], acc[i]);
    }
}

// Element-wise tail store for a partial output block or the last token rows: output o0 + v of token n.
template <int G, bool GELU, bool D4, class E>
__device__ __forceinline__ void store_quad_masked(const f32x4 (&acc)[G], uint16_t *__restrict__ y,
                                                  int64_t n, int64_t N, int o0, int C_out) {
    if (n >= N) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        if (o0 + v >= C_out) continue;
        float Y[G], out[G];
#pragma unroll
        for (int p = 0; p < G; ++p) Y[p] = acc[p][v];
        group_inverse<G, D4>(Y, out);
        apply_act<GELU>(out);
        uint16_t *dst = y + (n * C_out + o0 + v) * G;
#pragma unroll
        for (int h = 0; h < G; ++h) dst[h] = pack1<E>(out[h]);
    }
}

// ------------------------------------------------------------------------------------------------
// k_stream<G, KS>: small C_in (KS 32-channel steps held in registers). One persistent workgroup of
// NW waves per CU and per C_out tile. The tile's weight chunks are staged in LDS once; the
// workgroup's token range is an even share of the 16-token row blocks, dealt round-robin to its
// waves. Per row block a wave: DFTs the block (x already in registers), issues the loads of its
// next block, then for each 16-output block runs the K-step products and stores the result, so the
// stores of one output block overlap the products of the next and the next block's loads overlap
// both.
// grid = (token workgroups, C_out tiles); dynamic LDS = nb_tile * KS * G KB.
constexpr int kStreamWaves = 8;
constexpr int kStreamBiasPerThread = 8;  // bias values staged per thread: tiles of <= 4096 outputs

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory operations are
// outstanding and all LDS/scalar-memory operations are done; export counter not waited on.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }
static_assert(waitcnt_vm_lgkm0(0) == 0x70, "waitcnt encoding");

// Geometry of the stream kernel's data movement for group order G. Every global access moves whole
// 128-byte lines: x arrives through coalesced non-temporal loads and is re-ordered into matrix-core
// operands through a small per-wave LDS exchange buffer; y leaves the same way in reverse.
//   x exchange unit: U K-steps (32 channels each) of 16 rows; PX 16-byte pieces per row.
//   y store unit: UO 16-output blocks of 16 rows; PPR 16-byte pieces per row.
// A lane's operand for K-step ks, load q, lane group g = lane/16 is piece 4q + g of the K-step's
// 4G pieces of its row (whole channels: a piece holds 8/G channels x G samples); the prepared
// weights use the same k order.
template <int G>
struct StreamGeom {
    static constexpr int U = G == 1 ? 2 : 1;
    static constexpr int PX = 4 * G * U;
    static constexpr int XROWS = 64 / PX;   // rows per coalesced load instruction
    static constexpr int XINST = 16 / XROWS;
    static constexpr int UO = G >= 4 ? 1 : 4 / G;
    static constexpr int PPR = UO * 2 * G;
    static constexpr int OROWS = 64 / PPR;  // rows per store instruction
    static constexpr int OINST = 16 / OROWS;
    static constexpr int SCRATCH = 16 * 16 * (PX > PPR ? PX : PPR);  // bytes per wave
};

// XOR swizzle of a 16-row x P-piece tile in LDS: conflict-free for both the row-major coalesced side
// and the column-wise (16 rows, one piece) operand side.
template <int P>
__device__ __forceinline__ int swz(int r, int p) { return r * P + (p ^ (r & 7)); }

__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint4 *p, const uint4 &v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

// Coalesced non-temporal loads of one 16-token row block: exchange unit u, instruction i, lane l
// reads piece u*PX + l%PX of row i*XROWS + l/PX. Tokens past N re-read row N-1 and pieces past the
// row end re-read its last piece (both discarded: never stored / met by zero weight columns).
template <int G, int KS>
__device__ __forceinline__ void load_x_raw(const uint4 *__restrict__ x4, int64_t blk, int64_t N,
                                           int row_pieces, int lane,
                                           uint4 (&xr)[KS / StreamGeom<G>::U][StreamGeom<G>::XINST]) {
    using SG = StreamGeom<G>;
#pragma unroll
    for (int u = 0; u < KS / SG::U; ++u)
#pragma unroll
        for (int i = 0; i < SG::XINST; ++i) {
            const int64_t n = blk * 16 + i * SG::XROWS + lane / SG::PX;
            const int64_t nc = n < N ? n : N - 1;
            const int pc = min(u * SG::PX + lane % SG::PX, row_pieces - 1);
            xr[u][i] = ld_nt(x4 + nc * row_pieces + pc);
        }
}

template <int G, int KS, bool GELU, bool D4, class E>
__global__ __launch_bounds__(kStreamWaves * 64) void k_stream(const uint4 *__restrict__ x4,
                                                              const uint4 *__restrict__ wfrag,
                                                              const uint16_t *__restrict__ bias,
                                                              int bias_shift, uint16_t *__restrict__ y,
                                                              int64_t N, int C_in, int C_out,
                                                              int nb_tile) {
    using SG = StreamGeom<G>;
    static_assert(KS % SG::U == 0, "KS must be a multiple of the exchange unit");
    constexpr int NU = KS / SG::U;
    extern __shared__ uint4 lds[];
    constexpr int NW = kStreamWaves;
    const int lane = threadIdx.x & 63;
    // the wave index through a scalar register: the compiler then knows that the block index and the
    // buffer resources derived from it are wave-uniform (no per-lane loop around each buffer access)
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int g = lane >> 4;
    const int nb0 = blockIdx.y * nb_tile;
    const int64_t blocks = (N + 15) >> 4;
    const int64_t b0 = (int64_t)blockIdx.x * blocks / gridDim.x;
    const int64_t b1 = (int64_t)(blockIdx.x + 1) * blocks / gridDim.x;
    const int row_pieces = C_in * G / 8;             // 16-byte pieces per x row
    const int yrow_pieces = C_out * G / 8;           // 16-byte pieces per y row (when C_out*G % 8 == 0)

    // LDS: [weights: nb_tile*KS*G KB][bias: nb_tile*16 fp32][per-wave scratch: SCRATCH bytes each]
    const int chunks = nb_tile * KS * G;
    float *lbias = reinterpret_cast<float *>(lds + chunks * 64);
    uint4 *scratch = lds + chunks * 64 + nb_tile * 4 + wave * (SG::SCRATCH / 16);

    // Prologue, ordered so that the x loads of the wave's first block are the youngest memory
    // operations: (1) this thread's share of the tile's bias (raw bf16, clamped unconditional
    // loads), (2) the tile's weight chunks global -> LDS (contiguous in global memory for a tile),
    // (3) x. The barrier then waits only for (1) and (2) -- vector-memory counter down to the KS*G
    // x loads, which complete in order after them -- so each wave starts as soon as its own x has
    // arrived. s_barrier is issued without the block-wide memory fence of __syncthreads() (which
    // would wait for the x loads too). Without a bias the loads read the weight buffer instead
    // (valid memory, discarded), so no loaded value is selected before the wait.
    const int n_bias = nb_tile * 16;
    const int bias_len = (C_out + (1 << bias_shift) - 1) >> bias_shift;
    const uint16_t *bsrc = bias ? bias : reinterpret_cast<const uint16_t *>(wfrag);
    const int blen = bias ? bias_len : 1;
    uint32_t braw[kStreamBiasPerThread];
#pragma unroll
    for (int k = 0; k < kStreamBiasPerThread; ++k) {
        const int o = nb0 * 16 + threadIdx.x + k * NW * 64;
        braw[k] = bsrc[min(o >> bias_shift, blen - 1)];
    }
    const uint4 *src = wfrag + (size_t)nb0 * KS * G * 64;
    for (int c = wave; c < chunks; c += NW) chunk_to_lds(src + c * 64 + lane, lds + c * 64);

    // (a wave without a block of its own loads the workgroup's first block: cache hits, discarded)
    int64_t blk = b0 + wave;
    uint4 xr[NU][SG::XINST];
    __builtin_amdgcn_sched_barrier(0);
    load_x_raw<G, KS>(x4, blk < b1 ? blk : b0, N, row_pieces, lane, xr);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(KS * G));
#pragma unroll
    for (int k = 0; k < kStreamBiasPerThread; ++k) {
        const int t = threadIdx.x + k * NW * 64;
        if (t < n_bias) lbias[t] = (bias && nb0 * 16 + t < C_out) ? elem_to_float<E>((uint16_t)braw[k]) : 0.f;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    asm volatile("s_barrier" ::: "memory");

    const int nb_end = min(nb_tile, (C_out + 15) / 16 - nb0);
    const bool vec_rows = (C_out * G) % 8 == 0;  // 16-byte pieces tile the y rows exactly
    for (; blk < b1; blk += NW) {
        // x: exchange through LDS into operand order, then the group DFT -> bf16 planes
        uint4 a[KS][G], an[KS][G];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int i = 0; i < SG::XINST; ++i)
                scratch[swz<SG::PX>(i * SG::XROWS + lane / SG::PX, lane % SG::PX)] = xr[u][i];
#pragma unroll
            for (int ku = 0; ku < SG::U; ++ku) {
                uint4 r[G];
#pragma unroll
                for (int q = 0; q < G; ++q) r[q] = scratch[swz<SG::PX>(lane & 15, ku * 4 * G + 4 * q + g)];
                dft_to_frags<G, D4, E>(r, a[u * SG::U + ku]);
                if constexpr (!D4) negate_imag<G>(a[u * SG::U + ku], an[u * SG::U + ku]);
            }
        }
        const int64_t nxt = blk + NW;
        if (nxt < b1) load_x_raw<G, KS>(x4, nxt, N, row_pieces, lane, xr);

        const int64_t nrow0 = blk * 16;
        // the block's output rows, for range-checked stores: rows past N are dropped by the hardware
        const int64_t rows = N - nrow0 < 16 ? N - nrow0 : 16;
        const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
            y + nrow0 * C_out * G, (short)0, (int)(rows * yrow_pieces * 16), 0x00020000);
        // Weight fragments are read from LDS a whole 16-output block ahead of their products when the
        // block's KS*G fragments fit the register budget (else as the products need them).
        constexpr bool kWholeBlock = KS * G <= 12;
        constexpr int PF = kWholeBlock ? KS : 1;
        uint4 bw[2][PF][G];
        if constexpr (kWholeBlock) {
#pragma unroll
            for (int ks = 0; ks < PF; ++ks)
#pragma unroll
                for (int p = 0; p < G; ++p) bw[0][ks][p] = lds[(ks * G + p) * 64 + lane];
        }
        for (int nb = 0; nb < nb_end; ++nb) {
            const float4 bq = reinterpret_cast<const float4 *>(lbias)[nb * 4 + g];
            f32x4 acc[G];
            acc[0] = f32x4{bq.x, bq.y, bq.z, bq.w};
#pragma unroll
            for (int p = 1; p < G; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (kWholeBlock) {
                const int nbn = nb + 1 < nb_end ? nb + 1 : nb;  // last block: harmless re-read
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int p = 0; p < G; ++p) bw[1][ks][p] = lds[((nbn * KS + ks) * G + p) * 64 + lane];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) spectral_mfma_wx<G, D4, E>(bw[0][ks], a[ks], an[ks], acc);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int p = 0; p < G; ++p) bw[0][ks][p] = bw[1][ks][p];
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int p = 0; p < G; ++p) bw[0][0][p] = lds[((nb * KS + ks) * G + p) * 64 + lane];
                    spectral_mfma_wx<G, D4, E>(bw[0][0], a[ks], an[ks], acc);
                }
            }
            if (!vec_rows) {
                store_quad_masked<G, GELU, D4, E>(acc, y, nrow0 + (lane & 15), N, (nb0 + nb) * 16 + 4 * g, C_out);
                continue;
            }
            // inverse DFT (+ activation) -> this lane's 4 outputs x G (8G bytes) -> staging row lane%16,
            // one 16-byte piece (8 / G outputs) at a time to keep few values live
            const int ub = nb % SG::UO;  // block within the store unit
            if constexpr (G == 1) {
                float out[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) out[v] = acc[0][v];
                apply_act<GELU>(out);
                uint2 w;
                w.x = pack2<E>(out[0], out[1]);
                w.y = pack2<E>(out[2], out[3]);
                // 8 bytes at byte (ub*32 + g*8) of the row's 128-byte unit segment
                const int piece = ub * 2 + (g >> 1);
                reinterpret_cast<uint2 *>(scratch + swz<SG::PPR>(lane & 15, piece))[g & 1] = w;
            } else {
                constexpr int VP = 8 / G;  // outputs per piece
#pragma unroll
                for (int k = 0; k < G / 2; ++k) {
                    float out[8];
#pragma unroll
                    for (int vv = 0; vv < VP; ++vv) {
                        float Y[G];
#pragma unroll
                        for (int p = 0; p < G; ++p) Y[p] = acc[p][k * VP + vv];
                        group_inverse<G, D4>(Y, out + vv * G);
                    }
                    apply_act<GELU>(out);
                    scratch[swz<SG::PPR>(lane & 15, ub * 2 * G + g * (G / 2) + k)] = pack8<E>(out);
                }
            }
            if (ub == SG::UO - 1 || nb == nb_end - 1) {
                // whole 16-byte pieces of the unit's rows, full lines per instruction, non-temporal
                const int unit_o0 = (nb0 + nb - ub) * 16;  // first output of the unit
                const int piece0 = unit_o0 * G / 8;
#pragma unroll
                for (int j = 0; j < SG::OINST; ++j) {
                    const int r = j * SG::OROWS + lane / SG::PPR, pc = lane % SG::PPR;
                    const uint4 v = scratch[swz<SG::PPR>(r, pc)];
                    // only the pieces of blocks computed in this unit (a tile's last unit may be
                    // partial; the rest of its row belongs to the next tile or past C_out); others
                    // get an offset past the range, which drops them (no branches)
                    const int keep = -(int)((pc < (ub + 1) * 2 * G) & (piece0 + pc < yrow_pieces));
                    const int off = (r * yrow_pieces + piece0 + pc) * 16;
                    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
                    const u32x4 d = {v.x, v.y, v.z, v.w};
                    __builtin_amdgcn_raw_buffer_store_b128(d, yrs, (off & keep) | (0x7fffffff & ~keep), 0,
                                                           2 /* non-temporal */);
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Launchers and selection.

// Raise the kernel's dynamic-LDS limit above 64 KB where needed (gfx950 has 160 KB per CU). A refusal
// makes the selection below fall back to the large-channel kernel (static LDS, no attribute needed).
// EQLIN_FAULT_LDS_LIMIT=<bytes> (fault injection for the tests) refuses every request above <bytes>.
static hipError_t set_lds_limit(const void *fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    if (const char *cap = getenv("EQLIN_FAULT_LDS_LIMIT"))
        if (bytes > (size_t)strtoull(cap, nullptr, 10)) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    (void)hipGetLastError();
    return e;
}

static int g_num_cus = 0;

int device_num_cus() {
    if (g_num_cus <= 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            g_num_cus = n;
        else
            g_num_cus = 256;
    }
    return g_num_cus;
}

template <int G, int KS, bool D4>
static hipError_t launch_stream(const Plan *p, const void *x, const void *b, void *y, int64_t N, int act,
                                hipStream_t s) {
    const size_t lds = p->fwd.lds_bytes;
    const int64_t blocks = (N + 15) / 16;
    const int tiles = p->NB_total / p->fwd.nb_tile;
    // one workgroup per CU in total (over all C_out tiles), at least one row block each
    int64_t wg = std::max<int64_t>(1, p->fwd.num_cus / tiles);
    wg = std::min<int64_t>(wg, blocks);
    const dim3 grid((unsigned)wg, (unsigned)tiles), block(kStreamWaves * 64);
    const bool gelu = act == EQLIN_ACT_GELU;
    auto kern = p->dtype == EQLIN_F16 ? (gelu ? k_stream<G, KS, true, D4, F16> : k_stream<G, KS, false, D4, F16>)
                                      : (gelu ? k_stream<G, KS, true, D4, BF16> : k_stream<G, KS, false, D4, BF16>);
    hipLaunchKernelGGL(kern, grid, block, lds, s, (const uint4 *)x, (const uint4 *)p->planes, (const uint16_t *)b,
                       p->bias_shift, (uint16_t *)y, N, p->C_in, p->C_out, p->fwd.nb_tile);
    return hipGetLastError();
}

template <int G, int KS, bool D4>
static hipError_t init_stream(size_t lds) {
    const void *fns[] = {(const void *)k_stream<G, KS, false, D4, BF16>, (const void *)k_stream<G, KS, true, D4, BF16>,
                         (const void *)k_stream<G, KS, false, D4, F16>, (const void *)k_stream<G, KS, true, D4, F16>};
    for (const void *f : fns) {
        const hipError_t e = set_lds_limit(f, lds);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

struct StreamEntry {
    int G, KS;
    bool d4;
    LaunchFn launch;
    hipError_t (*init)(size_t);
};
#define SE(G, KS) {G, KS, false, launch_stream<G, KS, false>, init_stream<G, KS, false>}
#define SD(KS) {8, KS, true, launch_stream<8, KS, true>, init_stream<8, KS, true>}
static const StreamEntry kStream[] = {
    SE(1, 2), SE(1, 4), SE(1, 6), SE(1, 8), SE(1, 10), SE(1, 12), SE(1, 14), SE(1, 16),
    SE(2, 1), SE(2, 2), SE(2, 3), SE(2, 4), SE(2, 6), SE(2, 8),
    SE(4, 1), SE(4, 2), SE(4, 3), SE(4, 4),
    SE(8, 1), SE(8, 2),
    SD(1), SD(2),  // the dihedral group D4 (order 8)
};
#undef SE
#undef SD
static constexpr size_t kStreamLdsMax = 160 * 1024;
static constexpr int kStreamMaxTiles = 4;

static size_t stream_scratch(int G) {
    switch (G) {
        case 1: return StreamGeom<1>::SCRATCH;
        case 2: return StreamGeom<2>::SCRATCH;
        case 4: return StreamGeom<4>::SCRATCH;
        default: return StreamGeom<8>::SCRATCH;
    }
}

bool select_bf16(int G, bool d4, int C_in, int C_out, KernelChoice *out) {
    const int KS = (C_in + 31) / 32;
    const int nb_needed = (C_out + 15) / 16;
    // Stream kernel when x of a row block fits in registers (an instantiated KS) and the C_out tiles
    // whose weights fit LDS number at most kStreamMaxTiles (x is re-read and re-transformed per tile).
    for (const auto &e : kStream) {
        if (e.G != G || e.KS != KS || e.d4 != d4) continue;
        const size_t fixed = (size_t)kStreamWaves * stream_scratch(G);
        const size_t per_nb = (size_t)KS * G * 1024 + 16 * sizeof(float);
        const int nb_fit = (int)((kStreamLdsMax - fixed) / per_nb);
        if (nb_fit < 1) break;
        const int tiles = (nb_needed + nb_fit - 1) / nb_fit;
        if (tiles > kStreamMaxTiles) break;
        const int nb_tile = (nb_needed + tiles - 1) / tiles;
        if (nb_tile * 16 > kStreamBiasPerThread * kStreamWaves * 64) break;
        out->kind = KIND_STREAM;
        out->nb_tile = nb_tile;
        out->tokens_per_block = 16;
        out->block_threads = kStreamWaves * 64;
        out->lds_bytes = (size_t)nb_tile * per_nb + fixed;
        out->num_cus = device_num_cus();
        out->frag_kind = 1;
        out->rows_per_block = 16;
        out->kc = 32;
        out->ks_mult = 1;
        out->launch = e.launch;
        if (e.init(out->lds_bytes) != hipSuccess) break;  // LDS limit refused: the large-channel kernel
        snprintf(out->name, sizeof(out->name), "bf16 stream %s%d KS=%d nb_tile=%d tiles=%d waves=%d",
                 d4 ? "D" : "G=", d4 ? 4 : G, KS, nb_tile, tiles, kStreamWaves);
        return true;
    }
    return select_big(G, d4, C_in, C_out, out);
}

}  // namespace eqlin
