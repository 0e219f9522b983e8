// fwd_res.hip -- the p4 (G = 4) spectral EQ-Linear forward for wide layers whose input planes fit on
// chip (C_in up to 256 channels), bf16 / fp16 in and out, on v_mfma_f32_32x32x16.
//
// Method: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
// Transform" (gist.science explainer), "Enfoque Algorítmico" (group DFT, then one channel product per
// frequency k = 0..G/2), "Especialización para el Grupo de Rotación p4" (the p4 transforms are
// additions only; six real products per channel pair), "Implementación" (one fused kernel, the
// Fourier fragments kept on chip, no intermediate global writes).
//
// One workgroup per token tile of BT <= 64 tokens (BT = ceil(N / CUs) when that is at most 64, so
// every compute unit gets one tile and none a second). The tile's x is read from HBM once and its
// four frequency planes (all C_in channels, two 32-token MFMA blocks) stay in LDS for the whole
// workgroup: every output block of the layer is computed against them, so each token is transformed
// once however wide the layer is. The eight waves own distinct 32-output blocks (wave w: blocks w,
// w + 8, ...), so each streams only its own weight fragments from L2 (through a register ring four
// 16-channel steps deep) and no two waves wait for each other once the planes are complete:
//   - the planes are filled during each wave's first output block: the raw x of 32 channels (two
//     16-channel steps) is requested one such part ahead, transformed into the planes one part ahead
//     of its products, and the waves meet at an LDS barrier once per part;
//   - every later block reads the finished planes with no barrier at all;
//   - products: x planes as the A operand (rows = tokens), weight fragments as B (columns = outputs);
//     a complex frequency is four real products (Re = Xr Wr - Xi Wi via a sign-flipped Wi fragment);
//   - epilogue: inverse DFT in fp32 (the bias added to the k = 0 plane, i.e. to every sample), one
//     rounding, and 8-byte stores straight from the accumulator registers: for one accumulator row
//     the 32 lanes of a half-wave hold 32 consecutive outputs of one token, i.e. 256 contiguous bytes
//     of y, so every store instruction writes whole 128-byte lines.
#include <stdio.h>

#include <algorithm>

#include "act.h"
#include "device_common.h"
#include "eqlin_internal.h"

namespace eqlin {

namespace {

constexpr int kResWaves = 8, kResThreads = kResWaves * 64;
constexpr int kResMaxBT = 64;     // two 32-token blocks
constexpr int kResRing = 4;       // weight steps in flight per wave (16 channels each)
constexpr int kResMaxKS = 16;     // 16-channel steps of planes (8 KB each; C_in <= 256), plus two
constexpr int kResLdsSteps = kResMaxKS + 2;  // spare steps that past-the-end parts are written to
constexpr int kResStoreAux = 2;   // output stores non-temporal

// LDS chunk of (16-channel step ks, token block b, plane p): 64 lanes x 16 bytes, lane l holding token
// 32b + l % 32 and channels 16 ks + 8 (l / 32) .. + 7 (the 32x32x16 operand layout).
__device__ __forceinline__ int res_chunk(int ks, int b, int p) { return ((ks * 2 + b) * 4 + p) * 64; }

// One step of products for token block b: acc[0] += X0 W0, acc[1] += X2 W2 (the real k = 0 and k = 2
// planes), acc[2] (Re Y1) += Xr Wr + Xi (-Wi), acc[3] (Im Y1) += Xr Wi + Xi Wr. F: a block's first
// step, whose products start the accumulators from zero.
template <bool F, class E>
__device__ __forceinline__ void res_products(const uint4 (&xa)[4], const uint4 (&w)[4], const uint4 &wn,
                                             f32x16 (&acc)[4]) {
    auto c = [&](int p) { return F ? f32x16{} : acc[p]; };
    acc[0] = mma32<E>(xa[0], w[0], c(0));
    acc[1] = mma32<E>(xa[1], w[1], c(1));
    acc[2] = mma32<E>(xa[2], w[2], c(2));
    acc[3] = mma32<E>(xa[2], w[3], c(3));
    acc[2] = mma32<E>(xa[3], wn, acc[2]);
    acc[3] = mma32<E>(xa[3], w[2], acc[3]);
}

__device__ __forceinline__ void res_lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
    asm volatile("s_barrier" ::: "memory");
}

template <int V>
struct IC {
    static constexpr int value = V;
};

template <bool GELU, class E>
__global__ __launch_bounds__(kResThreads) void k_res(const uint4 *__restrict__ x4, const uint4 *__restrict__ wfrag,
                                                     const uint16_t *__restrict__ bias, uint16_t *__restrict__ y,
                                                     int64_t N, int C_in, int C_out, int KS, int NB, int BT) {
    constexpr int G = 4, R = kResRing;
    __shared__ uint4 planes[kResLdsSteps * 8 * 64];
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * BT;
    const int rows = (int)std::min<int64_t>(BT, N - n0);
    const int x_row = C_in * G * 2, y_row = C_out * G * 2;  // bytes per token row
    // x of this tile (rows past the tile read as zeros); y of this tile (stores past it are dropped)
    const __amdgpu_buffer_rsrc_t x_rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(x4 + n0 * C_in * G / 8), (short)0, rows * x_row, 0x00020000);
    const __amdgpu_buffer_rsrc_t y_rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(y + n0 * C_out * G), (short)0, rows * y_row, 0x00020000);
    // this wave's weight fragments: block wave + 8 u, step ks at chunk ((wave + 8u) KS + ks) G
    const int nu = (NB - wave + kResWaves - 1) / kResWaves;  // output blocks of this wave (>= 1)
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(wfrag + (size_t)wave * KS * G * 64), (short)0, ((nu - 1) * kResWaves * KS + KS) * G * 1024, 0x00020000);
    // step ks of block u (u past the wave's last block: the last block's, in range and unused)
    auto load_w = [&](int u, int ks, uint4 (&dst)[4]) {
        const bool past = u >= nu;  // uniform
        // (wave-uniform; said so, or the compiler may wrap each load in a loop over distinct values)
        const int soff =
            __builtin_amdgcn_readfirstlane((((past ? nu - 1 : u) * kResWaves) * KS + (past ? KS - 1 : ks)) * G * 1024);
#pragma unroll
        for (int p = 0; p < G; ++p) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(w_rs, lane * 16, soff + p * 1024, 0);
            dst[p] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    // raw x of step s: thread (token tl, channel pair cq) reads channels 16 s + 2 cq, + 1 (16 bytes)
    const int tl = tid >> 3, cq = tid & 7;
    auto load_x = [&](int s) {
        const int c = s * 16 + 2 * cq;
        const int vo = c < C_in ? tl * x_row + c * G * 2 : 0x7fffffff;  // channels past C_in: zeros
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(x_rs, vo, 0, 0);
        return make_uint4(v.x, v.y, v.z, v.w);
    };
    // transform of step s's pair into the planes: one 32-bit word (two channels) per plane
    uint32_t *const pw = reinterpret_cast<uint32_t *>(planes);
    const int slot = ((tl & 31) + 32 * (cq >> 2)) * 4 + (cq & 3);
    auto dft_store = [&](int s, const uint4 &r) {
        float v0[G], v1[G], P0[G], P1[G];
        v0[0] = elem_lo<E>(r.x); v0[1] = elem_hi<E>(r.x); v0[2] = elem_lo<E>(r.y); v0[3] = elem_hi<E>(r.y);
        v1[0] = elem_lo<E>(r.z); v1[1] = elem_hi<E>(r.z); v1[2] = elem_lo<E>(r.w); v1[3] = elem_hi<E>(r.w);
        forward_planes<G>(v0, P0);
        forward_planes<G>(v1, P1);
#pragma unroll
        for (int p = 0; p < G; ++p) pw[res_chunk(s, tl >> 5, p) * 4 + slot] = pack2<E>(P0[p], P1[p]);
    };

    // output column of this lane in each of its blocks: o = 32 (wave + 8 u) + lane % 32
    const int ocol = lane & 31, hrow = lane >> 5;
    // the lane's bias bits in block u (0: none); converted only where used (see epilogue)
    auto bias_bits = [&](int u) -> uint32_t {
        const int o = 32 * (wave + kResWaves * u) + ocol;
        return (bias && o < C_out) ? (uint32_t)bias[o] : 0u;
    };
    f32x16 acc[2][4];
    // products of step ks for both token blocks (weights w, planes from LDS); first: the block's step 0
    auto step_products = [&](auto first, int ks, const uint4 (&w)[4]) {
        constexpr bool F = decltype(first)::value;
        const uint4 wn = neg_bf16x8(w[3]);
        uint4 xa[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int p = 0; p < G; ++p) xa[b][p] = planes[res_chunk(ks, b, p) + lane];
        res_products<F, E>(xa[0], w, wn, acc[0]);
        res_products<F, E>(xa[1], w, wn, acc[1]);
    };
    // epilogue of block u: inverse DFT, activation, one rounding, 8-byte stores (row of 32 outputs per
    // half-wave = 256 contiguous bytes)
    // (bb: the lane's bias bits, added to Y_0, i.e. to every group sample; loaded at the block's start
    // and first read here -- the opaque copy keeps the conversion, and so the wait for the load, out of
    // the block's steps; a load issued here would be waited for together with every weight load and
    // store issued before it)
    auto epilogue = [&](int u, uint32_t bb) {
        asm volatile("" : "+v"(bb));
        const float bv = elem_to_float<E>((uint16_t)bb);
        const int o = 32 * (wave + kResWaves * u) + ocol;
        const int ooff = o < C_out ? o * G * 2 : -1;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float Y[G], out[G];
#pragma unroll
                for (int p = 0; p < G; ++p) Y[p] = acc[b][p][v];
                Y[0] += bv;
                inverse_planes<G>(Y, out);
                apply_act<GELU>(out);
                const int t = 32 * b + 8 * (v >> 2) + 4 * hrow + (v & 3);  // token within the tile
                const u32x2 d = {pack2<E>(out[0], out[1]), pack2<E>(out[2], out[3])};
                const int off = ooff >= 0 ? t * y_row + ooff : 0x7fffffff;
                __builtin_amdgcn_raw_buffer_store_b64(d, y_rs, off, 0, kResStoreAux);
            }
    };

    uint4 wr[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) load_w(0, r, wr[r]);  // KS >= R

    // Steps s + D0 .. s + D1 - 1 of block u (s a multiple of R), each refilling its ring slot with the
    // step R further on (in this block or the next); each step is its own scheduling region, so no
    // step's operand work is hoisted into an earlier one, where it would wait for loads still in flight.
    // FIRST: s = 0, whose step 0 starts the accumulators.
    // WIDE (blocks after the first, where no raw x is held): all eight plane reads of a step in flight
    // together; in block 0 the compiler pairs them (registers)
    auto steps = [&](auto first, auto d0, auto d1, auto wide, int u, int s) {
        constexpr int D0 = decltype(d0)::value, D1 = decltype(d1)::value;
        const bool wrap = s + R >= KS;
        const int un = wrap ? u + 1 : u, sn = wrap ? s + R - KS : s + R;
#pragma unroll
        for (int d = D0; d < D1; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            if (decltype(first)::value && d == 0)
                step_products(IC<true>{}, s + d, wr[d]);
            else
                step_products(IC<false>{}, s + d, wr[d]);
            load_w(un, sn + d, wr[d]);
            if constexpr (decltype(wide)::value) {
                // token block 0's four plane reads, its first two products, block 1's four reads (in flight
                // under block 0's products), the remaining products, then the ring refill
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- block 0 fills the planes on the way: the raw x arrives in parts of two steps (one uint4 per
    // thread and step), each part requested one part ahead of its transform and transformed one part
    // ahead of its products, so the HBM latency of x hides under the products of the part before ----
    {
        constexpr int PS = 2;  // steps per part (R / PS parts per ring body)
        uint4 xa[PS], xb[PS];
        auto load_part = [&](int q, uint4 (&dst)[PS]) {
#pragma unroll
            for (int j = 0; j < PS; ++j) dst[j] = load_x(q * PS + j);
        };
        auto dft_part = [&](int q, const uint4 (&src)[PS]) {
#pragma unroll
            for (int j = 0; j < PS; ++j) dft_store(q * PS + j, src[j]);
        };
        const uint32_t bb = bias_bits(0);
        load_part(0, xa);
        load_part(1, xb);  // KS >= R = 2 PS
        dft_part(0, xa);
        // Every body requests the next two parts and transforms them, unconditionally: parts past the
        // last read as zeros (channels past C_in) and are written to the two spare steps after the
        // planes. Each body starts with the barrier that publishes the part its first half reads, so a
        // load the compiler sinks into the next block still comes before that barrier. The first body
        // is its own copy: its first step starts the accumulators.
        auto body0 = [&](auto first, int s) {
            const int q = s / PS;
            res_lds_barrier();
            steps(first, IC<0>{}, IC<PS>{}, IC<0>{}, 0, s);  // part q's products, part q + 1 in flight
            dft_part(q + 1, xb);
            load_part(q + 2, xa);
            res_lds_barrier();
            steps(IC<false>{}, IC<PS>{}, IC<R>{}, IC<0>{}, 0, s);  // part q + 1's, part q + 2 in flight
            dft_part(q + 2, xa);
            load_part(q + 3, xb);
        };
        body0(IC<true>{}, 0);
        for (int s = R; s < KS; s += R) body0(IC<false>{}, s);
        epilogue(0, bb);
    }
    // ---- later blocks: the planes are complete; no barrier ----
    for (int u = 1; u < nu; ++u) {
        const uint32_t bb = bias_bits(u);
        steps(IC<true>{}, IC<0>{}, IC<R>{}, IC<1>{}, u, 0);
        for (int s = R; s < KS; s += R) steps(IC<false>{}, IC<0>{}, IC<R>{}, IC<1>{}, u, s);
        epilogue(u, bb);
    }
}

template <bool GELU, class E>
hipError_t launch_res_t(const Plan *p, const void *x, const void *b, void *y, int64_t N, hipStream_t s) {
    const int cus = std::max(1, p->fwd.num_cus);
    int64_t bt = (N + cus - 1) / cus;
    bt = std::min<int64_t>(std::max<int64_t>(bt, 1), kResMaxBT);
    const int64_t tiles = (N + bt - 1) / bt;
    if (tiles > 0x7fffffff || p->KS > kResMaxKS || p->KS % kResRing != 0 || p->NB_total < kResWaves)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_res<GELU, E>), dim3((unsigned)tiles), dim3(kResThreads), 0, s, (const uint4 *)x,
                       (const uint4 *)p->planes, (const uint16_t *)b, (uint16_t *)y, N, p->C_in, p->C_out, p->KS,
                       p->NB_total, (int)bt);
    return hipGetLastError();
}

hipError_t launch_res(const Plan *p, const void *x, const void *b, void *y, int64_t N, int act, hipStream_t s) {
    const bool gelu = act == EQLIN_ACT_GELU;
    if (p->dtype == EQLIN_F16)
        return gelu ? launch_res_t<true, F16>(p, x, b, y, N, s) : launch_res_t<false, F16>(p, x, b, y, N, s);
    return gelu ? launch_res_t<true, BF16>(p, x, b, y, N, s) : launch_res_t<false, BF16>(p, x, b, y, N, s);
}

}  // namespace

// G = 4 (cyclic), an even C_in whose padded steps fit the LDS, and at least one 32-output block per wave.
bool select_res(int G, bool d4, int C_in, int C_out, KernelChoice *out) {
    if (G != 4 || d4 || C_in % 2 != 0) return false;
    const int ks = ((C_in + 15) / 16 + kResRing - 1) / kResRing * kResRing;
    const int nb = (C_out + 31) / 32;
    if (ks > kResMaxKS || nb < kResWaves) return false;
    if ((int64_t)nb * ks * G * 1024 > 0x7fffffff) return false;  // weight offsets are 32-bit
    // the largest tile's output rows are addressed with 32-bit buffer offsets
    if ((int64_t)kResMaxBT * C_out * G * 2 > 0x7fffffff) return false;
    out->kind = KIND_RES;
    out->frag_kind = 2;
    out->rows_per_block = 32;
    out->kc = 16;
    out->ks_mult = kResRing;
    out->nb_tile = 1;
    out->tokens_per_block = kResMaxBT;
    out->block_threads = kResThreads;
    out->lds_bytes = (size_t)ks * 8 * 1024;
    out->num_cus = device_num_cus();
    out->launch = launch_res;
    snprintf(out->name, sizeof(out->name), "bf16 resident-planes G=4 BT<=%d KS=%d (%d waves) mfma32x32x16", kResMaxBT,
             ks, kResWaves);
    return true;
}

}  // namespace eqlin
