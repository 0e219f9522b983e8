// fwd_res8.hip -- the G = 8 spectral EQ-Linear forward (the cyclic group p8 and the dihedral group D4)
// for wide layers whose input planes fit on chip (C_in up to 256 channels), bf16 / fp16 in and out, on
// v_mfma_f32_32x32x16.
//
// Method: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
// Transform" (gist.science explainer), "Enfoque Algorítmico" (group DFT, then one channel product per
// frequency), "Implementación" (one fused kernel, the Fourier fragments kept on chip, no intermediate
// global writes); the EQ-VMamba page (lpnh.cn), section 5.2, for the order-8 groups. At G = 8 the
// cyclic DFT leaves two real frequencies (k = 0, 4) and three complex ones (k = 1, 2, 3): 2 + 3 x 4 =
// 14 real products per channel pair; D4's Fourier transform leaves four one-dimensional characters
// and one two-dimensional irreducible representation: 4 + 8 = 12.
//
// A token tile is 32 tokens (one matrix-core block); its eight frequency planes of all C_in channels
// (8 KB per 16 channels, 128 KB at 256) stay in LDS while the workgroup computes output blocks against
// them, so a token is transformed once per workgroup that touches its tile, not once per output tile.
//   - Work units are (token tile, quad of four 32-output blocks), tile-major. The workgroups are
//     persistent, one per compute unit, and each takes a contiguous range of units. A range covers
//     parts of one or a few tiles, and each tile's planes are filled during the first quad the
//     workgroup runs on it; a filling quad costs about 2.5 later ones, so the launch balances the
//     ranges on that cost, not on the unit count (at 12544 tokens and 1024 outputs: 3136 units over
//     256 CUs; equal counts leave 32 CUs with 13 quads and three fills, the balanced ranges give at
//     most 13 quads with two fills or 12 with three, and leave a few CUs idle).
//   - Four waves, one per SIMD (512 registers each): wave w computes block 4 q + w of quad q and
//     streams only that block's weight fragments from L2, through a register ring four 16-channel
//     steps deep, so the waves wait for each other only while a tile's planes are being filled.
//   - Filling: the raw x of 32 channels (two steps) is requested one part ahead, transformed into the
//     planes one part ahead of its products, and the waves meet at an LDS barrier once per part; the
//     quads after the first read the finished planes with no barrier.
//   - Products: x planes as the A operand (rows = tokens), weight fragments as B (columns = outputs).
//     For a complex frequency the real and imaginary cross terms go to separate accumulators (Re Y =
//     [Xr Wr] - [Xi Wi], Im Y = [Xr Wi + Xi Wr]), so no operand is negated in the loop: 11
//     accumulators for p8, 8 for D4 (the 2 x 2 block Y_ab = X_a0 W_0b + X_a1 W_1b).
//   - Epilogue: the subtraction, the inverse transform in fp32 (the bias added to the trivial
//     frequency, i.e. to every group sample), one rounding, and 16-byte stores straight from the
//     accumulators: for one accumulator row the 32 lanes of a half-wave hold 32 consecutive outputs of
//     one token, i.e. 512 contiguous bytes of y.
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "act.h"
#include "device_common.h"
#include "dft.h"
#include "eqlin_internal.h"

namespace eqlin {

namespace {

constexpr int kR8Waves = 4, kR8Threads = kR8Waves * 64;
constexpr int kR8BT = 32;                    // tokens per tile (one matrix-core block)
constexpr int kR8Ring = 4;                   // weight steps in flight per wave (16 channels each; 4 or 8)
constexpr int kR8MaxKS = 16;                 // 16-channel steps of planes (8 KB each; C_in <= 256), plus
constexpr int kR8LdsSteps = kR8MaxKS + 2;    // two spare steps that past-the-end parts are written to
constexpr int kR8StoreAux = 2;               // output stores non-temporal
constexpr int kR8Acc = 11;                   // accumulators (p8; D4 uses the first 8)
constexpr int kR8MaxTable = 320;             // workgroups whose unit ranges the launch hands over
// A quad that fills a tile's planes costs about 2.5 later quads (the transform, the waits for x and
// the barriers: measured 20 K cycles against 8-9 K, plus an epilogue of 2.5-3 K in both): the ranges
// are balanced on 16 per quad plus this per tile touched.
constexpr int kR8FillCost16 = 24;

// Per-workgroup unit ranges [lo, hi) within the workgroup's output group (by value: kernel argument).
struct R8Ranges {
    int lo[kR8MaxTable], hi[kR8MaxTable];
};

// LDS chunk of (16-channel step ks, plane p): 64 lanes x 16 bytes, lane l holding token l % 32 and
// channels 16 ks + 8 (l / 32) .. + 7 (the 32x32x16 operand layout).
__device__ __forceinline__ int r8_chunk(int ks, int p) { return (ks * 8 + p) * 64; }

// One step of products. Planes (x and weights alike): p8 -- 0 Re k=0, 1 Re k=4, 2 + 2c / 3 + 2c the
// real / imaginary part of k = c + 1; D4 -- 0..3 the characters, 4..7 the 2 x 2 block's entries
// (00, 01, 10, 11). Accumulators: p8 -- 0, 1 the real frequencies, 2 + 3c [Xr Wr], 3 + 3c [Xi Wi],
// 4 + 3c [Xr Wi + Xi Wr]; D4 -- one per plane. F: a block's first step (the products start the
// accumulators from zero). The order keeps every accumulator's two products apart.
template <bool F, bool D4, class E>
__device__ __forceinline__ void r8_products(const uint4 (&x)[8], const uint4 (&w)[8], f32x16 (&acc)[kR8Acc]) {
    auto c = [&](int a) __attribute__((always_inline)) { return F ? f32x16{} : acc[a]; };
    if constexpr (D4) {
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[p] = mma32<E>(x[p], w[p], c(p));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 + e] = mma32<E>(x[4 + 2 * (e >> 1)], w[4 + (e & 1)], c(4 + e));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 + e] = mma32<E>(x[5 + 2 * (e >> 1)], w[6 + (e & 1)], acc[4 + e]);
    } else {
        acc[0] = mma32<E>(x[0], w[0], c(0));
        acc[1] = mma32<E>(x[1], w[1], c(1));
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int r = 2 + 2 * k, a = 2 + 3 * k;
            acc[a] = mma32<E>(x[r], w[r], c(a));
            acc[a + 1] = mma32<E>(x[r + 1], w[r + 1], c(a + 1));
            acc[a + 2] = mma32<E>(x[r], w[r + 1], c(a + 2));
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int r = 2 + 2 * k, a = 2 + 3 * k;
            acc[a + 2] = mma32<E>(x[r + 1], w[r], acc[a + 2]);
        }
    }
}

// Two channels of G = 8 samples (one 16-byte piece each) -> their eight planes (the group's transform).
template <bool D4, class E>
__device__ __forceinline__ void dft_ch8(const uint4 (&r)[2], float (&pl)[8][2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float v[8], P[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) v[g] = elem_at<E>(r[j], g);
        group_forward<8, D4>(v, P);
#pragma unroll
        for (int p = 0; p < 8; ++p) pl[p][j] = P[p];
    }
}

__device__ __forceinline__ void r8_lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
    asm volatile("s_barrier" ::: "memory");
}

template <int V>
struct IC8 {
    static constexpr int value = V;
};

template <bool GELU, bool D4, class E>
__global__ __launch_bounds__(kR8Threads) void k_res8(const uint4 *__restrict__ x4, const uint4 *__restrict__ wfrag,
                                                     const uint16_t *__restrict__ bias, uint16_t *__restrict__ y,
                                                     int64_t N, int C_in, int C_out, int KS, int NQ, int S,
                                                     int tiles, int use_table, const R8Ranges ranges) {
    constexpr int G = 8, R = kR8Ring;
    __shared__ uint4 planes[kR8LdsSteps * 8 * 64];
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Output group g = blockIdx % S (S divides 8, and consecutive workgroups go to consecutive XCDs, so
    // the workgroups of one XCD all work on one group and its L2 holds that group's weights only):
    // quads [qb, qb + NQg) of every tile. This workgroup's units of its group: the launch's
    // cost-balanced range, or (grids past the table) Ug / nwg each, the first Ug % nwg workgroups one
    // more (32-bit, scalar).
    const int g = blockIdx.x % S, b = blockIdx.x / S, nwg = (gridDim.x - g + S - 1) / S;
    const int qb = g * NQ / S, NQg = (g + 1) * NQ / S - qb, Ug = tiles * NQg;
    const int per = Ug / nwg, extra = Ug % nwg;
    const int ub = use_table ? ranges.lo[blockIdx.x] : b * per + min(b, extra);
    const int ue = use_table ? ranges.hi[blockIdx.x] : ub + per + (b < extra ? 1 : 0);
    if (ub >= ue) return;
    const int x_row = C_in * G * 2, y_row = C_out * G * 2;  // bytes per token row

    // all weight fragments: block ob, step ks, plane p at chunk (ob KS + ks) 8 + p
    const __amdgpu_buffer_rsrc_t w_rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)wfrag, (short)0, NQ * 4 * KS * G * 1024, 0x00020000);
    auto load_w = [&](int q, int ks, uint4 (&dst)[8]) __attribute__((always_inline)) {
        // (wave-uniform; said so, or the compiler may wrap each load in a loop over distinct values)
        const int soff = __builtin_amdgcn_readfirstlane(((4 * q + wave) * KS + ks) * G * 1024);
#pragma unroll
        for (int p = 0; p < G; ++p) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(w_rs, lane * 16, soff + p * 1024, 0);
            dst[p] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    // raw x of step s: thread (token tl, channel pair cq) reads channels 16 s + 2 cq, + 1 (32 bytes)
    const int tl = tid >> 3, cq = tid & 7;
    auto load_x = [&](__amdgpu_buffer_rsrc_t x_rs, int s, uint4 (&dst)[2]) __attribute__((always_inline)) {
        const int c = s * 16 + 2 * cq;
        const int vo = c < C_in ? tl * x_row + c * G * 2 : 0x7fffffff;  // channels past C_in: zeros
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(x_rs, vo, 16 * j, 0);
            dst[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    // transform of step s's pair into the planes: one 32-bit word (two channels) per plane
    uint32_t *const pw = reinterpret_cast<uint32_t *>(planes);
    const int slot = (tl + 32 * (cq >> 2)) * 4 + (cq & 3);
    auto dft_store = [&](int s, const uint4 (&r)[2]) __attribute__((always_inline)) {
        float pl[G][2];
        dft_ch8<D4, E>(r, pl);
#pragma unroll
        for (int p = 0; p < G; ++p) pw[r8_chunk(s, p) * 4 + slot] = pack2<E>(pl[p][0], pl[p][1]);
    };

    // output column of this lane in block ob: o = 32 ob + lane % 32
    const int ocol = lane & 31, hrow = lane >> 5;
    auto bias_bits = [&](int q) __attribute__((always_inline)) -> uint32_t {
        const int o = 32 * (4 * q + wave) + ocol;
        return (bias && o < C_out) ? (uint32_t)bias[o] : 0u;
    };
    f32x16 acc[kR8Acc];
    // epilogue of quad q: inverse transform, activation, one rounding, 16-byte stores (row of 32
    // outputs per half-wave = 512 contiguous bytes)
    // (bb: the lane's bias bits, added to Y_0, i.e. to every group sample; loaded at the block's start
    // and first read here -- the opaque copy keeps the conversion, and so the wait for the load, out of
    // the block's steps; a load issued here would be waited for together with every weight load and
    // store issued before it)
    auto epilogue = [&](__amdgpu_buffer_rsrc_t y_rs, int q, uint32_t bb) __attribute__((always_inline)) {
        asm volatile("" : "+v"(bb));
        const float bv = elem_to_float<E>((uint16_t)bb);
        const int o = 32 * (4 * q + wave) + ocol;
        const int ooff = o < C_out ? o * G * 2 : -1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float Y[G], out[G];
            if constexpr (D4) {
#pragma unroll
                for (int p = 0; p < G; ++p) Y[p] = acc[p][v];
            } else {
                Y[0] = acc[0][v];
                Y[1] = acc[1][v];
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    Y[2 + 2 * k] = acc[2 + 3 * k][v] - acc[3 + 3 * k][v];
                    Y[3 + 2 * k] = acc[4 + 3 * k][v];
                }
            }
            Y[0] += bv;
            group_inverse<G, D4>(Y, out);
            apply_act<GELU>(out);
            const int t = 8 * (v >> 2) + 4 * hrow + (v & 3);  // token within the tile
            const uint4 pk = pack8<E>(out);
            const u32x4 d = {pk.x, pk.y, pk.z, pk.w};
            const int off = ooff >= 0 ? t * y_row + ooff : 0x7fffffff;
            __builtin_amdgcn_raw_buffer_store_b128(d, y_rs, off, 0, kR8StoreAux);
        }
    };

    uint4 wr[R][8];
    {
        const int q0 = qb + ub % NQg;
#pragma unroll
        for (int r = 0; r < R; ++r) load_w(q0, r, wr[r]);  // KS >= R
    }
    auto read_x = [&](int ks, uint4 (&dst)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < G; ++p) dst[p] = planes[r8_chunk(ks, p) + lane];
    };

    // Steps s + D0 .. s + D1 - 1 of quad q (s a multiple of R), each refilling its ring slot with the
    // step R further on (in this quad or in quad qn, the next one this workgroup runs); each step is its
    // own scheduling region, so no step's operand work is hoisted into an earlier one, where it would
    // wait for loads still in flight. FIRST: s = 0, whose step 0 starts the accumulators.
    // PF (quads whose planes are complete): each step's planes were read during the step before, and
    // it reads the next step's (step KS: a spare step, read and unused) under its products; in a
    // filling quad every step reads its own after the barrier that published them.
    auto steps = [&](auto first, auto d0, auto d1, auto pf, int q, int qn, int s, uint4 (&xq)[2][8]) __attribute__((always_inline)) {
        constexpr int D0 = decltype(d0)::value, D1 = decltype(d1)::value;
        constexpr bool PF = decltype(pf)::value;
        const bool wrap = s + R >= KS;
        const int q_next = wrap ? qn : q, s_next = wrap ? s + R - KS : s + R;
#pragma unroll
        for (int d = D0; d < D1; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            const int XB = PF ? (d & 1) : 0;
            if constexpr (PF)
                read_x(s + d + 1, xq[(d + 1) & 1]);
            else
                read_x(s + d, xq[0]);
            if (decltype(first)::value && d == 0)
                r8_products<true, D4, E>(xq[XB], wr[d], acc);
            else
                r8_products<false, D4, E>(xq[XB], wr[d], acc);
            load_w(q_next, s_next + d, wr[d]);
            if constexpr (PF) {
                // the next step's eight plane reads spread over the first products, the ring refill last
                constexpr int NM = D4 ? 12 : 14;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NM - 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    uint4 xq[2][8];
    for (int u = ub; u < ue;) {
        const int t = u / NQg;
        const int qa = qb + u % NQg;
        const int qe = min(qb + NQg, qa + (ue - u));
        const bool more_tiles = u + (qe - qa) < ue;  // then the range goes on with quad qb of tile t + 1
        // the quad this workgroup runs after q (past its last: q itself, whose weights are in range)
        auto next_q = [&](int q) __attribute__((always_inline)) { return q + 1 < qe ? q + 1 : (more_tiles ? qb : q); };
        const int64_t n0 = (int64_t)t * kR8BT;
        const int rows = (int)std::min<int64_t>(kR8BT, N - n0);
        // x of this tile (rows past the tile read as zeros); y of this tile (stores past it are dropped)
        const __amdgpu_buffer_rsrc_t x_rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(x4 + n0 * C_in * G / 8), (short)0, rows * x_row, 0x00020000);
        const __amdgpu_buffer_rsrc_t y_rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(y + n0 * C_out * G), (short)0, rows * y_row, 0x00020000);

        // ---- quad qa fills the planes on the way (parts of two steps: each part's raw x requested one
        // part ahead of its transform and transformed one part ahead of its products) ----
        {
            constexpr int PS = 2, NPB = R / PS;  // steps per part, parts per ring body
            uint4 xp[2][PS][2];                  // part k's raw x in xp[k % 2]
            auto load_part = [&](int p, uint4 (&dst)[PS][2]) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < PS; ++j) load_x(x_rs, p * PS + j, dst[j]);
            };
            auto dft_part = [&](int p, const uint4 (&src)[PS][2]) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < PS; ++j) dft_store(p * PS + j, src[j]);
            };
            const uint32_t bb = bias_bits(qa);
            const int qn = next_q(qa);
            load_part(0, xp[0]);
            load_part(1, xp[1]);  // KS >= R >= 2 PS
            // the previous tile's planes are no longer read by any wave
            r8_lds_barrier();
            dft_part(0, xp[0]);
            // Part J of the body at ring step s (part k = s / PS + J): the barrier that publishes it, its
            // products, the transform of part k + 1 and the request of part k + 2 into the buffer just
            // freed, unconditionally: parts past the last read as zeros (channels past C_in) and the one
            // of them transformed goes to the two spare steps after the planes. A load the compiler sinks
            // past the end of a part still comes before the next part's barrier. (The body starts at an
            // even part, so each part's buffers are known constants.)
            auto part = [&](auto first, auto jc, int s) __attribute__((always_inline)) {
                constexpr int J = decltype(jc)::value;
                const int k = s / PS + J;
                r8_lds_barrier();
                steps(first, IC8<J * PS>{}, IC8<(J + 1) * PS>{}, IC8<0>{}, qa, qn, s, xq);
                dft_part(k + 1, xp[(J + 1) & 1]);
                load_part(k + 2, xp[J & 1]);
            };
            // the first body is its own copy: its first step starts the accumulators
            auto body0 = [&](auto first, int s) __attribute__((always_inline)) {
                part(first, IC8<0>{}, s);
                part(IC8<false>{}, IC8<1>{}, s);
                if constexpr (NPB == 4) {
                    part(IC8<false>{}, IC8<2>{}, s);
                    part(IC8<false>{}, IC8<3>{}, s);
                }
            };
            body0(IC8<true>{}, 0);
            for (int s = R; s < KS; s += R) body0(IC8<false>{}, s);
            epilogue(y_rs, qa, bb);
        }
        // ---- later quads of the tile: the planes are complete; no barrier ----
        for (int q = qa + 1; q < qe; ++q) {
            const uint32_t bb = bias_bits(q);
            const int qn = next_q(q);
            read_x(0, xq[0]);
            steps(IC8<true>{}, IC8<0>{}, IC8<R>{}, IC8<1>{}, q, qn, 0, xq);
            for (int s = R; s < KS; s += R) steps(IC8<false>{}, IC8<0>{}, IC8<R>{}, IC8<1>{}, q, qn, s, xq);
            epilogue(y_rs, q, bb);
        }
        u += qe - qa;
    }
}

// Output groups: the fewest (1, 2, 4 or 8, at most the quads) whose weights fit kR8XcdWeightBudget of
// an XCD's 4 MB L2 each, leaving the rest to the streaming x and y; every further group transforms
// each token tile once more.
constexpr size_t kR8XcdWeightBudget = 4u << 20;
static int res8_groups(int NQ, int KS) {
    const size_t w = (size_t)NQ * 4 * KS * 8 * 1024;
    int S = 1;
    while (S < 8 && S * 2 <= NQ && w / S > kR8XcdWeightBudget) S *= 2;
    return S;
}

// The end of the longest run of units from a whose cost (16 per quad plus kR8FillCost16 per tile touched,
// NQg quads per tile) stays within T.
static int r8_run_end(int a, int64_t T, int Ug, int NQg) {
    int e = a;
    int64_t c = 0;
    while (e < Ug) {
        const int te = std::min(Ug, (e / NQg + 1) * NQg);  // end of e's tile
        const int64_t cf = c + kR8FillCost16;
        if (cf + 16 > T) break;
        const int k = (int)std::min<int64_t>(te - e, (T - cf) / 16);
        e += k;
        c = cf + 16 * (int64_t)k;
        if (e < te) break;
    }
    return e;
}

// Contiguous ranges of each output group's Ug = tiles x NQg units over its workgroups (g, g + S, ...)
// minimising the largest cost: the smallest T for which taking the longest run within T, workgroup
// after workgroup, covers every unit (binary search), then those runs.
static void r8_balance(int tiles, int NQ, int S, int grid, R8Ranges *r) {
    for (int g = 0; g < S; ++g) {
        const int qb = g * NQ / S, NQg = (g + 1) * NQ / S - qb, Ug = tiles * NQg;
        const int nwg = (grid - g + S - 1) / S;
        auto covers = [&](int64_t T) {
            int a = 0;
            for (int j = 0; j < nwg && a < Ug; ++j) a = r8_run_end(a, T, Ug, NQg);
            return a >= Ug;
        };
        int64_t lo = 16 + kR8FillCost16, hi = 16 * (int64_t)Ug + (int64_t)kR8FillCost16 * tiles;  // hi covers
        while (lo < hi) {
            const int64_t mid = (lo + hi) / 2;
            if (covers(mid))
                hi = mid;
            else
                lo = mid + 1;
        }
        int a = 0;
        for (int j = 0; j < nwg; ++j) {
            const int e = r8_run_end(a, lo, Ug, NQg);
            r->lo[g + j * S] = a;
            r->hi[g + j * S] = e;
            a = e;
        }
    }
}

// The ranges of a launch shape, kept for the last few shapes (a new shape computes them: microseconds),
// copied out under the lock.
static void r8_ranges(int tiles, int NQ, int S, int grid, R8Ranges *out) {
    struct Entry {
        int tiles = -1, NQ = 0, S = 0, grid = 0;
        R8Ranges r;
    };
    static std::mutex mu;
    static Entry cache[4];
    static int next = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (auto &e : cache)
        if (e.tiles == tiles && e.NQ == NQ && e.S == S && e.grid == grid) {
            *out = e.r;
            return;
        }
    Entry &e = cache[next];
    next = (next + 1) % 4;
    r8_balance(tiles, NQ, S, grid, &e.r);
    e.tiles = tiles, e.NQ = NQ, e.S = S, e.grid = grid;
    *out = e.r;
}

template <bool GELU, bool D4, class E>
hipError_t launch_res8_t(const Plan *p, const void *x, const void *b, void *y, int64_t N, hipStream_t s) {
    const int64_t tiles = (N + kR8BT - 1) / kR8BT;
    const int NQ = p->NB_total / 4;
    if (p->KS > kR8MaxKS || p->KS % kR8Ring != 0 || p->NB_total % 4 != 0 || NQ < 1) return hipErrorInvalidValue;
    if (tiles * NQ > 0x7fffffff) return hipErrorInvalidValue;  // units are counted in 32 bits
    const int S = res8_groups(NQ, p->KS);
    // every group needs a workgroup: at least S (S <= NQ <= the units)
    const int64_t grid = std::max<int64_t>(S, std::min<int64_t>(tiles * NQ, std::max(1, p->fwd.num_cus)));
    R8Ranges ranges{};  // copied into the launch's arguments
    const bool table = grid <= kR8MaxTable;
    if (table) r8_ranges((int)tiles, NQ, S, (int)grid, &ranges);
    hipLaunchKernelGGL((k_res8<GELU, D4, E>), dim3((unsigned)grid), dim3(kR8Threads), 0, s, (const uint4 *)x,
                       (const uint4 *)p->planes, (const uint16_t *)b, (uint16_t *)y, N, p->C_in, p->C_out, p->KS, NQ,
                       S, (int)tiles, table ? 1 : 0, ranges);
    return hipGetLastError();
}

template <bool D4>
hipError_t launch_res8_g(const Plan *p, const void *x, const void *b, void *y, int64_t N, int act, hipStream_t s) {
    const bool gelu = act == EQLIN_ACT_GELU;
    if (p->dtype == EQLIN_F16)
        return gelu ? launch_res8_t<true, D4, F16>(p, x, b, y, N, s) : launch_res8_t<false, D4, F16>(p, x, b, y, N, s);
    return gelu ? launch_res8_t<true, D4, BF16>(p, x, b, y, N, s) : launch_res8_t<false, D4, BF16>(p, x, b, y, N, s);
}

hipError_t launch_res8(const Plan *p, const void *x, const void *b, void *y, int64_t N, int act, hipStream_t s) {
    return p->d4 ? launch_res8_g<true>(p, x, b, y, N, act, s) : launch_res8_g<false>(p, x, b, y, N, act, s);
}

}  // namespace

// G = 8 (cyclic or D4), an even C_in whose padded steps fit the LDS, and at least one quad of 32-output
// blocks.
bool select_res8(int G, bool d4, int C_in, int C_out, KernelChoice *out) {
    if (G != 8 || C_in % 2 != 0) return false;
    const int ks = ((C_in + 15) / 16 + kR8Ring - 1) / kR8Ring * kR8Ring;
    const int nq = ((C_out + 31) / 32 + 3) / 4;
    if (ks > kR8MaxKS || nq < 1) return false;
    if ((int64_t)nq * 4 * ks * G * 1024 > 0x7fffffff) return false;  // weight offsets are 32-bit
    // a tile's output rows are addressed with 32-bit buffer offsets
    if ((int64_t)kR8BT * C_out * G * 2 > 0x7fffffff) return false;
    out->kind = KIND_RES;
    out->frag_kind = 2;
    out->rows_per_block = 32;
    out->kc = 16;
    out->ks_mult = kR8Ring;
    out->nb_tile = 4;
    out->tokens_per_block = kR8BT;
    out->block_threads = kR8Threads;
    out->lds_bytes = sizeof(uint4) * kR8LdsSteps * 8 * 64;
    out->num_cus = device_num_cus();
    out->launch = launch_res8;
    snprintf(out->name, sizeof(out->name), "bf16 resident-planes %s BT=%d KS=%d (%d waves) mfma32x32x16",
             d4 ? "D4" : "G=8", kR8BT, ks, kR8Waves);
    return true;
}

}  // namespace eqlin
