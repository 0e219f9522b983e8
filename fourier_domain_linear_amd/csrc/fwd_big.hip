// fwd_big.hip -- the spectral EQ-Linear forward for large channel counts (and the unrolled dense
// comparator at large sizes, run as G = 1), bf16 in/out, on v_mfma_f32_32x32x16_bf16.
//
// Method: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
// Transform" (gist.science explainer), "Enfoque Algorítmico" (group DFT -> per-frequency channel
// products, k = 0..G/2) and "Implementación" (one fused kernel, Fourier fragments on chip).
//
// Persistent workgroups, one per compute unit: each keeps one output tile (its weights and bias) and
// walks the token tiles tt0, tt0 + tstep, ... (block_tile: XCD-aware, so the workgroups sharing a
// token tile mostly share an L2). The load pipeline runs on across tile boundaries, and a tile's
// outputs, staged in LDS, are stored during the next tile's stages instead of in one burst at its
// end (every compute unit storing at once runs at the HBM write rate while the matrix cores idle).
//
// Tile: BO outputs x BT tokens, all G planes; OW x TW waves (4 or 8: one or two per SIMD), each
// owning WA x WB blocks of 32 outputs x 32 tokens (k_p8, for G = 8, splits the planes instead). The
// channel (K) loop runs in stages of SC input channels (SC*G*2 bytes per token row: whole 128-byte
// lines), two stages per loop trip so every register slot is fixed:
//   - x: raw rows are loaded into a two-slot register ring two stages ahead (HBM latency spans
//     several stages of products), transformed (group DFT, fp32) one stage ahead and written to one
//     of two LDS buffers as bf16 B operands (32 tokens x 16 channels x 1 plane per 1 KB chunk),
//     shared by every wave of the workgroup; each thread transforms distinct (token, 4 or 8
//     channel) items, so no transform is repeated;
//   - weights: each wave owns distinct output rows, so LDS staging would buy no reuse: fragment
//     chunks (32 outputs x 16 channels x 1 plane per 1 KB, one coalesced load per wave) go straight
//     into a two-slot register ring one stage ahead (they are L2 hits: the workgroup's output tile
//     never changes);
//   - products: weights as the A operand (rows = outputs), x planes as B (columns = tokens); a
//     complex frequency is four real products (Re = WrXr - WiXi via a sign-flipped Xi operand).
// All global loads are plain loads, so the compiler's waits count exactly the ones in flight; the
// per-stage barrier waits for LDS only. Vector-memory operations complete in issue order, so each
// stage issues its weight loads, then its x loads, then its share of stores: a wait for a load never
// waits for a store issued after it.
// Epilogue of a tile: inverse DFT in fp32 (the bias entered the k = 0 accumulators at the tile's
// start), outputs staged per wave in LDS (XOR-swizzled), then written as whole 16-byte pieces with
// range-checked non-temporal buffer stores.
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "act.h"
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

// The products of one K-step for all planes: Re += Wr Xr + (-Wi) Xi, Im += Wi Xr + Wr Xi (wn holds the
// negated Im weight fragments, indexed like w). F: the accumulators of planes 1.. start from zero
// (plane 0 always accumulates: it starts from the bias).
template <int G, bool F, class E>
__device__ __forceinline__ void spectral_mfma32(const uint4 (&w)[G], const uint4 (&wn)[G], const uint4 (&a)[G],
                                                f32x16 (&acc)[G]) {
    auto c = [&](int p) { return F ? f32x16{} : acc[p]; };
    acc[0] = mma32<E>(w[0], a[0], acc[0]);
    if constexpr (G >= 2) acc[1] = mma32<E>(w[1], a[1], c(1));
#pragma unroll
    for (int k = 1; k < G / 2; ++k) {
        const int r = 2 * k, i = 2 * k + 1;
        acc[r] = mma32<E>(w[r], a[r], c(r));
        acc[r] = mma32<E>(wn[i], a[i], acc[r]);
        acc[i] = mma32<E>(w[i], a[r], c(i));
        acc[i] = mma32<E>(w[r], a[i], acc[i]);
    }
}

// G samples of NCH channels (element j*G+g) -> G planes of NCH bf16 (NCH = 2, 4 or 8); D4: the
// dihedral group's Fourier transform instead of the cyclic DFT.
template <int G, int NCH, bool D4, class E>
__device__ __forceinline__ void dft_ch(const uint4 (&r)[NCH * G / 8], float (&pl)[G][NCH]) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        float v[G], P[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 &q = r[(j * G + g) >> 3];
            const int e = (j * G + g) & 7;
            const uint32_t wd = (e >> 1) == 0 ? q.x : (e >> 1) == 1 ? q.y : (e >> 1) == 2 ? q.z : q.w;
            v[g] = (e & 1) ? elem_hi<E>(wd) : elem_lo<E>(wd);
        }
        group_forward<G, D4>(v, P);
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

// Scheduling pattern for one stage: a 32x32x16 product keeps the matrix core busy for 32 cycles
// while the wave goes on issuing independent instructions, so the stage's global loads and the
// transform's vector ALU work are spread over the products (NM of them): the region's NR LDS reads
// first, then after each product one load (the first NV products) and up to VPM vector ALU
// instructions; the NS stores last (vector-memory operations complete in issue order, so a store
// issued ahead of a load would make every wait for that load wait for the store too).
template <int NR, int NM, int NV, int VPM, int NS = 0>
__device__ __forceinline__ void interleave_stage() {
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // the region's LDS reads first, as one batch
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // vector ALU
    }
    if (NS) __builtin_amdgcn_sched_group_barrier(0x040, NS, 0);  // global stores last
}

constexpr int kStoreAux = 2;  // cache policy of the output stores: non-temporal (measured faster than default)

template <int V>
struct IC {
    static constexpr int value = V;
};

// Workgroup -> (output tile, first token tile). Workgroups are dealt to the 8 XCDs (each with its own
// L2) round-robin: workgroup g runs on XCD g % 8. Workgroups are renumbered so that each XCD holds a
// contiguous run of the logical order, and the logical order is: groups of xg output tiles, within a
// group the token streams, within a stream the group's xg output tiles. An XCD then serves each x
// tile from its L2 to the xg workgroups that share it, while keeping only xg output tiles' weights.
// (xg divides tiles_o; xg = 1 puts one output tile per XCD when tiles_o = 8.)
__device__ __forceinline__ void block_tile(int tiles_o, int xg, int &ot, int &tt0, int &tstep) {
    const int grid = gridDim.x, g = blockIdx.x;
    const int xcd = g % 8, per = grid / 8, extra = grid % 8;
    const int L = xcd * per + min(xcd, extra) + g / 8;
    tstep = grid / tiles_o;  // token streams per output tile
    const int span = tstep * xg, og = L / span, r = L % span;
    ot = og * xg + r % xg;
    tt0 = r / xg;
}

template <int G, int WA, int WB, int OW, int TW>
struct BigCfg {
    static constexpr int NW = OW * TW, NT = NW * 64;
    static constexpr int BO = 32 * WA * OW, BT = 32 * WB * TW;
    static constexpr int SC = BigStage<G>::SC, KSS = BigStage<G>::KSS, GRP = BigStage<G>::GRP;
    static constexpr int SA = BigStage<G>::SA;
    // x work items: (token, NCH channels), as wide as possible while every thread has one
    static constexpr int NCH = BT * SC / 8 >= NT ? 8 : BT * SC / 4 >= NT ? 4 : 2;
    static constexpr int ITEMS = BT * (SC / NCH) / NT;      // x items per thread per stage
    static constexpr int XU4 = NCH * G / 8;                 // uint4 of raw x per item
    static constexpr int XST = (BT / 32) * KSS * G * 64;    // uint4 per x-plane buffer (1 KB chunks)
    static constexpr int WF = WA * KSS * G;                 // weight fragments per wave per stage
    static constexpr int VPM = G == 8 ? 10 : G == 2 ? 5 : G == 4 ? 4 : 3;  // transform ALU ops per product
    // output staging: a wave's tile is NU units of 32 tokens x (SA x 32 outputs x G), PR 16-byte
    // pieces per token row (XOR-swizzled); it leaves in NSTORE whole-wave stores, SPS per stage of
    // the next tile (the rest, if the tile has too few stages, before that tile's own epilogue)
    static constexpr int PR = 4 * SA * G;
    static constexpr int NU = WB * (WA / SA);
    static constexpr int UST = 32 * PR;                     // uint4 per unit
    static constexpr int STG = NU * UST;                    // uint4 of staging per wave
    static constexpr int NSTORE = NU * PR / 2;
    static constexpr int SPS = NW == 8 ? 1 : 2;  // stores per stage (measured: 8 waves 1, 4 waves 2)
    static constexpr int LDS_U4 = 2 * XST + NW * STG;
    static constexpr size_t LDS = (size_t)LDS_U4 * 16;
    static_assert(WA % SA == 0, "store unit must divide the wave's output blocks");
    static_assert(ITEMS >= 1 && ITEMS * NT == BT * (SC / NCH), "x items must split evenly over the threads");
    static_assert(XU4 >= 1, "an x item must fill at least one 16-byte piece");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Persistent: each workgroup keeps output tile ot (its weights, bias and L2 set) and walks the token
// tiles tt0, tt0 + tstep, ... (block_tile; tstep = gridDim.x / tiles_o). The load pipeline runs on
// across tile boundaries, and a tile's outputs are stored while the next tile computes.
//
// CONV: the input channels are the gathered channels of a p4 group convolution (conv.hip): token n is
// pixel n of a [B][img_h][img_w] grid and x holds x_elems elements per pixel. The stages come in groups
// of four that read the same four rows (16-channel pieces of a pixel's row): conv_tab[group] gives for
// row m its byte offset into the pixel's row (16 bits m of .x, .y) and the offset (dy, dx) of the
// pixel it is read from (byte m of .z, .w, signed); pixels outside the image read as zeros. A centre
// group (all offsets zero) is four channel blocks of the pixel itself, stage u reading row u; an orbit
// group is the four rotated neighbours R^m delta0 of one channel block, stage u taking sample g from
// row (g - u) mod 4 -- a gathered channel. Each row is loaded once per group (one row per stage, six
// stages ahead of the group's first use), so the four stages of a group cost one load per stage; the
// stage loop runs in bodies of 8 stages, so u and the two row sets are compile-time choices.
template <int G, int WA, int WB, int OW, int TW, bool VEC, bool GELU, class E, bool CONV = false>
__global__ __launch_bounds__(OW * TW * 64) void k_big(const uint4 *__restrict__ x4,
                                                      const uint4 *__restrict__ wfrag,
                                                      const uint16_t *__restrict__ bias, int bias_shift,
                                                      uint16_t *__restrict__ y, int64_t N, int C_in,
                                                      int C_out, int n_stages, int KS16, int tiles_t,
                                                      int tiles_o, int xg, const uint4 *__restrict__ conv_tab,
                                                      int img_h, int img_w, int x_elems) {
    using C = BigCfg<G, WA, WB, OW, TW>;
    constexpr int KSS = C::KSS, NCH = C::NCH;
    static_assert(!CONV || (C::XU4 == 1 && (G == 4 || G == 1)), "gathered loads: one 16-byte piece per item");
    constexpr int XL = CONV ? 4 : C::XU4;  // raw x per item and ring slot: CONV, a group's four rows
    __shared__ uint4 lds[C::LDS_U4];  // two x-plane buffers, then each wave's output staging
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wo = wave % OW, wt = wave / OW;
    int ot, tt0, tstep;
    block_tile(tiles_o, xg, ot, tt0, tstep);
    const int ntl = tt0 < tiles_t ? (tiles_t - 1 - tt0) / tstep + 1 : 0;  // token tiles of this workgroup
    if (ntl == 0) return;
    const int o0 = ot * C::BO, ob0 = o0 / 32;
    uint4 *const stg = lds + 2 * C::XST + wave * C::STG;
    constexpr bool vec_rows = VEC;  // output rows are whole 16-byte pieces: (C_out * G) % 8 == 0
    const int yrow_pieces = C_out * G / 8;
    const int yrow_bytes = C_out * G * 2;
    const int rcol = lane & 31;

    // ---- loaders: buffer loads whose per-stage offset is a scalar, so the stage loop spends no
    // vector ALU on addresses. x: one resource per token tile (rows past N read as zeros; past the
    // last tile, an empty range); a thread's (token, channel) offsets are the same in every tile.
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    // (item it of a thread is token tl + it * NT / (SC / NCH), same channels: a scalar row offset)
    static_assert(C::NT % (C::SC / NCH) == 0, "items of a thread differ by whole token rows");
    const int x_row = (CONV ? x_elems : C_in * G) * 2;  // bytes per token row
    const int x_tl = tid / (C::SC / NCH), x_c0 = (tid % (C::SC / NCH)) * NCH;
    const int x_vo = x_tl * x_row + x_c0 * G * 2;
    const int x_vo_last = x_tl * x_row + (C_in - NCH) * G * 2;  // the row's last channels
    constexpr int IT_ROWS = C::NT / (C::SC / NCH);  // token rows between a thread's items
    // The x source of token tile k: its buffer resource, and (CONV) each item's pixel and row offset.
    struct XSrc {
        __amdgpu_buffer_rsrc_t rs;
        int py[C::ITEMS], px[C::ITEMS], off[C::ITEMS];
    };
    auto x_src = [&](int k) {
        XSrc r;
        const int64_t n0 = (int64_t)(tt0 + k * tstep) * C::BT;
        if constexpr (CONV) {  // the whole tensor; rows past N or past the last tile read as zeros
            r.rs = __builtin_amdgcn_make_buffer_rsrc((void *)x4, (short)0, (int)(N * x_row), 0x00020000);
            const int hw = img_h * img_w;
#pragma unroll
            for (int it = 0; it < C::ITEMS; ++it) {
                const int64_t n = n0 + x_tl + it * IT_ROWS;
                const bool ok = k < ntl && n < N;
                const int nn = ok ? (int)n : 0, pix = nn % hw;
                r.py[it] = ok ? pix / img_w : -(1 << 24);
                r.px[it] = pix % img_w;
                r.off[it] = nn * x_row + x_c0 * G * 2;
            }
        } else {  // the tile's rows (rows past N read as zeros; past the last tile, an empty range)
            int64_t rows = N - n0 < C::BT ? N - n0 : C::BT;
            rows = k < ntl ? rows : 0;
            r.rs = __builtin_amdgcn_make_buffer_rsrc((void *)(x4 + (k < ntl ? n0 : 0) * C_in * G / 8), (short)0,
                                                     (int)(rows * x_row), 0x00020000);
#pragma unroll
            for (int it = 0; it < C::ITEMS; ++it) r.py[it] = r.px[it] = r.off[it] = 0;
        }
        return r;
    };
    // stage of the current tile (source src_c), or past its end: the next tile's (src_n)
    auto load_x = [&](const XSrc &src_c, const XSrc &src_n, int stage, uint4 (&dst)[C::ITEMS][XL]) {
        if constexpr (!CONV) {  // (CONV loads rows of stage groups: load_row)
            const bool next = stage >= n_stages;  // uniform
            const __amdgpu_buffer_rsrc_t rs = next ? src_n.rs : src_c.rs;
            stage = next ? stage - n_stages : stage;
            const int soff = stage * C::SC * G * 2;
            // channels past C_in (the stage count is padded) re-read the row's last channels: finite
            // values that meet zero weight columns
            const int vo = (stage * C::SC + x_c0 < C_in) ? x_vo : x_vo_last - soff;
#pragma unroll
            for (int it = 0; it < C::ITEMS; ++it)
#pragma unroll
                for (int q = 0; q < C::XU4; ++q) {
                    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, vo + 16 * q, soff + it * IT_ROWS * x_row,
                                                                          0);
                    dst[it][q] = make_uint4(v.x, v.y, v.z, v.w);
                }
        }
    };
    // CONV: the table entry of stage group `group` (past the tile's groups: the next tile's), wave-uniform
    const int n_groups = n_stages >> 2;
    auto group_entry = [&](int group) { return conv_tab[group < n_groups ? group : group - n_groups]; };
    // CONV: row r of a stage group (table entry t; next: a group of the next tile) into dst[.][r]
    auto load_row = [&](const XSrc &src_c, const XSrc &src_n, bool next, const uint4 &t, int r,
                        uint4 (&dst)[C::ITEMS][XL]) {
        const __amdgpu_buffer_rsrc_t rs = next ? src_n.rs : src_c.rs;
        const int chan = (int)(((r < 2 ? t.x : t.y) >> (16 * (r & 1))) & 0xffffu);
        const int sy = (int)(signed char)(t.z >> (8 * r)), sx = (int)(signed char)(t.w >> (8 * r));
        const int d = chan + (sy * img_w + sx) * x_row;  // uniform
#pragma unroll
        for (int it = 0; it < C::ITEMS; ++it) {
            const int py = next ? src_n.py[it] : src_c.py[it];
            const int px = next ? src_n.px[it] : src_c.px[it];
            const int off = next ? src_n.off[it] : src_c.off[it];
            const bool in = ((unsigned)(py + sy) < (unsigned)img_h) & ((unsigned)(px + sx) < (unsigned)img_w);
            const int vo = in ? off + d : 0x7fffffff;  // outside the image: zeros
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0);
            dst[it][r] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    // CONV: the item of stage u of a group from its rows. Element e = j * 4 + g (channel j, sample g);
    // orbit: element e of row (g - u) mod 4; centre: element e of row u.
    auto merge = [&](auto uc, bool centre, const uint4 (&rows)[C::ITEMS][XL], uint4 (&src)[C::ITEMS][C::XU4]) {
        constexpr int u = decltype(uc)::value;
        auto mix = [](uint32_t a, uint32_t b) { return (a & 0xffffu) | (b & 0xffff0000u); };
#pragma unroll
        for (int it = 0; it < C::ITEMS; ++it) {
            const uint4 *R = rows[it];
            const uint4 o = make_uint4(mix(R[(4 - u) & 3].x, R[(5 - u) & 3].x), mix(R[(6 - u) & 3].y, R[(7 - u) & 3].y),
                                       mix(R[(4 - u) & 3].z, R[(5 - u) & 3].z), mix(R[(6 - u) & 3].w, R[(7 - u) & 3].w));
            const uint4 c = R[u];
            src[it][0] = make_uint4(centre ? c.x : o.x, centre ? c.y : o.y, centre ? c.z : o.z, centre ? c.w : o.w);
        }
    };
    auto is_centre = [](const uint4 &t) { return (t.z | t.w) == 0u; };  // a centre group: no pixel offsets
    // weights: one resource per wave (its WA output blocks), block and stage as a scalar offset
    const int wo_u = __builtin_amdgcn_readfirstlane(wave) % OW;
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(wfrag + (size_t)((ob0 + wo_u * WA) * KS16) * G * 64), (short)0, WA * KS16 * G * 1024, 0x00020000);
    auto load_w = [&](int stage, uint4 (&dst)[C::WF]) {
        stage = stage < n_stages ? stage : stage - n_stages;
#pragma unroll
        for (int a = 0; a < WA; ++a)
#pragma unroll
            for (int r = 0; r < KSS * G; ++r) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(w_rs, lane * 16 + r * 1024,
                                                                      (a * KS16 + stage * KSS) * G * 1024, 0);
                dst[a * KSS * G + r] = make_uint4(v.x, v.y, v.z, v.w);
            }
    };
    // the transform of one stage's x items (for CONV the items merged from their group's rows)
    auto dft_store = [&](const uint4 (&src)[C::ITEMS][C::XU4], uint4 *xb) {
#pragma unroll
        for (int it = 0; it < C::ITEMS; ++it) {
            const int item = tid + it * C::NT;
            const int tl = item / (C::SC / NCH), cq = item % (C::SC / NCH);
            const int c0 = cq * NCH;  // first channel of the item within the stage
            uint4 *dst = xb + ((tl >> 5) * KSS + (c0 >> 4)) * G * 64 + ((c0 >> 3) & 1) * 32 + (tl & 31);
            float pl[G][NCH];
            dft_ch<G, NCH, false, E>(src[it], pl);
#pragma unroll
            for (int p = 0; p < G; ++p) {
                if constexpr (NCH == 8) {
                    dst[p * 64] = pack8<E>(pl[p]);
                } else if constexpr (NCH == 2) {
                    reinterpret_cast<uint32_t *>(dst + p * 64)[(c0 >> 1) & 3] = pack2<E>(pl[p][0], pl[p][1]);
                } else {
                    uint2 w;
                    w.x = pack2<E>(pl[p][0], pl[p][1]);
                    w.y = pack2<E>(pl[p][2], pl[p][3]);
                    reinterpret_cast<uint2 *>(dst + p * 64)[(c0 >> 2) & 1] = w;
                }
            }
        }
    };
    // Store j (0 <= j < NSTORE) of the staged tile: one 16-byte piece per lane, read from the staging
    // area, then written with a buffer store. Rows past N fall outside the buffer range and are
    // dropped by the hardware, as are pieces past the row end and every piece when `valid` is false.
    auto read_staged = [&](int j) {
        const int u = j / (C::PR / 2), jj = j % (C::PR / 2);
        const int r = jj * (64 / C::PR) + lane / C::PR, pc = lane % C::PR;
        return stg[u * C::UST + r * C::PR + (pc ^ (r & 7))];
    };
    auto store_staged = [&](int j, const uint4 &v, __amdgpu_buffer_rsrc_t rs, bool valid) {
        const int u = j / (C::PR / 2), jj = j % (C::PR / 2);
        const int r = jj * (64 / C::PR) + lane / C::PR, pc = lane % C::PR;
        const int b = u / (WA / C::SA), a0 = (u % (WA / C::SA)) * C::SA;
        const int piece = (o0 + (wo * WA + a0) * 32) * G / 8 + pc;
        const int off = ((wt * WB + b) * 32 + r) * yrow_bytes + piece * 16;
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 d = {v.x, v.y, v.z, v.w};
        // branch-free: an offset past the range drops the store (bitwise, no short-circuit jumps)
        const int keep = -(int)(valid & (piece < yrow_pieces));
        __builtin_amdgcn_raw_buffer_store_b128(d, rs, (off & keep) | (0x7fffffff & ~keep), 0, kStoreAux);
    };
    auto tile_rsrc = [&](int k) {
        const int64_t n0 = (int64_t)(tt0 + k * tstep) * C::BT;
        const int64_t rows = N - n0 < C::BT ? N - n0 : C::BT;
        return __builtin_amdgcn_make_buffer_rsrc(y + n0 * (C_out * G), (short)0, (int)(rows * yrow_bytes),
                                                 0x00020000);
    };

    // Bias: lane l keeps bias[row l % 32] of each of its output blocks (bf16 bits); a tile's k = 0
    // accumulators start as the product of that column with a row of ones (exact in fp32).
    uint32_t bcol[WA];
#pragma unroll
    for (int a = 0; a < WA; ++a) {
        const int o = o0 + (wo * WA + a) * 32 + rcol;
        bcol[a] = (bias && o < C_out) ? bias[o >> bias_shift] : 0u;
    }

    // ---- prologue: weights of stage 0 and raw x of positions 0 and 1 requested; x(0) transformed ----
    // (CONV: the rows of stage group 0 and rows 0, 1 of group 1 -- what stages -6 .. -1 would load)
    uint4 xr[2][C::ITEMS][XL];
    uint4 wr[2][C::WF];
    load_w(0, wr[0]);
    {
        const XSrc rs0 = x_src(0);
        if constexpr (CONV) {
            const uint4 t0 = group_entry(0), t1 = group_entry(1);
#pragma unroll
            for (int r = 0; r < 4; ++r) load_row(rs0, rs0, false, t0, r, xr[0]);
            load_row(rs0, rs0, false, t1, 0, xr[1]);
            load_row(rs0, rs0, false, t1, 1, xr[1]);
            uint4 xm[C::ITEMS][C::XU4];
            merge(IC<0>{}, is_centre(t0), xr[0], xm);
            dft_store(xm, lds);
        } else {
            load_x(rs0, rs0, 0, xr[0]);
            load_x(rs0, rs0, 1, xr[1]);
            dft_store(xr[0], lds);
        }
    }
    lds_barrier();

    f32x16 acc[WA][WB][G];
    // products of (K-step kk, token block b) pairs [lo, hi) of a stage, kk major
    // the x planes of (K-step kk, token block b) pair q = kk * WB + b of a stage
    auto read_planes = [&](int q, const uint4 *planes, uint4 (&xf)[G]) {
        const int kk = q / WB, b = q % WB;
#pragma unroll
        for (int p = 0; p < G; ++p) xf[p] = planes[(((wt * WB + b) * KSS + kk) * G + p) * 64 + lane];
    };
    // the products of pair q; first: the tile's first stage (its first K-step starts the accumulators)
    auto products = [&](auto first, int q, const uint4 (&xf)[G], const uint4 (&w_cur)[C::WF],
                        const uint4 (&w_neg)[C::WF]) {
        const int kk = q / WB, b = q % WB;
#pragma unroll
        for (int a = 0; a < WA; ++a) {
            uint4 wf[G], wn[G];
#pragma unroll
            for (int p = 0; p < G; ++p) {
                wf[p] = w_cur[(a * KSS + kk) * G + p];
                wn[p] = w_neg[(a * KSS + kk) * G + p];
            }
            if (decltype(first)::value && kk == 0)
                spectral_mfma32<G, true, E>(wf, wn, xf, acc[a][b]);
            else
                spectral_mfma32<G, false, E>(wf, wn, xf, acc[a][b]);
        }
    };
    // One stage (tile k, stage s) in two scheduling regions, so the loads leave in a fixed order:
    // the weights of s+1 under the first half of the products, then the raw x of position +2 and the
    // transform of x(+1) under the second half, and last this stage's share of the previous tile's
    // stores.
    // The next stage's products then wait for its weights only, with the raw x still in flight
    // (vector-memory operations complete in issue order).
    // CONV (bc: the stage's place b in its body of 8): the item of stage s + 1 is merged from its group's
    // rows in the first half, ahead of the second half's row load, which at b = 2 and 6 overwrites a row
    // of the set that merge reads; the load is row (b + 2) mod 4 of group (s + 6) / 4.
    auto step = [&](auto first, auto bc, const XSrc &xrs_c, const XSrc &xrs_n, int s, uint4 (&x_free)[C::ITEMS][XL],
                    const uint4 (&x_next)[C::ITEMS][XL], const uint4 (&w_cur)[C::WF], uint4 (&w_next)[C::WF],
                    const uint4 *planes, uint4 *planes_next, __amdgpu_buffer_rsrc_t rs_prev, bool has_prev,
                    const uint4 (&tg)[4], int g0) {
        constexpr int P = KSS * WB, H = P / 2;
        // the second half's planes are read with the first half's when they fit in 4 registers of 16
        // bytes, so its products do not wait for LDS after the first half's
        constexpr bool PRE = (P - H) * G <= 4;
        load_w(s + 1, w_next);
        // the Im weight fragments negated once per stage (each serves WB token blocks); only the
        // slots the products read are used, the rest is dead code
        uint4 w_neg[C::WF];
#pragma unroll
        for (int r = 0; r < C::WF; ++r) w_neg[r] = (r % G >= 3 && (r % G) % 2 == 1) ? neg_bf16x8(w_cur[r]) : w_cur[r];
        uint4 xa[H][G], xb[P - H][G];
#pragma unroll
        for (int q = 0; q < H; ++q) read_planes(q, planes, xa[q]);
        if constexpr (PRE)
#pragma unroll
            for (int q = H; q < P; ++q) read_planes(q, planes, xb[q - H]);
        constexpr int b = decltype(bc)::value;
        uint4 xm[C::ITEMS][C::XU4];
        // (CONV: stage s + 1 is in group g0 + (b + 1) / 4, the row load's group is g0 + (b + 6) / 4)
        if constexpr (CONV) merge(IC<(b + 1) % 4>{}, is_centre(tg[(b + 1) / 4]), xr[((b + 1) / 4) % 2], xm);
#pragma unroll
        for (int q = 0; q < H; ++q) products(first, q, xa[q], w_cur, w_neg);
        interleave_stage<(PRE ? P : H) * G, H * WA * real_products(G), C::WF, 1>();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (CONV)
            load_row(xrs_c, xrs_n, g0 + (b + 6) / 4 >= n_groups, tg[(b + 6) / 4], (b + 2) % 4, xr[((b + 6) / 4) % 2]);
        else
            load_x(xrs_c, xrs_n, s + 2, x_free);
        uint4 sv[C::SPS];
#pragma unroll
        for (int i = 0; i < C::SPS; ++i) sv[i] = read_staged(min(s * C::SPS + i, C::NSTORE - 1));
        if constexpr (!PRE)
#pragma unroll
            for (int q = H; q < P; ++q) read_planes(q, planes, xb[q - H]);
#pragma unroll
        for (int q = H; q < P; ++q) products(first, q, xb[q - H], w_cur, w_neg);
        if constexpr (CONV)
            dft_store(xm, planes_next);
        else
            dft_store(x_next, planes_next);  // past the last position: unused planes, harmless
        constexpr int XLOADS = CONV ? C::ITEMS : C::ITEMS * XL;  // x loads per stage
        interleave_stage<(PRE ? 0 : (P - H) * G) + C::SPS, (P - H) * WA * real_products(G), XLOADS, C::VPM>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < C::SPS; ++i) {
            const int j = s * C::SPS + i;
            store_staged(min(j, C::NSTORE - 1), sv[i], rs_prev, has_prev & (j < C::NSTORE));
        }
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);  // each stage is its own scheduling region
    };

    for (int k = 0; k < ntl; ++k) {
        // operands built here from one live register per block (constants and the thread id behind
        // opaque copies, so the compiler does not keep whole tuples live through the loop)
        int tid_b = threadIdx.x;
        asm volatile("" : "+v"(tid_b));
        const uint4 ones = make_uint4((tid_b & 63) < 32 ? E::kOne : 0u, 0u, 0u, 0u);  // 1.0 at k = 0
#pragma unroll
        for (int a = 0; a < WA; ++a) {
            uint32_t bc = bcol[a];
            asm volatile("" : "+v"(bc));
#pragma unroll
            for (int b = 0; b < WB; ++b) acc[a][b][0] = mma32<E>(make_uint4(bc, 0u, 0u, 0u), ones, f32x16{});
        }
        const bool has_prev = k > 0 && vec_rows;
        const __amdgpu_buffer_rsrc_t rs_prev = tile_rsrc(k > 0 ? k - 1 : 0);
        const XSrc xrs_c = x_src(k), xrs_n = x_src(k + 1);
        // n_stages is even (the channel padding sees to it); for G >= 2 the first pair is peeled so
        // the first products can start the accumulators of planes 1.. without clearing them (G = 1
        // has only the bias plane)
        if constexpr (CONV) {
            // n_stages is a multiple of 8: bodies of 8 stages, so each stage's place in its group of
            // four and the row set it uses are fixed; planes 1.. start from zero (no peeled first stage)
#pragma unroll
            for (int a = 0; a < WA; ++a)
#pragma unroll
                for (int b = 0; b < WB; ++b)
#pragma unroll
                    for (int p = 1; p < G; ++p) acc[a][b][p] = f32x16{};
            uint4(&x0)[C::ITEMS][XL] = xr[0];
            for (int s = 0; s < n_stages; s += 8) {
                // the table entries of the body's groups, read before its first stage: scalar loads
                // share the LDS wait counter, so waiting for one inside a stage would also wait for
                // that stage's LDS reads (the barrier that ended the last stage has drained the LDS)
                const int g0 = s >> 2;
                uint4 tg[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) tg[j] = group_entry(g0 + j);
                __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
                __builtin_amdgcn_sched_barrier(0);
#define CONV_STEP(B, WC, WN, PL, PN)                                                                        \
    step(IC<0>{}, IC<B>{}, xrs_c, xrs_n, s + B, x0, x0, wr[WC], wr[WN], PL, PN, rs_prev, has_prev, tg, g0)
                CONV_STEP(0, 0, 1, lds, lds + C::XST);
                CONV_STEP(1, 1, 0, lds + C::XST, lds);
                CONV_STEP(2, 0, 1, lds, lds + C::XST);
                CONV_STEP(3, 1, 0, lds + C::XST, lds);
                CONV_STEP(4, 0, 1, lds, lds + C::XST);
                CONV_STEP(5, 1, 0, lds + C::XST, lds);
                CONV_STEP(6, 0, 1, lds, lds + C::XST);
                CONV_STEP(7, 1, 0, lds + C::XST, lds);
#undef CONV_STEP
            }
        } else {
            const uint4 no_tab[4] = {};
            int s0 = 0;
            if constexpr (G >= 2) {
                step(IC<1>{}, IC<0>{}, xrs_c, xrs_n, 0, xr[0], xr[1], wr[0], wr[1], lds, lds + C::XST, rs_prev,
                     has_prev, no_tab, 0);
                step(IC<0>{}, IC<0>{}, xrs_c, xrs_n, 1, xr[1], xr[0], wr[1], wr[0], lds + C::XST, lds, rs_prev,
                     has_prev, no_tab, 0);
                s0 = 2;
            }
            for (int s = s0; s < n_stages; s += 2) {
                step(IC<0>{}, IC<0>{}, xrs_c, xrs_n, s, xr[0], xr[1], wr[0], wr[1], lds, lds + C::XST, rs_prev,
                     has_prev, no_tab, 0);
                step(IC<0>{}, IC<0>{}, xrs_c, xrs_n, s + 1, xr[1], xr[0], wr[1], wr[0], lds + C::XST, lds, rs_prev,
                     has_prev, no_tab, 0);
            }
        }
        // stores of the previous tile that did not fit in this tile's stages
        if (has_prev)
            for (int j = n_stages * C::SPS; j < C::NSTORE; ++j) store_staged(j, read_staged(j), rs_prev, true);

        // ---- epilogue of tile k: inverse DFT; stage the outputs (stored during the next tile) ----
        // lane-derived values are recomputed here (behind an opaque copy) rather than kept live
        // through the stage loop, where registers are scarce
        int tid_e = threadIdx.x;
        asm volatile("" : "+v"(tid_e));
        const int lane_e = tid_e & 63, wave_e = tid_e >> 6;
        const int wo_e = wave_e % OW, wt_e = wave_e / OW;
        const int h_e = lane_e >> 5, rcol_e = lane_e & 31;
        uint4 *const stg_e = lds + 2 * C::XST + wave_e * C::STG;
        const int64_t t0 = (int64_t)(tt0 + k * tstep) * C::BT;
#pragma unroll
        for (int b = 0; b < WB; ++b) {
#pragma unroll
            for (int a0 = 0; a0 < WA; a0 += C::SA) {
                if constexpr (!vec_rows) {  // rows not a whole number of 16-byte pieces: element stores
                    const int64_t nblk = t0 + (wt_e * WB + b) * 32;
#pragma unroll
                    for (int ai = 0; ai < C::SA; ++ai)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int o = o0 + (wo_e * WA + a0 + ai) * 32 + 8 * (v >> 2) + 4 * h_e + (v & 3);
                            const int64_t n = nblk + rcol_e;
                            if (o >= C_out || n >= N) continue;
                            float Y[G], out[G];
#pragma unroll
                            for (int p = 0; p < G; ++p) Y[p] = acc[a0 + ai][b][p][v];
                            inverse_planes<G>(Y, out);
                            apply_act<GELU>(out);
#pragma unroll
                            for (int g = 0; g < G; ++g) y[(n * C_out + o) * G + g] = pack1<E>(out[g]);
                        }
                    continue;
                }
                uint4 *ust = stg_e + (b * (WA / C::SA) + a0 / C::SA) * C::UST;
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
                        apply_act<GELU>(out);
                        const int ol = ai * 32 + 8 * vq + 4 * h_e;  // first of the 4 outputs in the unit row
                        if constexpr (G == 1) {
                            uint2 w;
                            w.x = pack2<E>(out[0], out[1]);
                            w.y = pack2<E>(out[2], out[3]);
                            const int piece = ol / 8;  // 8 outputs x 2 B per piece
                            reinterpret_cast<uint2 *>(ust + rcol_e * C::PR + (piece ^ (rcol_e & 7)))[(ol >> 2) & 1] = w;
                        } else {
#pragma unroll
                            for (int kq = 0; kq < G / 2; ++kq) {
                                const int piece = ol * G / 8 + kq;
                                ust[rcol_e * C::PR + (piece ^ (rcol_e & 7))] = pack8<E>(out + 8 * kq);
                            }
                        }
                    }
            }
        }
    }
    // the last tile's outputs
    if constexpr (vec_rows) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(ntl - 1);
#pragma unroll
        for (int j = 0; j < C::NSTORE; ++j) store_staged(j, read_staged(j), rs, true);
    }
}

// Output tiles per XCD group (see block_tile): the largest divisor of tiles_o whose weights fit in
// kXcdWeightBudget of an XCD's 4 MB L2, leaving the rest to the streaming x tiles.
constexpr size_t kXcdWeightBudget = 2u << 20;
static int xcd_group(int tiles_o, size_t weight_bytes_per_tile) {
    int best = 1;
    for (int d = 1; d <= tiles_o; ++d)
        if (tiles_o % d == 0 && d * weight_bytes_per_tile <= kXcdWeightBudget) best = d;
    return best;
}

// ------------------------------------------------------------------------------------------------
// k_p8: the G = 8 forward with two waves per SIMD. At G = 8 one wave needs all 256 accumulator
// registers to keep two token blocks per weight fragment, so instead of splitting the tile, the two
// waves of a SIMD split its frequency planes: both own the same 32 outputs and the same two 32-token
// blocks; role 0 holds planes Re0, Re4, Re1, Im1 (k = 0, 4 and 1: six products per block), role 1
// Re2, Im2, Re3, Im3 (k = 2 and 3: eight products). Each wave loads only its four weight planes (no
// weight is read twice) and reads only its four x planes. At a tile's end the pair hands over the
// four planes of one token block through LDS and each wave finishes one block (inverse DFT over all
// eight planes, staging). Everything else -- persistence, the load pipeline, the deferred stores --
// follows k_big.
struct P8Cfg {
    static constexpr int G = 8, OW = 4, NW = 8, NT = NW * 64, WB = 2;
    static constexpr int BO = 32 * OW, BT = 32 * WB;
    static constexpr int SC = 16, KSS = 1;
    static constexpr int NCH = 2, ITEMS = BT * (SC / NCH) / NT, XU4 = NCH * G / 8;
    static constexpr int XST = (BT / 32) * KSS * G * 64;  // uint4 per x-plane buffer
    static constexpr int HP = G / 2;                     // planes per wave
    static constexpr int WF = KSS * HP;                  // weight fragments per wave per stage
    static constexpr int VPM = 10;                       // transform ALU ops per product
    static constexpr int PR = 4 * G;                     // 16-byte pieces per staged row (32 outputs)
    static constexpr int STG = 32 * PR;                  // uint4 of staging per wave: one 32 x 32 block
    static constexpr int NSTORE = PR / 2;
    static constexpr int SPS = 1;
    static constexpr int LDS_U4 = 2 * XST + NW * STG;
    static constexpr size_t LDS = (size_t)LDS_U4 * 16;
    static_assert(ITEMS == 1 && XU4 == 2, "one 2-channel x item per thread");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(HP * 16 * 64 * 4 <= STG * 16, "a wave's staging holds the four planes it hands over");
};

template <bool GELU, bool D4, class E>
__global__ __launch_bounds__(P8Cfg::NT) void k_p8(const uint4 *__restrict__ x4, const uint4 *__restrict__ wfrag,
                                                  const uint16_t *__restrict__ bias, int bias_shift,
                                                  uint16_t *__restrict__ y, int64_t N, int C_in, int C_out,
                                                  int n_stages, int KS16, int tiles_t, int tiles_o, int xg) {
    using C = P8Cfg;
    constexpr int G = 8, KSS = C::KSS, NCH = C::NCH, WB = C::WB, HP = C::HP;
    __shared__ uint4 lds[C::LDS_U4];  // two x-plane buffers, then each wave's staging / hand-over area
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wo = wave & 3;  // waves w and w + 4 share a SIMD, the output block and the token blocks
    int ot, tt0, tstep;
    block_tile(tiles_o, xg, ot, tt0, tstep);
    const int ntl = tt0 < tiles_t ? (tiles_t - 1 - tt0) / tstep + 1 : 0;
    if (ntl == 0) return;
    const int o0 = ot * C::BO, ob0 = o0 / 32;
    uint4 *const stg = lds + 2 * C::XST + wave * C::STG;
    const int yrow_pieces = C_out * G / 8;
    const int yrow_bytes = C_out * G * 2;
    const int rcol = lane & 31;

    // Loads are buffer loads: the per-stage part of every address is a scalar offset, so the stage loop
    // spends no vector ALU on addresses. x: one resource per token tile (rows past N lie outside its
    // range and read as zeros); this thread's (token, channel pair) offset is the same in every tile.
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const int tl = tid / (C::SC / NCH), cq = tid % (C::SC / NCH);
    const int x_row = C_in * G * 2;                                  // bytes per token row
    const int x_vo = tl * x_row + cq * NCH * G * 2;                  // stage 0 offset in the tile
    const int x_vo_last = tl * x_row + (C_in - NCH) * G * 2;         // the row's last channel pair
    auto x_rsrc = [&](int k) {  // k >= ntl (past the last tile): an empty range, loads read zeros
        const int64_t n0 = (int64_t)(tt0 + k * tstep) * C::BT;
        int64_t rows = N - n0 < C::BT ? N - n0 : C::BT;
        rows = k < ntl ? rows : 0;
        return __builtin_amdgcn_make_buffer_rsrc((void *)(x4 + (k < ntl ? n0 : 0) * C_in * G / 8), (short)0,
                                                 (int)(rows * x_row), 0x00020000);
    };
    // stage of the current tile (resource rs_c), or past its end: the next tile's (rs_n)
    auto load_x = [&](__amdgpu_buffer_rsrc_t rs_c, __amdgpu_buffer_rsrc_t rs_n, int stage,
                      uint4 (&dst)[C::ITEMS][C::XU4]) {
        const bool next = stage >= n_stages;  // uniform
        const __amdgpu_buffer_rsrc_t rs = next ? rs_n : rs_c;
        stage = next ? stage - n_stages : stage;
        // channels past C_in (the stage count is padded) re-read the row's last pair: finite values
        // that meet zero weight columns
        const int soff = stage * C::SC * G * 2;
        const int vo = (stage * C::SC + cq * NCH < C_in) ? x_vo : x_vo_last - soff;
#pragma unroll
        for (int q = 0; q < C::XU4; ++q) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, vo + 16 * q, soff, 0);
            dst[0][q] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    // weights: one resource per wave (its output block and role's planes), stage as a scalar offset
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(wfrag + (size_t)((ob0 + (wave_u & 3)) * KS16) * G * 64 + (wave_u >> 2) * HP * 64), (short)0,
        KS16 * G * 1024 - (wave_u >> 2) * HP * 1024, 0x00020000);
    auto load_w = [&](int stage, uint4 (&dst)[C::WF]) {
        stage = stage < n_stages ? stage : stage - n_stages;
#pragma unroll
        for (int r = 0; r < HP; ++r) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(w_rs, lane * 16 + r * 1024, stage * G * 1024, 0);
            dst[r] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    auto dft_store = [&](const uint4 (&src)[C::ITEMS][C::XU4], uint4 *xb) {
        const int c0 = cq * NCH;
        uint4 *dst = xb + ((tl >> 5) * KSS + (c0 >> 4)) * G * 64 + ((c0 >> 3) & 1) * 32 + (tl & 31);
        float pl[G][NCH];
        dft_ch<G, NCH, D4, E>(src[0], pl);
#pragma unroll
        for (int p = 0; p < G; ++p)
            reinterpret_cast<uint32_t *>(dst + p * 64)[(c0 >> 1) & 3] = pack2<E>(pl[p][0], pl[p][1]);
    };
    // a wave's staged block: role r finishes token block r
    auto read_staged = [&](int j) {
        const int r = j * (64 / C::PR) + lane / C::PR, pc = lane % C::PR;
        return stg[r * C::PR + (pc ^ (r & 7))];
    };
    auto store_staged = [&](int j, int role, const uint4 &v, __amdgpu_buffer_rsrc_t rs, bool valid) {
        const int r = j * (64 / C::PR) + lane / C::PR, pc = lane % C::PR;
        const int piece = (o0 + wo * 32) * G / 8 + pc;
        const int off = (role * 32 + r) * yrow_bytes + piece * 16;
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 d = {v.x, v.y, v.z, v.w};
        const int keep = -(int)(valid & (piece < yrow_pieces));
        __builtin_amdgcn_raw_buffer_store_b128(d, rs, (off & keep) | (0x7fffffff & ~keep), 0, kStoreAux);
    };
    auto tile_rsrc = [&](int k) {
        const int64_t n0 = (int64_t)(tt0 + k * tstep) * C::BT;
        const int64_t rows = N - n0 < C::BT ? N - n0 : C::BT;
        return __builtin_amdgcn_make_buffer_rsrc(y + n0 * (C_out * G), (short)0, (int)(rows * yrow_bytes),
                                                 0x00020000);
    };

    const int o_b = o0 + wo * 32 + rcol;
    const uint32_t bcol = (bias && o_b < C_out) ? bias[o_b >> bias_shift] : 0u;

    uint4 xr[2][C::ITEMS][C::XU4];
    uint4 wr[2][C::WF];
    load_w(0, wr[0]);
    {
        const __amdgpu_buffer_rsrc_t rs0 = x_rsrc(0);
        load_x(rs0, rs0, 0, xr[0]);
        load_x(rs0, rs0, 1, xr[1]);
    }
    dft_store(xr[0], lds);
    lds_barrier();

    // the whole tile loop, once per role (wave-uniform), so each copy's stages are branch-free
    auto run = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        constexpr int NMB = D4 ? (R == 0 ? 4 : 8) : (R == 0 ? 6 : 8);  // products per token block per K-step
        f32x16 acc[WB][HP];
        // Re += Wr Xr + (-Wi) Xi and Im += Wi Xr + Wr Xi: the sign goes on the weight fragment (wn, one
        // negated copy per stage and Im plane), which serves both token blocks
        // (first: the tile's first stage, whose products start the accumulators from zero; role 0's
        // k = 0 plane starts from the bias instead)
        auto products = [&](auto first, int b, const uint4 (&w)[C::WF], const uint4 (&wn)[2], const uint4 *planes) {
            constexpr bool F = decltype(first)::value;
            uint4 xf[HP];
#pragma unroll
            for (int r = 0; r < HP; ++r) xf[r] = planes[((b * KSS) * G + R * HP + r) * 64 + lane];
            auto acc0 = [&](int q) { return F ? f32x16{} : acc[b][q]; };
            if constexpr (D4) {
                // D4, role 0: the four characters, one product each; role 1: the 2 x 2 irrep,
                // Y_ab += W_0b X_a0 + W_1b X_a1 (local planes 0..3 = entries 00, 01, 10, 11)
                if constexpr (R == 0) {
                    acc[b][0] = mma32<E>(w[0], xf[0], acc[b][0]);
#pragma unroll
                    for (int q = 1; q < 4; ++q) acc[b][q] = mma32<E>(w[q], xf[q], acc0(q));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int ra = e >> 1, cb = e & 1;
                        acc[b][e] = mma32<E>(w[cb], xf[2 * ra], acc0(e));
                        acc[b][e] = mma32<E>(w[2 + cb], xf[2 * ra + 1], acc[b][e]);
                    }
                }
            } else if constexpr (R == 0) {
                acc[b][0] = mma32<E>(w[0], xf[0], acc[b][0]);
                acc[b][1] = mma32<E>(w[1], xf[1], acc0(1));
                acc[b][2] = mma32<E>(w[2], xf[2], acc0(2));
                acc[b][2] = mma32<E>(wn[1], xf[3], acc[b][2]);
                acc[b][3] = mma32<E>(w[3], xf[2], acc0(3));
                acc[b][3] = mma32<E>(w[2], xf[3], acc[b][3]);
            } else {
#pragma unroll
                for (int c = 0; c < HP; c += 2) {
                    acc[b][c] = mma32<E>(w[c], xf[c], acc0(c));
                    acc[b][c] = mma32<E>(wn[c / 2], xf[c + 1], acc[b][c]);
                    acc[b][c + 1] = mma32<E>(w[c + 1], xf[c], acc0(c + 1));
                    acc[b][c + 1] = mma32<E>(w[c], xf[c + 1], acc[b][c + 1]);
                }
            }
        };
        auto step = [&](auto first, __amdgpu_buffer_rsrc_t xrs_c, __amdgpu_buffer_rsrc_t xrs_n, int s,
                        uint4 (&x_free)[C::ITEMS][C::XU4], const uint4 (&x_next)[C::ITEMS][C::XU4],
                        const uint4 (&w_cur)[C::WF], uint4 (&w_next)[C::WF], const uint4 *planes,
                        uint4 *planes_next, __amdgpu_buffer_rsrc_t rs_prev, bool has_prev) {
            load_w(s + 1, w_next);
            uint4 wn[2];  // role 0: -W(Im1) in slot 1; role 1: -W(Im2), -W(Im3)
            wn[0] = neg_bf16x8(w_cur[1]);
            wn[1] = neg_bf16x8(w_cur[3]);
            products(first, 0, w_cur, wn, planes);
            interleave_stage<HP, NMB, C::WF, 1>();
            __builtin_amdgcn_sched_barrier(0);
            load_x(xrs_c, xrs_n, s + 2, x_free);
            const int j = s * C::SPS;
            const uint4 sv = read_staged(min(j, C::NSTORE - 1));
            products(first, 1, w_cur, wn, planes);
            dft_store(x_next, planes_next);  // past the last position: unused planes, harmless
            interleave_stage<HP + 1, NMB, C::ITEMS * C::XU4, C::VPM>();
            __builtin_amdgcn_sched_barrier(0);
            store_staged(min(j, C::NSTORE - 1), R, sv, rs_prev, has_prev & (j < C::NSTORE));
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
        };

        for (int k = 0; k < ntl; ++k) {
            int tid_b = threadIdx.x;
            asm volatile("" : "+v"(tid_b));
            if constexpr (R == 0) {  // the bias enters plane k = 0: one product of the bias column with ones
                const uint4 ones = make_uint4((tid_b & 63) < 32 ? E::kOne : 0u, 0u, 0u, 0u);
                uint32_t bc = bcol;
                asm volatile("" : "+v"(bc));
#pragma unroll
                for (int b = 0; b < WB; ++b) acc[b][0] = mma32<E>(make_uint4(bc, 0u, 0u, 0u), ones, f32x16{});
            }
            const bool has_prev = k > 0;
            const __amdgpu_buffer_rsrc_t rs_prev = tile_rsrc(k > 0 ? k - 1 : 0);
            const __amdgpu_buffer_rsrc_t xrs_c = x_rsrc(k), xrs_n = x_rsrc(k + 1);
            // n_stages is even (the channel padding sees to it); the first pair is peeled so the first
            // products can start the accumulators without clearing them
            step(IC<1>{}, xrs_c, xrs_n, 0, xr[0], xr[1], wr[0], wr[1], lds, lds + C::XST, rs_prev, has_prev);
            step(IC<0>{}, xrs_c, xrs_n, 1, xr[1], xr[0], wr[1], wr[0], lds + C::XST, lds, rs_prev, has_prev);
            for (int s = 2; s < n_stages; s += 2) {
                step(IC<0>{}, xrs_c, xrs_n, s, xr[0], xr[1], wr[0], wr[1], lds, lds + C::XST, rs_prev, has_prev);
                step(IC<0>{}, xrs_c, xrs_n, s + 1, xr[1], xr[0], wr[1], wr[0], lds + C::XST, lds, rs_prev, has_prev);
            }
            if (has_prev)
                for (int j = n_stages * C::SPS; j < C::NSTORE; ++j) store_staged(j, R, read_staged(j), rs_prev, true);

            // ---- epilogue: hand the partner the planes of the block it finishes, take ours ----
            int tid_e = threadIdx.x;
            asm volatile("" : "+v"(tid_e));
            const int lane_e = tid_e & 63, wave_e = tid_e >> 6;
            float *const mine = reinterpret_cast<float *>(lds + 2 * C::XST + wave_e * C::STG);
            const float *const theirs = reinterpret_cast<const float *>(lds + 2 * C::XST + (wave_e ^ 4) * C::STG);
#pragma unroll
            for (int q = 0; q < HP; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v) mine[(q * 16 + v) * 64 + lane_e] = acc[1 - R][q][v];
            lds_barrier();
            float recv[HP][16];
#pragma unroll
            for (int q = 0; q < HP; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v) recv[q][v] = theirs[(q * 16 + v) * 64 + lane_e];
            lds_barrier();
            // inverse DFT of token block R over all eight planes, staged for the next tile's stages
            const int h_e = lane_e >> 5, rcol_e = lane_e & 31;
            auto plane = [&](int p, int v) { return (p / HP == R) ? acc[R][p % HP][v] : recv[p % HP][v]; };
#pragma unroll
            for (int vq = 0; vq < 4; ++vq) {
                float out[4 * G];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float Y[G];
#pragma unroll
                    for (int p = 0; p < G; ++p) Y[p] = plane(p, 4 * vq + v);
                    group_inverse<G, D4>(Y, out + v * G);
                }
                apply_act<GELU>(out);
                const int ol = 8 * vq + 4 * h_e;  // first of the 4 outputs in the staged row
#pragma unroll
                for (int kq = 0; kq < G / 2; ++kq) {
                    const int piece = ol * G / 8 + kq;
                    reinterpret_cast<uint4 *>(mine)[rcol_e * C::PR + (piece ^ (rcol_e & 7))] = pack8<E>(out + 8 * kq);
                }
            }
        }
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(ntl - 1);
#pragma unroll
        for (int j = 0; j < C::NSTORE; ++j) store_staged(j, R, read_staged(j), rs, true);
    };
    if (wave < 4)
        run(IC<0>{});
    else
        run(IC<1>{});
}

static hipError_t launch_p8(const Plan *p, const void *x, const void *b, void *y, int64_t N, int act,
                            hipStream_t s) {
    using C = P8Cfg;
    const int64_t tiles_t = (N + C::BT - 1) / C::BT;
    const int tiles_o = p->NB_total / (C::BO / 32);
    const int n_stages = p->KS / C::KSS;
    if (tiles_t > 0x7fffffff || (int64_t)C::BT * p->C_out * C::G * 2 > 0x7fffffff) return hipErrorInvalidValue;
    int64_t per_o = std::max(1, p->fwd.num_cus / tiles_o);
    per_o = std::min<int64_t>(per_o, tiles_t);
    // the fewest token streams per output tile that keep the number of tile rounds: every stream then
    // gets the same number of tiles (196 tiles: 28 streams of 7, not 32 of which 4 run a 7th)
    const int64_t rounds = (tiles_t + per_o - 1) / per_o;
    per_o = (tiles_t + rounds - 1) / rounds;
    const int64_t grid = per_o * tiles_o;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const int xg = xcd_group(tiles_o, (size_t)C::BO * p->KS * 16 * C::G * 2);
    const bool gelu = act == EQLIN_ACT_GELU, f16 = p->dtype == EQLIN_F16;
    auto kern = p->d4 ? (f16 ? (gelu ? k_p8<true, true, F16> : k_p8<false, true, F16>)
                             : (gelu ? k_p8<true, true, BF16> : k_p8<false, true, BF16>))
                      : (f16 ? (gelu ? k_p8<true, false, F16> : k_p8<false, false, F16>)
                             : (gelu ? k_p8<true, false, BF16> : k_p8<false, false, BF16>));
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), 0, s, (const uint4 *)x, (const uint4 *)p->planes,
                       (const uint16_t *)b, p->bias_shift, (uint16_t *)y, N, p->C_in, p->C_out, n_stages, p->KS,
                       (int)tiles_t, tiles_o, xg);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------

template <int G, int WA, int WB, int OW, int TW>
static hipError_t launch_big(const Plan *p, const void *x, const void *b, void *y, int64_t N, int act,
                             hipStream_t s) {
    using C = BigCfg<G, WA, WB, OW, TW>;
    const int64_t tiles_t = (N + C::BT - 1) / C::BT;
    const int tiles_o = p->NB_total / (C::BO / 32);
    const int n_stages = p->KS / C::KSS;
    // a token tile's output rows are addressed with 32-bit buffer offsets
    if (tiles_t > 0x7fffffff || (int64_t)C::BT * p->C_out * G * 2 > 0x7fffffff) return hipErrorInvalidValue;
    // one workgroup per compute unit, a whole number of them per output tile
    int64_t per_o = std::max(1, p->fwd.num_cus / tiles_o);
    per_o = std::min<int64_t>(per_o, tiles_t);
    const int64_t grid = per_o * tiles_o;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const int xg = xcd_group(tiles_o, (size_t)C::BO * p->KS * 16 * G * 2);
    const bool vec = (p->C_out * G) % 8 == 0, gelu = act == EQLIN_ACT_GELU;
    auto pick = [&](auto e) {
        using E = decltype(e);
        return vec ? (gelu ? k_big<G, WA, WB, OW, TW, true, true, E> : k_big<G, WA, WB, OW, TW, true, false, E>)
                   : (gelu ? k_big<G, WA, WB, OW, TW, false, true, E> : k_big<G, WA, WB, OW, TW, false, false, E>);
    };
    auto kern = p->dtype == EQLIN_F16 ? pick(F16{}) : pick(BF16{});
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), 0, s, (const uint4 *)x, (const uint4 *)p->planes,
                       (const uint16_t *)b, p->bias_shift, (uint16_t *)y, N, p->C_in, p->C_out, n_stages, p->KS,
                       (int)tiles_t, tiles_o, xg, (const uint4 *)nullptr, 0, 0, 0);
    return hipGetLastError();
}

// The gathered-load instances (the p4 group convolution and its unrolled comparator): like launch_big,
// plus the stage table and the image geometry (token n = pixel n of a [N / (H W)][H][W] grid).
template <int G, int WA, int WB, int OW, int TW>
static hipError_t launch_big_conv(const Plan *p, const void *x, const void *b, void *y, int64_t N, int img_h,
                                  int img_w, hipStream_t s) {
    using C = BigCfg<G, WA, WB, OW, TW>;
    const int64_t tiles_t = (N + C::BT - 1) / C::BT;
    const int tiles_o = p->NB_total / (C::BO / 32);
    const int n_stages = p->KS / C::KSS;
    if (n_stages % 8 != 0) return hipErrorInvalidValue;  // the stage loop's bodies of 8
    const int x_elems = p->conv_cin * 4;  // elements per pixel row of x (C_in channels x 4 samples)
    // x is one buffer resource addressed with 32-bit offsets; output rows as in launch_big
    if (tiles_t > 0x7fffffff || (int64_t)C::BT * p->C_out * G * 2 > 0x7fffffff || N * x_elems * 2 > 0x7fffffff)
        return hipErrorInvalidValue;
    int64_t per_o = std::max(1, p->fwd.num_cus / tiles_o);
    per_o = std::min<int64_t>(per_o, tiles_t);
    const int64_t grid = per_o * tiles_o;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const int xg = xcd_group(tiles_o, (size_t)C::BO * p->KS * 16 * G * 2);
    auto kern = p->dtype == EQLIN_F16 ? k_big<G, WA, WB, OW, TW, true, false, F16, true>
                                      : k_big<G, WA, WB, OW, TW, true, false, BF16, true>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), 0, s, (const uint4 *)x, (const uint4 *)p->planes,
                       (const uint16_t *)b, p->bias_shift, (uint16_t *)y, N, p->C_in, p->C_out, n_stages, p->KS,
                       (int)tiles_t, tiles_o, xg, (const uint4 *)p->conv_tab, img_h, img_w, x_elems);
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
    // two waves per SIMD (8 waves, 128 accumulators each) where one wave's 32-output blocks keep
    // the weight reuse: the waves of a SIMD hide each other's waits. At G = 8 a wave needs all 256
    // accumulators for two token blocks (fewer would double the L2 traffic per product), so one.
    BE(1, 2, 4, 8, 1),
    BE(2, 1, 4, 8, 1),
    BE(4, 1, 2, 8, 1),
    {8, P8Cfg::BO, P8Cfg::BT, P8Cfg::KSS, P8Cfg::NT, P8Cfg::LDS, launch_p8, "planes split over 2 waves/SIMD, 4x2 waves"},
};
#undef BE

// The gathered-load tiles: G = 4 as the layer's (8 waves, two per SIMD); the unrolled comparator
// (G = 1) on 4 waves, one per SIMD: its two x items per thread keep two sets of four rows each in
// registers, which 8 waves' 256 registers per wave cannot hold beside the 2x4 blocks' accumulators
// (spilled: 606 us vs 333 us at 3x3 256->256 over 4x64x64 pixels).
template <int G, int WA, int WB, int OW, int TW>
static void conv_choice(KernelChoice *out) {
    using C = BigCfg<G, WA, WB, OW, TW>;
    out->kind = KIND_BIG;
    out->frag_kind = 2;
    out->rows_per_block = 32;
    out->kc = 16;
    out->ks_mult = 8 * C::KSS;  // stages in bodies of 8 (two groups of four that share their rows)
    out->nb_tile = C::BO / 32;
    out->tokens_per_block = C::BT;
    out->block_threads = C::NT;
    out->lds_bytes = C::LDS;
    out->num_cus = device_num_cus();
    out->launch = nullptr;  // a convolution plan runs only through conv_launch
    out->conv_launch = launch_big_conv<G, WA, WB, OW, TW>;
    snprintf(out->name, sizeof(out->name), "bf16 big G=%d BO=%d BT=%d (%dx%d blocks/wave, %dx%d waves) mfma32x32x16 gathered",
             G, C::BO, C::BT, WA, WB, OW, TW);
}

bool select_big_conv(int G, int C_in, int C_out, KernelChoice *out) {
    (void)C_in;
    if (G != 4 && G != 1) return false;
    if ((C_out * G) % 8 != 0) return false;  // whole 16-byte pieces per output row
    if (G == 4) {
        if ((int64_t)BigCfg<4, 1, 2, 8, 1>::BT * C_out * G * 2 > 0x7fffffff) return false;
        conv_choice<4, 1, 2, 8, 1>(out);
    } else {
        if ((int64_t)BigCfg<1, 2, 4, 4, 1>::BT * C_out * G * 2 > 0x7fffffff) return false;
        conv_choice<1, 2, 4, 4, 1>(out);
    }
    return true;
}

bool select_big(int G, bool d4, int C_in, int C_out, KernelChoice *out) {
    (void)C_in;
    for (const auto &e : kBig) {
        if (e.G != G || (d4 && G != 8)) continue;  // D4 runs on the plane-split G = 8 kernel
        // a token tile's output rows are addressed with 32-bit buffer offsets
        if ((int64_t)e.BT * C_out * G * 2 > 0x7fffffff) return false;
        out->kind = KIND_BIG;
        out->frag_kind = 2;
        out->rows_per_block = 32;
        out->kc = 16;
        out->ks_mult = 2 * e.KSS;  // an even number of stages: the main loop runs them in pairs
        out->nb_tile = e.BO / 32;
        out->tokens_per_block = e.BT;
        out->block_threads = e.NT;
        out->lds_bytes = e.lds;
        out->num_cus = device_num_cus();
        out->launch = e.launch;
        snprintf(out->name, sizeof(out->name), "bf16 big %s%d BO=%d BT=%d (%s) mfma32x32x16", d4 ? "D" : "G=",
                 d4 ? 4 : G, e.BO, e.BT, e.tile);
        return true;
    }
    return false;
}

}  // namespace eqlin
