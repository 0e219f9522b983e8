// eqlin_internal.h -- the plan behind an eqlin_handle_t and the kernel launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/eqlin.h"

namespace eqlin {

// Forward-kernel families.
enum KernelKind {
    KIND_STREAM = 0,    // bf16, small C_in: persistent workgroup per CU, the C_out tile's weights in
                        // LDS, 16-token row blocks streamed through the waves, x straight to registers
    KIND_BIG = 1,       // bf16, large C: persistent workgroups, each keeping one output tile and
                        // walking token tiles on 32x32x16 matrix cores; x planes transformed once per
                        // stage into LDS, weights straight to registers, outputs stored a tile later
    KIND_F32 = 2,       // fp32: vector-ALU spectral kernel
    KIND_RES = 3        // bf16, G = 4, C_in planes fit on chip: one token tile per workgroup, its
                        // planes resident in LDS for every output block, weights streamed per wave
};

struct Plan;

// act: an eqlin_act_t applied to every output value in the epilogue
typedef hipError_t (*LaunchFn)(const Plan *p, const void *x, const void *b, void *y, int64_t N, int act,
                               hipStream_t s);
// the p4 group convolution's forward (conv.hip): x, y one token per pixel of a [N / (H W)][H][W] grid
typedef hipError_t (*ConvLaunchFn)(const Plan *p, const void *x, const void *b, void *y, int64_t N, int H, int W,
                                   hipStream_t s);

// Kernel choice for one plan. The weight layout (padding of C_in and C_out) depends on it.
struct KernelChoice {
    int kind = -1;
    int nb_tile = 1;        // 16-wide output blocks per workgroup tile
    int tokens_per_block = 0;
    int block_threads = 0;
    int num_cus = 0;        // compute units of the device the plan was made on
    int frag_kind = 1;      // weight fragment layout (prepare.hip): 1 = 16x32 chunks, stream k order;
                            // 2 = 32x16 chunks, natural k order
    int rows_per_block = 16;  // outputs per fragment chunk
    int kc = 32;            // input channels per K-step (per fragment chunk)
    int ks_mult = 1;        // K-steps are padded to a multiple of this
    size_t lds_bytes = 0;
    LaunchFn launch = nullptr;
    ConvLaunchFn conv_launch = nullptr;  // convolution plans: the gathered-load instance
    char name[96] = {0};
};

struct Plan {
    int C_out = 0, C_in = 0, G = 0;
    bool d4 = false;   // the group is the dihedral D4 (G = 8), not the cyclic group of order G
    eqlin_dtype_t dtype = EQLIN_BF16;
    unsigned flags = 0;
    int device = 0;
    int bias_shift = 0;  // the bias index is o >> bias_shift (expanded plans: log2 of the parent's G)

    // spectral weights. bf16: fragment-ordered chunks (see prepare.hip); f32: planes [G][C_out][C_in]
    void *planes = nullptr;
    size_t planes_bytes = 0;
    int KS = 0;        // bf16: K-steps of fwd.kc channels (C_in padded up; a multiple of ks_mult)
    int NB_total = 0;  // bf16: output blocks of fwd.rows_per_block (C_out padded to the tile)
    KernelChoice fwd;
    // bf16 / fp16: the kernel for batches of at most small_max_n tokens (launch == nullptr: none), run
    // on the same spectral weights (its padding of KS and NB_total agrees with fwd's)
    KernelChoice fwd_small;
    int64_t small_max_n = 0;

    // unrolled weight (flags & EQLIN_PREPARE_EXPANDED): a G = 1 plan over E, plus E itself
    Plan *expanded = nullptr;
    void *wexp = nullptr;  // [C_out*G][C_in*G] of dtype

    // data gradient (flags & EQLIN_PREPARE_BACKWARD): a plan over Wt[i][o][d] = W[o][i][-d mod G]
    // (C_in and C_out swapped), whose forward is dx; plus Wt itself
    Plan *backward = nullptr;
    void *wt = nullptr;  // [C_in][C_out][G] of dtype

    // p4 group convolution (eqlin_prepare_conv_weights): C_in above is the gathered channel count
    // conv_cin * conv_k^2; conv_tab the kernels' per-stage source table (conv.hip); wconv the gathered
    // weight W'[C_out][C_in][G] the spectral planes (and the unrolled weight) were built from
    int conv_k = 0, conv_cin = 0;
    void *conv_tab = nullptr;
    void *wconv = nullptr;
};

// ---- fwd_bf16.hip ----
bool select_bf16(int G, bool d4, int C_in, int C_out, KernelChoice *out);
int device_num_cus();  // compute units of the current device (queried once)
// ---- fwd_big.hip ----
bool select_big(int G, bool d4, int C_in, int C_out, KernelChoice *out);
// the gathered-load (convolution) instance for G = 4 (spectral) or G = 1 (the unrolled comparator)
bool select_big_conv(int G, int C_in, int C_out, KernelChoice *out);
// ---- fwd_res.hip ----
bool select_res(int G, bool d4, int C_in, int C_out, KernelChoice *out);
bool select_res8(int G, bool d4, int C_in, int C_out, KernelChoice *out);
// ---- fwd_f32.hip ----
bool select_f32(int G, bool d4, int C_in, int C_out, KernelChoice *out);

// ---- bwd.hip ----
// Workspace bytes eqlin_backward_weights needs for N tokens (0: none).
size_t bw_workspace_bytes(const Plan *p, int64_t N);
// dW [C_out][C_in][G] fp32 and db [C_out] fp32 (or null) from x and dy of the plan's dtype.
hipError_t launch_backward_weights(const Plan *p, const void *x, const void *dy, float *dW, float *db, int64_t N,
                                   void *ws, hipStream_t s);
const char *bw_kernel_name(const Plan *p);
// p[0..n) = 0 on stream s (a fill kernel: no memset node when the caller captures a graph)
hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t s);

// ---- conv.hip ----
// gathered channels of the layer a k x k convolution over C_in channels runs as: C_in * k * k, plus the
// zero channels that fill the centre's last group of four stages
int conv_gathered_channels(int C_in, int k);
// psi[C_out][C_in][4][k][k] -> the gathered layer's weight W'[C_out][conv_gathered_channels][4] (2- or
// 4-byte elements; the filling channels' weights are zero)
hipError_t launch_conv_weight(const void *psi, int elem_bytes, int C_out, int C_in, int k, void *wp, hipStream_t s);
// the kernels' source table, one entry per group of four stages, for n_groups groups (host side;
// uploaded by the caller)
std::vector<uint4> conv_group_table(int C_in, int k, int elem_bytes, int n_groups);

// ---- prepare.hip ----
// W [C_out][C_in][G] (16-bit elements of the half type when w_is_half, else fp32) -> fragment-ordered
// spectral planes in the half type (fp16 when f16, else bf16).
hipError_t launch_prep_frag(const void *W, bool w_is_half, bool f16, bool d4, int G, int C_out, int C_in, int KS,
                            int NB_total, int frag_kind, void *frag, hipStream_t s);
// W fp32 -> planes [G][C_out][C_in] fp32.
hipError_t launch_prep_plain_f32(const float *W, bool d4, int G, int C_out, int C_in, float *planes,
                                 hipStream_t s);
// W -> Wt[C_in][C_out][G], Wt[i][o][d] = W[o][i][(G - d) mod G] (same element size, 2 or 4 bytes).
hipError_t launch_transpose_reverse(const void *W, int elem_bytes, bool d4, int G, int C_out, int C_in, void *Wt,
                                   hipStream_t s);
// W -> E[C_out*G][C_in*G] (same element size, 2 or 4 bytes).
hipError_t launch_expand(const void *W, int elem_bytes, bool d4, int G, int C_out, int C_in, void *E,
                         hipStream_t s);
// stored spectral weights -> canonical fp32 [G][C_out][C_in] with the scaling undone.
hipError_t launch_export_frag(const void *frag, bool f16, bool d4, int G, int C_out, int C_in, int KS, int NB_total,
                              int frag_kind, float *out, hipStream_t s);
hipError_t launch_export_plain_f32(const float *planes, bool d4, int G, int C_out, int C_in, float *out,
                                   hipStream_t s);

}  // namespace eqlin

struct eqlin_plan : public eqlin::Plan {};
