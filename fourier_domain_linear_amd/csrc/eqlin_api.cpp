// eqlin_api.cpp -- the C ABI (include/eqlin.h): argument checks, plans, dispatch, status codes.
// Nothing here computes the layer; every step of the forward runs in the HIP kernels.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "eqlin_internal.h"

using eqlin::Plan;

namespace {

thread_local char g_err[512] = "";

eqlin_status_t fail(eqlin_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

eqlin_status_t hip_fail(hipError_t e, const char *what) {
    return fail(EQLIN_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int ilog2(int g) {
    int s = 0;
    while ((1 << s) < g) ++s;
    return s;
}

void free_plan(Plan *p) {
    if (!p) return;
    if (p->expanded) free_plan(p->expanded);
    if (p->backward) free_plan(p->backward);
    if (p->planes) (void)hipFree(p->planes);
    if (p->wexp) (void)hipFree(p->wexp);
    if (p->wt) (void)hipFree(p->wt);
    if (p->conv_tab) (void)hipFree(p->conv_tab);
    if (p->wconv) (void)hipFree(p->wconv);
    delete static_cast<eqlin_plan *>(p);
}

// Fill p->planes from a weight W[C_out][C_in][G] of p->dtype (W may be the unrolled E, G = 1). A plan
// with conv_k > 0 gets the gathered-load kernel and its stage table.
eqlin_status_t build_spectral(Plan *p, const void *W, hipStream_t s) {
    hipError_t e;
    if (p->dtype != EQLIN_F32) {  // bf16 or fp16: the matrix-core kernels
        bool ok = p->conv_k > 0 ? eqlin::select_big_conv(p->G, p->C_in, p->C_out, &p->fwd)
                                : eqlin::select_bf16(p->G, p->d4, p->C_in, p->C_out, &p->fwd);
        // layers too wide for the stream kernel whose input planes fit on chip: the resident-planes
        // kernels (a token tile's planes kept for every output block, each token transformed once per
        // workgroup) instead of the large-channel ones
        eqlin::KernelChoice big;
        bool res4 = false;
        if (ok && p->conv_k == 0 && p->fwd.kind == eqlin::KIND_BIG) {
            eqlin::KernelChoice r;
            big = p->fwd;
            res4 = eqlin::select_res(p->G, p->d4, p->C_in, p->C_out, &r);
            if (res4 || eqlin::select_res8(p->G, p->d4, p->C_in, p->C_out, &r)) p->fwd = r;
        }
        if (!ok)
            return fail(EQLIN_ERR_UNSUPPORTED, "no half-precision kernel for G=%d C_in=%d C_out=%d", p->G, p->C_in,
                        p->C_out);
        if (p->dtype == EQLIN_F16 && strncmp(p->fwd.name, "bf16", 4) == 0) memcpy(p->fwd.name, "f16 ", 4);
        const int ks = (p->C_in + p->fwd.kc - 1) / p->fwd.kc;
        p->KS = (ks + p->fwd.ks_mult - 1) / p->fwd.ks_mult * p->fwd.ks_mult;
        const int nb = (p->C_out + p->fwd.rows_per_block - 1) / p->fwd.rows_per_block;
        p->NB_total = (nb + p->fwd.nb_tile - 1) / p->fwd.nb_tile * p->fwd.nb_tile;
        // G = 4: at 32 tokens per compute unit or fewer (one 32-token block per resident tile) every CU of
        // the resident-planes kernel still streams the whole weight set for its few tokens, and the
        // large-channel kernel, which splits the outputs over the CUs, is faster (measured at
        // 192 -> 768: 13.3 against 27.6 us at 3136 tokens, 24.1 against 29.5 at 6272, equal at 12544).
        // It reads the same weights when both kernels pad the channels alike.
        if (res4 && !(p->flags & EQLIN_PREPARE_FIXED_KERNEL) && big.frag_kind == p->fwd.frag_kind &&
            big.kc == p->fwd.kc && big.rows_per_block == p->fwd.rows_per_block && p->KS % big.ks_mult == 0 &&
            p->NB_total % big.nb_tile == 0) {
            p->fwd_small = big;
            p->small_max_n = (int64_t)32 * std::max(1, p->fwd.num_cus);
            if (p->dtype == EQLIN_F16 && strncmp(p->fwd_small.name, "bf16", 4) == 0) memcpy(p->fwd_small.name, "f16 ", 4);
        }
        p->planes_bytes = (size_t)p->NB_total * p->KS * p->G * 1024;
        e = hipMalloc(&p->planes, p->planes_bytes);
        if (e != hipSuccess) {
            p->planes = nullptr;
            return fail(EQLIN_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) for spectral weights: %s", p->planes_bytes,
                        hipGetErrorString(e));
        }
        e = eqlin::launch_prep_frag(W, true, p->dtype == EQLIN_F16, p->d4, p->G, p->C_out, p->C_in, p->KS, p->NB_total, p->fwd.frag_kind,
                                    p->planes, s);
        if (e != hipSuccess) return hip_fail(e, "spectral weight preparation");
        if (p->conv_k > 0) {  // the gathered loads' table (one entry per group of four stages of 16 channels)
            const int n_stages = p->G == 1 ? p->KS / 4 : p->KS;
            const std::vector<uint4> tab = eqlin::conv_group_table(p->conv_cin, p->conv_k, 2, n_stages / 4);
            e = hipMalloc(&p->conv_tab, tab.size() * sizeof(uint4));
            if (e != hipSuccess) {
                p->conv_tab = nullptr;
                return fail(EQLIN_ERR_OUT_OF_MEMORY, "hipMalloc for the convolution's stage table");
            }
            // the host vector dies with this call: a synchronous copy (a few KB, at prepare only)
            e = hipMemcpy(p->conv_tab, tab.data(), tab.size() * sizeof(uint4), hipMemcpyHostToDevice);
            if (e != hipSuccess) return hip_fail(e, "convolution stage table");
        }
    } else {
        if (!eqlin::select_f32(p->G, p->d4, p->C_in, p->C_out, &p->fwd))
            return fail(EQLIN_ERR_UNSUPPORTED, "no f32 kernel for G=%d", p->G);
        p->planes_bytes = (size_t)p->G * p->C_out * p->C_in * sizeof(float);
        e = hipMalloc(&p->planes, p->planes_bytes);
        if (e != hipSuccess) {
            p->planes = nullptr;
            return fail(EQLIN_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) for spectral weights: %s", p->planes_bytes,
                        hipGetErrorString(e));
        }
        e = eqlin::launch_prep_plain_f32((const float *)W, p->d4, p->G, p->C_out, p->C_in, (float *)p->planes, s);
        if (e != hipSuccess) return hip_fail(e, "spectral weight preparation");
    }
    return EQLIN_OK;
}

// The unrolled comparator of plan p, whose weight W[C_out][C_in][G] (p's dtype) is given: E = unroll(W)
// and a G = 1 plan over it (p->wexp, p->expanded).
eqlin_status_t add_expanded(Plan *p, const void *W, hipStream_t s) {
    const int G = p->G;
    const size_t eb = p->dtype == EQLIN_F32 ? 4 : 2;
    const size_t ebytes = (size_t)p->C_out * G * p->C_in * G * eb;
    hipError_t e = hipMalloc(&p->wexp, ebytes);
    if (e != hipSuccess) {
        p->wexp = nullptr;
        return fail(EQLIN_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) for the unrolled weight", ebytes);
    }
    e = eqlin::launch_expand(W, (int)eb, p->d4, G, p->C_out, p->C_in, p->wexp, s);
    if (e != hipSuccess) return hip_fail(e, "unrolled weight");
    Plan *q = new (std::nothrow) eqlin_plan();
    if (!q) return fail(EQLIN_ERR_OUT_OF_MEMORY, "host allocation");
    q->C_out = p->C_out * G;
    q->C_in = p->C_in * G;
    q->G = 1;
    q->dtype = p->dtype;
    q->device = p->device;
    q->bias_shift = ilog2(G);
    p->expanded = q;  // owned by p from here (freed with it)
    return build_spectral(q, p->wexp, s);
}

eqlin_status_t check_forward_args(const Plan *h, const void *x, const void *b, const void *y, int64_t N,
                                  int C_in, int C_out, int G) {
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (N < 0) return fail(EQLIN_ERR_INVALID_ARG, "N = %lld < 0", (long long)N);
    if (N == 0) return EQLIN_OK;
    if (!x || !y) return fail(EQLIN_ERR_INVALID_ARG, "null x or y");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(EQLIN_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    const size_t eb = h->dtype == EQLIN_F32 ? 4 : 2;
    if (b && !aligned(b, eb)) return fail(EQLIN_ERR_INVALID_ARG, "b misaligned");
    const int64_t lim = INT64_C(1) << 60;
    if (N > lim / ((int64_t)C_in * G) || N > lim / ((int64_t)C_out * G))
        return fail(EQLIN_ERR_INVALID_ARG, "N = %lld overflows the index range", (long long)N);
    if (N > INT64_C(1) << 35) return fail(EQLIN_ERR_INVALID_ARG, "N = %lld exceeds the grid range", (long long)N);
    // x and y must not overlap
    const char *xs = (const char *)x, *ys = (const char *)y;
    const size_t xb = (size_t)N * C_in * G * eb, yb = (size_t)N * C_out * G * eb;
    if (xs < ys + yb && ys < xs + xb) return fail(EQLIN_ERR_INVALID_ARG, "x and y overlap");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != h->device)
        return fail(EQLIN_ERR_INVALID_ARG, "handle belongs to device %d, current device is %d", h->device, dev);
    return EQLIN_OK;
}

// The scratch of eqlin_backward_weights_static: a static device array in this library's code object,
// so each device the library runs on holds its own copy, from the first use until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device (static_scratch), and only that address is handed to kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[EQLIN_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on device `dev`, which must be the current device (looked up on the
// first call for that device, then kept).
static eqlin_status_t static_scratch(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(EQLIN_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(EQLIN_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return EQLIN_OK;
}

extern "C" {

eqlin_status_t eqlin_prepare_weights(const void *W, int C_out, int C_in, int G, eqlin_dtype_t dtype,
                                     unsigned flags, eqlin_stream_t stream, eqlin_handle_t *out) {
    g_err[0] = 0;
    if (!out) return fail(EQLIN_ERR_INVALID_ARG, "null out");
    *out = nullptr;
    if (!W) return fail(EQLIN_ERR_INVALID_ARG, "null W");
    if (C_out < 1 || C_in < 1) return fail(EQLIN_ERR_INVALID_ARG, "C_out = %d, C_in = %d must be >= 1", C_out, C_in);
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return fail(EQLIN_ERR_INVALID_ARG, "G = %d not in {1, 2, 4, 8}", G);
    if (dtype != EQLIN_F32 && dtype != EQLIN_BF16 && dtype != EQLIN_F16)
        return fail(EQLIN_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    if (flags & ~(EQLIN_PREPARE_EXPANDED | EQLIN_PREPARE_BACKWARD | EQLIN_PREPARE_D4 | EQLIN_PREPARE_FIXED_KERNEL))
        return fail(EQLIN_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    const bool d4 = (flags & EQLIN_PREPARE_D4) != 0;
    if (d4 && G != 8) return fail(EQLIN_ERR_INVALID_ARG, "EQLIN_PREPARE_D4 needs G = 8 (got G = %d)", G);
    if ((int64_t)C_out * G > (1 << 20) || (int64_t)C_in * G > (1 << 20))
        return fail(EQLIN_ERR_UNSUPPORTED, "channel counts beyond 2^20 unrolled columns");
    if (!aligned(W, 16)) return fail(EQLIN_ERR_INVALID_ARG, "W must be 16-byte aligned");
    if (dtype != EQLIN_F32 && C_in % 8 != 0)
        return fail(EQLIN_ERR_UNSUPPORTED, "bf16/f16 path needs C_in %% 8 == 0 (C_in = %d)", C_in);
    if ((flags & EQLIN_PREPARE_BACKWARD) && dtype != EQLIN_F32 && C_out % 8 != 0)
        return fail(EQLIN_ERR_UNSUPPORTED, "bf16/f16 backward needs C_out %% 8 == 0 (C_out = %d)", C_out);

    hipStream_t s = (hipStream_t)stream;
    Plan *p = new (std::nothrow) eqlin_plan();
    if (!p) return fail(EQLIN_ERR_OUT_OF_MEMORY, "host allocation");
    p->C_out = C_out;
    p->C_in = C_in;
    p->G = G;
    p->d4 = d4;
    p->dtype = dtype;
    p->flags = flags;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        free_plan(p);
        return hip_fail(e, "hipGetDevice");
    }
    eqlin_status_t st = build_spectral(p, W, s);
    if (st != EQLIN_OK) {
        free_plan(p);
        return st;
    }
    {  // set-up of this device: the address of eqlin_backward_weights_static's scratch
        void *ws = nullptr;
        st = static_scratch(p->device, &ws);
        if (st != EQLIN_OK) {
            free_plan(p);
            return st;
        }
    }
    if (flags & EQLIN_PREPARE_EXPANDED) {
        st = add_expanded(p, W, s);
        if (st != EQLIN_OK) {
            free_plan(p);
            return st;
        }
    }
    if (flags & EQLIN_PREPARE_BACKWARD) {
        const size_t eb = dtype == EQLIN_F32 ? 4 : 2;
        const size_t bytes = (size_t)C_out * C_in * G * eb;
        e = hipMalloc(&p->wt, bytes);
        if (e != hipSuccess) {
            p->wt = nullptr;
            free_plan(p);
            return fail(EQLIN_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) for the backward weight", bytes);
        }
        e = eqlin::launch_transpose_reverse(W, (int)eb, d4, G, C_out, C_in, p->wt, s);
        if (e != hipSuccess) {
            free_plan(p);
            return hip_fail(e, "backward weight");
        }
        Plan *q = new (std::nothrow) eqlin_plan();
        if (!q) {
            free_plan(p);
            return fail(EQLIN_ERR_OUT_OF_MEMORY, "host allocation");
        }
        q->C_out = C_in;
        q->C_in = C_out;
        q->G = G;
        q->d4 = d4;
        q->dtype = dtype;
        q->device = p->device;
        q->flags = flags & EQLIN_PREPARE_FIXED_KERNEL;  // dx runs this plan's forward kernels
        p->backward = q;
        st = build_spectral(q, p->wt, s);
        // with both flags, the data gradient's own unrolled comparator: the G = 1 product with E^T
        if (st == EQLIN_OK && (flags & EQLIN_PREPARE_EXPANDED)) st = add_expanded(q, p->wt, s);
        if (st != EQLIN_OK) {
            free_plan(p);
            return st;
        }
    }
    *out = static_cast<eqlin_handle_t>(static_cast<eqlin_plan *>(p));
    return EQLIN_OK;
}

static eqlin_status_t run_forward(const Plan *h, const void *x, const void *b, void *y, int64_t N, int act,
                                  eqlin_stream_t stream, const char *what) {
    (void)hipGetLastError();  // drop a stale error left by someone else's call on this thread
    const eqlin::KernelChoice &k = (h->fwd_small.launch && N <= h->small_max_n) ? h->fwd_small : h->fwd;
    hipError_t e = k.launch(h, x, b, y, N, act, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, what);
    return EQLIN_OK;
}

static bool valid_act(int act) { return act == EQLIN_ACT_NONE || act == EQLIN_ACT_GELU; }

eqlin_status_t eqlin_forward_act(eqlin_handle_t h, const void *x, const void *b, void *y, int64_t N, int act,
                                 eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (h->conv_k > 0) return fail(EQLIN_ERR_INVALID_ARG, "a convolution handle: use eqlin_conv_forward");
    if (!valid_act(act)) return fail(EQLIN_ERR_INVALID_ARG, "unknown activation %d", act);
    eqlin_status_t st = check_forward_args(h, x, b, y, N, h->C_in, h->C_out, h->G);
    if (st != EQLIN_OK || N == 0) return st;
    return run_forward(h, x, b, y, N, act, stream, "eqlin_forward launch");
}

eqlin_status_t eqlin_forward(eqlin_handle_t h, const void *x, const void *b, void *y, int64_t N,
                             eqlin_stream_t stream) {
    return eqlin_forward_act(h, x, b, y, N, EQLIN_ACT_NONE, stream);
}

eqlin_status_t eqlin_forward_expanded_act(eqlin_handle_t h, const void *x, const void *b, void *y, int64_t N,
                                          int act, eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (h->conv_k > 0) return fail(EQLIN_ERR_INVALID_ARG, "a convolution handle: use eqlin_conv_forward_expanded");
    if (!h->expanded)
        return fail(EQLIN_ERR_INVALID_ARG, "handle was prepared without EQLIN_PREPARE_EXPANDED");
    if (!valid_act(act)) return fail(EQLIN_ERR_INVALID_ARG, "unknown activation %d", act);
    eqlin_status_t st = check_forward_args(h, x, b, y, N, h->C_in, h->C_out, h->G);
    if (st != EQLIN_OK || N == 0) return st;
    return run_forward(h->expanded, x, b, y, N, act, stream, "eqlin_forward_expanded launch");
}

eqlin_status_t eqlin_forward_expanded(eqlin_handle_t h, const void *x, const void *b, void *y, int64_t N,
                                      eqlin_stream_t stream) {
    return eqlin_forward_expanded_act(h, x, b, y, N, EQLIN_ACT_NONE, stream);
}

eqlin_status_t eqlin_backward_data(eqlin_handle_t h, const void *dy, void *dx, int64_t N, eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (!h->backward) return fail(EQLIN_ERR_INVALID_ARG, "handle was prepared without EQLIN_PREPARE_BACKWARD");
    eqlin_status_t st = check_forward_args(h, dy, nullptr, dx, N, h->C_out, h->C_in, h->G);
    if (st != EQLIN_OK || N == 0) return st;
    return run_forward(h->backward, dy, nullptr, dx, N, EQLIN_ACT_NONE, stream, "eqlin_backward_data launch");
}

eqlin_status_t eqlin_backward_data_expanded(eqlin_handle_t h, const void *dy, void *dx, int64_t N,
                                            eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (!h->backward || !h->backward->expanded)
        return fail(EQLIN_ERR_INVALID_ARG, "handle was not prepared with EQLIN_PREPARE_BACKWARD | EQLIN_PREPARE_EXPANDED");
    eqlin_status_t st = check_forward_args(h, dy, nullptr, dx, N, h->C_out, h->C_in, h->G);
    if (st != EQLIN_OK || N == 0) return st;
    return run_forward(h->backward->expanded, dy, nullptr, dx, N, EQLIN_ACT_NONE, stream,
                       "eqlin_backward_data_expanded launch");
}

size_t eqlin_backward_weights_workspace(eqlin_handle_t h, int64_t N) {
    if (!h || N <= 0) return 0;
    return eqlin::bw_workspace_bytes(h, N);
}

// The gradient passes of eqlin_backward_weights after its argument checks; ws: workspace of at least
// eqlin::bw_workspace_bytes(h, N) bytes (or null when that is 0).
static eqlin_status_t backward_weights_run(const Plan *h, const void *x, const void *dy, float *dW, float *db,
                                           int64_t N, void *ws, hipStream_t stream) {
    (void)hipGetLastError();
    hipError_t e;
    if (N == 0) {  // no tokens: zero gradients (fill kernels, no memset nodes under graph capture)
        e = eqlin::launch_zero_f32(dW, (int64_t)h->C_out * h->C_in * h->G, stream);
        if (e == hipSuccess && db) e = eqlin::launch_zero_f32(db, h->C_out, stream);
        return e == hipSuccess ? EQLIN_OK : hip_fail(e, "eqlin_backward_weights clear");
    }
    e = eqlin::launch_backward_weights(h, x, dy, dW, db, N, ws, stream);
    return e == hipSuccess ? EQLIN_OK : hip_fail(e, "eqlin_backward_weights launch");
}

static eqlin_status_t check_backward_weights_args(const Plan *h, const void *x, const void *dy, const float *dW,
                                                  const float *db, int64_t N) {
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (h->conv_k > 0) return fail(EQLIN_ERR_INVALID_ARG, "a convolution handle has no gradient entry points");
    if (!dW) return fail(EQLIN_ERR_INVALID_ARG, "null dW");
    if (!aligned(dW, 4) || (db && !aligned(db, 4))) return fail(EQLIN_ERR_INVALID_ARG, "dW and db must be 4-byte aligned");
    // x plays the forward's x, dy the forward's y (shapes, alignment, overlap, device)
    return check_forward_args(h, x, nullptr, dy, N, h->C_in, h->C_out, h->G);
}

eqlin_status_t eqlin_backward_weights(eqlin_handle_t h, const void *x, const void *dy, float *dW, float *db,
                                      int64_t N, void *workspace, size_t workspace_bytes, eqlin_stream_t stream) {
    g_err[0] = 0;
    eqlin_status_t st = check_backward_weights_args(h, x, dy, dW, db, N);
    if (st != EQLIN_OK) return st;
    const size_t need = eqlin::bw_workspace_bytes(h, N);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(EQLIN_ERR_INVALID_ARG, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (need > 0 && !aligned(workspace, 256)) return fail(EQLIN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    return backward_weights_run(h, x, dy, dW, db, N, workspace, (hipStream_t)stream);
}

eqlin_status_t eqlin_backward_weights_static(eqlin_handle_t h, const void *x, const void *dy, float *dW, float *db,
                                             int64_t N, eqlin_stream_t stream) {
    g_err[0] = 0;
    eqlin_status_t st = check_backward_weights_args(h, x, dy, dW, db, N);
    if (st != EQLIN_OK) return st;
    const size_t need = eqlin::bw_workspace_bytes(h, N);
    if (need > EQLIN_STATIC_SCRATCH_BYTES)
        return fail(EQLIN_ERR_UNSUPPORTED, "N = %lld needs %zu bytes of scratch, above the static %zu (use "
                    "eqlin_backward_weights with a workspace)", (long long)N, need, (size_t)EQLIN_STATIC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0) {
        st = static_scratch(h->device, &ws);
        if (st != EQLIN_OK) return st;
    }
    return backward_weights_run(h, x, dy, dW, db, N, ws, (hipStream_t)stream);
}

eqlin_status_t eqlin_prepare_conv_weights(const void *psi, int C_out, int C_in, int G, int k, eqlin_dtype_t dtype,
                                          unsigned flags, eqlin_stream_t stream, eqlin_handle_t *out) {
    g_err[0] = 0;
    if (!out) return fail(EQLIN_ERR_INVALID_ARG, "null out");
    *out = nullptr;
    if (!psi) return fail(EQLIN_ERR_INVALID_ARG, "null psi");
    if (G != 4) return fail(EQLIN_ERR_INVALID_ARG, "the convolution is over p4: G must be 4 (got %d)", G);
    if (k < 1 || k > 15 || k % 2 == 0) return fail(EQLIN_ERR_INVALID_ARG, "k = %d: odd, 1..15", k);
    if (C_out < 1 || C_in < 1) return fail(EQLIN_ERR_INVALID_ARG, "C_out = %d, C_in = %d must be >= 1", C_out, C_in);
    if (!aligned(psi, 16)) return fail(EQLIN_ERR_INVALID_ARG, "psi must be 16-byte aligned");
    if (dtype != EQLIN_BF16 && dtype != EQLIN_F16)
        return fail(EQLIN_ERR_UNSUPPORTED, "the convolution runs in bf16 or fp16 (dtype %d)", (int)dtype);
    if (C_in % 16 != 0 || C_out % 8 != 0)
        return fail(EQLIN_ERR_UNSUPPORTED, "the convolution needs C_in %% 16 == 0 and C_out %% 8 == 0 (%d, %d)", C_in, C_out);
    if (flags & ~EQLIN_PREPARE_EXPANDED) return fail(EQLIN_ERR_UNSUPPORTED, "flags 0x%x: only EQLIN_PREPARE_EXPANDED", flags);
    if (C_in > 8192) return fail(EQLIN_ERR_UNSUPPORTED, "the convolution takes C_in <= 8192 (got %d)", C_in);
    const int64_t cg = eqlin::conv_gathered_channels(C_in, k);
    if (cg * G > (1 << 20) || (int64_t)C_out * G > (1 << 20))
        return fail(EQLIN_ERR_UNSUPPORTED, "channel counts beyond 2^20 unrolled columns");
    hipStream_t s = (hipStream_t)stream;
    Plan *p = new (std::nothrow) eqlin_plan();
    if (!p) return fail(EQLIN_ERR_OUT_OF_MEMORY, "host allocation");
    p->C_out = C_out;
    p->C_in = (int)cg;
    p->G = G;
    p->dtype = dtype;
    p->flags = flags;
    p->conv_k = k;
    p->conv_cin = C_in;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        free_plan(p);
        return hip_fail(e, "hipGetDevice");
    }
    const size_t wbytes = (size_t)C_out * cg * G * 2;
    e = hipMalloc(&p->wconv, wbytes);
    if (e != hipSuccess) {
        p->wconv = nullptr;
        free_plan(p);
        return fail(EQLIN_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) for the gathered weight", wbytes);
    }
    e = eqlin::launch_conv_weight(psi, 2, C_out, C_in, k, p->wconv, s);
    if (e != hipSuccess) {
        free_plan(p);
        return hip_fail(e, "gathered weight");
    }
    eqlin_status_t st = build_spectral(p, p->wconv, s);
    if (st != EQLIN_OK) {
        free_plan(p);
        return st;
    }
    {  // set-up of this device (as eqlin_prepare_weights)
        void *ws = nullptr;
        st = static_scratch(p->device, &ws);
        if (st != EQLIN_OK) {
            free_plan(p);
            return st;
        }
    }
    if (flags & EQLIN_PREPARE_EXPANDED) {  // the unrolled gathered layer, run as G = 1 with the same gather
        const size_t ebytes = (size_t)C_out * G * cg * G * 2;
        e = hipMalloc(&p->wexp, ebytes);
        if (e != hipSuccess) {
            p->wexp = nullptr;
            free_plan(p);
            return fail(EQLIN_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) for the unrolled weight", ebytes);
        }
        e = eqlin::launch_expand(p->wconv, 2, false, G, C_out, (int)cg, p->wexp, s);
        if (e != hipSuccess) {
            free_plan(p);
            return hip_fail(e, "unrolled weight");
        }
        Plan *q = new (std::nothrow) eqlin_plan();
        if (!q) {
            free_plan(p);
            return fail(EQLIN_ERR_OUT_OF_MEMORY, "host allocation");
        }
        q->C_out = C_out * G;
        q->C_in = (int)cg * G;
        q->G = 1;
        q->dtype = dtype;
        q->device = p->device;
        q->bias_shift = 2;
        q->conv_k = k;
        q->conv_cin = C_in;
        p->expanded = q;
        st = build_spectral(q, p->wexp, s);
        if (st != EQLIN_OK) {
            free_plan(p);
            return st;
        }
    }
    *out = static_cast<eqlin_handle_t>(static_cast<eqlin_plan *>(p));
    return EQLIN_OK;
}

static eqlin_status_t run_conv(const Plan *h, const Plan *run, const void *x, const void *b, void *y, int64_t B, int H,
                               int W, eqlin_stream_t stream, const char *what) {
    if (B < 0 || H < 0 || W < 0) return fail(EQLIN_ERR_INVALID_ARG, "B = %lld, H = %d, W = %d", (long long)B, H, W);
    if (B == 0 || H == 0 || W == 0) return EQLIN_OK;
    if ((int64_t)H * W > INT32_MAX || B > (INT64_C(1) << 40) / ((int64_t)H * W))
        return fail(EQLIN_ERR_INVALID_ARG, "B x H x W overflows");
    const int64_t N = B * H * W;
    // x plays the layer's x with its real channel count, y the layer's y
    eqlin_status_t st = check_forward_args(h, x, b, y, N, h->conv_cin, h->C_out, h->G);
    if (st != EQLIN_OK) return st;
    if (N * h->conv_cin * h->G * 2 >= (INT64_C(1) << 31))
        return fail(EQLIN_ERR_UNSUPPORTED, "x of %lld bytes: the gathered loads address x with 32-bit offsets",
                    (long long)(N * h->conv_cin * h->G * 2));
    (void)hipGetLastError();
    hipError_t e = run->fwd.conv_launch(run, x, b, y, N, H, W, (hipStream_t)stream);
    return e == hipSuccess ? EQLIN_OK : hip_fail(e, what);
}

eqlin_status_t eqlin_conv_forward(eqlin_handle_t h, const void *x, const void *bias, void *y, int64_t B, int H, int W,
                                  eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (h->conv_k <= 0) return fail(EQLIN_ERR_INVALID_ARG, "not a convolution handle (eqlin_prepare_conv_weights)");
    return run_conv(h, h, x, bias, y, B, H, W, stream, "eqlin_conv_forward launch");
}

eqlin_status_t eqlin_conv_forward_expanded(eqlin_handle_t h, const void *x, const void *bias, void *y, int64_t B,
                                           int H, int W, eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (h->conv_k <= 0) return fail(EQLIN_ERR_INVALID_ARG, "not a convolution handle (eqlin_prepare_conv_weights)");
    if (!h->expanded) return fail(EQLIN_ERR_INVALID_ARG, "handle was prepared without EQLIN_PREPARE_EXPANDED");
    return run_conv(h, h->expanded, x, bias, y, B, H, W, stream, "eqlin_conv_forward_expanded launch");
}

eqlin_status_t eqlin_destroy(eqlin_handle_t h) {
    g_err[0] = 0;
    free_plan(h);
    return EQLIN_OK;
}

eqlin_status_t eqlin_export_spectral_weights(eqlin_handle_t h, float *out, eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h || !out) return fail(EQLIN_ERR_INVALID_ARG, "null handle or out");
    hipError_t e;
    if (h->dtype != EQLIN_F32)
        e = eqlin::launch_export_frag(h->planes, h->dtype == EQLIN_F16, h->d4, h->G, h->C_out, h->C_in, h->KS, h->NB_total,
                                      h->fwd.frag_kind, out, (hipStream_t)stream);
    else
        e = eqlin::launch_export_plain_f32((const float *)h->planes, h->d4, h->G, h->C_out, h->C_in, out,
                                           (hipStream_t)stream);
    return e == hipSuccess ? EQLIN_OK : hip_fail(e, "export of spectral weights");
}

eqlin_status_t eqlin_export_expanded_weight(eqlin_handle_t h, void *out, eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h || !out) return fail(EQLIN_ERR_INVALID_ARG, "null handle or out");
    if (!h->wexp) return fail(EQLIN_ERR_INVALID_ARG, "handle was prepared without EQLIN_PREPARE_EXPANDED");
    const size_t eb = h->dtype == EQLIN_F32 ? 4 : 2;
    const size_t bytes = (size_t)h->C_out * h->G * h->C_in * h->G * eb;
    hipError_t e = hipMemcpyAsync(out, h->wexp, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream);
    return e == hipSuccess ? EQLIN_OK : hip_fail(e, "export of the unrolled weight");
}

int eqlin_describe(eqlin_handle_t h, char *buf, size_t len) {
    if (!h) return snprintf(buf, len, "(null handle)");
    if (h->conv_k > 0)
        return snprintf(buf, len, "p4 conv %dx%d C_in=%d (gathered %d) C_out=%d %s | forward: %s | expanded: %s", h->conv_k,
                        h->conv_k, h->conv_cin, h->C_in, h->C_out, h->dtype == EQLIN_BF16 ? "bf16" : "f16", h->fwd.name,
                        h->expanded ? h->expanded->fwd.name : "(not prepared)");
    char fw[224];
    if (h->fwd_small.launch)
        snprintf(fw, sizeof(fw), "%s; at N <= %lld: %s", h->fwd.name, (long long)h->small_max_n, h->fwd_small.name);
    else
        snprintf(fw, sizeof(fw), "%s", h->fwd.name);
    return snprintf(buf, len,
                    "%s%d C_in=%d C_out=%d %s | forward: %s | expanded: %s | backward data: %s | backward weights: %s",
                    h->d4 ? "D" : "G=", h->d4 ? 4 : h->G, h->C_in, h->C_out, h->dtype == EQLIN_BF16 ? "bf16" : h->dtype == EQLIN_F16 ? "f16" : "f32", fw,
                    h->expanded ? h->expanded->fwd.name : "(not prepared)",
                    h->backward ? h->backward->fwd.name : "(not prepared)", eqlin::bw_kernel_name(h));
}

const char *eqlin_status_string(eqlin_status_t s) {
    switch (s) {
        case EQLIN_OK: return "EQLIN_OK";
        case EQLIN_ERR_INVALID_ARG: return "EQLIN_ERR_INVALID_ARG";
        case EQLIN_ERR_UNSUPPORTED: return "EQLIN_ERR_UNSUPPORTED";
        case EQLIN_ERR_OUT_OF_MEMORY: return "EQLIN_ERR_OUT_OF_MEMORY";
        case EQLIN_ERR_HIP: return "EQLIN_ERR_HIP";
    }
    return "EQLIN_ERR_UNKNOWN";
}

const char *eqlin_last_error(void) { return g_err; }

const char *eqlin_version(void) { return "0.1.0"; }

}  // extern "C"
