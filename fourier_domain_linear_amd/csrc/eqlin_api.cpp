// eqlin_api.cpp -- the C ABI (include/eqlin.h): argument checks, plans, dispatch, status codes.
// Nothing here computes the layer; every step of the forward runs in the HIP kernels.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

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
    delete static_cast<eqlin_plan *>(p);
}

// Fill p->planes from a weight W[C_out][C_in][G] of p->dtype (W may be the unrolled E, G = 1).
eqlin_status_t build_spectral(Plan *p, const void *W, hipStream_t s) {
    hipError_t e;
    if (p->dtype != EQLIN_F32) {  // bf16 or fp16: the matrix-core kernels
        if (!eqlin::select_bf16(p->G, p->d4, p->C_in, p->C_out, &p->fwd))
            return fail(EQLIN_ERR_UNSUPPORTED, "no half-precision kernel for G=%d C_in=%d C_out=%d", p->G, p->C_in,
                        p->C_out);
        if (p->dtype == EQLIN_F16 && strncmp(p->fwd.name, "bf16", 4) == 0) memcpy(p->fwd.name, "f16 ", 4);
        const int ks = (p->C_in + p->fwd.kc - 1) / p->fwd.kc;
        p->KS = (ks + p->fwd.ks_mult - 1) / p->fwd.ks_mult * p->fwd.ks_mult;
        const int nb = (p->C_out + p->fwd.rows_per_block - 1) / p->fwd.rows_per_block;
        p->NB_total = (nb + p->fwd.nb_tile - 1) / p->fwd.nb_tile * p->fwd.nb_tile;
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

}  // namespace

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
    if (flags & ~(EQLIN_PREPARE_EXPANDED | EQLIN_PREPARE_BACKWARD | EQLIN_PREPARE_D4))
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
    if (flags & EQLIN_PREPARE_EXPANDED) {
        const size_t eb = dtype == EQLIN_F32 ? 4 : 2;
        const size_t ebytes = (size_t)C_out * G * C_in * G * eb;
        e = hipMalloc(&p->wexp, ebytes);
        if (e != hipSuccess) {
            p->wexp = nullptr;
            free_plan(p);
            return fail(EQLIN_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) for the unrolled weight", ebytes);
        }
        e = eqlin::launch_expand(W, (int)eb, d4, G, C_out, C_in, p->wexp, s);
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
        q->C_in = C_in * G;
        q->G = 1;
        q->dtype = dtype;
        q->device = p->device;
        q->bias_shift = ilog2(G);
        p->expanded = q;
        st = build_spectral(q, p->wexp, s);
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
        p->backward = q;
        st = build_spectral(q, p->wt, s);
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
    hipError_t e = h->fwd.launch(h, x, b, y, N, act, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, what);
    return EQLIN_OK;
}

static bool valid_act(int act) { return act == EQLIN_ACT_NONE || act == EQLIN_ACT_GELU; }

eqlin_status_t eqlin_forward_act(eqlin_handle_t h, const void *x, const void *b, void *y, int64_t N, int act,
                                 eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
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

size_t eqlin_backward_weights_workspace(eqlin_handle_t h, int64_t N) {
    if (!h || N <= 0) return 0;
    return eqlin::bw_workspace_bytes(h, N);
}

eqlin_status_t eqlin_backward_weights(eqlin_handle_t h, const void *x, const void *dy, float *dW, float *db,
                                      int64_t N, void *workspace, size_t workspace_bytes, eqlin_stream_t stream) {
    g_err[0] = 0;
    if (!h) return fail(EQLIN_ERR_INVALID_ARG, "null handle");
    if (!dW) return fail(EQLIN_ERR_INVALID_ARG, "null dW");
    if (!aligned(dW, 4) || (db && !aligned(db, 4))) return fail(EQLIN_ERR_INVALID_ARG, "dW and db must be 4-byte aligned");
    // x plays the forward's x, dy the forward's y (shapes, alignment, overlap, device)
    eqlin_status_t st = check_forward_args(h, x, nullptr, dy, N, h->C_in, h->C_out, h->G);
    if (st != EQLIN_OK) return st;
    const size_t need = eqlin::bw_workspace_bytes(h, N);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(EQLIN_ERR_INVALID_ARG, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (need > 0 && !aligned(workspace, 256)) return fail(EQLIN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    (void)hipGetLastError();
    hipError_t e;
    if (N == 0) {  // no tokens: zero gradients
        e = hipMemsetAsync(dW, 0, (size_t)h->C_out * h->C_in * h->G * sizeof(float), (hipStream_t)stream);
        if (e == hipSuccess && db) e = hipMemsetAsync(db, 0, (size_t)h->C_out * sizeof(float), (hipStream_t)stream);
        return e == hipSuccess ? EQLIN_OK : hip_fail(e, "eqlin_backward_weights clear");
    }
    e = eqlin::launch_backward_weights(h, x, dy, dW, db, N, workspace, (hipStream_t)stream);
    return e == hipSuccess ? EQLIN_OK : hip_fail(e, "eqlin_backward_weights launch");
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
    return snprintf(buf, len,
                    "%s%d C_in=%d C_out=%d %s | forward: %s | expanded: %s | backward data: %s | backward weights: %s",
                    h->d4 ? "D" : "G=", h->d4 ? 4 : h->G, h->C_in, h->C_out, h->dtype == EQLIN_BF16 ? "bf16" : h->dtype == EQLIN_F16 ? "f16" : "f32", h->fwd.name,
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
