// act.h -- element-wise activations applied in the forward kernels' epilogues, after the inverse
// DFT and the bias and before the single rounding to the output type.
//
// The transformer MLP block the layer is built into (EQ-Linear, GELU, EQ-Linear; "Flash EQ-Linear",
// explainer page, "Resultados Experimentales", network level) returns to the group domain between
// its two layers for the activation. Applied to each value alone, the activation commutes with the
// cyclic shift of the group axis, so it may run on the outputs a lane already holds.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/eqlin.h"

namespace eqlin {

// GELU(v) = v * Phi(v), Phi the standard normal CDF (the activation the ViT-on-mobile page names,
// "El Efecto GELU"; the erf form v * Phi(v), not the tanh approximation). With Q(|v|) = 1 - Phi(|v|), the
// upper tail, GELU(v) = max(v, 0) - |v| * Q(|v|) for either sign of v. Q comes from Abramowitz &
// Stegun's rational approximation 7.1.28 (Hastings): erf(z) = 1 - (1 + a1 z + ... + a6 z^6)^-16 with
// |error| <= 3e-7 for z >= 0, so Q(u) = (1 - erf(u / sqrt 2)) / 2 = (1/2) p(u)^-16, where p has the
// 1/sqrt(2) scaling folded into its coefficients (c_k = a_k / 2^(k/2)). One reciprocal, six fused
// multiply-adds and four squarings, branch-free: the error in GELU is at most 1.5e-7 |v| plus fp32
// rounding, well under a bf16 output's rounding and the fp32 path's tolerance.
__host__ __device__ __forceinline__ float gelu_erf_form(float v) {
    constexpr float c1 = 0.04986734696679053f, c2 = 0.02114100615f, c3 = 0.0032776263241471684f,
                    c4 = 3.8003575e-05f, c5 = 4.889063564344402e-05f, c6 = 5.382975e-06f;
    const float u = fabsf(v);
    float p = fmaf(c6, u, c5);
    p = fmaf(p, u, c4);
    p = fmaf(p, u, c3);
    p = fmaf(p, u, c2);
    p = fmaf(p, u, c1);
    p = fmaf(p, u, 1.0f);
#ifdef __HIP_DEVICE_COMPILE__
    float r = __builtin_amdgcn_rcpf(p);  // 1 ulp; p >= 1
#else
    float r = 1.0f / p;
#endif
    r *= r;  // p^-2
    r *= r;  // p^-4
    r *= r;  // p^-8
    r *= r;  // p^-16 = 2 Q(u)
    // |v| clamped in the tail's factor only: at |v| = inf the tail is 0 * finite (GELU(inf) = inf,
    // GELU(-inf) = 0), while a NaN still reaches the result through r
    return fmaf(-0.5f * fminf(u, 64.0f), r, fmaxf(v, 0.0f));
}

// out[j] <- GELU(out[j]) for the M values a lane is about to store, when the kernel is the GELU
// instance (a template flag, so the plain forward carries none of its code or registers).
template <bool GELU, int M>
__device__ __forceinline__ void apply_act(float (&out)[M]) {
    if constexpr (GELU) {
#pragma unroll
        for (int j = 0; j < M; ++j) out[j] = gelu_erf_form(out[j]);
    }
}

}  // namespace eqlin
