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

// GELU in its exact form v * Phi(v) = v/2 * (1 + erf(v / sqrt(2))) (the activation the ViT-on-mobile
// page names, "El Efecto GELU"); erff is the device math library's.
__device__ __forceinline__ float gelu_exact(float v) {
    return 0.5f * v * (1.0f + erff(v * 0.707106781186547524f));
}

// out[j] <- GELU(out[j]) for the M values a lane is about to store, when the kernel is the GELU
// instance (a template flag, so the plain forward carries none of its code or registers).
template <bool GELU, int M>
__device__ __forceinline__ void apply_act(float (&out)[M]) {
    if constexpr (GELU) {
#pragma unroll
        for (int j = 0; j < M; ++j) out[j] = gelu_exact(out[j]);
    }
}

}  // namespace eqlin
