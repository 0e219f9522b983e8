// conv.hip -- the p4 group convolution with k x k spatial kernels, run as an EQ-Linear layer over
// gathered channels.
//
// Flash EQ-Linear page ("Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise
// Discrete Fourier Transform", gist.science explainer), "Limitaciones y Trabajo Futuro": carrying the
// principle over to other equivariant operators, equivariant convolutions among them. The layer is the
// rotation-group convolution on the square pixel grid whose 1 x 1 case is the EQ-Linear layer:
//
//     y[p, o, h] = b[o] + sum_{i, g} sum_{delta} psi[o, i, (h - g) mod 4, R^-h delta] x[p + delta, i, g]
//
// (R(dy, dx) = (-dx, dy) the quarter turn of an offset, |dy|, |dx| <= r = k / 2, zero padding).
//
// Reduction to the layer. The nonzero offsets fall into orbits {R^j delta0} of four under R (one
// representative per orbit in the quadrant dy in [1, r], dx in [0, r]); the centre is its own orbit.
// For an orbit and an input channel i, the four rotated neighbours' 16 values x[p + R^j delta0, i, g]
// split into four gathered channels u = 0..3 with group index g:
//
//     xt[(i, delta0, u), g] = x[p + R^(g - u) delta0, i, g],
//
// and the term of the sum that reads them is W'[o, (i, delta0, u), (h - g) mod 4] xt[(i, delta0, u), g]
// with W'[o, (i, delta0, u), m] = psi[o, i, m, R^-(m + u) delta0]: the weight over (h, g) depends on
// h - g alone, so the convolution is an EQ-Linear layer over C_in * k^2 gathered channels (the centre
// orbit contributes x[p, i, g] itself with W'[o, (i, centre), m] = psi[o, i, m, 0]), which the group
// DFT diagonalises as before. The forward kernels gather xt while loading x (CONV in fwd_big.hip):
// sample g of a gathered channel is sample g of the pixel at offset R^(g - u) delta0, so the gather is
// only a choice of load address per sample, never a shuffle of loaded values.
//
// Gathered channel order (the K axis the kernels stream in stages of 16 channels): stage s < nib
// (nib = C_in / 16) is the centre, channels i = 16 s .. 16 s + 15; stage nib + t, t = 4 (q nib + ib) + u,
// is orbit q, channels 16 ib .. 16 ib + 15, gathered channel u.
#include <algorithm>
#include <vector>

#include "device_common.h"
#include "eqlin_internal.h"

namespace eqlin {

// quarter turns of an offset
__host__ __device__ inline void turn(int &dy, int &dx, int m) {
    m &= 3;
    for (int t = 0; t < m; ++t) {
        const int ny = -dx;
        dx = dy;
        dy = ny;
    }
}

// orbit q's representative: the quadrant dy in [1, r], dx in [0, r], row-major
__host__ __device__ inline void orbit_rep(int r, int q, int &dy, int &dx) {
    dy = q / (r + 1) + 1;
    dx = q % (r + 1);
}

// stage s -> (orbit q or -1 for the centre, channel block ib, gathered channel u)
__host__ __device__ inline void conv_stage(int s, int nib, int &q, int &ib, int &u) {
    if (s < nib) {
        q = -1;
        ib = s;
        u = 0;
        return;
    }
    const int t = s - nib;
    u = t & 3;
    ib = (t >> 2) % nib;
    q = (t >> 2) / nib;
}

// W'[o][c'][m] (c' the gathered channel, order above) from psi[o][i][m][ky][kx]: a gather, exact.
// T: the 2- or 4-byte element (the value is copied bit for bit).
template <typename T>
__global__ __launch_bounds__(256) void k_conv_weight(const T *__restrict__ psi, int C_out, int C_in, int k,
                                                     T *__restrict__ wp) {
    const int cg = C_in * k * k, nib = C_in / 16, r = k / 2;
    const int64_t total = (int64_t)C_out * cg * 4;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int m = (int)(e & 3);
        const int c = (int)((e >> 2) % cg);
        const int o = (int)((e >> 2) / cg);
        int q, ib, u;
        conv_stage(c / 16, nib, q, ib, u);
        const int i = ib * 16 + c % 16;
        int fy = 0, fx = 0;
        if (q >= 0) {
            orbit_rep(r, q, fy, fx);
            turn(fy, fx, -(m + u));  // R^-(m + u) delta0
        }
        wp[e] = psi[((((int64_t)o * C_in + i) * 4 + m) * k + fy + r) * k + fx + r];
    }
}

hipError_t launch_conv_weight(const void *psi, int elem_bytes, int C_out, int C_in, int k, void *wp, hipStream_t s) {
    const int64_t total = (int64_t)C_out * C_in * k * k * 4;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(k_conv_weight<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t *)psi, C_out, C_in, k,
                           (uint16_t *)wp);
    else
        hipLaunchKernelGGL(k_conv_weight<float>, dim3(blocks), dim3(256), 0, s, (const float *)psi, C_out, C_in, k,
                           (float *)wp);
    return hipGetLastError();
}

// The kernels' per-stage source table: .x the stage's byte offset into a pixel's row of x (channel
// block ib: 16 channels x 4 samples x elem bytes), bytes g of .y / .z the pixel offset (dy, dx) that
// sample g is read from, R^(g - u) delta0 (0 for the centre). Stages past the real ones (padding to
// the kernels' stage multiple) repeat the first centre stage; their weights are zero.
std::vector<uint4> conv_stage_table(int C_in, int k, int elem_bytes, int n_stages) {
    const int nib = C_in / 16, r = k / 2, real = nib * k * k;
    std::vector<uint4> tab((size_t)n_stages);
    for (int s = 0; s < n_stages; ++s) {
        int q, ib, u;
        conv_stage(s < real ? s : 0, nib, q, ib, u);
        uint32_t ys = 0, xs = 0;
        for (int g = 0; g < 4; ++g) {
            int dy = 0, dx = 0;
            if (q >= 0) {
                orbit_rep(r, q, dy, dx);
                turn(dy, dx, g - u);
            }
            ys |= (uint32_t)(uint8_t)(int8_t)dy << (8 * g);
            xs |= (uint32_t)(uint8_t)(int8_t)dx << (8 * g);
        }
        tab[s] = make_uint4((uint32_t)(ib * 16 * 4 * elem_bytes), ys, xs, 0u);
    }
    return tab;
}

}  // namespace eqlin
