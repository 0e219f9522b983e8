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
// the four gathered channels u of one (orbit, channel block) read the same four rows of x -- the
// block at the four rotated offsets R^m delta0 -- sample g of channel u from row (g - u) mod 4, so
// each row is loaded once and the gather is a choice of 16-bit halves among rows in registers.
//
// Gathered channel order (the K axis the kernels stream in stages of 16 channels, four stages to a
// group that reads the same four 16-channel rows of x): nib = C_in / 16 channel blocks, taken four at
// a time (a quad Q: blocks 4Q .. 4Q + 3). A quad's groups are its centre group, stage u being channel
// block 4Q + u (blocks past nib are zero-weight filling), then for each of its blocks ib the orbit
// groups q = 0 .. n_orb - 1 (n_orb = (k^2 - 1) / 4), stage u the gathered channel u of (q, ib) and
// row m the block at offset R^m delta0. All reads of a block's rows then fall within one quad's
// groups, so the rows that neighbouring token tiles share are still in the L2 when they are re-read.
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

__host__ __device__ inline int centre_groups(int nib) { return (nib + 3) / 4; }

__host__ __device__ inline int gathered(int C_in, int k) {
    const int nib = C_in / 16;
    return 64 * (centre_groups(nib) + (k * k - 1) / 4 * nib);
}

int conv_gathered_channels(int C_in, int k) { return gathered(C_in, k); }

// group T -> (orbit q, or -1 for the centre; channel block ib of an orbit group, or the centre group's
// first block). n_orb: orbits of nonzero offsets.
__host__ __device__ inline void conv_group(int T, int nib, int n_orb, int &q, int &ib) {
    const int per_quad = 1 + 4 * n_orb, Q = T / per_quad, t = T % per_quad;
    if (t == 0) {
        q = -1;
        ib = 4 * Q;
        return;
    }
    q = (t - 1) % n_orb;
    ib = 4 * Q + (t - 1) / n_orb;
}

// W'[o][c'][m] (c' the gathered channel, order above) from psi[o][i][m][ky][kx]: a gather, exact
// (zeros for the filling channels). T: the 2- or 4-byte element (the value is copied bit for bit).
template <typename T>
__global__ __launch_bounds__(256) void k_conv_weight(const T *__restrict__ psi, int C_out, int C_in, int k,
                                                     T *__restrict__ wp) {
    const int cg = gathered(C_in, k), nib = C_in / 16, r = k / 2;
    const int64_t total = (int64_t)C_out * cg * 4;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int m = (int)(e & 3);
        const int c = (int)((e >> 2) % cg);
        const int o = (int)((e >> 2) / cg);
        const int stage = c / 16, u = stage & 3;
        int q, ib;
        conv_group(stage >> 2, nib, (k * k - 1) / 4, q, ib);
        if (q < 0) ib += u;  // centre: stage u is block 4 T + u
        int fy = 0, fx = 0;
        if (q >= 0) {
            orbit_rep(r, q, fy, fx);
            turn(fy, fx, -(m + u));  // R^-(m + u) delta0
        }
        const int i = ib * 16 + c % 16;
        wp[e] = ib < nib ? psi[((((int64_t)o * C_in + i) * 4 + m) * k + fy + r) * k + fx + r] : T(0);
    }
}

hipError_t launch_conv_weight(const void *psi, int elem_bytes, int C_out, int C_in, int k, void *wp, hipStream_t s) {
    const int64_t total = (int64_t)C_out * conv_gathered_channels(C_in, k) * 4;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(k_conv_weight<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t *)psi, C_out, C_in, k,
                           (uint16_t *)wp);
    else
        hipLaunchKernelGGL(k_conv_weight<float>, dim3(blocks), dim3(256), 0, s, (const float *)psi, C_out, C_in, k,
                           (float *)wp);
    return hipGetLastError();
}

// The kernels' per-group source table: row m's byte offset into a pixel's row of x (channel block:
// 16 channels x 4 samples x elem bytes) in 16 bits m of .x, .y, and the pixel offset (dy, dx) it is
// read from in byte m of .z, .w (R^m delta0 for an orbit group, 0 for the centre). Centre filling
// rows re-read the last block (zero weights); groups past the real ones (the stage count is padded)
// repeat the first centre group, their weights zero as well.
std::vector<uint4> conv_group_table(int C_in, int k, int elem_bytes, int n_groups) {
    const int nib = C_in / 16, r = k / 2, real = conv_gathered_channels(C_in, k) / 64;
    std::vector<uint4> tab((size_t)n_groups);
    for (int T = 0; T < n_groups; ++T) {
        int q, ib;
        conv_group(T < real ? T : 0, nib, (k * k - 1) / 4, q, ib);
        uint32_t chan[4], ys = 0, xs = 0;
        for (int m = 0; m < 4; ++m) {
            int dy = 0, dx = 0, blk = ib;
            if (q >= 0) {
                orbit_rep(r, q, dy, dx);
                turn(dy, dx, m);
            } else {
                blk = std::min(ib + m, nib - 1);
            }
            chan[m] = (uint32_t)(blk * 16 * 4 * elem_bytes);
            ys |= (uint32_t)(uint8_t)(int8_t)dy << (8 * m);
            xs |= (uint32_t)(uint8_t)(int8_t)dx << (8 * m);
        }
        tab[T] = make_uint4(chan[0] | chan[1] << 16, chan[2] | chan[3] << 16, ys, xs);
    }
    return tab;
}

}  // namespace eqlin
