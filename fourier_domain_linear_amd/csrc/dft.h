// dft.h -- G-point real DFT butterflies along the group axis (G in {1, 2, 4, 8}), in registers.
//
// Flash EQ-Linear page ("Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise
// Discrete Fourier Transform", gist.science explainer), section "Enfoque Algorítmico": a DFT along
// the group axis turns the group convolution into a pointwise product per frequency, and because x
// and W are real only k = 0..G/2 is kept (conjugate symmetry). Section "Especialización para el Grupo
// de Rotación p4": for G = 4 both transforms need only additions, subtractions and power-of-two
// scalings. For G = 8 (the p8 extension) the odd frequencies add the twiddle sqrt(2)/2.
//
// Plane order (G real planes per channel, used for x, W and the products alike):
//   p = 0          : Re X_0                (real)
//   p = 1          : Re X_{G/2}            (real; G >= 2)
//   p = 2k, 2k + 1 : Re X_k, Im X_k        (k = 1 .. G/2 - 1)
// with X_k = sum_g x_g exp(-2 pi i g k / G).
//
// Inverse. With Y_k = What_k X_k, the real inverse over the half spectrum is
//   y_h = (1/G) [ Y_0 + (-1)^h Y_{G/2} + 2 sum_{k=1}^{G/2-1} Re(Y_k exp(+2 pi i h k / G)) ].
// The library folds the 1/G (real planes) and 2/G (complex planes) factors into the stored weight
// planes (exact: powers of two), so inverse_planes() below takes the already-scaled products and is
// additions only for G <= 4. plane_scale() gives those factors.
//
// This header is plain C++ so the host test suite can compile it and check it against numpy's FFT.
#pragma once

#if defined(__HIPCC__)
#define EQLIN_HD __host__ __device__ __forceinline__
#else
#define EQLIN_HD inline
#endif

namespace eqlin {

constexpr float kSqrtHalf = 0.70710678118654752440f;

// Scale folded into weight plane p (see above).
EQLIN_HD float plane_scale(int G, int p) {
    if (G == 1) return 1.0f;
    return (p < 2) ? 1.0f / (float)G : 2.0f / (float)G;
}

// Forward: v[0..G-1] (group samples) -> P[0..G-1] (planes, order above).
template <int G>
EQLIN_HD void forward_planes(const float *v, float *P) {
    if constexpr (G == 1) {
        P[0] = v[0];
    } else if constexpr (G == 2) {
        P[0] = v[0] + v[1];
        P[1] = v[0] - v[1];
    } else if constexpr (G == 4) {
        const float a = v[0] + v[2], c = v[0] - v[2];
        const float b = v[1] + v[3], d = v[1] - v[3];
        P[0] = a + b;  // X0
        P[1] = a - b;  // X2
        P[2] = c;      // Re X1 = v0 - v2
        P[3] = -d;     // Im X1 = v3 - v1
    } else {
        static_assert(G == 8, "G must be 1, 2, 4 or 8");
        const float a0 = v[0] + v[4], a1 = v[1] + v[5], a2 = v[2] + v[6], a3 = v[3] + v[7];
        const float d0 = v[0] - v[4], d1 = v[1] - v[5], d2 = v[2] - v[6], d3 = v[3] - v[7];
        const float e0 = a0 + a2, e1 = a1 + a3, f0 = a0 - a2;
        const float t1 = d1 - d3, t2 = d1 + d3;
        // the signs sit on the operands (exactly equal to negating the results; saves an instruction)
        P[0] = e0 + e1;                      // X0
        P[1] = e0 - e1;                      // X4
        P[2] = d0 + kSqrtHalf * t1;          // Re X1
        P[3] = -kSqrtHalf * t2 - d2;         // Im X1
        P[4] = f0;                           // Re X2
        P[5] = a3 - a1;                      // Im X2
        P[6] = d0 - kSqrtHalf * t1;          // Re X3
        P[7] = d2 - kSqrtHalf * t2;          // Im X3
    }
}

// Inverse: scaled products Y[0..G-1] (plane order) -> y[0..G-1] (group samples).
template <int G>
EQLIN_HD void inverse_planes(const float *Y, float *y) {
    if constexpr (G == 1) {
        y[0] = Y[0];
    } else if constexpr (G == 2) {
        y[0] = Y[0] + Y[1];
        y[1] = Y[0] - Y[1];
    } else if constexpr (G == 4) {
        const float u = Y[0] + Y[1], w = Y[0] - Y[1];
        y[0] = u + Y[2];
        y[1] = w - Y[3];
        y[2] = u - Y[2];
        y[3] = w + Y[3];
    } else {
        static_assert(G == 8, "G must be 1, 2, 4 or 8");
        // even part (period 4 in h): Y0, Y4, Y2
        const float u = Y[0] + Y[1], w = Y[0] - Y[1];
        const float E0 = u + Y[4], E1 = w - Y[5], E2 = u - Y[4], E3 = w + Y[5];
        // odd part (antiperiodic, period 8): Y1, Y3
        const float r1 = Y[2], i1 = Y[3], r3 = Y[6], i3 = Y[7];
        const float O0 = r1 + r3;
        const float O1 = kSqrtHalf * ((r1 - i1) - (r3 + i3));
        const float O2 = i3 - i1;
        const float O3 = kSqrtHalf * ((r3 - i3) - (r1 + i1));
        y[0] = E0 + O0; y[4] = E0 - O0;
        y[1] = E1 + O1; y[5] = E1 - O1;
        y[2] = E2 + O2; y[6] = E2 - O2;
        y[3] = E3 + O3; y[7] = E3 - O3;
    }
}

// ---- The dihedral group D4 (p4's rotations plus reflections; order 8) ----
//
// The Flash EQ-Linear page names reflection groups as the method's next generalisation
// ("Limitaciones y Trabajo Futuro"). The layer is the group convolution y(h) = sum_g W(g^-1 h) x(g).
// Element e = a + 4b is r^a s^b (rotation by 90a degrees after the mirror s when b = 1; s r = r^-1 s).
// Its Fourier transform F(rho) = sum_g f(g) rho(g) runs over the irreducible representations: four
// characters (1, (-1)^b, (-1)^a, (-1)^(a+b)) and the 2-D one rho(r^a s^b) = R^a S^b with R the
// 90-degree rotation [[0, -1], [1, 0]] and S = diag(1, -1). The layer becomes, per irrep and channel
// pair, Y(rho) = X(rho) W(rho): four real products for the characters and a 2 x 2 matrix product
// (eight real products) for rho -- twelve in all, against 64 for the unrolled 8 x 8 block.
//
// Plane order: P0..P3 the characters' values, P4..P7 the entries (0,0), (0,1), (1,0), (1,1) of F(rho).
// All coefficients are 0 or +-1. Inverse (Schur orthogonality):
//   f(g) = (1/8) sum_k chi_k(g) F_k + (2/8) sum_{jk} rho(g)_jk F(rho)_jk,
// with the 1/8 and 2/8 folded into the stored weight planes (plane_scale_d4), as for the cyclic case.
EQLIN_HD float plane_scale_d4(int p) { return p < 4 ? 0.125f : 0.25f; }

EQLIN_HD void forward_planes_d4(const float *v, float *P) {
    // rotations v0..v3 and reflections v4..v7, each split into even/odd rotation parts
    const float A = v[0] + v[2], B = v[1] + v[3], C = v[0] - v[2], D = v[1] - v[3];
    const float A2 = v[4] + v[6], B2 = v[5] + v[7], C2 = v[4] - v[6], D2 = v[5] - v[7];
    const float s0 = A + B, s1 = A2 + B2, t0 = A - B, t1 = A2 - B2;
    P[0] = s0 + s1;  // trivial
    P[1] = s0 - s1;  // (-1)^b
    P[2] = t0 + t1;  // (-1)^a
    P[3] = t0 - t1;  // (-1)^(a+b)
    P[4] = C + C2;   // rho_00 = v0 - v2 + v4 - v6
    P[5] = D2 - D;   // rho_01 = -v1 + v3 + v5 - v7
    P[6] = D + D2;   // rho_10 = v1 - v3 + v5 - v7
    P[7] = C - C2;   // rho_11 = v0 - v2 - v4 + v6
}

EQLIN_HD void inverse_planes_d4(const float *Y, float *y) {
    const float p = Y[0] + Y[1], m = Y[0] - Y[1], q = Y[2] + Y[3], n = Y[2] - Y[3];
    const float e0 = p + q, e1 = p - q, e2 = m + n, e3 = m - n;  // characters at (b, a mod 2)
    const float m0 = Y[4] + Y[7], m1 = Y[6] - Y[5];               // trace terms, rotations
    const float n0 = Y[4] - Y[7], n1 = Y[5] + Y[6];               // trace terms, reflections
    y[0] = e0 + m0; y[2] = e0 - m0;
    y[1] = e1 + m1; y[3] = e1 - m1;
    y[4] = e2 + n0; y[6] = e2 - n0;
    y[5] = e3 + n1; y[7] = e3 - n1;
}

// The group's own transform for kernels templated on (G, D4); D4 requires G = 8.
template <int G, bool D4>
EQLIN_HD void group_forward(const float *v, float *P) {
    if constexpr (D4) {
        static_assert(G == 8, "D4 has order 8");
        forward_planes_d4(v, P);
    } else {
        forward_planes<G>(v, P);
    }
}
template <int G, bool D4>
EQLIN_HD void group_inverse(const float *Y, float *y) {
    if constexpr (D4) {
        static_assert(G == 8, "D4 has order 8");
        inverse_planes_d4(Y, y);
    } else {
        inverse_planes<G>(Y, y);
    }
}
EQLIN_HD float group_plane_scale(int G, bool d4, int p) { return d4 ? plane_scale_d4(p) : plane_scale(G, p); }

}  // namespace eqlin
