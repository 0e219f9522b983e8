// Host build of the library's group-DFT butterflies (fourier_domain_linear_amd/csrc/dft.h) so the
// CPU test suite can check them against numpy's FFT. Test-only; not part of libeqlin.so.
#include "../../fourier_domain_linear_amd/csrc/dft.h"

extern "C" {
int dft_forward(int G, const float *v, float *P) {
    switch (G) {
        case 1: eqlin::forward_planes<1>(v, P); return 0;
        case 2: eqlin::forward_planes<2>(v, P); return 0;
        case 4: eqlin::forward_planes<4>(v, P); return 0;
        case 8: eqlin::forward_planes<8>(v, P); return 0;
    }
    return -1;
}
int dft_inverse(int G, const float *Y, float *y) {
    switch (G) {
        case 1: eqlin::inverse_planes<1>(Y, y); return 0;
        case 2: eqlin::inverse_planes<2>(Y, y); return 0;
        case 4: eqlin::inverse_planes<4>(Y, y); return 0;
        case 8: eqlin::inverse_planes<8>(Y, y); return 0;
    }
    return -1;
}
float dft_plane_scale(int G, int p) { return eqlin::plane_scale(G, p); }
void d4_forward(const float *v, float *P) { eqlin::forward_planes_d4(v, P); }
void d4_inverse(const float *Y, float *y) { eqlin::inverse_planes_d4(Y, y); }
float d4_plane_scale(int p) { return eqlin::plane_scale_d4(p); }
}
