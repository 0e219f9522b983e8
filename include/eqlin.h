/*
 * eqlin.h -- C ABI of the MI355X (gfx950) EQ-Linear library, libeqlin.so: the spectral forward, its
 * dense comparator, the fused-activation variants and the gradients.
 *
 * The operation. A cyclic-group equivariant linear layer (EQ-Linear) over tokens shaped
 * [channels, G], G the order of the rotation group (p4: G = 4; p8: G = 8; G = 1 and 2 also work):
 *
 *     y[n, o, h] = b[o] + sum_{i < C_in} sum_{g < G} W[o, i, (h - g) mod G] * x[n, i, g]
 *
 * Source: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
 * Transform" (explainer page, gist.science/es/paper/2607.21271). Section "Percepción Central": the
 * layer's unrolled weight is group-circulant (cyclic shifts of one parameter set), i.e. a circular
 * convolution along the group axis composed with a channel linear map. Section "Enfoque
 * Algorítmico": a DFT along the group axis turns the convolution into independent per-frequency
 * channel products, and conjugate symmetry leaves only k = 0..G/2 to compute. The bias b[o] is
 * broadcast over h (the pages name no bias; this is the only bias that keeps the layer equivariant).
 *
 * Layouts (row-major, contiguous, group index innermost):
 *   x[N][C_in][G], y[N][C_out][G], W[C_out][C_in][G], b[C_out].
 * Element type: EQLIN_BF16 (bfloat16 in and out, fp32 transforms and accumulation, one
 * round-to-nearest-even at the store), EQLIN_F16 (the same with IEEE half precision: the page's FP16
 * kernels, "Implementación"; values beyond +-65504 overflow to infinity) or EQLIN_F32 (fp32 throughout).
 *
 * Memory. Every data pointer is a DEVICE pointer on the current HIP device. The caller owns x, W, b
 * and y; the handle owns the spectral weights (and the unrolled weight, when asked for) until
 * eqlin_destroy. x, y and W must be 16-byte aligned; b (optional) 4-byte aligned for f32, 2-byte
 * for bf16 and fp16. x and y must not overlap.
 *
 * Streams. All device work is enqueued on `stream` (NULL = the legacy default stream) and nothing
 * synchronises the host, except where an entry point says otherwise. A handle is immutable after
 * eqlin_prepare_weights returns; forwards on several streams may share it once the preparing stream
 * has passed the prepare (the caller orders that).
 *
 * Errors. Arguments are checked on the host before anything is enqueued; a bad argument returns a
 * status code and enqueues nothing. A failed HIP call returns EQLIN_ERR_HIP. Nothing throws or aborts
 * across this ABI. eqlin_last_error() gives a message for the calling thread's most recent failure.
 * A device-side fault would surface at the caller's next synchronisation, as for any HIP kernel.
 */
#ifndef EQLIN_H
#define EQLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t (HIP defines hipStream_t as struct ihipStream_t*). */
struct ihipStream_t;
typedef struct ihipStream_t *eqlin_stream_t;

/* Opaque plan: spectral weights + kernel choice for one weight set. Owned by the library. */
typedef struct eqlin_plan *eqlin_handle_t;

typedef enum {
    EQLIN_OK = 0,
    EQLIN_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, G not in {1,2,4,8}, ... */
    EQLIN_ERR_UNSUPPORTED = 2,   /* valid layer the kernels do not cover (bf16/fp16 with C_in % 8 != 0;
                                    C_out * G or C_in * G above 2^20) */
    EQLIN_ERR_OUT_OF_MEMORY = 3, /* device allocation failed */
    EQLIN_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} eqlin_status_t;

typedef enum { EQLIN_F32 = 0, EQLIN_BF16 = 1, EQLIN_F16 = 2 } eqlin_dtype_t;

/* Element-wise activation applied to the layer's output (after the bias, before the store's single
 * rounding). EQLIN_ACT_GELU is GELU in its exact form, y * Phi(y) = y/2 (1 + erf(y / sqrt 2)): the
 * activation between the two EQ-Linear layers of a transformer MLP block (EQ-ViT / EQ-Swin,
 * "Resultados Experimentales", network level; GELU as the ViT-on-mobile page names it, "El Efecto
 * GELU"). Acting on each value alone, it keeps the layer equivariant. */
typedef enum { EQLIN_ACT_NONE = 0, EQLIN_ACT_GELU = 1 } eqlin_act_t;

/* flags for eqlin_prepare_weights */
#define EQLIN_PREPARE_EXPANDED 1u /* also build the unrolled weight for eqlin_forward_expanded */
#define EQLIN_PREPARE_BACKWARD 2u /* also build the data-gradient weights for eqlin_backward_data */
#define EQLIN_PREPARE_D4 4u       /* the group is the dihedral group D4 (needs G = 8), see below */
#define EQLIN_PREPARE_FIXED_KERNEL 8u /* one forward kernel for every batch size (see eqlin_forward) */

/*
 * The dihedral group D4 (EQLIN_PREPARE_D4). The p4 rotations plus the mirror images: the reflection
 * groups the Flash EQ-Linear page names as the method's next generalisation ("Limitaciones y Trabajo
 * Futuro"; reflection symmetry also in the EQ-VMamba page's section 5.2). The group axis has 8
 * entries, element e = a + 4b being r^a s^b (rotation by 90a degrees after the mirror s when b = 1;
 * s r = r^-1 s), and the layer is the group convolution
 *
 *     y[n, o, h] = b[o] + sum_{i, g} W[o, i, g^-1 h] * x[n, i, g]
 *
 * (the cyclic layer is the case g^-1 h = h - g mod G). The kernels use D4's Fourier transform over its
 * irreducible representations (four characters and one 2-D representation): per channel pair four
 * real products and one 2 x 2 matrix product, twelve real products against 64 for the unrolled block.
 * Every entry point takes a D4 handle.
 */

/*
 * eqlin_prepare_weights -- W -> spectral weights, once per weight set.
 *
 * Computes What[o, i, k] = sum_d W[o, i, d] exp(-2 pi i d k / G) for k = 0..G/2 (the DFT along the
 * group axis, same sign as the input's, no conjugate; "Enfoque Algorítmico") in fp32 and stores it
 * as G real planes in the layout the forward kernels read (bf16 / fp16 for EQLIN_BF16 / EQLIN_F16). It takes the very
 * W a naive EQ-Linear uses: the method is a drop-in replacement that needs no retraining
 * ("Implementación": training-free, plug-and-play).
 *
 *   W      device [C_out][C_in][G] of `dtype`; read once, stream-ordered. The caller may free or
 *          overwrite W once `stream` has passed this call.
 *   C_out, C_in >= 1; G in {1, 2, 4, 8}; C_out * G and C_in * G <= 2^20 (else UNSUPPORTED).
 *          EQLIN_BF16 and EQLIN_F16 need C_in % 8 == 0 (else UNSUPPORTED).
 *   flags  EQLIN_PREPARE_EXPANDED to also build the unrolled weight for eqlin_forward_expanded;
 *          EQLIN_PREPARE_BACKWARD to also build the weights of eqlin_backward_data (bf16/fp16 then
 *          also needs C_out % 8 == 0, else UNSUPPORTED); EQLIN_PREPARE_D4 for the dihedral group
 *          (G must be 8, else INVALID_ARG; W's group axis in the element order above);
 *          EQLIN_PREPARE_FIXED_KERNEL to run one forward kernel whatever the batch size (below).
 *   out    receives the new handle (set to NULL on failure).
 * Allocates device memory (hipMalloc) on the current device; synchronises nothing.
 */
eqlin_status_t eqlin_prepare_weights(const void *W, int C_out, int C_in, int G, eqlin_dtype_t dtype,
                                     unsigned flags, eqlin_stream_t stream, eqlin_handle_t *out);

/*
 * eqlin_forward -- the spectral forward, one fused kernel: load a token tile (G contiguous), group
 * DFT in registers, per-frequency channel products on the matrix cores (bf16 or fp16 in, fp32 accumulate;
 * a complex frequency as four real products), inverse DFT + bias in registers, one store
 * ("Enfoque Algorítmico"; "Implementación": fused dataflow with no intermediate global writes).
 *
 *   h      handle from eqlin_prepare_weights.
 *   x      device [N][C_in][G]; b device [C_out] or NULL (no bias); y device [N][C_out][G].
 *   N      >= 0 tokens; N == 0 enqueues nothing and returns EQLIN_OK.
 * Must be called with the handle's device current. Asynchronous on `stream`; allocates nothing.
 * Kernel by batch size: a wide p4 layer (C_in <= 256, C_out >= 256) runs the resident-planes kernel,
 * which gives each compute unit one token tile and every output, while N exceeds 32 tokens per compute
 * unit; at smaller N it runs the large-channel kernel, which splits the outputs over the compute units
 * instead (the same prepared weights; eqlin_describe names both). The two sum in different orders, so
 * results can differ in the last bits between batch sizes on either side of that point; a handle
 * prepared with EQLIN_PREPARE_FIXED_KERNEL always runs the first (eqlin_backward_data, which runs
 * these kernels on the transposed weight, follows the same rule).
 */
eqlin_status_t eqlin_forward(eqlin_handle_t h, const void *x, const void *b, void *y, int64_t N,
                             eqlin_stream_t stream);

/*
 * eqlin_forward_expanded -- the naive comparator: y_flat = x_flat E^T + b_exp with the unrolled
 * block-circulant weight E[o*G+h][i*G+g] = W[o, i, (h-g) mod G] and b_exp[o*G+h] = b[o], as one
 * dense matrix product on the matrix cores ("Declaración del Problema": replicate the shared
 * weights into a dense matrix, then multiply densely). Same arguments and rules as eqlin_forward;
 * needs a handle prepared with EQLIN_PREPARE_EXPANDED (else EQLIN_ERR_INVALID_ARG).
 */
eqlin_status_t eqlin_forward_expanded(eqlin_handle_t h, const void *x, const void *b, void *y,
                                      int64_t N, eqlin_stream_t stream);

/*
 * eqlin_forward_act, eqlin_forward_expanded_act -- eqlin_forward and eqlin_forward_expanded with
 * `act` applied to every output value in the kernel's epilogue (no extra pass over y):
 *     y[n, o, h] = act(b[o] + sum_{i, g} W[o, i, (h - g) mod G] * x[n, i, g]).
 * act is an eqlin_act_t (else EQLIN_ERR_INVALID_ARG); EQLIN_ACT_NONE is eqlin_forward itself. Same
 * arguments, rules and handle requirements as the entry points they extend.
 */
eqlin_status_t eqlin_forward_act(eqlin_handle_t h, const void *x, const void *b, void *y, int64_t N, int act,
                                 eqlin_stream_t stream);
eqlin_status_t eqlin_forward_expanded_act(eqlin_handle_t h, const void *x, const void *b, void *y, int64_t N,
                                          int act, eqlin_stream_t stream);

/*
 * eqlin_backward_data -- the data gradient of the layer ("Implementación": the operator has forward
 * and backward passes; "Resultados Experimentales": backward speedups):
 *
 *     dx[n, i, g] = sum_{o < C_out} sum_{h < G} W[o, i, (h - g) mod G] * dy[n, o, h]
 *
 * i.e. the transpose of the unrolled product. It is itself an EQ-Linear layer -- with the weight
 * Wt[i, o, d] = W[o, i, (-d) mod G] (C_in and C_out swapped, group axis reversed; the DFT of Wt is
 * the conjugate of the DFT of W) and no bias -- and runs on the forward kernels.
 *   dy     device [N][C_out][G] of the handle's dtype; dx device [N][C_in][G] (same type).
 *   N      >= 0; N == 0 enqueues nothing.
 * Needs a handle prepared with EQLIN_PREPARE_BACKWARD (else EQLIN_ERR_INVALID_ARG). Same alignment,
 * overlap, device and stream rules as eqlin_forward; allocates nothing.
 */
eqlin_status_t eqlin_backward_data(eqlin_handle_t h, const void *dy, void *dx, int64_t N, eqlin_stream_t stream);

/*
 * eqlin_backward_data_expanded -- the naive comparator of eqlin_backward_data: dx_flat = dy_flat E, the
 * dense product with the unrolled weight E[o*G+h][i*G+g] = W[o, i, (h-g) mod G] (the gradient of the
 * replicate-then-multiply layer of "Declaración del Problema"), on the matrix cores as one G = 1
 * product over E^T. Same arguments and rules as eqlin_backward_data; needs a handle prepared with both
 * EQLIN_PREPARE_BACKWARD and EQLIN_PREPARE_EXPANDED (else EQLIN_ERR_INVALID_ARG). Allocates nothing.
 */
eqlin_status_t eqlin_backward_data_expanded(eqlin_handle_t h, const void *dy, void *dx, int64_t N,
                                            eqlin_stream_t stream);

/*
 * eqlin_backward_weights -- the weight and bias gradients (same passages):
 *
 *     dW[o, i, d] = sum_n sum_{h < G} dy[n, o, h] * x[n, i, (h - d) mod G],   db[o] = sum_{n, h} dy[n, o, h]
 *
 * computed per frequency as C_k = sum_n DY_k conj(X_k) (the same group DFT as the forward) followed
 * by the inverse DFT (D4: its irreps' adjoint products and inverse). bf16 or fp16 with G = 4, 8 or D4:
 * x and dy are transformed into half-type planes, multiplied on the matrix cores with fp32
 * accumulation over token splits, and the splits summed in fp32; small channel counts (C_in * C_out * G
 * up to about 40960) run one fused matrix-core pass per token range instead; other cases (fp32,
 * G = 1 or 2) evaluate the definition in fp32 on the vector ALU.
 *   x      device [N][C_in][G], dy device [N][C_out][G], both of the handle's dtype.
 *   dW     device float [C_out][C_in][G] (overwritten); db device float [C_out] or NULL (overwritten).
 *   workspace, workspace_bytes: device scratch of at least eqlin_backward_weights_workspace(h, N)
 *          bytes, 256-byte aligned (may be NULL when that is 0); owned by the caller, not kept.
 *   N      >= 0; N == 0 writes zeros.
 * Any handle (no prepare flag needed). Asynchronous on `stream`; allocates nothing. Calls sharing a
 * workspace must not overlap.
 */
size_t eqlin_backward_weights_workspace(eqlin_handle_t h, int64_t N);
eqlin_status_t eqlin_backward_weights(eqlin_handle_t h, const void *x, const void *dy, float *dW, float *db,
                                      int64_t N, void *workspace, size_t workspace_bytes, eqlin_stream_t stream);

/*
 * eqlin_backward_weights_static -- eqlin_backward_weights with no workspace argument and no device
 * allocation, for callers that cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The same gradients from the same kernels, with the same arguments
 * (less the workspace), alignment, device and stream rules.
 *
 * Its scratch is a static device array of EQLIN_STATIC_SCRATCH_BYTES (64 MiB) inside the library:
 * each device holds its own copy, from when the library first runs there until the process ends. Its
 * device address is looked up once per device, when eqlin_prepare_weights (or else the first call of
 * this function) runs there. A call whose scratch need, eqlin_backward_weights_workspace(h, N),
 * exceeds the array returns EQLIN_ERR_UNSUPPORTED and enqueues nothing. (The fused small-channel pass
 * keeps one partial spectrum per compute unit, so its need does not grow with N: the p4 96 x 96 and
 * p8 64 x 64 layers fit at any token count. The large-channel passes hold transformed copies of x and
 * dy, so they fit only small batches, e.g. about 1000 tokens at p4 192 -> 768.)
 *
 * Calls no hipMalloc, hipFree or other allocating routine. All calls on one device share its array,
 * which keeps the last call's contents; no pass reads scratch that the same call has not written, so
 * nothing needs to start at zero. Calls that overlap on one device (several streams, or several
 * threads without an order between them) race on the array: the caller must order them.
 */
#define EQLIN_STATIC_SCRATCH_BYTES (64u << 20)
eqlin_status_t eqlin_backward_weights_static(eqlin_handle_t h, const void *x, const void *dy, float *dW, float *db,
                                             int64_t N, eqlin_stream_t stream);

/*
 * The p4 group convolution with k x k spatial kernels -- the equivariant convolutions the Flash
 * EQ-Linear page names among the operators the method extends to ("Limitaciones y Trabajo Futuro"):
 *
 *     y[b, p, o, h] = bias[o] + sum_{i, g} sum_{delta} psi[o, i, (h - g) mod 4, R^-h delta] * x[b, p + delta, i, g]
 *
 * over the pixels p = (row, column) of H x W images, offsets delta = (dy, dx) with |dy|, |dx| <= k / 2,
 * R(dy, dx) = (-dx, dy) the quarter turn of an offset (the filter turns with the output orientation h),
 * pixels outside the image reading as zero. Turning the image a quarter and shifting the group axis by
 * one commutes with it; k = 1 is the EQ-Linear layer (W = psi[:, :, :, 0, 0]). The library runs it as an
 * EQ-Linear layer over C_in * k * k gathered channels -- for each orbit {R^j delta0} of offsets,
 * gathered channel (i, delta0, u) holds sample g of pixel p + R^(g - u) delta0 -- whose weight
 * psi[o, i, m, R^-(m + u) delta0] depends on h - g alone, so the group DFT diagonalises it; the gather
 * happens while x is loaded, in the layer's own spectral kernel: the four gathered channels u of one
 * (orbit, 16-channel block) read the same four neighbour rows, each loaded once.
 *
 * Layouts (row-major, contiguous): x[B][H][W][C_in][4], y[B][H][W][C_out][4] (one token per pixel, the
 * layer's rows), psi[C_out][C_in][4][k][k] (psi[o][i][d][ky][kx]: the filter at offset
 * (ky - k/2, kx - k/2)), bias[C_out]. Element type EQLIN_BF16 or EQLIN_F16 (fp32 transforms and
 * accumulation, one rounding of y).
 *
 * eqlin_prepare_conv_weights -- psi -> the gathered layer's spectral weights (and, with
 * EQLIN_PREPARE_EXPANDED, its unrolled weight for eqlin_conv_forward_expanded).
 *   G must be 4 and k odd in 1..15 (else EQLIN_ERR_INVALID_ARG); C_in % 16 == 0, C_in <= 8192,
 *   C_out % 8 == 0, dtype EQLIN_BF16 or EQLIN_F16 and flags within EQLIN_PREPARE_EXPANDED (else
 *   EQLIN_ERR_UNSUPPORTED).
 *   Allocates device memory; synchronises nothing; psi may be freed once `stream` has passed the call.
 *   The handle serves eqlin_conv_forward(_expanded), eqlin_describe, eqlin_export_* (the gathered
 *   layer's weights: C_in * k * k input channels, plus zero-weight filling channels up to a multiple of
 *   64 centre channels when C_in / 16 is not a multiple of 4) and eqlin_destroy; the layer's entry
 *   points reject it.
 * eqlin_conv_forward -- y from x for B images of H x W pixels (B, H, W >= 0; an empty batch enqueues
 *   nothing). bias may be NULL. B * H * W * C_in * 8 must stay below 2^31 (x is addressed with 32-bit
 *   offsets; else EQLIN_ERR_UNSUPPORTED). Alignment, overlap, device and stream rules as eqlin_forward;
 *   allocates nothing.
 * eqlin_conv_forward_expanded -- the same through the unrolled gathered layer, one dense product on the
 *   matrix cores (the comparator); needs EQLIN_PREPARE_EXPANDED (else EQLIN_ERR_INVALID_ARG).
 */
eqlin_status_t eqlin_prepare_conv_weights(const void *psi, int C_out, int C_in, int G, int k, eqlin_dtype_t dtype,
                                          unsigned flags, eqlin_stream_t stream, eqlin_handle_t *out);
eqlin_status_t eqlin_conv_forward(eqlin_handle_t h, const void *x, const void *bias, void *y, int64_t B, int H, int W,
                                  eqlin_stream_t stream);
eqlin_status_t eqlin_conv_forward_expanded(eqlin_handle_t h, const void *x, const void *bias, void *y, int64_t B,
                                           int H, int W, eqlin_stream_t stream);

/* Frees the handle's device memory (hipFree, which synchronises the device). NULL is a no-op. */
eqlin_status_t eqlin_destroy(eqlin_handle_t h);

/*
 * eqlin_export_spectral_weights -- copy the stored spectral weights out, for checking.
 * out: device float [G][C_out][C_in], plane order: k = 0 (real); k = G/2 (real, when G >= 2);
 * then Re and Im of each k = 1..G/2-1 in turn. Values are What itself (the forward's internal
 * 1/G and 2/G scalings are undone exactly), as stored: rounded to the handle's half type for EQLIN_BF16
 * and EQLIN_F16. A D4
 * handle's planes are sum_g W[., ., g] chi_k(g) for its four characters chi_k = 1, (-1)^b, (-1)^a,
 * (-1)^(a+b), then the entries (0,0), (0,1), (1,0), (1,1) of sum_g W[., ., g] rho(g), rho(r^a s^b) =
 * R^a S^b with R = [[0, -1], [1, 0]] and S = diag(1, -1).
 */
eqlin_status_t eqlin_export_spectral_weights(eqlin_handle_t h, float *out, eqlin_stream_t stream);

/*
 * eqlin_export_expanded_weight -- copy the unrolled weight out, for checking.
 * out: device [C_out*G][C_in*G] of the handle's dtype. Needs EQLIN_PREPARE_EXPANDED.
 */
eqlin_status_t eqlin_export_expanded_weight(eqlin_handle_t h, void *out, eqlin_stream_t stream);

/* Writes a one-line description of the kernels the handle dispatches to (for logs and reports).
 * Returns the length it wanted to write (like snprintf); buf may be NULL when len == 0. */
int eqlin_describe(eqlin_handle_t h, char *buf, size_t len);

/* Static text for a status code. */
const char *eqlin_status_string(eqlin_status_t s);

/* Message for the calling thread's most recent failed call ("" if none). Valid until the thread's
 * next call into the library. */
const char *eqlin_last_error(void);

/* Library version string, "major.minor.patch". */
const char *eqlin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EQLIN_H */
