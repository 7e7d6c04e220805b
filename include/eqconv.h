/*
 * eqconv.h -- C ABI of the MI355X (gfx950) p4 group convolution built on the
 * group-circulant linear layer of eqlin.h.
 *
 * The Flash EQ-Linear technical summary (gist.science 2607.21271, section
 * "Limitations and future work") names the extension of its Fourier route to
 * other equivariant operators, equivariant convolution first, without
 * formulas.  This library takes the p4 group convolution of regular feature
 * maps whose 1 x 1 case is exactly the layer of eqlin.h with T = 4
 * ("Key insight"):
 *
 *   X [N][H][W][C]   channel c'*4 + s   (rotation s = 0..3 fastest)
 *   psi [D'][C'][K][K][4]               (filter tap (a - p, b - p), K = 2p + 1,
 *                                        group offset u)
 *   Y[n, x, d'*4 + r] = sum_{c', s, delta} X[n, x + delta, c'*4 + s]
 *                                          psi[d', c', R^-r delta, (r - s) mod 4]
 *
 * delta runs over the K x K window {-p..p}^2 with zero padding outside the
 * image (output size = input size), and R is the quarter turn of the pixel
 * grid R(di, dj) = (-dj, di) (the turn of numpy.rot90 on the (H, W) axes).
 * Turning the input image by R^g and shifting its rotation index by g turns
 * and shifts the output the same way (p4 equivariance).
 *
 * How it is computed: the taps split into the centre and the quarter-turn
 * orbits {R^m delta_o, m = 0..3} of the others; gathering, per output pixel,
 * the centre values X[x, c'*4 + m] and, per orbit and shift b, the values
 * X[x + R^m delta_o, c'*4 + (m + b) mod 4], turns the convolution into one
 * group-circulant layer (C'K^2 input group channels, D' output group
 * channels) with weight w_lin[d', (c', o, b), u] = psi[d', c', R^-u delta_o,
 * (u - b) mod 4] (centre: psi[d', c', 0, u]) -- each filter entry used once.
 * The forward kernel of eqlin.h runs that layer with the gather done by its
 * loads (no gathered copy in global memory).  dX is the same kind of
 * convolution of dY with psi'[c', d', delta, v] = psi[d', c', -R^v delta,
 * -v mod 4]; the filter gradient is the layer's dw, gathered the same way.
 *
 * Conventions (as eqlin.h unless stated):
 *   - dtype EQLIN_F32 or EQLIN_F16 with the arithmetic of eqlin.h; dpsi is
 *     float32 for both.
 *   - C, D: positive multiples of 4; C' = C/4 and D' = D/4 must be multiples
 *     of 4 (EQLIN_F32) or 8 (EQLIN_F16), else EQLIN_ENOTSUP.
 *   - K: odd, 1 <= K <= 15, else EQLIN_ENOTSUP (K <= 0 or even: EQLIN_EINVAL).
 *   - N, H, W >= 0; N*H*W == 0 is an empty batch (forward and dX enqueue
 *     nothing; dpsi is written as zeros).  The maps a launch gathers from (X
 *     for the forward and for dpsi, dY for dX) must be smaller than 2^31
 *     bytes, else EQLIN_ENOTSUP.
 *   - Device pointers, caller-owned, 16-byte aligned (else EQLIN_EALIGN); the
 *     library allocates nothing; calls only enqueue work on `stream`; all
 *     arguments are validated before anything is enqueued; a HIP launch
 *     failure returns EQLIN_EHIP (eqlin_last_hip_error()).
 */
#ifndef EQCONV_H
#define EQCONV_H

#include <stddef.h>
#include <stdint.h>

#include "eqlin.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Size in bytes of the prepared filter buffer, or 0 for invalid arguments.
 * Layout: the forward set of the gathered layer (D' rows, C'K^2 group
 * channels padded to whole 16 (EQLIN_F32) / 32 (EQLIN_F16) channel blocks,
 * the block layout of eqlin.h's forward set) at offset 0, then the adjoint
 * set (C' rows over D'K^2 channels) at eqconv_prepared_adjoint_offset() (a
 * multiple of 256).  Within a block the channel order is that of the gather:
 * block cb (4 G channels, G = 1 for EQLIN_F32, 2 for EQLIN_F16) is either a
 * centre block (cb < C'/(4G): channels 4 G cb .. ) or orbit block (o, cg)
 * with cb = C'/(4G) + o C'/G + cg, orbit o = (a - 1)(p + 1) + b of the tap
 * (a, b), a = 1..p, b = 0..p.
 */
size_t eqconv_prepared_weight_bytes(int C, int D, int K, int dtype);
size_t eqconv_prepared_adjoint_offset(int C, int D, int K, int dtype);

/*
 * Group DFT of the gathered layer's weights (both sets) from psi
 * [D'][C'][K][K][4] (device, storage dtype).  prepared_bytes must be >=
 * eqconv_prepared_weight_bytes (else EQLIN_EWORKSPACE).  Run once per filter
 * version.
 */
int eqconv_prepare_weights(const void* psi, int C, int D, int K, int dtype,
                           void* prepared, size_t prepared_bytes, void* stream);

/*
 * Y = act(conv(X, psi) + b): X [N][H][W][C] -> Y [N][H][W][D].  bias (NULL
 * or D' values of the storage dtype, element-aligned) is added to the four
 * rotations of output channel d'; act is EQLIN_ACT_NONE or EQLIN_ACT_GELU
 * (else EQLIN_EINVAL); both run in the register epilogue as in
 * eqlin_forward_ex.  Reproducibility as eqlin_forward (per output pixel;
 * EQLIN_FWD_SPLIT=0 keeps every pixel in the fixed summation order).
 */
int eqconv_forward(const void* X, int64_t N, int H, int W, int C, int D, int K,
                   const void* prepared, const void* bias, int act, void* Y,
                   int dtype, void* stream);

/* Workspace bytes eqconv_backward needs when dpsi is requested. */
size_t eqconv_backward_workspace_bytes(int64_t N, int H, int W, int C, int D, int K, int dtype);

/*
 * Backward for upstream gradient dY [N][H][W][D]:
 *   dX [N][H][W][C] = d<dY, Y>/dX   (skipped if dX == NULL)
 *   dpsi [D'][C'][K][K][4] float32 = d<dY, Y>/dpsi   (skipped if dpsi == NULL)
 * dpsi is the gathered layer's dw, with the gather done by the loads of its
 * reduction, reduced over row splits in a fixed order (deterministic) and
 * permuted onto the filter.  The workspace holds the split partials and the
 * gathered layer's gradient; it may be NULL only when dpsi == NULL, and X
 * may be NULL only when dpsi == NULL.  At least one output is required.
 */
int eqconv_backward(const void* dY, const void* X, int64_t N, int H, int W, int C, int D, int K,
                    const void* prepared, void* dX, float* dpsi,
                    void* workspace, size_t workspace_bytes, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EQCONV_H */
