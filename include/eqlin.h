/*
 * eqlin.h -- C ABI of the MI355X (gfx950) group-circulant linear layer
 * ("Flash EQ-Linear") for the cyclic groups of order 4 (the p4 rotation
 * group) and 8 (C8), and for the dihedral group p4m (order 8).
 *
 * The layer (Flash EQ-Linear technical summary, gist.science 2607.21271,
 * section "Key insight"): the dense weight W (D x C) is made of
 * (D/T) x (C/T) blocks, block (d', c') being the T x T circulant of a
 * learnable vector w[d', c', 0..T-1]:
 *
 *     W[T d' + t, T c' + s] = w[d', c', (t - s) mod T]
 *     Y = X W^T,  Y[n, T d' + t] = sum_{c', s} w[d', c', (t - s) mod T] X[n, T c' + s]
 *
 * It is computed exactly through the group DFT ("Algorithmic approach",
 * items 1-2; "Specialisation for the p4 rotation group"): only the
 * non-redundant frequencies of the real signals are formed and the
 * contraction becomes real per-frequency matrix products.  For T = 4: f0, f2
 * (real) and f1 (complex), add/sub-only transforms, six real products
 * instead of sixteen.  For T = 8 (the summary names other groups as future
 * work, "Limitations"; this is the same route for the next cyclic group):
 * f0, f4 (real) and f1, f2, f3 (complex), transforms with the factor
 * sqrt(1/2), fourteen real products instead of sixty-four.
 *
 * p4m (the rotations and reflections of the square, a non-abelian group of
 * order 8; "Limitations" names reflection groups as future work): the same
 * layer as a group convolution, with the group elements u = k + 4m standing
 * for r^k s^m (r: rotation by 90 degrees, s: a reflection, s r s = r^-1):
 *
 *     W[8 d' + g, 8 c' + h] = w[d', c', h^-1 g]
 *
 * (for the cyclic groups h^-1 g = (g - h) mod T, the circulant above).  It is
 * computed through the irreducible representations of p4m: four characters
 * and one 2 x 2 block per group channel, add/sub-only transforms, twelve real
 * products instead of sixty-four.
 *
 * Conventions shared by every entry point
 *   - T selects the group: 4 or 8 (cyclic, order T) or EQLIN_P4M (order 8);
 *     any other value -> EQLIN_ENOTSUP.  Below, "T" in sizes and layouts is
 *     the group order.
 *   - C, D are the full channel widths, positive multiples of T; C' = C/T
 *     and D' = D/T are the group-channel counts.  The channel index is
 *     group_channel * T + group_element (group element fastest).
 *   - All matrices are row-major and contiguous:
 *       X, dX  [N][C]      Y, dY  [N][D]      w  [D'][C'][T]     dw [D'][C'][T]
 *   - dtype EQLIN_F32: X, Y, dY, dX, w in float32, arithmetic in float32
 *     (true fp32 matrix-core products).
 *     dtype EQLIN_F16: X, Y, dY, dX, w stored as IEEE binary16; the group
 *     transforms run in float32, the Fourier operands are rounded once
 *     (nearest-even) to binary16 for the matrix cores, products accumulate in
 *     float32, and outputs are rounded nearest-even to binary16.  dw is float32
 *     for both dtypes.  With EQLIN_F16 and T = 4, C' and D' must be
 *     even (otherwise EQLIN_ENOTSUP).
 *   - f16 range.  A plane of a group transform can be as large as T times its
 *     inputs (the zero frequency sums all T values of a group), so before the
 *     rounding to binary16 every Fourier operand plane (of X, of dY and of the
 *     prepared weights) is multiplied by a fixed power of two that keeps it
 *     within the largest magnitude of its inputs; the exact inverse power is
 *     applied to the float32 accumulators in the inverse transform.  The
 *     summary's dyadic coefficients ("Specialisation for the p4 rotation
 *     group", first bullet) allow the normalisation on either side.  Scales
 *     per plane, in the plane order of eqlin_prepared_weight_bytes below:
 *       f16 operand scales, T = 4: (1/4, 1/4, 1/2, 1/2)
 *       f16 operand scales, T = 8: (1/8, 1/8, 1/8, 1/8, 1/4, 1/4, 1/8, 1/8)
 *       f16 operand scales, EQLIN_P4M: (1/8, 1/8, 1/8, 1/8, 1/4, 1/4, 1/4, 1/4)
 *     Consequences: every finite binary16 input (|x| <= 65504) gives finite
 *     operands; an output is inf only where the exact result itself exceeds
 *     the binary16 range (Y, dX; dw is float32).  At the small end a scaled
 *     operand below 2^-14 is a binary16 subnormal (spacing 2^-24): an operand
 *     plane whose inputs are near the smallest normal 2^-14 keeps an absolute
 *     rounding error of at most 2^-25 per operand instead of a relative one.
 *     float32 has no such scaling (its planes overflow only past about 8e37).
 *   - Every data pointer is a DEVICE pointer on the current HIP device, owned
 *     by the caller, 16-byte aligned (else EQLIN_EALIGN).  The library never
 *     allocates, frees or retains memory and keeps no mutable global state
 *     (apart from eqlin_backward_noalloc's static scratch, see there); calls
 *     are thread-safe.  Outputs must not alias inputs.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns without synchronising.
 *   - All arguments are validated before any kernel is enqueued: on any error
 *     nothing is launched and no output is touched.  A launch the device
 *     cannot take returns EQLIN_EHIP and records the hipError_t for
 *     eqlin_last_hip_error(): a launch error the HIP runtime reports, or a
 *     grid beyond 2^31 - 1 workgroups (hipErrorInvalidConfiguration, refused
 *     before anything of that launch is enqueued; e.g. more than 2^37 rows).
 *   - N == 0 is a valid empty batch: forward and dX enqueue nothing, dw is
 *     written as zeros.
 *   - Kernels address one tile (at most 256 rows) with 32-bit offsets: C and D
 *     must keep 256 rows of X, Y, dY and dX below 1 GiB (C, D < 2^20 in
 *     float32), else EQLIN_ENOTSUP.
 */
#ifndef EQLIN_H
#define EQLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtypes. */
enum { EQLIN_F32 = 0, EQLIN_F16 = 1 };

/* Group code of p4m (order 8) for the T argument; 4 and 8 select the cyclic groups. */
enum { EQLIN_P4M = 108 };

/* Status codes returned by every int-returning entry point. */
enum {
  EQLIN_OK = 0,
  EQLIN_EINVAL = 1,     /* bad size, negative N, null required pointer, unknown dtype */
  EQLIN_ENOTSUP = 2,    /* T not 4, 8 or EQLIN_P4M, an odd group count with EQLIN_F16 and T = 4, or
                           rows so wide that 256 of them (input or output) pass 1 GiB */
  EQLIN_EALIGN = 3,     /* a data pointer is not 16-byte aligned */
  EQLIN_EWORKSPACE = 4, /* workspace / prepared-weight buffer too small */
  EQLIN_EHIP = 5        /* the HIP runtime reported an error for a launch */
};

/* Library ABI version (major * 100 + minor). */
int eqlin_version(void);

/* Static string for a status code ("unknown status" for others). */
const char* eqlin_status_str(int status);

/* hipError_t value that produced the calling thread's last EQLIN_EHIP (0 if none). */
int eqlin_last_hip_error(void);

/*
 * Size in bytes of the prepared-weight buffer W_hat for a layer, or 0 if the
 * arguments are invalid.
 *
 * W_hat layout (element = the storage dtype; S = 16 for EQLIN_F32, 32 for
 * EQLIN_F16 group channels per 64-byte block):
 *   offset 0: forward set  [D'][ceil(C'/S)][T planes][S]
 *   offset eqlin_prepared_transpose_offset() (a multiple of 256):
 *             transpose set [C'][ceil(D'/S)][T planes][S]
 * With F_k = sum_u w[d', c', u] exp(-2 pi i k u / T) the group DFT of each
 * circulant vector ("Algorithmic approach", item 1; F_{T-k} = conj(F_k) is
 * redundant for real w, item 2), the planes of the forward set are
 *   T = 4: (F0, F2, Re F1, Im F1)
 *   T = 8: (F0, F4, Re F1, Im F1, Re F2, Im F2, Re F3, Im F3)
 * and the transpose set holds the same planes with every Im negated: the
 * spectrum of the transposed, group-reversed weight (a conjugate) used by
 * the dX pass.  With EQLIN_F16 each plane is stored multiplied by its f16
 * operand scale (see "f16 range" above).  For EQLIN_P4M the planes are w_hat(rho) = sum_u w(u) rho(u)
 * for the characters A1, A2, B1, B2 (r -> 1, 1, -1, -1; s -> 1, -1, 1, -1)
 * and the 2 x 2 representation E (r -> [[0,-1],[1,0]], s -> diag(1,-1)),
 * ordered (A1, A2, B1, B2, E00, E01, E10, E11); the transpose set holds the
 * spectrum of u -> w(u^-1), i.e. the same planes with E01 and E10 swapped.  Within block ks of a row, slot s holds group channel
 * ks*S + g(s); with V = 16 / element bytes (4 or 8) and G = the number of
 * whole groups in one 16-byte piece (2 for EQLIN_F16 with T = 4, else 1),
 *   g(s) = G ((s / V) + 4 ((s % V) / G)) + (s % V) % G
 * which for T = 4 reads
 *   g(s) = (s >> 2) + 4 (s & 3)                              (EQLIN_F32)
 *   g(s) = 2 ((s >> 3) + 4 ((s >> 1) & 3)) + (s & 1)          (EQLIN_F16)
 * (the order in which the forward kernel's loaders deposit the transformed
 * input on chip), and slots past the last group channel hold zeros.  The
 * layout depends on the group order only (EQLIN_P4M as T = 8).
 */
size_t eqlin_prepared_weight_bytes(int C, int D, int T, int dtype);
size_t eqlin_prepared_transpose_offset(int C, int D, int T, int dtype);

/*
 * a1: group DFT of the weights.  w [D'][C'][T] (device, storage dtype) ->
 * W_hat (device, W_hat_bytes >= eqlin_prepared_weight_bytes, else
 * EQLIN_EWORKSPACE).  Run it once per weight version; the forward and
 * backward calls consume W_hat read-only.  For T = 4 the transform uses adds
 * and subtracts only ("Specialisation for the p4 rotation group").
 */
int eqlin_prepare_weights(const void* w, int C, int D, int T, int dtype,
                          void* W_hat, size_t W_hat_bytes, void* stream);

/*
 * a2-a4: Y = X W^T.  X [N][C], Y [N][D] (device, storage dtype), W_hat from
 * eqlin_prepare_weights for the same (C, D, T, dtype).  One fused kernel:
 * group DFT of X tiles into on-chip Fourier planes, the real per-frequency
 * products on the matrix cores (6 for T = 4, 14 for T = 8), inverse DFT in
 * registers and a single store of Y; no intermediate global-memory writes
 * ("Implementation" section).
 * Reproducibility: for given (N, C, D, T, dtype) the result is the same on
 * every call.  Every row normally sums its k range in one fixed order, so a
 * row does not depend on N either, except in float32 when the last, at most
 * half-full round of tiles runs split (the rows of those tiles add two
 * partial sums over the two halves of every k stage): there a row can
 * differ in the last bits from the same row computed with another N.
 * Setting the environment variable EQLIN_FWD_SPLIT=0 keeps every row in
 * the fixed order (and may run slower).  The same holds for dX below.
 */
int eqlin_forward(const void* X, int64_t N, int C, int D, int T,
                  const void* W_hat, void* Y, int dtype, void* stream);

/*
 * Launch plan of eqlin_forward (and of eqlin_backward_dx, whose launch has
 * the same structure with C and D exchanged) for this shape, in the
 * environment of the call (EQLIN_FWD_TILE, EQLIN_FWD_SPLIT); enqueues
 * nothing and needs no device.  Writes, for non-NULL pointers:
 *   tile   the tile code, FM FN WM WN NBUF PF [P] as EQLIN_FWD_TILE takes it:
 *          (32 FM WM) rows x (32 FN WN) output groups, WM x WN waves;
 *   tiles  the number of tiles (0 for N == 0);
 *   whole  how many run as one workgroup each; the other tiles - whole run
 *          as two workgroups of half the rows (the float32 tail split).
 * Returns EQLIN_OK, or the status eqlin_forward would return for the shape.
 */
int eqlin_forward_plan(int64_t N, int C, int D, int T, int dtype, int* tile, int64_t* tiles,
                       int64_t* whole);

/* Epilogue activations for eqlin_forward_ex. */
enum { EQLIN_ACT_NONE = 0, EQLIN_ACT_GELU = 1 };

/*
 * Forward with a fused epilogue: Y = act(X W^T + b).
 *   bias: NULL or a device pointer to D' = D/T values in the storage dtype
 *         (element-aligned).  The bias is group-invariant: b[d'] is added to
 *         all T outputs T d'+0..T-1 of output group d', which keeps the layer
 *         equivariant (the summary is silent on bias; this is the reading).
 *   act:  EQLIN_ACT_NONE or EQLIN_ACT_GELU (GELU(z) = z/2 (1 + erf(z/sqrt 2)),
 *         pointwise, so it commutes with the group shift), else EQLIN_EINVAL.
 * The bias add and the activation run in float32 in the register epilogue
 * of the same kernel, before the single rounding to the storage dtype.
 * Forward only (inference); everything else as eqlin_forward.
 */
int eqlin_forward_ex(const void* X, int64_t N, int C, int D, int T, const void* W_hat,
                     const void* bias, int act, void* Y, int dtype, void* stream);

/*
 * Forward with a fused epilogue and a residual: Y = act(X W^T + b) + R.
 * The residual is the transformer block's skip connection around the MLP
 * (x + MLP(x)) of the ViT networks the summary measures ("Network-level
 * results"; the pages do not spell it out: this is the reading).  Adding a
 * tensor that is itself laid out by group channel keeps the layer
 * equivariant.
 *   R: NULL (then exactly eqlin_forward_ex) or a device pointer to [N][D] in
 *      the storage dtype, 16-byte aligned (else EQLIN_EALIGN).  R may be Y
 *      itself (an in-place update: every element is read before it is
 *      written, by the same lane); otherwise R must not overlap Y.
 * The residual is added in float32 after the activation, before the single
 * rounding to the storage dtype.  Everything else as eqlin_forward_ex.
 */
int eqlin_forward_residual(const void* X, int64_t N, int C, int D, int T, const void* W_hat,
                           const void* bias, int act, const void* R, void* Y, int dtype, void* stream);

/*
 * Workspace bytes eqlin_forward_ws needs for this shape, or 0 when its launch
 * has no K split (then it needs none; also 0 for invalid arguments).  If
 * parts is non-NULL it receives the part count of each split tile (0, or 2
 * to 4).  Depends on the environment as eqlin_forward_plan does.
 */
size_t eqlin_forward_workspace_bytes(int64_t N, int C, int D, int T, int dtype, int* parts);

/*
 * a2-a4 with a workspace: eqlin_forward_residual (the same fused kernel,
 * "Implementation" section, and the same arguments), where the float32 tiles
 * of the last, partial round of workgroups may each run as 2 to 4
 * workgroups over consecutive ranges of the k axis.  The summary's kernel
 * design leaves the division of the work over the GPU open; this one keeps
 * every CU within a third or a quarter of a tile of the others where the
 * tail split of eqlin_forward leaves half a tile (ViT-B attention: 591
 * tiles of 64 x 64 on 256 CUs).
 *   workspace: NULL (then exactly eqlin_forward_residual), or a device
 *     buffer, 16-byte aligned, of workspace_bytes >=
 *     eqlin_forward_workspace_bytes (else EQLIN_EWORKSPACE).  Its first
 *     1024 bytes are arrival counters: they must be zero before the first
 *     call that uses the buffer (e.g. allocate it zero-filled), and every
 *     call leaves them zero when its kernel completes.  The rest holds the
 *     parts' partial sums (float32), written before they are read.  Calls
 *     that overlap in time (other streams, other threads) must not share a
 *     workspace.  The library does not retain it.
 * Each split tile's parts are added in a fixed order by whichever part
 * finishes last, so for given (N, C, D, T, dtype) the result is the same on
 * every call; a row of a split tile can differ in the last bits from the
 * same row computed by eqlin_forward (a different summation order).
 * EQLIN_FWD_SPLIT=0 turns the K split off with the tail split.
 */
int eqlin_forward_ws(const void* X, int64_t N, int C, int D, int T, const void* W_hat,
                     const void* bias, int act, const void* R, void* Y,
                     void* workspace, size_t workspace_bytes, int dtype, void* stream);

/* Workspace bytes eqlin_backward / eqlin_backward_dw need for this shape. */
size_t eqlin_backward_workspace_bytes(int64_t N, int C, int D, int T, int dtype);

/*
 * a5 + a6: backward pass for upstream gradient dY [N][D].  The summary's
 * kernels cover the backward pass as well as the forward ("Implementation",
 * first bullet: dedicated forward and backward kernels); its operator-level
 * results report the backward speed-up beside the forward's ("Experimental
 * results", "Operator level").  It gives no formulas for it: the two
 * gradients below are plain calculus on the layer's definition ("Key
 * insight"), computed through the same group DFT ("Algorithmic approach",
 * items 1-2).
 *   dX [N][C] = dY W   (transposed group-circulant; skipped if dX == NULL)
 *   dw [D'][C'][T] (float32) = d<dY, Y>/dw
 *      = sum_n sum_t dY[n, T d'+t] X[n, T c' + (t-u) mod T]   (skipped if dw == NULL)
 *      (EQLIN_P4M: sum_n sum_h dY[n, 8 d' + h u] X[n, 8 c' + h])
 * dX runs the forward's fused structure on the transpose spectra; dw is
 * formed per frequency as sum_n G_k conj(Xhat_k) (G = group DFT of dY;
 * for EQLIN_P4M per representation sum_n Xhat^T G), reduced over row splits
 * in a fixed order (deterministic) and inverse transformed along u.
 * `workspace` (device, >= eqlin_backward_workspace_bytes) holds the
 * per-split partial spectra; it may be NULL only when dw == NULL.
 * X may be NULL when dw == NULL.  With both outputs asked for, dX and the dw
 * partials run in one launch (both read dY), then the ordered finalize.
 * Errors as for every entry point: EINVAL, ENOTSUP, EALIGN, EWORKSPACE
 * (workspace_bytes too small), EHIP; both halves are validated before
 * either is launched.
 */
int eqlin_backward(const void* dY, const void* X, int64_t N, int C, int D, int T,
                   const void* W_hat, void* dX, float* dw,
                   void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * a5 alone: dX = dY W (the transpose of the layer's circulant blocks: the
 * backward of "Key insight"'s map, run as the forward structure of
 * "Implementation", first bullet, on the transpose spectra).  Same contract
 * as eqlin_backward with dw == NULL.
 */
int eqlin_backward_dx(const void* dY, int64_t N, int C, int D, int T,
                      const void* W_hat, void* dX, int dtype, void* stream);

/*
 * a6 alone: dw only, the weight gradient of "Key insight"'s map formed per
 * frequency ("Algorithmic approach", items 1-2) as a row reduction over the
 * batch ("Experimental results", "Operator level": the backward pass).  Same
 * contract as eqlin_backward with dX == NULL.
 */
int eqlin_backward_dw(const void* dY, const void* X, int64_t N, int C, int D, int T,
                      float* dw, void* workspace, size_t workspace_bytes,
                      int dtype, void* stream);

/* Bytes of the per-device scratch of eqlin_backward_noalloc (32 MiB). */
#define EQLIN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * eqlin_backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, outputs and errors as eqlin_backward, without the
 * workspace: the dw split partials go to a scratch array inside the library
 * (EQLIN_NOALLOC_SCRATCH_BYTES per device, a static device array that every
 * device the library runs on holds until the process ends).  The call
 * allocates and frees nothing.
 *   - The row splits of the dw reduction are capped to what the scratch
 *     holds (each split T x D' x C' float32 values).  Where the cap binds,
 *     dw is summed in fewer, longer splits than eqlin_backward uses (the
 *     same values to rounding; the p4 layers of the ViT-B shapes are not
 *     capped and give the same bits as eqlin_backward; the ViT-H layers,
 *     whose dw runs in 6 (float32, fused with dX) or 8 (f16, 128-wide tiles)
 *     splits of 6.5 MB, run 5).  A layer one split
 *     of which does not fit (T D' C' > 8 Mi values) -> EQLIN_EWORKSPACE.
 *   - Every call on a device shares that device's scratch, which keeps the
 *     last call's partials; nothing in it needs clearing (every partial is
 *     written before it is read).  Calls that overlap on one device (other
 *     streams, other threads) race on the scratch: serialise them.
 *   - dw == NULL needs no scratch (dX only, as eqlin_backward).
 */
int eqlin_backward_noalloc(const void* dY, const void* X, int64_t N, int C, int D, int T,
                           const void* W_hat, void* dX, float* dw, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EQLIN_H */
