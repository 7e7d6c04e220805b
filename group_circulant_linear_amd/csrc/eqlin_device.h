// Device code of the group-circulant (EQ-)linear layer for gfx950 (CDNA4):
// group transforms, the matrix-core "complex core", the forward / dX tile
// (one tile per workgroup, or the persistent stage stream), the dw
// split-partial tile, the dw finalize and the weight preparation, all
// templated on the storage type E (float or _Float16) and the group G: 4 (the
// p4 rotation group, cyclic of order 4), 8 (the cyclic group C8) or kP4M (the
// dihedral group p4m of order 8).  The forward and dw tiles also have a p4
// convolution mode (ConvGeom) whose operand loads gather a K x K window;
// the convolution's own kernels are in eqconv_kernels.hip.
//
// Method (Flash EQ-Linear technical summary, gist.science 2607.21271):
//   * "Key insight": the weight is group-circulant, so the layer is a circular
//     convolution over the group axis combined with a channel contraction.
//   * "Algorithmic approach", items 1-2: a DFT over the group axis turns each
//     circulant block into a pointwise product per frequency; for real data
//     only the non-redundant frequencies are formed.
//   * "Specialisation for the p4 rotation group": for T = 4 the transforms use
//     only 0, +-1 and the power-of-two rescales 1/4, 1/2 (adds and subtracts),
//     and the contraction is six real matrix products: f0 (1), f2 (1) and the
//     complex f1 (4: Re/Im cross terms).
//   * "Limitations": the specialisation is to p4; other groups (reflections
//     among them) and other equivariant operators (convolution) are future
//     work.  C8 here follows the same route with the general real-signal DFT:
//     real f0 and f4, complex f1..f3, 2 + 3 * 4 = 14 real products.  p4m uses
//     its irreducible representations: four 1-D and one 2-D, 4 + 8 = 12 real
//     products.  The p4 convolution is the p4 layer over a gathered window.
//   * "Implementation": fused dataflow (no intermediate global writes), Fourier
//     fragments resident in registers / on-chip memory, shape-specialised
//     tiles on the matrix cores.
//
// gfx950 mapping.  Work is expressed as one "structured GEMM":
//   out_plane[m][n] = sum_k A_plane[m][k] (*) B_plane[n][k]
// where (*) is a fixed list of plane products (Grp<G>::kFwd / kDw): for a
// cyclic group the real planes pointwise and the (Re, Im) plane pairs as
// complex numbers, for p4m the 1-D planes pointwise and the 2 x 2 blocks as
// matrices.  Both operands are staged per pipeline stage into LDS as
// T planes [plane][row][k] with k contiguous in 64-byte rows whose four 16-byte
// slots are XOR-swizzled (see swz_slot).  Every lane reads 16 bytes per plane
// per 32x32 fragment: 4 fp32 k-values (four 32x32x2 f32 MFMAs) or 8 f16
// k-values (one 32x32x16 f16 MFMA).  Waves are 64 wide; each wave owns
// FM x FN fragments of 32 x 32 for each of the T accumulator planes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "eqlin_kernels.h"

namespace eqlin {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// Stage timestamps of the forward tile, for the diagnostic program
// stage_trace.hip, which defines EQLIN_STAGE_TRACE before including this
// header; in the library the hook is empty.  Event ev of workgroup b: the
// shader clock and the 100 MHz real-time counter, written by thread 0 to
// g_stage_trace[(b * 64 + ev) * 2 + {0, 1}] (b < 8192; event 61 holds the
// wave's hardware id and its XCC id).  Events: 0 start, 1 first stage in LDS, 2 first stage
// multiplied, 3 last stage multiplied, 62 output stores issued, 63 stores
// completed.
#ifdef EQLIN_STAGE_TRACE
__device__ unsigned long long* g_stage_trace;
__device__ __forceinline__ void stage_mark(int ev) {
  unsigned long long* t = g_stage_trace;
  if (threadIdx.x == 0 && t != nullptr && blockIdx.x < 8192) {
    t[(blockIdx.x * 64 + ev) * 2] = __builtin_amdgcn_s_memtime();
    t[(blockIdx.x * 64 + ev) * 2 + 1] = __builtin_amdgcn_s_memrealtime();
    if (ev == 0) {
      unsigned id, xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(id));
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      t[(blockIdx.x * 64 + 61) * 2] = id;
      t[(blockIdx.x * 64 + 61) * 2 + 1] = xcc & 0xf;
    }
  }
}
// the tile's output stores have completed
__device__ __forceinline__ void stage_mark_drained() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  stage_mark(63);
}
#else
__device__ __forceinline__ void stage_mark(int) {}
__device__ __forceinline__ void stage_mark_drained() {}
#endif
constexpr int kNumXcd = 8;
// LDS stage buffers of the dw partial tiles and of the dX tiles inside the
// fused backward (1: smaller LDS, more resident workgroups per CU), and the
// register prefetch depth of those dX tiles.
constexpr int kDwBufs = 1;
constexpr int kBwdFwdBufs = 1;
constexpr int kBwdFwdPrefetch = 1;

// LDS plane rows are 64 bytes (four 16-byte slots) with no padding; the slot
// index is XOR-swizzled with bits 2-3 of the row, which keeps both the
// 4-lanes-per-row stores and the 32-rows-per-wave fragment reads free of bank
// conflicts on gfx950 (checked with the LDS bank-conflict counter).
constexpr int kRowBytes = 64;
__device__ __forceinline__ int swz_slot(int row, int slot) { return slot ^ ((row >> 2) & 3); }

// The dw tile's placement of the same 64-byte plane rows (rows = group
// channels, k along the batch rows).  Its f16 p4 writes are transposed: a
// 32-lane write covers eight rows two apart (the two groups' rows of eight
// consecutive unit columns), four 8-byte runs in each.  Row r goes to
// physical row dw_row(r) (the low three bits rotated to b1 b2 b0) and its
// 16-byte slots are XOR-ed with bits 0 and 3 of r, which spreads those 32
// runs over all 64 banks; sixteen consecutive rows of a fragment read also
// meet all 64 banks once.
__device__ __forceinline__ int dw_row(int r) { return (r & ~7) | ((r >> 1) & 3) | ((r & 1) << 2); }
__device__ __forceinline__ int dw_slot(int r, int slot) { return slot ^ ((r & 1) | (((r >> 3) & 1) << 1)); }
__device__ __forceinline__ int dw_off(int r, int kb) {
  return dw_row(r) * kRowBytes + dw_slot(r, kb >> 4) * 16 + (kb & 15);
}

// Group channels whose values one lane holds per 16-byte LDS slot of a plane
// (= k-values per lane and fragment): 4 fp32, 8 f16.  A pipeline stage covers
// four slots, i.e. 16 fp32 / 32 f16 group channels along k.
template <typename E>
struct Traits {
  static constexpr int kVals = 16 / (int)sizeof(E);
  static constexpr int kStageGroups = 4 * kVals;
};

// How one lane's slot worth of groups (kVals groups of T values) is fetched:
// as kUnits units of kPiecesPerUnit consecutive 16-byte pieces, each unit
// holding kGroupsPerUnit whole groups (a group of T fp32 values spans T/4
// pieces; a 16-byte piece holds 2 f16 groups of 4 or one of 8).
template <typename E, int T>
struct Units {
  static constexpr int kVals = Traits<E>::kVals;
  static constexpr int kGroupBytes = T * (int)sizeof(E);
  static constexpr int kGroupsPerUnit = kGroupBytes >= 16 ? 1 : 16 / kGroupBytes;
  static constexpr int kPiecesPerUnit = kGroupBytes >= 16 ? kGroupBytes / 16 : 1;
  static constexpr int kUnits = kVals / kGroupsPerUnit;
  static constexpr int kPieces = kUnits * kPiecesPerUnit;  // = T
  static_assert(kPieces == T, "a lane's slot of every plane is fed by T pieces");
};

// Group channel held by slot value s (0 .. kStageGroups-1) of a stage block:
// lane block q = s / kVals fetches units q, q+4, q+8, ... of the stage, so
// value v of block q is group kGroupsPerUnit * (q + 4 (v / kGroupsPerUnit)) +
// v % kGroupsPerUnit.  The prepared weights are stored in this order so that
// both operands of every product meet at the same k.
template <typename E, int T>
__host__ __device__ constexpr int slot_group(int s) {
  constexpr int V = Traits<E>::kVals, G = Units<E, T>::kGroupsPerUnit;
  return G * (s / V + 4 * ((s % V) / G)) + (s % V) % G;
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ void dft4(float z0, float z1, float z2, float z3,
                                     float& f0, float& f2, float& f1r, float& f1i) {
  const float a = z0 + z2, b = z1 + z3;
  f0 = a + b;
  f2 = a - b;
  f1r = z0 - z2;
  f1i = z3 - z1;
}

__device__ __forceinline__ void idft4(float f0, float f2, float f1r, float f1i, float y[4]) {
  const float s = 0.25f * (f0 + f2), d = 0.25f * (f0 - f2);
  const float r = 0.5f * f1r, i = 0.5f * f1i;
  y[0] = s + r;
  y[1] = d - i;
  y[2] = s - r;
  y[3] = d + i;
}

// ------------------------------------------------------------------ groups
//
// Grp<G> describes one group: its order T (= number of real planes per group
// channel), the forward transform dft (T values -> T planes), the inverse
// idft, the adjoint (the spectrum of the transposed kernel u -> w(u^-1): the
// conjugate for a cyclic group, the transposed 2 x 2 block for p4m), and the
// plane products of the contraction.  A product {out, a, b, neg} accumulates
// (neg ? -1 : 1) * A[a] * B[b] into plane out.  kFwd serves the forward and
// dX passes (out = A * B per representation); kDw the dw pass, which needs
// B * A (the same list for the commutative cyclic groups).  Every
// accumulator's first product comes before any second one, so dependent
// matrix-core operations on one accumulator are far apart.
struct Prod {
  int out, a, b;
  bool neg;
};

template <int G>
struct Grp;

// Cyclic groups: a real signal z[0..T-1] has T real Fourier degrees of
// freedom (F_k = sum_u z_u exp(-2 pi i k u / T) is conjugate symmetric), kept
// as T planes in the order
//   F_0, F_{T/2}, Re F_1, Im F_1, ..., Re F_{T/2-1}, Im F_{T/2-1}
// (for T = 4: F0, F2, Re F1, Im F1).  idft maps any such planes back to the
// real signal (1/T) sum_k F_k exp(+2 pi i k u / T) with F_{T-k} = conj F_k.
__host__ __device__ constexpr bool imag_plane(int p) { return p >= 2 && (p & 1); }

template <int T>
__device__ __forceinline__ void conj_planes(float* f) {
#pragma unroll
  for (int p = 0; p < T; ++p)
    if (imag_plane(p)) f[p] = -f[p];
}

// Range of the f16 Fourier operands.  A plane of the transform of T values
// bounded by M is bounded by b_p M (F0 sums all T values).  In f16 every
// operand plane p (the transformed input, dY and the prepared weights) is
// multiplied by kF16Scale[p], the largest power of two with
// kF16Scale[p] b_p <= 1, before its one rounding to binary16, so no finite
// binary16 input can overflow an operand (the page's dyadic coefficients
// put the normalisation on either side; here part of it moves to the forward
// transform).  Every product of an output plane p meets operands of equal
// scale, so the accumulated plane carries kF16Scale[p]^2, which the epilogue
// and the dw finalize multiply back out (exact powers of two).
template <int G>
__host__ __device__ constexpr float f16_unscale(int p) {
  return 1.0f / (Grp<G>::kF16Scale[p] * Grp<G>::kF16Scale[p]);
}

template <>
struct Grp<4> {
  static constexpr int kOrder = 4;
  static constexpr int kProducts = 6;
  static constexpr Prod kFwd[kProducts] = {{0, 0, 0, false}, {2, 2, 2, false}, {1, 1, 1, false},
                                           {3, 2, 3, false}, {2, 3, 3, true},  {3, 3, 2, false}};
  static constexpr const Prod* kDw = kFwd;
  // |F0|, |F2| <= 4 M; |Re F1|, |Im F1| <= 2 M
  static constexpr float kF16Scale[kOrder] = {0.25f, 0.25f, 0.5f, 0.5f};
  __device__ __forceinline__ static void dft(const float* z, float* f) {
    dft4(z[0], z[1], z[2], z[3], f[0], f[1], f[2], f[3]);
  }
  __device__ __forceinline__ static void idft(const float* f, float* y) { idft4(f[0], f[1], f[2], f[3], y); }
  __device__ __forceinline__ static void adjoint(float* f) { conj_planes<4>(f); }
};

// C8 by one radix-2 split: the even frequencies are the 4-point DFT of
// s_u = z_u + z_{u+4}; the odd ones come from a_u = z_u - z_{u+4}, where with
// c = sqrt(1/2):  F1 = (a0 + c (a1 - a3)) - i (a2 + c (a1 + a3)),
//                 F3 = (a0 - c (a1 - a3)) + i (a2 - c (a1 + a3)).
// Inverse: s = 4-point inverse of (F0, F4, F2) and
//   a0 = (Re F1 + Re F3)/2           a2 = (Im F3 - Im F1)/2
//   a1 = c/2 ((Re F1 - Im F1) - (Re F3 + Im F3))
//   a3 = c/2 ((Re F3 - Im F3) - (Re F1 + Im F1))
//   z_u = (s_u + a_u)/2,  z_{u+4} = (s_u - a_u)/2.
// Planes: 0 F0, 1 F4, 2/3 F1, 4/5 F2, 6/7 F3.
template <>
struct Grp<8> {
  static constexpr int kOrder = 8;
  static constexpr int kProducts = 14;
  static constexpr Prod kFwd[kProducts] = {
      {0, 0, 0, false}, {2, 2, 2, false}, {1, 1, 1, false}, {3, 2, 3, false}, {4, 4, 4, false},
      {5, 4, 5, false}, {6, 6, 6, false}, {7, 6, 7, false}, {2, 3, 3, true},  {3, 3, 2, false},
      {4, 5, 5, true},  {5, 5, 4, false}, {6, 7, 7, true},  {7, 7, 6, false}};
  static constexpr const Prod* kDw = kFwd;
  static constexpr float kC = 0.70710678118654752f;
  // |F0|, |F4| <= 8 M; |Re F2|, |Im F2| <= 4 M; the parts of F1 and F3 <= (2 + 4c) M < 8 M
  static constexpr float kF16Scale[kOrder] = {0.125f, 0.125f, 0.125f, 0.125f, 0.25f, 0.25f, 0.125f, 0.125f};
  __device__ __forceinline__ static void dft(const float* z, float* f) {
    float s[4], a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s[u] = z[u] + z[u + 4];
      a[u] = z[u] - z[u + 4];
    }
    dft4(s[0], s[1], s[2], s[3], f[0], f[1], f[4], f[5]);
    const float p = kC * (a[1] - a[3]), q = kC * (a[1] + a[3]);
    f[2] = a[0] + p;
    f[3] = -a[2] - q;
    f[6] = a[0] - p;
    f[7] = a[2] - q;
  }
  __device__ __forceinline__ static void idft(const float* f, float* y) {
    float s[4], a[4];
    idft4(f[0], f[1], f[4], f[5], s);
    a[0] = 0.5f * (f[2] + f[6]);
    a[2] = 0.5f * (f[7] - f[3]);
    a[1] = (0.5f * kC) * ((f[2] - f[3]) - (f[6] + f[7]));
    a[3] = (0.5f * kC) * ((f[6] - f[7]) - (f[2] + f[3]));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      y[u] = 0.5f * (s[u] + a[u]);
      y[u + 4] = 0.5f * (s[u] - a[u]);
    }
  }
  __device__ __forceinline__ static void adjoint(float* f) { conj_planes<8>(f); }
};

// p4m, the symmetry group of the square: element u = k + 4m is r^k s^m (r the
// rotation by 90 degrees, s a reflection, s r s = r^-1).  The group
// convolution y(g) = sum_h x(h) w(h^-1 g) becomes y_hat(rho) = x_hat(rho)
// w_hat(rho) for every irreducible representation rho, with
// f_hat(rho) = sum_g f(g) rho(g).  The irreducible representations are four
// characters A1, A2, B1, B2 (r -> 1, 1, -1, -1; s -> 1, -1, 1, -1) and the 2-D
// representation E (r -> [[0, -1], [1, 0]], s -> diag(1, -1)).  All their
// entries are 0 or +-1, so with p_k = z_k (rotations), q_k = z_{4+k}
// (reflections), a = p0 + p2, b = p1 + p3, c = q0 + q2, d = q1 + q3 and
// al = p0 - p2, be = p1 - p3, ga = q0 - q2, de = q1 - q3:
//   A1 = a + b + c + d   A2 = a + b - c - d   B1 = a - b + c - d   B2 = a - b - c + d
//   E00 = al + ga   E01 = de - be   E10 = be + de   E11 = al - ga
// Planes: 0 A1, 1 A2, 2 B1, 3 B2, 4 E00, 5 E01, 6 E10, 7 E11.  Inverse
// (Fourier inversion f(g) = 1/8 [sum_chi chi(g) f_chi + 2 tr(E(g)^T F)]):
//   z_0 = P + Q + U   z_1 = P - Q + V   z_2 = P + Q - U   z_3 = P - Q - V
//   z_4 = P' + Q' + U'  z_5 = P' - Q' + V'  z_6 = P' + Q' - U'  z_7 = P' - Q' - V'
// with P = (A1 + A2)/8, Q = (B1 + B2)/8, P' = (A1 - A2)/8, Q' = (B1 - B2)/8,
// U = (E00 + E11)/4, V = (E10 - E01)/4, U' = (E00 - E11)/4, V' = (E01 + E10)/4.
// Products: the four characters pointwise and the 2 x 2 block as a matrix
// product (8 real products).  dX uses the spectrum of w(u^-1), i.e. the 2 x 2
// block transposed; dw_hat = x_hat^T dy_hat per representation.
template <>
struct Grp<kP4M> {
  static constexpr int kOrder = 8;
  static constexpr int kProducts = 12;
  // out[ij] += A[ik] B[kj]
  static constexpr Prod kFwd[kProducts] = {
      {0, 0, 0, false}, {1, 1, 1, false}, {2, 2, 2, false}, {3, 3, 3, false}, {4, 4, 4, false}, {5, 4, 5, false},
      {6, 6, 4, false}, {7, 6, 5, false}, {4, 5, 6, false}, {5, 5, 7, false}, {6, 7, 6, false}, {7, 7, 7, false}};
  // out[ij] += B[ik] A[kj]
  static constexpr Prod kDw[kProducts] = {
      {0, 0, 0, false}, {1, 1, 1, false}, {2, 2, 2, false}, {3, 3, 3, false}, {4, 4, 4, false}, {5, 5, 4, false},
      {6, 4, 6, false}, {7, 5, 6, false}, {4, 6, 5, false}, {5, 7, 5, false}, {6, 6, 7, false}, {7, 7, 7, false}};
  // the characters sum all eight values (<= 8 M); the entries of E four (<= 4 M)
  static constexpr float kF16Scale[kOrder] = {0.125f, 0.125f, 0.125f, 0.125f, 0.25f, 0.25f, 0.25f, 0.25f};
  __device__ __forceinline__ static void dft(const float* z, float* f) {
    const float a = z[0] + z[2], b = z[1] + z[3], c = z[4] + z[6], d = z[5] + z[7];
    const float al = z[0] - z[2], be = z[1] - z[3], ga = z[4] - z[6], de = z[5] - z[7];
    const float ab = a + b, amb = a - b, cd = c + d, cmd = c - d;
    f[0] = ab + cd;
    f[1] = ab - cd;
    f[2] = amb + cmd;
    f[3] = amb - cmd;
    f[4] = al + ga;
    f[5] = de - be;
    f[6] = be + de;
    f[7] = al - ga;
  }
  __device__ __forceinline__ static void idft(const float* f, float* y) {
    const float P = 0.125f * (f[0] + f[1]), Q = 0.125f * (f[2] + f[3]);
    const float P2 = 0.125f * (f[0] - f[1]), Q2 = 0.125f * (f[2] - f[3]);
    const float U = 0.25f * (f[4] + f[7]), V = 0.25f * (f[6] - f[5]);
    const float U2 = 0.25f * (f[4] - f[7]), V2 = 0.25f * (f[5] + f[6]);
    y[0] = (P + Q) + U;
    y[1] = (P - Q) + V;
    y[2] = (P + Q) - U;
    y[3] = (P - Q) - V;
    y[4] = (P2 + Q2) + U2;
    y[5] = (P2 - Q2) + V2;
    y[6] = (P2 + Q2) - U2;
    y[7] = (P2 - Q2) - V2;
  }
  __device__ __forceinline__ static void adjoint(float* f) {
    const float t = f[5];
    f[5] = f[6];
    f[6] = t;
  }
};

// erf(z) by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: for z >= 0, erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5)
// exp(-z^2) with t = 1 / (1 + p z); |error| <= 1.5e-7.  Odd extension for
// z < 0.  exp(-z^2) uses the hardware base-2 exponential.
__device__ __forceinline__ float erf_as7126(float z) {
  const float a = fabsf(z);
  const float t = __frcp_rn(1.0f + 0.3275911f * a);
  const float poly = t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float e = __builtin_amdgcn_exp2f(-a * a * 1.4426950408889634f);
  const float r = 1.0f - poly * e;
  return copysignf(r, z);
}

// erf(z) by Abramowitz & Stegun formula 7.1.27: for z >= 0,
// erf(z) = 1 - 1 / (1 + a1 z + a2 z^2 + a3 z^3 + a4 z^4)^4, |error| <= 5e-4;
// one reciprocal and no exponential.  Odd extension for z < 0.  Used for
// binary16 outputs, whose own rounding (2^-11 relative) is of the same size.
__device__ __forceinline__ float erf_as7127(float z) {
  const float a = fabsf(z);
  const float p = 1.0f + a * (0.278393f + a * (0.230389f + a * (0.000972f + a * 0.078108f)));
  const float p2 = p * p;
  return copysignf(1.0f - __frcp_rn(p2 * p2), z);
}

// GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))), evaluated in float32
// with erf by 7.1.26 for float32 outputs and by 7.1.27 for binary16 ones
template <typename E>
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = x * 0.70710678118654752f;
  return 0.5f * x * (1.0f + (sizeof(E) == 2 ? erf_as7127(z) : erf_as7126(z)));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Buffer resource over [base, base + bytes): raw buffer loads at offsets past
// the range return zeros.  Ranges are clamped below 2^31 so that kOob is
// always out of range.
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7ffffff0ull ? 0x7ffffff0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
// The same resource as four scalar words (an inline-assembly operand).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7ffffff0ull ? 0x7ffffff0u : (uint32_t)bytes;
  const uint64_t a = (uint64_t)(uintptr_t)base;
  auto uni = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); };
  return u32x4{uni((uint32_t)a), uni((uint32_t)(a >> 32) & 0xffffu), uni(n), 0x00020000u};
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Same with a wave-uniform offset added in the scalar operand (a stage
// advance); the range test is made on `off`, which alone decides whether the
// lane reads memory or zeros.
__device__ __forceinline__ u32x4 bload16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Direct global-to-LDS load of 16 bytes per lane (gfx950): lane l's bytes land
// at LDS address lds_addr + 16 l (wave-uniform lds_addr, through M0); a lane
// whose offset is out of the buffer's range writes zeros.  Issued from inline
// assembly so that the compiler's wait-count analysis does not see it: the
// compiler would otherwise wait for every such load before each LDS read.
// The caller orders it so that a wait the compiler emits for a later
// ordinary load also covers it (vector-memory loads complete in issue order),
// and `dep` (any register the asm must follow) pins it after a given
// instruction.  M0 is saved and restored around it.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff, uint32_t dep) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0 ; after %5"
      : "=&s"(keep)
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff), "v"(dep)
      : "memory");
}
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ uint32_t lds_address(const char* p) { return (uint32_t)(uintptr_t)(lds_char*)p; }

// Blocks are dispatched round-robin over the 8 XCDs.  Renumber so that
// consecutive logical tile ids land on the same XCD (and share its L2).
__device__ __forceinline__ int64_t xcd_logical_id(int64_t bid, int64_t nblocks) {
  const int64_t xcd = bid % kNumXcd;
  const int64_t per = nblocks / kNumXcd, rem = nblocks % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + bid / kNumXcd;
}

// Stores the T outputs of one group (float32 results) in the storage type.
template <typename E, int T>
// Output stores are non-temporal (streaming): the layer's output is written
// once and not read back by the kernel, and keeping it out of the caches
// shortens the store bursts of the tile epilogues (measured 6% on the fp32
// ViT-B attention forward, 10-15% on the f16 MLP layers).
__device__ __forceinline__ void store_group(E* dst, const float* y) {
  if constexpr (sizeof(E) == 4) {
#pragma unroll
    for (int i = 0; i < T / 4; ++i)
      __builtin_nontemporal_store(
          __builtin_bit_cast(u32x4, f32x4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]}),
          reinterpret_cast<u32x4*>(dst + 4 * i));
  } else {
    // Every kernel rounds the float32 result to binary16 the same way (float32
    // first, then nearest-even): the empty asm keeps the compiler from folding
    // the inverse transform's last multiply-add into a mixed-precision FMA that
    // rounds once, which it does in some kernels and not in others, so the
    // same output would differ by one unit in the last place between paths.
    float v[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      v[i] = y[i];
      asm volatile("" : "+v"(v[i]));
    }
    if constexpr (T == 4) {
      const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
      __builtin_nontemporal_store(__builtin_bit_cast(u32x2, h), reinterpret_cast<u32x2*>(dst));
    } else {
#pragma unroll
      for (int i = 0; i < T / 8; ++i) {
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (_Float16)v[8 * i + e];
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h), reinterpret_cast<u32x4*>(dst + 8 * i));
      }
    }
  }
}

// The same group store through a buffer resource: offsets at or past its
// range (a row beyond the last, or kOob for a column beyond the last) drop
// the store.  aux 2 = non-temporal.
template <typename E, int T>
__device__ __forceinline__ void store_group_buf(__amdgpu_buffer_rsrc_t dst, uint32_t off, const float* y) {
  constexpr int kNt = 2;
  if constexpr (sizeof(E) == 4) {
#pragma unroll
    for (int i = 0; i < T / 4; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, f32x4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]}), dst, off + 16u * i,
          0, kNt);
  } else {
    // float32 first, then binary16, in every kernel (see store_group); the
    // p4 epilogue without activation instead rounds each output once from
    // its mixed-precision FMA, also alike in every kernel that runs it
    float v[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      v[i] = y[i];
      asm volatile("" : "+v"(v[i]));
    }
    if constexpr (T == 4) {
      const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), dst, off, 0, kNt);
    } else {
#pragma unroll
      for (int i = 0; i < T / 8; ++i) {
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (_Float16)v[8 * i + e];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, h), dst, off + 16u * i, 0, kNt);
      }
    }
  }
}

// T values of one output group (a residual) as float32, read through a buffer
// range like store_group_buf's (out of range: zeros).
template <typename E, int T>
__device__ __forceinline__ void load_group_buf(__amdgpu_buffer_rsrc_t src, uint32_t off, float* v) {
  if constexpr (sizeof(E) == 4) {
#pragma unroll
    for (int i = 0; i < T / 4; ++i) {
      const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(src, off + 16u * i, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = x[e];
    }
  } else if constexpr (T == 4) {
    const f16x4 h = __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(src, off, 0, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (float)h[e];
  } else {
#pragma unroll
    for (int i = 0; i < T / 8; ++i) {
      const f16x8 h = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(src, off + 16u * i, 0, 0));
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * i + e] = (float)h[e];
    }
  }
}

// ------------------------------------------------------ input transforms
//
// T 16-byte pieces fetched in unit order (see Units) hold kVals whole groups
// one after another: group v occupies values v*T .. v*T+T-1.  The transform
// writes the T plane vectors pl[p] whose value v is plane p of group v.
// kConj applies the group's adjoint (conjugate / transposed spectrum).

// f16, T = 4: group DFT of the two groups of one 16-byte piece (registers
// z01 = (z0, z1), z23 = (z2, z3) of group 0 and z45 / z67 of group 1), written
// as packed f16 plane values scaled by Grp<4>::kF16Scale: p0 = (F0_g0,
// F0_g1) / 4, p2 = (F2_g0, F2_g1) / 4, p1r = (Re F1_g0, Re F1_g1) / 2,
// p1i = (+-Im F1_g0, +-Im F1_g1) / 2.  The mixed precision FMA reads f16
// halves (or f32 registers) directly, computes in f32 and rounds the result
// once (nearest-even) into the low or high half of the destination:
//   a = z0 + z2, b = z1 + z3 (f32);  F0/4 = a/4 + b/4;  F2/4 = a/4 - b/4;
//   Re F1/2 = a/2 - z2 (= (z0 - z2)/2);  Im F1/2 = b/2 - z1 (= (z3 - z1)/2,
//   negated when kConj).
template <bool kConj>
__device__ __forceinline__ void dft4_f16_pair(uint32_t z01, uint32_t z23, uint32_t z45, uint32_t z67,
                                              uint32_t& p0, uint32_t& p2, uint32_t& p1r, uint32_t& p1i) {
  static_assert(Grp<4>::kF16Scale[0] == 0.25f && Grp<4>::kF16Scale[1] == 0.25f && Grp<4>::kF16Scale[2] == 0.5f &&
                    Grp<4>::kF16Scale[3] == 0.5f,
                "the p4 f16 transform applies the scales 1/4, 1/4, 1/2, 1/2");
  float a0, b0, a1, b1;
  asm volatile(
      "v_fma_mix_f32 %0, %4, 1.0, %5 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mix_f32 %1, %4, 1.0, %5 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mix_f32 %2, %6, 1.0, %7 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mix_f32 %3, %6, 1.0, %7 op_sel:[1,0,1] op_sel_hi:[1,0,1]"
      : "=&v"(a0), "=&v"(b0), "=&v"(a1), "=&v"(b1)
      : "v"(z01), "v"(z23), "v"(z45), "v"(z67));
  const float bq0 = 0.25f * b0, bq1 = 0.25f * b1;
  asm volatile(
      "v_fma_mixlo_f16 %0, %2, %6, %4 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %3, %6, %5 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixlo_f16 %1, %2, %6, -%4 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %1, %3, %6, -%5 op_sel_hi:[0,0,0]"
      : "=&v"(p0), "=&v"(p2)
      : "v"(a0), "v"(a1), "v"(bq0), "v"(bq1), "s"(0.25f));
  // src2 an f16 half (op_sel_hi 1), selected by op_sel
  asm volatile(
      "v_fma_mixlo_f16 %0, %1, 0.5, -%3 op_sel:[0,0,0] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, 0.5, -%4 op_sel:[0,0,0] op_sel_hi:[0,0,1]"
      : "=&v"(p1r)
      : "v"(a0), "v"(a1), "v"(z23), "v"(z67));
  if constexpr (!kConj) {
    asm volatile(
        "v_fma_mixlo_f16 %0, %1, 0.5, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %0, %2, 0.5, -%4 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
        : "=&v"(p1i)
        : "v"(b0), "v"(b1), "v"(z01), "v"(z45));
  } else {
    asm volatile(
        "v_fma_mixlo_f16 %0, %1, -0.5, %3 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %0, %2, -0.5, %4 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
        : "=&v"(p1i)
        : "v"(b0), "v"(b1), "v"(z01), "v"(z45));
  }
}

// f16, C8: group DFT of two groups (x: group 0, y: group 1; word k holds
// (z_2k, z_2k+1)), written as packed f16 plane values o[p] = (plane p of
// group 0, plane p of group 1) in the plane order of Grp<8>, scaled by
// Grp<8>::kF16Scale (1/8, except 1/4 for F2).  As in dft4_f16_pair the
// mixed-precision FMAs read the f16 halves directly and every plane is
// rounded once to f16 from a float32 expression:
//   s_u = z_u + z_u+4, a_u = z_u - z_u+4 (f32);  A = s0 + s2, B = s1 + s3,
//   t = a1 - a3, v = a1 + a3;  F0/8 = A/8 + B/8, F4/8 = A/8 - B/8,
//   Re F2/4 = A/4 - s2/2, Im F2/4 = B/4 - s1/2, Re F1/8 = a0/8 + (c/8) t,
//   Im F1/8 = -a2/8 - (c/8) v, Re F3/8 = a0/8 - (c/8) t, Im F3/8 = a2/8 - (c/8) v
//   (c = sqrt 1/2; the imaginary planes negated when kConj).
template <bool kConj>
__device__ __forceinline__ void dft8_f16_pair(const u32x4& x, const u32x4& y, uint32_t (&o)[8]) {
  float s[2][4], a[2][4];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const u32x4& z = g == 0 ? x : y;
    asm volatile(
        "v_fma_mix_f32 %0, %8, 1.0, %10 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %1, %8, 1.0, %10 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %2, %9, 1.0, %11 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %3, %9, 1.0, %11 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %4, %8, 1.0, -%10 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %5, %8, 1.0, -%10 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %6, %9, 1.0, -%11 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %7, %9, 1.0, -%11 op_sel:[1,0,1] op_sel_hi:[1,0,1]"
        : "=&v"(s[g][0]), "=&v"(s[g][1]), "=&v"(s[g][2]), "=&v"(s[g][3]), "=&v"(a[g][0]), "=&v"(a[g][1]),
          "=&v"(a[g][2]), "=&v"(a[g][3])
        : "v"(z[0]), "v"(z[1]), "v"(z[2]), "v"(z[3]));
  }
  static_assert(Grp<8>::kF16Scale[0] == 0.125f && Grp<8>::kF16Scale[1] == 0.125f &&
                    Grp<8>::kF16Scale[2] == 0.125f && Grp<8>::kF16Scale[3] == 0.125f &&
                    Grp<8>::kF16Scale[4] == 0.25f && Grp<8>::kF16Scale[5] == 0.25f &&
                    Grp<8>::kF16Scale[6] == 0.125f && Grp<8>::kF16Scale[7] == 0.125f,
                "the C8 f16 transform applies the scales 1/8 (F0, F4, F1, F3) and 1/4 (F2)");
  float A[2], Bq[2], t[2], v[2], s1h[2], s2h[2], a0q[2], a2q[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    A[g] = s[g][0] + s[g][2];
    Bq[g] = 0.125f * (s[g][1] + s[g][3]);
    t[g] = a[g][1] - a[g][3];
    v[g] = a[g][1] + a[g][3];
    s1h[g] = 0.5f * s[g][1];
    s2h[g] = 0.5f * s[g][2];
    a0q[g] = 0.125f * a[g][0];
    a2q[g] = 0.125f * a[g][2];
  }
  const float c8 = 0.125f * Grp<8>::kC;
  // planes 0, 1 (F0/8, F4/8) and 4 (Re F2/4)
  asm volatile(
      "v_fma_mixlo_f16 %0, %3, %9, %5 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %4, %9, %6 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixlo_f16 %1, %3, %9, -%5 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %1, %4, %9, -%6 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixlo_f16 %2, %3, %10, -%7 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %2, %4, %10, -%8 op_sel_hi:[0,0,0]"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[4])
      : "v"(A[0]), "v"(A[1]), "v"(Bq[0]), "v"(Bq[1]), "v"(s2h[0]), "v"(s2h[1]), "s"(0.125f), "s"(0.25f));
  // plane 5 (Im F2/4 = B/4 - s1/2, or its negative), B/4 = 2 Bq
  if constexpr (!kConj) {
    asm volatile(
        "v_fma_mixlo_f16 %0, %1, 2.0, -%3 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %2, 2.0, -%4 op_sel_hi:[0,0,0]"
        : "=&v"(o[5])
        : "v"(Bq[0]), "v"(Bq[1]), "v"(s1h[0]), "v"(s1h[1]));
  } else {
    asm volatile(
        "v_fma_mixlo_f16 %0, %1, -2.0, %3 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %2, -2.0, %4 op_sel_hi:[0,0,0]"
        : "=&v"(o[5])
        : "v"(Bq[0]), "v"(Bq[1]), "v"(s1h[0]), "v"(s1h[1]));
  }
  // planes 2 and 6 (real parts of F1, F3, over 8): a0/8 +- (c/8) t
  asm volatile(
      "v_fma_mixlo_f16 %0, %2, %6, %4 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %3, %6, %5 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixlo_f16 %1, %2, -%6, %4 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %1, %3, -%6, %5 op_sel_hi:[0,0,0]"
      : "=&v"(o[2]), "=&v"(o[6])
      : "v"(t[0]), "v"(t[1]), "v"(a0q[0]), "v"(a0q[1]), "s"(c8));
  // planes 3 and 7 (imaginary parts, over 8): -a2/8 - (c/8) v and a2/8 - (c/8) v, or their negatives
  if constexpr (!kConj) {
    asm volatile(
        "v_fma_mixlo_f16 %0, %2, -%6, -%4 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %3, -%6, -%5 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixlo_f16 %1, %2, -%6, %4 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixhi_f16 %1, %3, -%6, %5 op_sel_hi:[0,0,0]"
        : "=&v"(o[3]), "=&v"(o[7])
        : "v"(v[0]), "v"(v[1]), "v"(a2q[0]), "v"(a2q[1]), "s"(c8));
  } else {
    asm volatile(
        "v_fma_mixlo_f16 %0, %2, %6, %4 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %3, %6, %5 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixlo_f16 %1, %2, %6, -%4 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixhi_f16 %1, %3, %6, -%5 op_sel_hi:[0,0,0]"
        : "=&v"(o[3]), "=&v"(o[7])
        : "v"(v[0]), "v"(v[1]), "v"(a2q[0]), "v"(a2q[1]), "s"(c8));
  }
}

template <typename E, int G, bool kConj>
__device__ __forceinline__ void pieces_to_planes(const u32x4 (&pc)[Grp<G>::kOrder], u32x4 (&pl)[Grp<G>::kOrder]) {
  constexpr int V = Traits<E>::kVals, T = Grp<G>::kOrder;
  if constexpr (sizeof(E) == 2 && G == 8) {
    // piece j is group j; groups 2k and 2k + 1 fill word k of every plane
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t o[8];
      dft8_f16_pair<kConj>(pc[2 * k], pc[2 * k + 1], o);
#pragma unroll
      for (int p = 0; p < 8; ++p) pl[p][k] = o[p];
    }
  } else if constexpr (sizeof(E) == 2 && G == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p0, p2, p1r, p1i;
      dft4_f16_pair<kConj>(pc[j][0], pc[j][1], pc[j][2], pc[j][3], p0, p2, p1r, p1i);
      pl[0][j] = p0;
      pl[1][j] = p2;
      pl[2][j] = p1r;
      pl[3][j] = p1i;
    }
  } else {
    // unpack whole vectors, then index (a bit-cast of one vector element
    // would reinterpret the vector's first element)
    float z[V * T];
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if constexpr (sizeof(E) == 4) {
        const f32x4 x = __builtin_bit_cast(f32x4, pc[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[4 * j + e] = x[e];
      } else {
        const f16x8 x = __builtin_bit_cast(f16x8, pc[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[8 * j + e] = (float)x[e];
      }
    }
    float f[V][T];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      Grp<G>::dft(&z[v * T], f[v]);
      if constexpr (kConj) Grp<G>::adjoint(f[v]);
    }
#pragma unroll
    for (int p = 0; p < T; ++p) {
      if constexpr (sizeof(E) == 4) {
        pl[p] = __builtin_bit_cast(u32x4, f32x4{f[0][p], f[1][p], f[2][p], f[3][p]});
      } else {
        // scaled into the f16 operand range (Grp<G>::kF16Scale, exact)
        f16x8 o;
#pragma unroll
        for (int v = 0; v < 8; ++v) o[v] = (_Float16)(f[v][p] * Grp<G>::kF16Scale[p]);
        pl[p] = __builtin_bit_cast(u32x4, o);
      }
    }
  }
}

// ----------------------------------------------------------- MFMA core
//
// One 16-byte slot per operand plane and fragment; the plane products of the
// group's list (kDwRole: the dw list) run as MFMAs into the T accumulators.
template <int G, bool kDwRole, int I>
__host__ __device__ constexpr Prod product() {
  return (kDwRole ? Grp<G>::kDw : Grp<G>::kFwd)[I];
}

template <int G, bool kDwRole, int FM, int FN, int... I>
__device__ __forceinline__ void products_f32(std::integer_sequence<int, I...>,
                                             f32x16 (&acc)[Grp<G>::kOrder][FM][FN],
                                             const f32x4 (&af)[Grp<G>::kOrder][FM],
                                             const f32x4 (&bf)[Grp<G>::kOrder][FN], int j, int fm, int fn) {
  ((acc[product<G, kDwRole, I>().out][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
        product<G, kDwRole, I>().neg ? -af[product<G, kDwRole, I>().a][fm][j]
                                     : af[product<G, kDwRole, I>().a][fm][j],
        bf[product<G, kDwRole, I>().b][fn][j], acc[product<G, kDwRole, I>().out][fm][fn], 0, 0, 0)),
   ...);
}

// kNegB: a negated product flips the sign of its B operand instead of its A
// operand (the same products; the sign flips cost 4 XORs per plane and
// fragment, so they go to the operand with fewer fragments).
template <int G, bool kDwRole, int FM, int FN, bool kNegB, int... I>
__device__ __forceinline__ void products_f16(std::integer_sequence<int, I...>,
                                             f32x16 (&acc)[Grp<G>::kOrder][FM][FN],
                                             const f16x8 (&av)[Grp<G>::kOrder], const f16x8 (&nav)[Grp<G>::kOrder],
                                             const f16x8 (&bv)[Grp<G>::kOrder], const f16x8 (&nbv)[Grp<G>::kOrder],
                                             int fm, int fn) {
  ((acc[product<G, kDwRole, I>().out][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
        product<G, kDwRole, I>().neg && !kNegB ? nav[product<G, kDwRole, I>().a] : av[product<G, kDwRole, I>().a],
        product<G, kDwRole, I>().neg && kNegB ? nbv[product<G, kDwRole, I>().b] : bv[product<G, kDwRole, I>().b],
        acc[product<G, kDwRole, I>().out][fm][fn], 0, 0, 0)),
   ...);
}

template <typename E, int G, bool kDwRole, int FM, int FN>
struct Core;

template <int G, bool kDwRole, int FM, int FN>
struct Core<float, G, kDwRole, FM, FN> {
  static constexpr int T = Grp<G>::kOrder;
  __device__ __forceinline__ static void mma(f32x16 (&acc)[T][FM][FN], const u32x4 (&a)[T][FM],
                                             const u32x4 (&b)[T][FN]) {
    // bit-cast whole vectors, then index (a bit-cast of one vector element
    // would reinterpret the vector's first element)
    f32x4 af[T][FM], bf[T][FN];
#pragma unroll
    for (int p = 0; p < T; ++p) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) af[p][fm] = __builtin_bit_cast(f32x4, a[p][fm]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) bf[p][fn] = __builtin_bit_cast(f32x4, b[p][fn]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          products_f32<G, kDwRole, FM, FN>(std::make_integer_sequence<int, Grp<G>::kProducts>{}, acc, af, bf, j,
                                           fm, fn);
  }
};

template <int G, bool kDwRole, int FM, int FN>
struct Core<_Float16, G, kDwRole, FM, FN> {
  static constexpr int T = Grp<G>::kOrder;
  __device__ __forceinline__ static void mma(f32x16 (&acc)[T][FM][FN], const u32x4 (&a)[T][FM],
                                             const u32x4 (&b)[T][FN]) {
    constexpr u32x4 kSign = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    constexpr bool kNegB = FN < FM;
    // nbv / nav: the negated operands (only those named by a product are used)
    f16x8 bv[FN][T], nbv[FN][T];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int p = 0; p < T; ++p) {
        bv[fn][p] = __builtin_bit_cast(f16x8, b[p][fn]);
        nbv[fn][p] = __builtin_bit_cast(f16x8, kNegB ? b[p][fn] ^ kSign : b[p][fn]);
      }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      f16x8 av[T], nav[T];
#pragma unroll
      for (int p = 0; p < T; ++p) {
        av[p] = __builtin_bit_cast(f16x8, a[p][fm]);
        nav[p] = __builtin_bit_cast(f16x8, kNegB ? a[p][fm] : a[p][fm] ^ kSign);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        products_f16<G, kDwRole, FM, FN, kNegB>(std::make_integer_sequence<int, Grp<G>::kProducts>{}, acc, av, nav,
                                                bv[fn], nbv[fn], fm, fn);
    }
  }
};

// Reads this lane's 16-byte operand slot of one chunk from every LDS plane
// and runs the core.  a_lds / b_lds point at the lane's slot in plane 0 of its
// first fragment row; plane p is p * a_plane further, fragment fm 32 rows
// further.
template <typename E, int G, bool kDwRole, int FM, int FN>
__device__ __forceinline__ void mma_chunk(f32x16 (&acc)[Grp<G>::kOrder][FM][FN], const char* a_lds, int a_plane,
                                          const char* b_lds, int b_plane, int stride) {
  constexpr int T = Grp<G>::kOrder;
  u32x4 a[T][FM], b[T][FN];
#pragma unroll
  for (int p = 0; p < T; ++p) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) a[p][fm] = ld16(a_lds + p * a_plane + fm * 32 * stride);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) b[p][fn] = ld16(b_lds + p * b_plane + fn * 32 * stride);
  }
  Core<E, G, kDwRole, FM, FN>::mma(acc, a, b);
}

// Instruction interleaving for one pipeline stage of fwd_kernel: spread the
// operand reads of the second chunk, the global loads of a later stage and
// the next stage's transform and LDS writes between the MFMAs, so that one
// wave keeps its matrix core busy while it prepares the next stage.
// Masks: 0x008 MFMA, 0x100 DS read, 0x200 DS write, 0x020 VMEM read, 0x002 VALU.
// CH: k chunks a wave multiplies per stage (2, or 1 in a tail-split half).
template <typename E, int G, int FM, int FN, int PA, int PB, int CH = 2>
__device__ __forceinline__ void interleave_schedule() {
  constexpr int T = Grp<G>::kOrder;
  constexpr int kMfma = (sizeof(E) == 4 ? 4 : 1) * Grp<G>::kProducts * FM * FN * CH;
  constexpr int kDsRead = CH * T * (FM + FN);
  constexpr int kVmem = T * (PA + PB);
  constexpr int kDsWrite = T * (PA + PB);
  constexpr int kHalf = kDsRead / 2;
  __builtin_amdgcn_sched_group_barrier(0x100, kHalf, 0);
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < kHalf) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (i >= kMfma / 4 && i < kMfma / 4 + kVmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    if (i >= kMfma / 2) {
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      if ((i - kMfma / 2) % ((kMfma / 2 + kDsWrite - 1) / kDsWrite) == 0) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
  }
}

// ============================================================ forward / dX
//
// out[n][T m + t] = IDFT_t( sum_k Ahat[n][k] (*) Bhat[m][k] )
// A = in [nrows][T kg] (raw groups, transformed on the fly),
// B = prepared spectra in stage blocks (see prepare_kernel), out [nrows][T mg].
// A stage covers 64 bytes of every plane row: SG = 16 fp32 or 32 f16 groups
// along k.  Thread t owns row t / 4 (+ NT/4 per pass) and 16-byte slot block
// q = t % 4 of that row: it loads the units q + 4i of the stage window
// (coalesced), transforms them and writes the contiguous LDS block q of each
// plane; the prepared weights are stored in that same slot order, so their
// 16-byte pieces are copied to LDS unchanged.  Global loads are buffer loads:
// addresses past the end of the tile's range (rows >= nrows) or flagged out
// of range (groups >= kg) return zeros without branches.
// NBUF = 3 and 4 copy the weight operand by DMA (see fwd_tile): NBUF = 3
// keeps two buffers of the transformed input and three of the weight
// planes, NBUF = 4 one of the input and two of the weights.
template <typename E, int T, int FM, int FN, int WM, int WN, int NBUF>
constexpr int fwd_lds_bytes() {
  return NBUF == 3   ? T * (2 * 32 * FM * WM + 3 * 32 * FN * WN) * kRowBytes
         : NBUF == 4 ? T * (32 * FM * WM + 2 * 32 * FN * WN) * kRowBytes
                     : NBUF * T * (32 * FM * WM + 32 * FN * WN) * kRowBytes;
}

// Epilogue of a forward / dX tile: inverse group DFT in registers, optional
// group-invariant bias and GELU, one vector store per (row, group).
// HALF: a tail-split half, whose fragments all start at the half's row 0.
template <typename E, int G, int FM, int FN, int WM, int WN, bool HALF = false>
__device__ __forceinline__ void fwd_epilogue(const f32x16 (&acc)[Grp<G>::kOrder][FM][FN], int64_t row0, int col0,
                                             E* __restrict__ out, int64_t nrows, int mg,
                                             const E* __restrict__ bias, int act, const E* __restrict__ res) {
  constexpr int T = Grp<G>::kOrder;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = HALF ? 0 : wave / WN, wc = wave % WN;
  const int li = lane & 31, lh = lane >> 5;
  const uint32_t row_bytes = (uint32_t)(T * mg) * (uint32_t)sizeof(E);
  // The tile's rows as one buffer: rows past nrows lie beyond its range and
  // their stores are dropped, as are those of a column past mg (kOob), so the
  // row loop needs no bounds test and only 32-bit offsets.
  const __amdgpu_buffer_rsrc_t dst = make_rsrc(out + row0 * (int64_t)T * mg, (uint64_t)(nrows - row0) * row_bytes);
  // residual rows, read through the same offsets as the stores
  const __amdgpu_buffer_rsrc_t rsd = make_rsrc(res != nullptr ? res + row0 * (int64_t)T * mg : out,
                                               res != nullptr ? (uint64_t)(nrows - row0) * row_bytes : 0);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int m = col0 + wc * 32 * FN + fn * 32 + li;
      const bool mok = m < mg;
      const float bm = (bias != nullptr && mok) ? (float)bias[m] : 0.f;
      const uint32_t lane_off =
          mok ? (uint32_t)(wr * 32 * FM + fm * 32 + 4 * lh) * row_bytes + (uint32_t)m * (uint32_t)(T * sizeof(E))
              : kOob;
      if constexpr (sizeof(E) == 2 && G == 4) {
        if (act == 0 && res == nullptr) {
          // f16 p4 without activation: the accumulators hold F0/16, F2/16
          // and F1/4 (the operand scales), so with a = F0 + F2 and
          // b = F0 - F2 in float32, a / 4 + bias and b / 4 + bias are
          // 4 (acc0 +- acc2) + bias; then each output is one mixed-precision
          // FMA (+- Re F1 / 2 or +- Im F1 / 2, i.e. +- 2 acc) rounded once
          // into its half of the packed store
          static_assert(f16_unscale<4>(0) == 16.f && f16_unscale<4>(1) == 16.f && f16_unscale<4>(2) == 4.f &&
                            f16_unscale<4>(3) == 4.f,
                        "p4 f16 accumulator scales");
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float f0 = acc[0][fm][fn][r], f2 = acc[1][fm][fn][r];
            const float f1r = acc[2][fm][fn][r], f1i = acc[3][fm][fn][r];
            const float qa = __builtin_fmaf(f0 + f2, 4.0f, bm), qb = __builtin_fmaf(f0 - f2, 4.0f, bm);
            uint32_t w0, w1;
            asm volatile(
                "v_fma_mixlo_f16 %0, %2, 2.0, %3 op_sel_hi:[0,0,0]\n\t"
                "v_fma_mixhi_f16 %0, %4, -2.0, %5 op_sel_hi:[0,0,0]\n\t"
                "v_fma_mixlo_f16 %1, %2, -2.0, %3 op_sel_hi:[0,0,0]\n\t"
                "v_fma_mixhi_f16 %1, %4, 2.0, %5 op_sel_hi:[0,0,0]"
                : "=&v"(w0), "=&v"(w1)
                : "v"(f1r), "v"(qa), "v"(f1i), "v"(qb));
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, dst,
                                                  lane_off + (uint32_t)(8 * (r >> 2) + (r & 3)) * row_bytes, 0, 2);
          }
          continue;
        }
      }
      // The residual rows of a chunk of RC rows are all read before any of
      // them is written.  The residual may be `out` itself (in place), so the
      // compiler cannot move a row's load above the previous row's store;
      // each thread reads and writes only its own elements, so reading ahead
      // is safe, and the loads' latencies then overlap instead of adding up
      // row by row.
      constexpr int RC = T == 4 ? 16 : 8;
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += RC) {
        float rv[RC][T];
        if (res != nullptr) {
#pragma unroll
          for (int i = 0; i < RC; ++i) {
            const int r = r0 + i;
            load_group_buf<E, T>(rsd, lane_off + (uint32_t)(8 * (r >> 2) + (r & 3)) * row_bytes, rv[i]);
          }
        }
#pragma unroll
        for (int i = 0; i < RC; ++i) {
          const int r = r0 + i;
          float f[T], y[T];
          // f16: undo the operand scales (exact powers of two)
#pragma unroll
          for (int p = 0; p < T; ++p)
            f[p] = sizeof(E) == 2 ? acc[p][fm][fn][r] * f16_unscale<G>(p) : acc[p][fm][fn][r];
          Grp<G>::idft(f, y);
          if (bias != nullptr) {
#pragma unroll
            for (int t = 0; t < T; ++t) y[t] += bm;
          }
          if (act == 1) {
#pragma unroll
            for (int t = 0; t < T; ++t) y[t] = gelu_erf<E>(y[t]);
          }
          if (res != nullptr) {
#pragma unroll
            for (int t = 0; t < T; ++t) y[t] += rv[i][t];
          }
          store_group_buf<E, T>(dst, lane_off + (uint32_t)(8 * (r >> 2) + (r & 3)) * row_bytes, y);
        }
      }
    }
  }
}

// ============================================================ p4 group convolution gather
//
// A p4 group convolution with a K x K filter (K = 2p + 1) is one group-
// circulant layer over a gathered row per output pixel.  The row's group
// channels are the centre taps (channel c', rotations m = 0..3 read at the
// pixel itself) and, for every quarter-turn orbit {R^m delta_o, m = 0..3} of
// the other taps (delta_o = (a, b), a = 1..p, b = 0..p; R(a, b) = (-b, a))
// and every shift b of the rotation axis, the four values
// f[x + R^m delta_o, c', (m + b) mod 4].  The lane slot of a stage is filled
// by one block: a centre block holds 4 G consecutive channels at the pixel
// (G = group channels per 16-byte load), an orbit block the G channels
// cg G .. cg G + G - 1 at the four taps of one orbit, one 16-byte load per
// tap; the shifts b are the diagonals of those loads' (tap, rotation) values.
// Block cb's unit i lands at group channel (cb / 4) 16 G + G (cb % 4 + 4 i).
struct ConvGeom {
  int H, W;              // image height and width (pixels)
  int cpix;              // group channels per input pixel
  int p;                 // filter half width
  int ncb;               // centre blocks: cpix / (4 G)
  int bpo;               // blocks per orbit: cpix / G
  int nblk;              // blocks per gathered row: cpix K^2 / (4 G)
  float inv_bpo, inv_p1; // 1 / bpo and 1 / (p + 1), for the block decode
  uint32_t in_bytes;     // bytes of the input map (< 2^31)
  uint32_t w_mul, hw_mul;  // floor(n / W) = (n w_mul) >> w_shift for n < 2^31 (same for H W)
  int w_shift, hw_shift;
};

// floor(n / d) for n < 2^31 with mul = ceil(2^shift / d), shift = 31 + ceil(log2 d)
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t mul, int shift) {
  return (uint32_t)(((uint64_t)n * mul) >> shift);
}

struct ConvBlock {
  int ch0, chstep;  // group channel of unit i: ch0 + chstep i
  int di[4], dj[4]; // tap of unit i (pixel offset)
  bool live, centre;
};

// floor(n / d) for 0 <= n < 2^22 from a float estimate, corrected by one either way.
__device__ __forceinline__ int div_small(int n, int d, float inv_d) {
  int q = (int)((float)n * inv_d);
  q += (q + 1) * d <= n ? 1 : 0;
  q -= q * d > n ? 1 : 0;
  return q;
}

template <int G>
__device__ __forceinline__ ConvBlock conv_block(int cb, const ConvGeom& g) {
  ConvBlock k;
  k.live = cb < g.nblk;
  k.centre = cb < g.ncb;
  const int cbo = k.centre ? 0 : cb - g.ncb;
  const int o = div_small(cbo, g.bpo, g.inv_bpo);
  const int oa = div_small(o, g.p + 1, g.inv_p1);
  const int a = 1 + oa, b = o - oa * (g.p + 1);
  k.ch0 = k.centre ? cb * 4 * G : (cbo - o * g.bpo) * G;
  k.chstep = k.centre ? G : 0;
  const int ta[4] = {a, -b, -a, b}, tb[4] = {b, a, -b, -a};  // R^m (a, b)
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    k.di[m] = k.centre ? 0 : ta[m];
    k.dj[m] = k.centre ? 0 : tb[m];
  }
  return k;
}

// The four loads M[m] of a block -> the four pieces of its group channels:
// orbit block, piece b value m = M[m] at rotation (m + b) mod 4 (per channel
// of the piece); centre block, the loads themselves.
template <typename E>
__device__ __forceinline__ void conv_diag(const u32x4 (&M)[4], bool centre, u32x4 (&pc)[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t d;
      if constexpr (sizeof(E) == 4) {
        d = M[k][(k + b) & 3];
      } else {
        const int e = k >> 1, m0 = 2 * (k & 1);
        const int hl = 4 * e + ((m0 + b) & 3), hh = 4 * e + ((m0 + 1 + b) & 3);
        const uint32_t lo = (M[m0][hl >> 1] >> (16 * (hl & 1))) & 0xffffu;
        const uint32_t hi = (M[m0 + 1][hh >> 1] >> (16 * (hh & 1))) & 0xffffu;
        d = lo | (hi << 16);
      }
      pc[b][k] = centre ? M[b][k] : d;
    }
  }
}

// K split of a tail tile (float32): the tile's k stages are cut into
// `nparts` consecutive ranges, each multiplied by its own workgroup (a
// part).  Every part writes its accumulators to its slot of the workspace
// and counts itself in the tile's arrival counter; the part that arrives
// last adds the parts' sums in the fixed order 0, 1, .., nparts - 1 (so the
// result does not depend on which part came last), runs the tile's epilogue
// and returns the counter to zero for the next launch.  Nothing waits on
// another workgroup: each part only counts and leaves, or, if last, reduces.
struct KPiece {
  float* ws;       // the tile's nparts slots of kpiece_slot_bytes
  uint32_t* cnt;   // the tile's arrival counter (zero between launches)
  int part, nparts, k0, kn;   // this part, the part count (<= kMaxKParts), its first stage and stage count
};

// Cache policy of a buffer access with device scope (the SC1 bit): the
// access is coherent across the whole GPU, past the per-XCD L2 caches.
constexpr int kScopeDevice = 16;

// Bytes of one part's accumulators: every lane's T FM FN 32 x 32 fragments
// as 16-byte pieces, lane-minor (each store instruction writes 1 KB).
template <int T, int FM, int FN, int NT>
constexpr uint32_t kpiece_slot_bytes() {
  return (uint32_t)(NT / 64) * T * FM * FN * 4 * 64 * 16;
}

// Returns true in the part that arrived last, with acc holding the tile's
// whole sums; false in every other part (which then has nothing left to do).
// LDS must be free (after the stage loop's last barrier): one word of it
// broadcasts the arrival count.
template <int T, int FM, int FN, int NT>
__device__ __forceinline__ bool kpiece_reduce(f32x16 (&acc)[T][FM][FN], char* lds, const KPiece& kp) {
  constexpr int CH = T * FM * FN * 4;   // 16-byte pieces per lane
  constexpr uint32_t kSlot = kpiece_slot_bytes<T, FM, FN, NT>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t slots = make_rsrc(kp.ws, (uint64_t)kp.nparts * kSlot);
  const uint32_t base = (uint32_t)(wave * CH * 64 + lane) * 16u;
  const uint32_t mine = (uint32_t)kp.part * kSlot + base;
  // planes per round of reads: eight 16-byte pieces of every part in
  // flight for the tiles of one or two fragments per wave and plane (one
  // plane, sixteen pieces, for four), few enough registers to keep the
  // kernel's occupancy (the 64 x 64 tile: 166 registers, three waves per SIMD)
  constexpr int kPlanesPerRound = FM * FN == 1 ? 2 : 1;
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = ((p * FM + fm) * FN + fn) * 4 + j;
          const f32x4 v = {acc[p][fm][fn][4 * j], acc[p][fm][fn][4 * j + 1], acc[p][fm][fn][4 * j + 2],
                           acc[p][fm][fn][4 * j + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), slots, mine + (uint32_t)c * 1024u, 0,
                                                 kScopeDevice);
        }
  // The sums are written and read with device scope (coherent across the
  // XCDs' L2 caches, as the device-scope atomics are), so no cache-wide
  // write-back or invalidation is needed, which an agent-scope fence would
  // issue (and which costs every other workgroup on the XCD its cached
  // operands).  Ordering: every lane's stores have completed (vmcnt 0)
  // before the barrier that precedes the count, and the reads below are
  // issued after the count has returned.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint32_t* flag = reinterpret_cast<uint32_t*>(lds);
  if (threadIdx.x == 0) *flag = __hip_atomic_fetch_add(kp.cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*flag != (uint32_t)(kp.nparts - 1)) return false;   // workgroup-uniform
  if (threadIdx.x == 0) __hip_atomic_store(kp.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // every part's sums, this one's included (its own stores are visible to
  // it), read a round of planes at a time: all of a round's reads are issued
  // before any is added, so that their latencies overlap
  constexpr int kRounds = T / kPlanesPerRound, kRc = kPlanesPerRound * FM * FN * 4;   // pieces per round
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    f32x4 v[kRc][kMaxKParts];
#pragma unroll
    for (int c = 0; c < kRc; ++c) {
      const uint32_t off = base + (uint32_t)(r * kRc + c) * 1024u;
#pragma unroll
      for (int i = 0; i < kMaxKParts; ++i)   // parts past nparts read as zeros (no memory access)
        v[c][i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                slots, i < kp.nparts ? (uint32_t)i * kSlot + off : kOob, 0,
                                                kScopeDevice));
    }
#pragma unroll
    for (int c = 0; c < kRc; ++c) {
      // ((v0 + v1) + v2) + v3: a fixed order; the zeros past nparts add exactly
      f32x4 sum = v[c][0];
#pragma unroll
      for (int i = 1; i < kMaxKParts; ++i)
        sum = f32x4{sum[0] + v[c][i][0], sum[1] + v[c][i][1], sum[2] + v[c][i][2], sum[3] + v[c][i][3]};
      asm volatile("" : "+v"(sum));   // the sum is formed here, not sunk into the epilogue
      const int cc = r * kRc + c, j = cc % 4, fn = (cc / 4) % FN, fm = (cc / (4 * FN)) % FM, p = cc / (4 * FN * FM);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[p][fm][fn][4 * j + e] = sum[e];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return true;
}

// One forward (or dX) tile: workgroup-level logical tile id `lid`.  NBUF = 2
// double-buffers the LDS stages (one barrier per stage); NBUF = 1 halves the
// LDS footprint (two barriers per stage) so that more workgroups fit a CU.
// PF (1 or 2) is the number of stages whose global loads are in flight in
// registers ahead of the stage being transformed into LDS.
// CONV: the A rows are output pixels of a p4 group convolution whose
// gathered rows (see ConvGeom) are read straight from the input map `in`.
// HALF: lid = 2 tile + h runs rows h BM/2 .. h BM/2 + BM/2 - 1 of the tile
// (tail split): wave row wr multiplies k chunk wr of every stage for all of
// those rows and the two rows' sums are added through LDS.
// KS: one part of a K-split tail tile (see KPiece): stages kp.k0 ..
// kp.k0 + kp.kn - 1 of tile lid, then kpiece_reduce before the epilogue.
template <typename E, int G, int FM, int FN, int WM, int WN, int NBUF, int PF, int SCHED, bool CONV = false,
          bool HALF = false, bool KS = false>
__device__ __forceinline__ void fwd_tile(char* lds, int64_t lid, const E* __restrict__ in,
                                         const E* __restrict__ wp, E* __restrict__ out, int64_t nrows, int kg,
                                         int mg, int tiles_n, const E* __restrict__ bias, int act,
                                         const E* __restrict__ res, const ConvGeom& geo = ConvGeom{},
                                         const KPiece& kp = KPiece{}) {
  constexpr int T = Grp<G>::kOrder;
  using U = Units<E, T>;
  constexpr int NT = 64 * WM * WN;
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  constexpr int SG = Traits<E>::kStageGroups;
  constexpr int STRIDE = kRowBytes;
  constexpr int A_PLANE = BM * STRIDE, B_PLANE = BN * STRIDE;
  constexpr int BUF = T * (A_PLANE + B_PLANE);
  constexpr int BLOCK = T * kRowBytes;      // bytes of one prepared stage block
  constexpr int RPP = NT / 4;               // tile rows covered per load pass
  constexpr int PA = (BM + RPP - 1) / RPP, PB = (BN + RPP - 1) / RPP;
  // NBUF = 3: the weight operand goes from memory straight into LDS (dma16)
  // through three buffers, two stages ahead like the input's register ring;
  // the transformed input keeps two buffers.  NBUF = 4: one input buffer
  // (two barriers per stage, as NBUF = 1) and two weight buffers, the copy
  // one stage ahead.  Otherwise NBUF buffers of both.
  constexpr bool kDma = NBUF >= 3;
  constexpr int kXB = NBUF == 3 ? 2 : 1, kWB = NBUF == 3 ? 3 : 2;
  constexpr int XBUF = kDma ? T * A_PLANE : BUF, WBUF = kDma ? T * B_PLANE : BUF;
  static_assert((kDma ? kXB * XBUF + kWB * WBUF : NBUF * BUF) == fwd_lds_bytes<E, T, FM, FN, WM, WN, NBUF>(),
                "LDS size");
  static_assert(!HALF || fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF), "tail split");
  static_assert(!kDma || (PF == 1 && !HALF), "weight DMA: one register stage, whole tiles");
  static_assert(!KS || (!kDma && !HALF && !CONV && fwd_ksplit_fits(sizeof(E) == 4, T, NBUF, 0)),
                "K split: float32 p4 register-path tiles");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tile = HALF ? lid >> 1 : lid;
  const int64_t row0 = (tile / tiles_n) * BM + (HALF ? (lid & 1) * (BM / 2) : 0);
  const int col0 = (int)(tile % tiles_n) * BN;
  // kst: stages of the whole k range (the prepared rows' stride); a K-split
  // part multiplies stages kb .. kb + ksteps - 1, whose groups end at kend
  const int kst = (kg + SG - 1) / SG;
  const int kb = KS ? kp.k0 : 0;
  const int ksteps = KS ? kp.kn : kst;
  const int kend = KS ? (kg < (kp.k0 + kp.kn) * SG ? kg : (kp.k0 + kp.kn) * SG) : kg;
  if (HALF && row0 >= nrows) return;   // second half of a last tile with no rows there (uniform)
  // this workgroup's rows end at row_end; the A range stops there, so the
  // unused rows of a half read zeros without memory traffic
  const int64_t row_end = HALF ? (nrows < row0 + BM / 2 ? nrows : row0 + BM / 2) : nrows;

  const uint32_t row_bytes = (uint32_t)kg * (uint32_t)(T * sizeof(E));
  const __amdgpu_buffer_rsrc_t a_src =
      CONV ? make_rsrc(in, geo.in_bytes) : make_rsrc(in + row0 * T * (int64_t)kg, (uint64_t)(row_end - row0) * row_bytes);
  const __amdgpu_buffer_rsrc_t b_src =
      make_rsrc(wp + (int64_t)col0 * kst * SG * T, (uint64_t)(mg - col0) * (uint64_t)kst * BLOCK);

  const int q = tid & 3, rl = tid >> 2;
  // Weight DMA: a stage's T x BN plane rows are blocks of 16 rows (1 KB,
  // one DMA of a wave); wave w copies blocks w KD .. w KD + KD - 1.  Lane l
  // fills physical slot l % 4 of block row l / 4, so it reads the logical
  // slot that the XOR swizzle puts there (bits 2-3 of the row are bits 4-5
  // of l).  Rows past the layer's groups are out of range and land as zeros.
  constexpr int KD = kDma ? T * BN / 16 / (NT / 64) : 1;
  static_assert(!kDma || KD * (NT / 64) * 16 == T * BN, "whole 16-row blocks per wave");
  u32x4 b_words{};
  uint32_t dma_off[KD], dma_lds[KD];
  if constexpr (kDma) {
    b_words = rsrc_words(wp + (int64_t)col0 * kst * SG * T, (uint64_t)(mg - col0) * (uint64_t)kst * BLOCK);
#pragma unroll
    for (int i = 0; i < KD; ++i) {
      const int j = wave * KD + i, p = j / (BN / 16), blk = j % (BN / 16);
      const int m = blk * 16 + (lane >> 2), slot = (lane & 3) ^ ((lane >> 4) & 3);
      dma_off[i] = (uint32_t)m * (uint32_t)kst * BLOCK + p * 64 + slot * 16;
      dma_lds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(p * B_PLANE + blk * 16 * STRIDE));
    }
  }
  // W buffer of stage s (DMA mode) and its LDS address
  auto wbuf = [&](int s) -> char* { return lds + kXB * XBUF + (s % kWB) * WBUF; };
  // copy the weight block of stage ks into its buffer; `dep` orders the copy
  // after the input loads it follows (see step)
  auto dma_w = [&](int ks, uint32_t dep) {
    const uint32_t soffb = __builtin_amdgcn_readfirstlane((uint32_t)(kb + (ks < ksteps ? ks : ksteps - 1)) * (uint32_t)BLOCK);
    const uint32_t base = lds_address(wbuf(ks));
#pragma unroll
    for (int i = 0; i < KD; ++i) dma16(b_words, __builtin_amdgcn_readfirstlane(base + dma_lds[i]), dma_off[i], soffb, dep);
  };
  u32x4 ra[PF][PA][T], rb[PF][PB][T];   // register ring of PF stages of loads

  // convolution: pixel of each A row this lane loads, and per ring slot
  // whether its block is a centre block
  int py[PA], px[PA];
  uint32_t pbase[PA];
  bool prow[PA], cen[PF];
  if constexpr (CONV) {
    static_assert(T == 4 && U::kPiecesPerUnit == 1, "p4 convolution");
#pragma unroll
    for (int ps = 0; ps < PA; ++ps) {
      const int64_t n = row0 + ps * RPP + rl;
      prow[ps] = n < row_end;
      const int nn = prow[ps] ? (int)n : 0;
      const int hw = geo.H * geo.W;
      const int img = nn / hw, rem = nn - img * hw;
      py[ps] = rem / geo.W;
      px[ps] = rem - py[ps] * geo.W;
      pbase[ps] = (uint32_t)nn * (uint32_t)(geo.cpix * T * sizeof(E));
    }
  }
  auto load = [&](int ks, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
    if constexpr (CONV) {
      const ConvBlock k = conv_block<U::kGroupsPerUnit>(4 * ks + q, geo);
      cen[sl] = k.centre;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int delta = ((k.di[i] * geo.W + k.dj[i]) * geo.cpix + k.ch0 + k.chstep * i) * (int)(T * sizeof(E));
#pragma unroll
        for (int ps = 0; ps < PA; ++ps) {
          const bool ok = k.live && prow[ps] && (unsigned)(py[ps] + k.di[i]) < (unsigned)geo.H &&
                          (unsigned)(px[ps] + k.dj[i]) < (unsigned)geo.W;
          ra[sl][ps][i] = bload16(a_src, ok ? pbase[ps] + (uint32_t)delta : kOob);
        }
      }
    } else {
      // the stage advance is wave-uniform (scalar offset); a unit reads only
      // below the row's last group channel (lim <= 0 past the last stage)
      const int lim = kend - (kb + ks) * SG;
      const uint32_t soff = (uint32_t)((kb + ks) * SG) * (uint32_t)(T * sizeof(E));
#pragma unroll
      for (int ps = 0; ps < PA; ++ps) {
        const uint32_t r = (uint32_t)(ps * RPP + rl);
#pragma unroll
        for (int i = 0; i < U::kUnits; ++i) {
          const int u = (q + 4 * i) * U::kGroupsPerUnit;
#pragma unroll
          for (int h = 0; h < U::kPiecesPerUnit; ++h) {
            const uint32_t off = u < lim ? r * row_bytes + (uint32_t)u * (uint32_t)(T * sizeof(E)) + 16u * h : kOob;
            ra[sl][ps][i * U::kPiecesPerUnit + h] = bload16s(a_src, off, soff);
          }
        }
      }
    }
    // weights: past the last stage the loads re-read it (the pipeline's idle
    // stage, never multiplied), so the scalar offset stays inside each row
    if constexpr (!kDma) {
      const uint32_t soffb = (uint32_t)(kb + (ks < ksteps ? ks : ksteps - 1)) * (uint32_t)BLOCK;
#pragma unroll
      for (int ps = 0; ps < PB; ++ps) {
        const uint32_t m = (uint32_t)(ps * RPP + rl);
#pragma unroll
        for (int p = 0; p < T; ++p)
          rb[sl][ps][p] = bload16s(b_src, m * (uint32_t)kst * BLOCK + p * 64 + q * 16, soffb);
      }
    }
  };
  // Transform the input registers of a stage into buf; in DMA mode first
  // copy the weight block of stage dma_ks, after every input register of the
  // stage has arrived (the copy's operand `dep` is made of them).
  auto store = [&](char* buf, auto slot_c, int dma_ks) {
    constexpr int sl = decltype(slot_c)::value;
    if constexpr (NBUF == 3) {
      uint32_t dep = 0;
#pragma unroll
      for (int ps = 0; ps < PA; ++ps)
#pragma unroll
        for (int i = 0; i < T; ++i) dep ^= ra[sl][ps][i][0];
      dma_w(dma_ks, dep);
    }
#pragma unroll
    for (int ps = 0; ps < PA; ++ps) {
      const int r = ps * RPP + rl;
      if (BM % RPP == 0 || r < BM) {
        u32x4 pl[T];
        if constexpr (CONV) {
          u32x4 pcs[T];
          conv_diag<E>(ra[sl][ps], cen[sl], pcs);
          pieces_to_planes<E, G, false>(pcs, pl);
        } else {
          pieces_to_planes<E, G, false>(ra[sl][ps], pl);
        }
#pragma unroll
        for (int p = 0; p < T; ++p) st16(buf + p * A_PLANE + r * STRIDE + swz_slot(r, q) * 16, pl[p]);
      }
    }
#pragma unroll
    for (int ps = 0; ps < (kDma ? 0 : PB); ++ps) {
      const int m = ps * RPP + rl;
      if (BN % RPP == 0 || m < BN) {
#pragma unroll
        for (int p = 0; p < T; ++p)
          st16(buf + T * A_PLANE + p * B_PLANE + m * STRIDE + swz_slot(m, q) * 16, rb[sl][ps][p]);
      }
    }
  };

  f32x16 acc[T][FM][FN];
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[p][fm][fn] = f32x16{};

  const int wr = wave / WN, wc = wave % WN;
  const int li = lane & 31, lh = lane >> 5;
  // fragment rows differ from li by multiples of 32, so the swizzle of every
  // row this lane reads is that of li
  const int a_frag = ((HALF ? 0 : wr * 32 * FM) + li) * STRIDE;
  const int b_frag = T * A_PLANE + (wc * 32 * FN + li) * STRIDE;
  const int c0 = swz_slot(li, lh) * 16, c1 = swz_slot(li, 2 + lh) * 16;
  const int cw = swz_slot(li, 2 * wr + lh) * 16;   // HALF: this wave row's k chunk

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, PF - 1>;
  // One pipeline step: multiply stage ks (LDS buffer of ks), then transform
  // the registers of stage ks + 1 into the other (or, single-buffered, the
  // same) buffer and issue the loads of stage ks + 1 + PF into the slot just
  // freed.  Past the last stage the loads read zeros (out of range) and the
  // stores fill an idle buffer, so the body is one basic block in which the
  // scheduler can interleave MFMAs with the transform, LDS writes and loads.
  //
  // DMA mode: the weight block of stage ks + 2 is copied during step ks, into
  // the buffer stage ks - 1 used (free since the previous barrier), right
  // after the input registers of stage ks + 1 have arrived and before the
  // input loads of stage ks + 2 are issued.  Loads complete in issue order,
  // so the wait for those input registers in step ks + 1 (before they are
  // transformed, and so before that step's barrier) also covers the copy.
  auto step = [&](int ks, auto slot_next) {
    // NBUF = 4: the next stage's weight block goes into the buffer stage
    // ks - 1 read (free since the barrier that closed step ks - 1).  The copy
    // follows the input loads of stage ks + 1 and precedes, as a memory
    // barrier in program order, every load issued after it; the compiler's
    // wait for those input registers in this step's store (before the second
    // barrier) may leave only such later loads outstanding, so it completes
    // the copy too (loads complete in issue order)
    if constexpr (NBUF == 4) dma_w(ks + 1, 0u);
    const char* cur = lds + (NBUF == 3 ? (ks & 1) * XBUF : NBUF == 2 ? (ks & 1) * BUF : 0);
    const char* bcur = kDma ? wbuf(ks) - T * A_PLANE : cur;   // b_frag counts from the A planes
    if constexpr (HALF) {
      mma_chunk<E, G, false, FM, FN>(acc, cur + a_frag + cw, A_PLANE, bcur + b_frag + cw, B_PLANE, STRIDE);
    } else {
      mma_chunk<E, G, false, FM, FN>(acc, cur + a_frag + c0, A_PLANE, bcur + b_frag + c0, B_PLANE, STRIDE);
      mma_chunk<E, G, false, FM, FN>(acc, cur + a_frag + c1, A_PLANE, bcur + b_frag + c1, B_PLANE, STRIDE);
    }
    if constexpr (NBUF == 1 || NBUF == 4) __syncthreads();   // every wave is done reading the only buffer
    store(lds + (NBUF == 3 ? ((ks + 1) & 1) * XBUF : NBUF == 2 ? ((ks + 1) & 1) * BUF : 0), slot_next, ks + 2);
    load(ks + 1 + PF, slot_next);
    // (the DMA mode runs faster with the compiler's own order: measured)
    if constexpr (SCHED == 1 && NBUF == 2 && !HALF) interleave_schedule<E, G, FM, FN, PA, PB>();
    __syncthreads();
  };

  stage_mark(0);
  if constexpr (kDma) dma_w(0, 0u);   // issued before the input loads of stage 0
  load(0, S0{});
  store(lds, S0{}, 1);
  if constexpr (PF == 1) {
    load(1, S0{});
    __syncthreads();
    stage_mark(1);
    for (int ks = 0; ks < ksteps; ++ks) {
      step(ks, S0{});
      if (ks == 0) stage_mark(2);
    }
    stage_mark(3);
    // the last steps' copies (of the idle stages past the end) must land
    // before the workgroup can leave its LDS
    if constexpr (kDma) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    // ring: stage s lives in slot (s + 1) % 2 once stage 0 has been stored
    load(1, S1{});
    load(2, S0{});
    __syncthreads();
    for (int ks = 0; ks < ksteps; ks += 2) {
      step(ks, S1{});
      if (ks + 1 >= ksteps) break;
      step(ks + 1, S0{});
    }
  }

  if constexpr (KS) {
    if (!kpiece_reduce<T, FM, FN, NT>(acc, lds, kp)) return;
  }
  if constexpr (HALF) {
    // after the last stage's barrier LDS is free: wave row 1 leaves its sums
    // there (16-byte pieces, lane-minor) and wave row 0 adds them
    f32x4* red = reinterpret_cast<f32x4*>(lds) + wc * (T * FM * FN * 4 * 64) + lane;
    if (wr == 1) {
#pragma unroll
      for (int p = 0; p < T; ++p)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              red[(((p * FM + fm) * FN + fn) * 4 + j) * 64] =
                  f32x4{acc[p][fm][fn][4 * j], acc[p][fm][fn][4 * j + 1], acc[p][fm][fn][4 * j + 2],
                        acc[p][fm][fn][4 * j + 3]};
    }
    __syncthreads();
    if (wr == 1) return;
#pragma unroll
    for (int p = 0; p < T; ++p) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 v = red[(((p * FM + fm) * FN + fn) * 4 + j) * 64];
            f32x4 s = {acc[p][fm][fn][4 * j] + v[0], acc[p][fm][fn][4 * j + 1] + v[1],
                       acc[p][fm][fn][4 * j + 2] + v[2], acc[p][fm][fn][4 * j + 3] + v[3]};
            asm volatile("" : "+v"(s));   // the sum is formed here, not in the epilogue
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[p][fm][fn][4 * j + e] = s[e];
          }
      asm volatile("" ::: "memory");   // one plane's reads in flight at a time
    }
  }
  fwd_epilogue<E, G, FM, FN, WM, WN, HALF>(acc, row0, col0, out, row_end, mg, bias, act, res);
  stage_mark(62);
  stage_mark_drained();
}

// Persistent forward: workgroup `first` runs the tiles first, first + stride,
// first + 2 stride, ... (< ntiles) as one stream of pipeline stages.  A tile's
// epilogue runs right after its last stage, when the loads of the next tile's
// first stages are already in flight and its LDS stage is stored, and its
// global stores drain behind the next tile's MFMAs; no workgroup launch,
// prologue or store drain separates the tiles.  The stage pipeline, LDS
// layout and transforms are those of fwd_tile.
template <typename E, int G, int FM, int FN, int WM, int WN, int NBUF, int PF, int SCHED>
__device__ __forceinline__ void fwd_stream(char* lds, int64_t first, int64_t stride, int64_t ntiles,
                                           const E* __restrict__ in, const E* __restrict__ wp, E* __restrict__ out,
                                           int64_t nrows, int kg, int mg, int tiles_n, const E* __restrict__ bias,
                                           int act, const E* __restrict__ res) {
  constexpr int T = Grp<G>::kOrder;
  using U = Units<E, T>;
  constexpr int NT = 64 * WM * WN;
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  constexpr int SG = Traits<E>::kStageGroups;
  constexpr int STRIDE = kRowBytes;
  constexpr int A_PLANE = BM * STRIDE, B_PLANE = BN * STRIDE;
  constexpr int BUF = T * (A_PLANE + B_PLANE);
  constexpr int BLOCK = T * kRowBytes;
  constexpr int RPP = NT / 4;
  constexpr int PA = (BM + RPP - 1) / RPP, PB = (BN + RPP - 1) / RPP;

  if (first >= ntiles) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ksteps = (kg + SG - 1) / SG;
  const int64_t nt = (ntiles - first + stride - 1) / stride;
  const int64_t S = nt * ksteps;
  const uint32_t row_bytes = (uint32_t)kg * (uint32_t)(T * sizeof(E));

  const int q = tid & 3, rl = tid >> 2;
  u32x4 ra[PF][PA][T], rb[PF][PB][T];
  // Load cursor: the loads are issued for consecutive global stages, so the
  // cursor steps through (tile, stage) with selects only (no division, no
  // branch: the stage loop stays one basic block).  Past the stream's last
  // stage the loads read zeros.
  const int64_t sq = stride / tiles_n;
  const int sr = (int)(stride % tiles_n);
  int lks = 0, lcol = (int)(first % tiles_n);
  int64_t lrow = first / tiles_n, lleft = S;
  auto load = [&](auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
    const int ks = lks;
    const int kcap = lleft > 0 ? kg : 0;           // no live stage left: every load out of range
    const int64_t row0 = lrow * BM;
    const int col0 = lcol * BN;
    const __amdgpu_buffer_rsrc_t a_src =
        make_rsrc(in + row0 * T * (int64_t)kg, (uint64_t)(nrows > row0 ? nrows - row0 : 0) * row_bytes);
    const __amdgpu_buffer_rsrc_t b_src =
        make_rsrc(wp + (int64_t)col0 * ksteps * SG * T, (uint64_t)(mg - col0) * (uint64_t)ksteps * BLOCK);
#pragma unroll
    for (int ps = 0; ps < PA; ++ps) {
      const uint32_t r = (uint32_t)(ps * RPP + rl);
#pragma unroll
      for (int i = 0; i < U::kUnits; ++i) {
        const int g = ks * SG + (q + 4 * i) * U::kGroupsPerUnit;
#pragma unroll
        for (int h = 0; h < U::kPiecesPerUnit; ++h) {
          const uint32_t off = g < kcap ? r * row_bytes + (uint32_t)g * (uint32_t)(T * sizeof(E)) + 16u * h : kOob;
          ra[sl][ps][i * U::kPiecesPerUnit + h] = bload16(a_src, off);
        }
      }
    }
#pragma unroll
    for (int ps = 0; ps < PB; ++ps) {
      const uint32_t m = (uint32_t)(ps * RPP + rl);
#pragma unroll
      for (int p = 0; p < T; ++p)
        rb[sl][ps][p] =
            bload16(b_src, kcap > 0 ? (m * (uint32_t)ksteps + (uint32_t)ks) * BLOCK + p * 64 + q * 16 : kOob);
    }
    // advance the cursor by one stage (selects only)
    --lleft;
    const bool wrap = ++lks == ksteps;
    lks = wrap ? 0 : lks;
    const int c = lcol + sr;
    const bool carry = c >= tiles_n;
    lcol = wrap ? (carry ? c - tiles_n : c) : lcol;
    lrow = wrap ? lrow + sq + (carry ? 1 : 0) : lrow;
  };
  auto store = [&](char* buf, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int ps = 0; ps < PA; ++ps) {
      const int r = ps * RPP + rl;
      if (BM % RPP == 0 || r < BM) {
        u32x4 pl[T];
        pieces_to_planes<E, G, false>(ra[sl][ps], pl);
#pragma unroll
        for (int p = 0; p < T; ++p) st16(buf + p * A_PLANE + r * STRIDE + swz_slot(r, q) * 16, pl[p]);
      }
    }
#pragma unroll
    for (int ps = 0; ps < PB; ++ps) {
      const int m = ps * RPP + rl;
      if (BN % RPP == 0 || m < BN) {
#pragma unroll
        for (int p = 0; p < T; ++p)
          st16(buf + T * A_PLANE + p * B_PLANE + m * STRIDE + swz_slot(m, q) * 16, rb[sl][ps][p]);
      }
    }
  };

  f32x16 acc[T][FM][FN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int p = 0; p < T; ++p)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[p][fm][fn] = f32x16{};
  };
  zero_acc();

  const int wr = wave / WN, wc = wave % WN;
  const int li = lane & 31, lh = lane >> 5;
  const int a_frag = (wr * 32 * FM + li) * STRIDE;
  const int b_frag = T * A_PLANE + (wc * 32 * FN + li) * STRIDE;
  const int c0 = swz_slot(li, lh) * 16, c1 = swz_slot(li, 2 + lh) * 16;

  using S0 = std::integral_constant<int, 0>;
  static_assert(PF == 1, "the persistent stream keeps one stage of loads in flight");
  auto step = [&](int64_t gs) {
    char* cur = lds + (NBUF == 2 ? (int)(gs & 1) * BUF : 0);
    mma_chunk<E, G, false, FM, FN>(acc, cur + a_frag + c0, A_PLANE, cur + b_frag + c0, B_PLANE, STRIDE);
    mma_chunk<E, G, false, FM, FN>(acc, cur + a_frag + c1, A_PLANE, cur + b_frag + c1, B_PLANE, STRIDE);
    if constexpr (NBUF == 1) __syncthreads();
    store(lds + (NBUF == 2 ? (int)((gs + 1) & 1) * BUF : 0), S0{});
    load(S0{});
    if constexpr (SCHED == 1 && NBUF == 2) interleave_schedule<E, G, FM, FN, PA, PB>();
    __syncthreads();
  };

  load(S0{});
  store(lds, S0{});
  load(S0{});
  __syncthreads();
  int64_t gs = 0, tile = first;
  for (int64_t j = 0; j < nt; ++j) {
    for (int ks = 0; ks < ksteps; ++ks) step(gs++);
    fwd_epilogue<E, G, FM, FN, WM, WN>(acc, (tile / tiles_n) * BM, (int)(tile % tiles_n) * BN, out, nrows, mg, bias,
                                       act, res);
    zero_acc();
    tile += stride;
  }
}

// Two waves per SIMD (256 registers per lane) unless a wave holds 16+
// accumulator fragments (planes x FM x FN) or, for f16 C8, the operands with
// their negated imaginary planes would not fit besides the eight accumulators.
// The p4 tiles of one fragment per plane in a single wave column (32 output
// groups: the narrow-layer tiles, whose time goes to HBM latency) ask for
// three, so that more of their workgroups, and so more loads, are resident.
template <typename E, int T, int FM, int FN, int WN = 0>
constexpr int fwd_waves_per_simd() {
  return (T * FM * FN >= 16 || (T == 8 && sizeof(E) == 2)) ? 1 : (T == 4 && FM * FN == 1 && WN == 1) ? 3 : 2;
}

// The forward kernel's bound.  The library's fp32 p4 one-fragment,
// single-buffered tiles fit three waves per SIMD (three workgroups per CU,
// as their LDS allows) under the bound of two; the stage-timeline build's
// timestamp stores would push them past it, so there the bound asks for
// three, keeping the traced launch's occupancy that of the library.
template <typename E, int T, int FM, int FN, int WN, int NBUF, int PF>
constexpr int fwd_kernel_waves() {
#ifdef EQLIN_STAGE_TRACE
  if (sizeof(E) == 4 && T == 4 && FM * FN == 1 && NBUF == 1 && PF == 1) return 3;
#endif
  return fwd_waves_per_simd<E, T, FM, FN, WN>();
}

// PERSIST = 0: one workgroup per tile.  PERSIST = 1: a grid of resident
// workgroups, each running every gridDim.x-th tile (fwd_stream); ntiles is the
// tile count.
// nparts >= 2 (K split of the tail, the tiles that fwd_ksplit_fits): the
// grid holds nfull whole tiles and the parts of tiles nfull .. ntiles - 1,
// nparts per tile, with their slots and arrival counters in ws / cnt (see
// KPiece).
template <typename E, int G, int FM, int FN, int WM, int WN, int NBUF, int PF, int SCHED, int PERSIST>
__global__ void __launch_bounds__(64 * WM * WN, (fwd_kernel_waves<E, Grp<G>::kOrder, FM, FN, WN, NBUF, PF>()))
fwd_kernel(const E* __restrict__ in, const E* __restrict__ wp, E* __restrict__ out,
           int64_t nrows, int kg, int mg, int tiles_n, const E* __restrict__ bias, int act,
           const E* __restrict__ res, int64_t ntiles, int64_t nfull, float* __restrict__ ws,
           uint32_t* __restrict__ cnt, int nparts) {
  __shared__ __attribute__((aligned(16))) char lds[fwd_lds_bytes<E, Grp<G>::kOrder, FM, FN, WM, WN, NBUF>()];
  if constexpr (PERSIST) {
    fwd_stream<E, G, FM, FN, WM, WN, NBUF, PF, SCHED>(lds, xcd_logical_id(blockIdx.x, gridDim.x), gridDim.x, ntiles,
                                                      in, wp, out, nrows, kg, mg, tiles_n, bias, act, res);
  } else {
    int64_t bid = blockIdx.x;
    if constexpr (fwd_ksplit_fits(sizeof(E) == 4, Grp<G>::kOrder, NBUF, PERSIST)) {
      // Where every CU gets at most one part, the parts are dispatched
      // first: the oldest waves of their CUs, they run their few stages
      // ahead of the whole tiles instead of behind them (the instruction
      // arbiter favours older waves), and the whole tiles end as on the CUs
      // without a part plus the part's matrix-core work.  Measured at the
      // ViT-B attention projection: 55.9 -> 52.9 us; with more parts than
      // CUs (ViT-H fc2) dispatching them first delays the whole tiles
      // instead (333 -> 428 us), so they go last there, at the highest wave
      // priority so that they are not starved until the whole tiles end
      // (ViT-H fc2 334 -> 326 us; their stages end at 96-204 us instead of
      // 210-319 us).
      const int64_t nkp = (int64_t)gridDim.x - nfull;   // part workgroups
      const bool first = nkp <= kNumCu;
      const bool is_part = nparts > 1 && (first ? bid < nkp : bid >= nfull);
      const int64_t pbid = first ? bid : bid - nfull;
      if (nparts > 1 && first && !is_part) bid -= nkp;
      if (is_part) {
        if (!first) __builtin_amdgcn_s_setprio(3);
        // consecutive logical ids share an XCD: a tile's parts mostly meet in one L2
        const int64_t lp = xcd_logical_id(pbid, nkp);
        const int64_t t = lp / nparts;
        const int part = (int)(lp - t * nparts);
        const int kst = (kg + Traits<E>::kStageGroups - 1) / Traits<E>::kStageGroups;
        const int k0 = part * kst / nparts, k1 = (part + 1) * kst / nparts;
        constexpr uint32_t kSlot = kpiece_slot_bytes<Grp<G>::kOrder, FM, FN, 64 * WM * WN>();
        const KPiece kp{ws + t * nparts * (int64_t)(kSlot / 4), cnt + t, part, nparts, k0, k1 - k0};
        fwd_tile<E, G, FM, FN, WM, WN, NBUF, PF, SCHED, false, false, true>(
            lds, nfull + t, in, wp, out, nrows, kg, mg, tiles_n, bias, act, res, ConvGeom{}, kp);
        return;
      }
    }
    // workgroups 0 .. nfull - 1 run whole tiles; the rest, dispatched last
    // and so at most one per CU beyond the whole rounds, run the halves of
    // tiles nfull .. ntiles - 1 (tail split)
    if constexpr (fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF)) {
      if (bid >= nfull) {
        fwd_tile<E, G, FM, FN, WM, WN, NBUF, PF, SCHED, false, true>(
            lds, 2 * nfull + xcd_logical_id(bid - nfull, (int64_t)gridDim.x - nfull), in, wp, out, nrows, kg, mg,
            tiles_n, bias, act, res);
        return;
      }
    }
    fwd_tile<E, G, FM, FN, WM, WN, NBUF, PF, SCHED>(lds, xcd_logical_id(bid, nfull), in, wp, out, nrows, kg, mg,
                                                    tiles_n, bias, act, res);
  }
}

// ============================================================ dw partials
//
// P_k[m][n] = sum_rows G_k[row][m] conj(Xhat_k[row][n])   (m = d', n = c';
// for p4m per representation Xhat^T G: the adjoint of Xhat and the dw product
// list) over the rows of one split; the T planes are written to
// ws[split][plane][mg][ng] (float32).  Tiles W x W: W = 64 with four waves of
// one 32 x 32 fragment per plane, or W = 128 with eight waves (two rows of
// four) of two fragments each (each dY and X column slab is then read by half
// as many tiles).  The k axis is the row axis: thread (unit column pc, row
// block rq) loads KV consecutive rows of one unit (kGroupsPerUnit groups),
// transforms them and writes, per group and plane, the KV rows as one
// contiguous LDS run (KV = 4 for both widths: twice the threads cover the
// twice wider rows).  A stage is 64 bytes of every plane row (16 fp32 / 32
// f16 rows); LDS is single- or double-buffered as in fwd_kernel.
template <int W>
struct DwShape {
  static_assert(W == 64 || W == 128, "dw tile width");
  static constexpr int kThreads = W == 64 ? 256 : 512;
  static constexpr int kWaveRows = 2, kWaveCols = W == 64 ? 2 : 4;
  static constexpr int kFragRows = W / (32 * kWaveRows), kFragCols = W / (32 * kWaveCols);
};

template <int T, int NBUF, int W = 64>
constexpr int dw_lds_bytes() {
  return NBUF * 2 * T * W * kRowBytes;
}

// CONV: x is the input map of a p4 group convolution and the n axis runs over
// the gathered group channels (see ConvGeom): each lane reads, per row, the
// one value of each of the four taps (or, for a centre block, the four values
// of its channel) that its gathered group channel needs, as 32-bit loads.
template <typename E, int G, int NBUF, bool CONV = false, int W = 64>
__device__ __forceinline__ void dw_tile(char* lds, int64_t lid, const E* __restrict__ dy, const E* __restrict__ x,
                                        float* __restrict__ ws, int64_t nrows, int mg, int ng,
                                        int64_t rows_per_split, int tiles_m, int tiles_n, int cw_m, int cw_n,
                                        const ConvGeom& geo = ConvGeom{}) {
  constexpr int T = Grp<G>::kOrder;
  using U = Units<E, T>;
  using S = DwShape<W>;
  constexpr int NT = S::kThreads;
  constexpr int WC = S::kWaveCols, FR = S::kFragRows, FC = S::kFragCols;
  constexpr int GPU = U::kGroupsPerUnit, PPU = U::kPiecesPerUnit;
  constexpr int PR = W / GPU;                      // units per tile row (W groups)
  constexpr int RB = NT / PR;                      // row blocks per stage
  constexpr int SR = 64 / (int)sizeof(E);          // rows per stage: 16 (fp32) / 32 (f16)
  constexpr int KV = SR / RB;                      // rows per thread per stage
  constexpr int RUN = KV * (int)sizeof(E);         // LDS bytes per (group, plane) per thread
  constexpr int STRIDE = kRowBytes;
  constexpr int PLANE = W * STRIDE;
  constexpr int BUF = 2 * T * PLANE;
  static_assert(RB * KV == SR && (RUN == 8 || RUN == 16), "stage shape");
  static_assert(NBUF * BUF == dw_lds_bytes<T, NBUF, W>(), "LDS size");
  static_assert(!CONV || W == 64, "the convolution's gathered loads use the 64-wide tile");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = tiles_m * tiles_n;
  const int64_t split = lid / ntiles;
  const int tile = (int)(lid % ntiles);
  const int m0 = (tile / tiles_n) * W, n0 = (tile % tiles_n) * W;
  const int64_t rbeg = split * rows_per_split;
  const int64_t rend = (rbeg + rows_per_split < nrows) ? rbeg + rows_per_split : nrows;
  const int nstages = (int)((rend - rbeg + SR - 1) / SR);

  const uint32_t a_row = (uint32_t)mg * (uint32_t)(T * sizeof(E));
  const uint32_t b_row = (uint32_t)ng * (uint32_t)(T * sizeof(E));
  const __amdgpu_buffer_rsrc_t a_src = make_rsrc(dy + rbeg * T * (int64_t)mg, (uint64_t)(rend - rbeg) * a_row);
  const __amdgpu_buffer_rsrc_t b_src =
      CONV ? make_rsrc(x, geo.in_bytes) : make_rsrc(x + rbeg * T * (int64_t)ng, (uint64_t)(rend - rbeg) * b_row);

  // thread (unit column pc, row block rq).  With two groups per unit (f16
  // p4) a wave's 32-lane half holds eight consecutive unit columns (128
  // contiguous bytes of a row per load) of four row blocks, so that its
  // transposed LDS writes cover all 64 banks (see dw_row); otherwise the unit
  // column runs fastest.
  static_assert(GPU != 2 || RB == 8, "eight row blocks per stage");
  const int pc = GPU == 2 ? (tid & 7) | ((tid >> 6) << 3) : tid % PR;
  const int rq = GPU == 2 ? ((tid >> 3) & 3) | (((tid >> 5) & 1) << 2) : tid / PR;
  const int ga = m0 + pc * GPU, gb = n0 + pc * GPU;
  const bool a_ok = ga < mg, b_ok = gb < ng;
  const uint32_t a_col = (uint32_t)ga * (uint32_t)(T * sizeof(E));
  const uint32_t b_col = (uint32_t)gb * (uint32_t)(T * sizeof(E));

  // convolution: the sources of this lane's gathered group channel gb (fixed
  // for the tile).  Source m is tap m of the block (orbit) or the lane's
  // channel at the pixel (centre); jj[m] is the rotation read from it.
  constexpr int NW = CONV ? 2 * GPU : 1;       // 32-bit loads per source and row
  bool c_live = false;
  int c_dy[4], c_dx[4], c_jj[4], c_off[4];
  if constexpr (CONV) {
    static_assert(T == 4 && PPU == 1, "p4 convolution");
    constexpr int SGc = 16 * GPU;
    const int w = (gb % SGc) / GPU, ui = w >> 2;
    const ConvBlock k = conv_block<GPU>((gb / SGc) * 4 + (w & 3), geo);
    c_live = b_ok && k.live;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      c_dy[m] = k.centre ? 0 : k.di[m];
      c_dx[m] = k.centre ? 0 : k.dj[m];
      c_jj[m] = k.centre ? m : ((m + ui) & 3);
      const int ch = k.centre ? k.ch0 + k.chstep * ui : k.ch0;
      c_off[m] = ((c_dy[m] * geo.W + c_dx[m]) * geo.cpix + ch) * (int)(T * sizeof(E));
    }
  }

  u32x4 ra[KV][PPU], rb[CONV ? 1 : KV][PPU];
  uint32_t rc[CONV ? KV : 1][4][NW];
  auto load = [&](int st) {
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const uint32_t row = (uint32_t)(st * SR + rq * KV + v);
#pragma unroll
      for (int h = 0; h < PPU; ++h) {
        ra[v][h] = bload16(a_src, a_ok ? row * a_row + a_col + 16u * h : kOob);
        if constexpr (!CONV) rb[v][h] = bload16(b_src, b_ok ? row * b_row + b_col + 16u * h : kOob);
      }
      if constexpr (CONV) {
        const int64_t n = rbeg + row;
        const bool rok = c_live && n < rend;
        const uint32_t nn = rok ? (uint32_t)n : 0u;
        const uint32_t img = div_magic(nn, geo.hw_mul, geo.hw_shift);
        const uint32_t rem = nn - img * (uint32_t)(geo.H * geo.W);
        const uint32_t py = div_magic(rem, geo.w_mul, geo.w_shift);
        const uint32_t px = rem - py * (uint32_t)geo.W;
        const uint32_t base = nn * (uint32_t)(geo.cpix * T * sizeof(E));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bool ok = rok && (unsigned)((int)py + c_dy[m]) < (unsigned)geo.H &&
                          (unsigned)((int)px + c_dx[m]) < (unsigned)geo.W;
          const uint32_t src = base + (uint32_t)c_off[m];
          if constexpr (sizeof(E) == 4) {
            rc[v][m][0] = bload4(b_src, ok ? src + 4u * (uint32_t)c_jj[m] : kOob);
          } else {
            // halves jj (channel e = 0) and 4 + jj (e = 1) of the 8-half source
            rc[v][m][0] = bload4(b_src, ok ? src + 4u * (uint32_t)(c_jj[m] >> 1) : kOob);
            rc[v][m][1] = bload4(b_src, ok ? src + 8u + 4u * (uint32_t)(c_jj[m] >> 1) : kOob);
          }
        }
      }
    }
  };
  // transform one operand's KV rows and write the (group, plane) runs
  auto put = [&](char* plane0, const u32x4 (&r)[KV][PPU], auto conj_c) {
    constexpr bool kConj = decltype(conj_c)::value;
    if constexpr (sizeof(E) == 2 && G == 4 && KV == 4 && PPU == 1) {
      // f16 p4: the mixed-precision DFT of group e of rows (2 j, 2 j + 1)
      // yields each plane's values of that row pair, packed as the run needs
#pragma unroll
      for (int e = 0; e < GPU; ++e) {
        u32x2 run[T];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t q0, q2, q1r, q1i;
          dft4_f16_pair<kConj>(r[2 * j][0][2 * e], r[2 * j][0][2 * e + 1], r[2 * j + 1][0][2 * e],
                               r[2 * j + 1][0][2 * e + 1], q0, q2, q1r, q1i);
          run[0][j] = q0;
          run[1][j] = q2;
          run[2][j] = q1r;
          run[3][j] = q1i;
        }
        const int off = dw_off(pc * GPU + e, rq * RUN);
#pragma unroll
        for (int p = 0; p < T; ++p) *reinterpret_cast<u32x2*>(plane0 + p * PLANE + off) = run[p];
      }
      return;
    }
    if constexpr (sizeof(E) == 2 && G == 8 && KV == 8 && PPU == 1 && GPU == 1) {
      // f16 C8: rows 2 j and 2 j + 1 of the one group fill word j of every run
      u32x4 run[T];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t o[8];
        dft8_f16_pair<kConj>(r[2 * j][0], r[2 * j + 1][0], o);
#pragma unroll
        for (int p = 0; p < T; ++p) run[p][j] = o[p];
      }
      const int off = dw_off(pc, rq * RUN);
#pragma unroll
      for (int p = 0; p < T; ++p) st16(plane0 + p * PLANE + off, run[p]);
      return;
    }
    float f[KV][GPU][T];
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      float z[GPU * T];
#pragma unroll
      for (int h = 0; h < PPU; ++h) {
        if constexpr (sizeof(E) == 4) {
          const f32x4 xv = __builtin_bit_cast(f32x4, r[v][h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) z[4 * h + e] = xv[e];
        } else {
          const f16x8 xv = __builtin_bit_cast(f16x8, r[v][h]);
#pragma unroll
          for (int e = 0; e < 8; ++e) z[8 * h + e] = (float)xv[e];
        }
      }
#pragma unroll
      for (int e = 0; e < GPU; ++e) {
        Grp<G>::dft(&z[e * T], f[v][e]);
        if constexpr (kConj) Grp<G>::adjoint(f[v][e]);
      }
    }
#pragma unroll
    for (int e = 0; e < GPU; ++e) {
      const int off = dw_off(pc * GPU + e, rq * RUN);
#pragma unroll
      for (int p = 0; p < T; ++p) {
        if constexpr (sizeof(E) == 4) {
          st16(plane0 + p * PLANE + off, __builtin_bit_cast(u32x4, f32x4{f[0][e][p], f[1][e][p], f[2][e][p], f[3][e][p]}));
        } else if constexpr (KV == 4) {
          // f16: scaled into the operand range (Grp<G>::kF16Scale, exact)
          const float sc = Grp<G>::kF16Scale[p];
          const f16x4 hv = {(_Float16)(f[0][e][p] * sc), (_Float16)(f[1][e][p] * sc), (_Float16)(f[2][e][p] * sc),
                            (_Float16)(f[3][e][p] * sc)};
          *reinterpret_cast<u32x2*>(plane0 + p * PLANE + off) = __builtin_bit_cast(u32x2, hv);
        } else {
          const float sc = Grp<G>::kF16Scale[p];
          f16x8 hv;
#pragma unroll
          for (int v = 0; v < 8; ++v) hv[v] = (_Float16)(f[v][e][p] * sc);
          st16(plane0 + p * PLANE + off, __builtin_bit_cast(u32x4, hv));
        }
      }
    }
  };
  auto store = [&](char* buf) {
    put(buf, ra, std::false_type{});
    if constexpr (CONV) {
      // the gathered pieces: value m of channel e = the selected rotation of source m
      u32x4 pcs[KV][PPU];
#pragma unroll
      for (int v = 0; v < KV; ++v) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (sizeof(E) == 4) {
            pcs[v][0][k] = rc[v][k][0];
          } else {
            const int e = k >> 1, m0 = 2 * (k & 1);
            const uint32_t lo = (rc[v][m0][e] >> (16 * (c_jj[m0] & 1))) & 0xffffu;
            const uint32_t hi = (rc[v][m0 + 1][e] >> (16 * (c_jj[m0 + 1] & 1))) & 0xffffu;
            pcs[v][0][k] = lo | (hi << 16);
          }
        }
      }
      put(buf + T * PLANE, pcs, std::true_type{});
    } else {
      put(buf + T * PLANE, rb, std::true_type{});
    }
  };

  f32x16 acc[T][FR][FC];
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int fm = 0; fm < FR; ++fm)
#pragma unroll
      for (int fn = 0; fn < FC; ++fn) acc[p][fm][fn] = f32x16{};

  const int wr = wave / WC, wc = wave % WC;
  const int li = lane & 31, lh = lane >> 5;
  // fragment rows differ from li by multiples of 32, which dw_row and
  // dw_slot leave unchanged
  const int a_frag = (wr * 32 * FR + dw_row(li)) * STRIDE;
  const int b_frag = T * PLANE + (wc * 32 * FC + dw_row(li)) * STRIDE;
  const int c0 = dw_slot(li, lh) * 16, c1 = dw_slot(li, 2 + lh) * 16;

  if (nstages > 0) {
    load(0);
    store(lds);
    if (nstages > 1) load(1);
    __syncthreads();
  }
  // Row chunks (cw_m < mg, fp32): the rows of a narrow layer are read as rows of
  // CH = mg / cw_m = ng / cw_n consecutive rows, so the tile is CH x CH blocks
  // of cw_m x cw_n and only the diagonal blocks (block c of dY against block c
  // of X, the same rows) belong to dw.  A p4 fp32 wave whose 32 x 32 fragment
  // meets no diagonal block, or lies wholly past mg or ng, loads and
  // transforms its share of the stages but issues no MFMA: its products
  // would be dropped.
  const int fr = m0 + wr * 32 * FR, fc = n0 + wc * 32 * FC;
  const bool live = W != 64 || (fr < mg && fc < ng &&
                                (fr / cw_m > fc / cw_n ? fr / cw_m <= (min(fc + 31, ng - 1) / cw_n)
                                                       : fc / cw_n <= (min(fr + 31, mg - 1) / cw_m)));
  // Only the p4 fp32 tiles skip: in f16 the MFMAs are short, and for the
  // order-8 groups, whose eight planes fill the registers, a branch around
  // them inside the loop costs more than it saves (the compiler guards MFMA
  // hazards at block edges; measured: C8 ViT-B fp32 dw 86.6 -> 94.4 us),
  // while a second copy of the loop without them costs occupancy.
  const bool mma = !(sizeof(E) == 4 && T == 4) || live;
  // multiply stage st, then transform stage st + 1 (slot of st + 1) into LDS
  // and refill that slot with the loads of stage st + 1 + PF
  for (int st = 0; st < nstages; ++st) {
    char* cur = lds + (NBUF == 2 ? (st & 1) * BUF : 0);
    if (mma) {
      mma_chunk<E, G, true, FR, FC>(acc, cur + a_frag + c0, PLANE, cur + b_frag + c0, PLANE, STRIDE);
      mma_chunk<E, G, true, FR, FC>(acc, cur + a_frag + c1, PLANE, cur + b_frag + c1, PLANE, STRIDE);
    }
    if (st + 1 < nstages) {
      if constexpr (NBUF == 1) __syncthreads();   // every wave is done reading the only buffer
      store(lds + (NBUF == 2 ? ((st + 1) & 1) * BUF : 0));
      if (st + 2 < nstages) load(st + 2);
    }
    __syncthreads();
  }

  if constexpr (W == 64) {   // row chunks: narrow fp32 layers (64-wide tile only)
    const int n = n0 + wc * 32 + li;
    if (sizeof(E) == 4 && cw_m < mg) {
      // row chunks (fp32): the CH diagonal blocks meet in LDS (free after the
      // stage loop's last barrier), are added in block order and written as
      // one cw_m x cw_n partial per plane
      const int CH = mg / cw_m, cell = cw_m * cw_n;
      // [T][CH][cw_m][cw_n]: T mg ng / CH <= T x 2048 floats (CH >= 2, mg, ng <= 64),
      // the size of the dw stage buffers (T x 2 x 64 x 64 bytes per buffer)
      static_assert(BUF >= T * 2048 * (int)sizeof(float), "chunk reduction fits the stage buffer");
      float* red = reinterpret_cast<float*>(lds);
      const int nblk = n / cw_n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wr * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (m < mg && n < ng && m / cw_m == nblk) {
          const int o = nblk * cell + (m - nblk * cw_m) * cw_n + (n - nblk * cw_n);
#pragma unroll
          for (int p = 0; p < T; ++p) red[p * CH * cell + o] = acc[p][0][0][r];
        }
      }
      __syncthreads();
      float* dstc = ws + split * T * (int64_t)cell;
      for (int i = tid; i < T * cell; i += NT) {
        const int p = i / cell, e = i - p * cell;
        float sum = red[p * CH * cell + e];
        for (int c = 1; c < CH; ++c) sum += red[(p * CH + c) * cell + e];
        dstc[i] = sum;
      }
      return;
    }
  }
  const int64_t plane_elems = (int64_t)mg * ng;
  float* dst = ws + split * T * plane_elems;
#pragma unroll
  for (int fm = 0; fm < FR; ++fm)
#pragma unroll
    for (int fn = 0; fn < FC; ++fn) {
      const int n = n0 + wc * 32 * FC + fn * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wr * 32 * FR + fm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (m < mg && n < ng) {
#pragma unroll
          for (int p = 0; p < T; ++p) dst[p * plane_elems + (int64_t)m * ng + n] = acc[p][fm][fn][r];
        }
      }
    }
}

// C8 tiles hold eight 32 x 32 accumulators per wave next to the operands
// and the load ring: one wave per SIMD (512 registers) avoids spills.
template <int T>
constexpr int bwd_waves_per_simd() {
  return T == 4 ? 2 : 1;
}

// W = 128 (p4 only: two fragments of eight planes would not fit the registers
// of two waves per SIMD) runs one 512-thread workgroup per CU.
template <typename E, int G, int W = 64>
__global__ void __launch_bounds__(DwShape<W>::kThreads, bwd_waves_per_simd<Grp<G>::kOrder>())
dw_partial_kernel(const E* __restrict__ dy, const E* __restrict__ x, float* __restrict__ ws,
                  int64_t nrows, int mg, int ng, int64_t rows_per_split, int tiles_m, int tiles_n, int cw_m,
                  int cw_n) {
  static_assert(W == 64 || G == 4, "the 128-wide dw tile is built for p4");
  // The 128-wide tile runs one workgroup per CU (registers), so its LDS has
  // room for two stage buffers: the next chunk's loads are written while the
  // current one is multiplied, one barrier per chunk instead of two.  The
  // 64-wide tile gained nothing from a second buffer (measured), so it keeps one.
  constexpr int NB = W == 128 ? 2 : kDwBufs;
  __shared__ __attribute__((aligned(16))) char lds[dw_lds_bytes<Grp<G>::kOrder, NB, W>()];
  dw_tile<E, G, NB, false, W>(lds, xcd_logical_id(blockIdx.x, gridDim.x), dy, x, ws, nrows, mg, ng,
                              rows_per_split, tiles_m, tiles_n, cw_m, cw_n);
}

// Backward in one launch: the first ndw_pad workgroups are dw split partials,
// the rest are dX tiles (the forward structure on the transpose spectra).
// Both roles read dY; running them in one grid lets the dispatcher fill the
// tail of one role with work of the other.  ndw_pad is a multiple of 8, so
// each role keeps its own XCD-aware numbering.
template <typename E, int G, int SCHED>
__global__ void __launch_bounds__(kThreads, bwd_waves_per_simd<Grp<G>::kOrder>())
bwd_fused_kernel(const E* __restrict__ dy, const E* __restrict__ x, const E* __restrict__ wb,
                 E* __restrict__ dx, float* __restrict__ ws, int64_t nrows, int dg, int cg,
                 int64_t rows_per_split, int dw_tiles_m, int dw_tiles_n, int64_t ndw, int64_t ndw_pad,
                 int dx_tiles_n, int64_t ndx_full, int chunks) {
  constexpr int T = Grp<G>::kOrder;
  constexpr int kFwd = fwd_lds_bytes<E, T, 1, 1, 2, 2, kBwdFwdBufs>();
  constexpr int kDw = dw_lds_bytes<T, kDwBufs>();
  __shared__ __attribute__((aligned(16))) char lds[kFwd > kDw ? kFwd : kDw];
  const int64_t b = blockIdx.x;
  if (b < ndw_pad) {
    const int64_t lid = xcd_logical_id(b, ndw_pad);
    if (lid < ndw)
      dw_tile<E, G, kDwBufs>(lds, lid, dy, x, ws, (sizeof(E) == 2 || chunks == 1) ? nrows : nrows / chunks,
                             chunks * dg, chunks * cg, rows_per_split, dw_tiles_m, dw_tiles_n, dg, cg);
  } else {
    // dX tiles past ndx_full run as halves (the tail split of fwd_kernel)
    const int64_t bx = b - ndw_pad;
    if constexpr (fwd_tail_split_fits(sizeof(E) == 4, 1, 1, 2, 2, kBwdFwdBufs)) {
      if (bx >= ndx_full) {
        fwd_tile<E, G, 1, 1, 2, 2, kBwdFwdBufs, kBwdFwdPrefetch, SCHED, false, true>(
            lds, 2 * ndx_full + xcd_logical_id(bx - ndx_full, (int64_t)gridDim.x - ndw_pad - ndx_full), dy, wb, dx,
            nrows, dg, cg, dx_tiles_n, nullptr, 0, nullptr);
        return;
      }
    }
    fwd_tile<E, G, 1, 1, 2, 2, kBwdFwdBufs, kBwdFwdPrefetch, SCHED>(lds, xcd_logical_id(bx, ndx_full), dy, wb, dx,
                                                                     nrows, dg, cg, dx_tiles_n, nullptr, 0, nullptr);
  }
}

// Sum the split partials (deterministic), inverse group DFT along u, write
// dw[m][n][0..T-1] (float32).  A 256-thread block covers EB = 256 / (T R)
// consecutive entries: thread (part r, plane p, entry e) sums the splits
// s = r, r + R, r + 2R, ... of plane p in increasing s, the R part sums of
// a (plane, entry) meet in LDS and are added in part order, then the T plane
// sums of an entry meet and one thread per entry applies the inverse DFT.
// R (a power of two, T R <= 256) is set by the host from the entry and split
// counts alone (dw_finalize_parts), so a given call always adds in the same
// order; R = 1 is the plain split-order sum.  nsplit == 0 writes zeros.
// kF16: the partials are products of f16 operands, which carry the operand
// scales (Grp<G>::kF16Scale); they are multiplied back out before the
// inverse DFT.
template <int G, bool kF16>
__global__ void __launch_bounds__(kThreads)
dw_finalize_kernel(const float* __restrict__ ws, float* __restrict__ dw, int mg, int ng, int nsplit, int R) {
  constexpr int T = Grp<G>::kOrder;
  __shared__ float red[kThreads];
  const int cols = kThreads / R;  // (plane, entry) columns of the block
  const int EB = cols / T;
  const int t = threadIdx.x;
  const int col = t % cols, r = t / cols;
  const int e = col % EB, p = col / EB;
  const int64_t plane = (int64_t)mg * ng;
  const int64_t idx = (int64_t)blockIdx.x * EB + e;
  float acc = 0.f;
  if (idx < plane) {
    const float* src = ws + p * plane + idx;
    const int64_t step = T * plane;
    int s = r;
    for (; s + 3 * R < nsplit; s += 4 * R) {
      const float v0 = src[(int64_t)s * step], v1 = src[(int64_t)(s + R) * step];
      const float v2 = src[(int64_t)(s + 2 * R) * step], v3 = src[(int64_t)(s + 3 * R) * step];
      acc += v0;
      acc += v1;
      acc += v2;
      acc += v3;
    }
    for (; s < nsplit; s += R) acc += src[(int64_t)s * step];
  }
  red[t] = acc;
  __syncthreads();
  if (r == 0) {  // each column reads its own chunk slots only: no race with the writes
    float sum = red[t];
    for (int q = 1; q < R; ++q) sum += red[q * cols + t];
    red[t] = sum;
  }
  __syncthreads();
  if (t < EB && idx < plane) {
    float f[T], y[T];
#pragma unroll
    for (int k = 0; k < T; ++k) f[k] = kF16 ? red[k * EB + t] * f16_unscale<G>(k) : red[k * EB + t];
    Grp<G>::idft(f, y);
    store_group<float, T>(dw + idx * T, y);
  }
}

// Parts per (plane, entry) of dw_finalize_kernel: doubled while the launch
// holds fewer than two blocks per CU and every part keeps at least four
// splits, so a layer with few weight entries and many row splits (narrow
// layers over many rows) reads its partials with the whole chip rather than
// a few CUs each walking every split.
inline int dw_finalize_parts(int64_t entries, int T, int nsplit) {
  int R = 1;
  while (2 * R * T <= kThreads && (int64_t)nsplit >= 8 * R &&
         (entries + kThreads / (T * R) - 1) / (kThreads / (T * R)) < 2 * kNumCu)
    R *= 2;
  return R;
}

template <typename E, int G>
hipError_t launch_dw_finalize(const float* ws, float* dw, int mg, int ng, int nsplit, hipStream_t s) {
  constexpr int T = Grp<G>::kOrder;
  const int64_t entries = (int64_t)mg * ng;
  const int R = dw_finalize_parts(entries, T, nsplit);
  const int64_t grid = (entries + kThreads / (T * R) - 1) / (kThreads / (T * R));
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (grid > 0)
    hipLaunchKernelGGL((dw_finalize_kernel<G, sizeof(E) == 2>), dim3((unsigned)grid), dim3(kThreads), 0, s, ws, dw, mg,
                       ng, nsplit, R);
  return hipGetLastError();
}

// ============================================================ prepare
//
// Weight spectra in the stage-block layout read by fwd_kernel:
//   dst[row][ks][plane][s]   (SG = 16 fp32 / 32 f16 slots per 64-byte block)
// where slot s of stage ks holds group channel ks * SG + slot_group(s) (the
// slot order fwd_kernel's loaders produce for the transformed input) and
// groups past the end are zero.
//   forward planes:   row = d', groups = c',  spectrum of w[d'][c'][.]
//   transpose planes: row = c', groups = d',  adjoint spectrum of w[d'][c'][.]
// The second set is the spectrum of the transposed weight (u -> w(u^-1): a
// conjugate for cyclic groups, the transposed 2 x 2 block for p4m), used by
// the dX pass.  Both sets are written by one launch: blocks below nbf write
// the forward set, the others the transpose set.
template <typename E, int G, bool kTranspose>
__device__ __forceinline__ void prepare_entry(const E* __restrict__ w, E* __restrict__ dst, int mg, int ng,
                                              int64_t idx) {
  constexpr int SG = Traits<E>::kStageGroups, T = Grp<G>::kOrder;
  const int rows = kTranspose ? ng : mg;
  const int kgr = kTranspose ? mg : ng;
  const int nks = (kgr + SG - 1) / SG;
  if (idx >= (int64_t)rows * nks * SG) return;
  const int s = (int)(idx % SG);
  const int64_t t = idx / SG;
  const int ks = (int)(t % nks);
  const int64_t row = t / nks;
  const int g = ks * SG + slot_group<E, T>(s);
  float f[T];
#pragma unroll
  for (int p = 0; p < T; ++p) f[p] = 0.f;
  if (g < kgr) {
    const E* src = kTranspose ? w + ((int64_t)g * ng + row) * T : w + (row * ng + g) * T;
    float z[T];
#pragma unroll
    for (int u = 0; u < T; ++u) z[u] = (float)src[u];
    Grp<G>::dft(z, f);
    if (kTranspose) Grp<G>::adjoint(f);
  }
  // f16: scaled into the operand range of the f16 products (Grp<G>::kF16Scale)
  E* o = dst + (row * nks + ks) * T * SG + s;
#pragma unroll
  for (int p = 0; p < T; ++p) o[p * SG] = (E)(sizeof(E) == 2 ? f[p] * Grp<G>::kF16Scale[p] : f[p]);
}

template <typename E, int G>
__global__ void __launch_bounds__(kThreads)
prepare_kernel(const E* __restrict__ w, E* __restrict__ wf, E* __restrict__ wb, int mg, int ng, int64_t nbf) {
  const int64_t b = blockIdx.x;
  if (b < nbf)
    prepare_entry<E, G, false>(w, wf, mg, ng, b * kThreads + threadIdx.x);
  else
    prepare_entry<E, G, true>(w, wb, mg, ng, (b - nbf) * kThreads + threadIdx.x);
}

// ============================================================ launchers

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Resident workgroups of one kernel on the current device (occupancy x CUs),
// queried once per kernel instantiation.
template <typename K>
int64_t resident_workgroups(K kernel, int threads) {
  static const int64_t n = [&] {
    int dev = 0, per_cu = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return int64_t(0);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return int64_t(0);
    return int64_t(per_cu) * prop.multiProcessorCount;
  }();
  return n;
}

// ks: the K split of the tail (fwd_ksplit_plan for this tile; ks.nparts == 0:
// none, and then the tail split where it fits).  The caller has checked that
// ks.ws holds the plan's counters and slots.
template <typename E, int G, int FM, int FN, int WM, int WN, int NBUF, int PF, int SCHED, int PERSIST>
hipError_t launch_fwd_s(const void* in, const void* wp, void* out, int64_t nrows, int kg, int mg,
                        const void* bias, int act, const void* res, hipStream_t s, const FwdKSplit& ks = FwdKSplit{}) {
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  const int64_t tiles_m = cdiv(nrows, BM);
  const int tiles_n = (int)cdiv(mg, BN);
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles <= 0) return hipSuccess;
  int64_t grid = tiles, nfull = tiles;
  int nparts = 0;
  float* slots = nullptr;
  uint32_t* cnt = nullptr;
  auto kernel = fwd_kernel<E, G, FM, FN, WM, WN, NBUF, PF, SCHED, PERSIST>;
  if constexpr (PERSIST) {
    const int64_t resident = resident_workgroups(kernel, 64 * WM * WN);
    if (resident > 0 && resident < grid) grid = resident;
  } else {
    bool ksplit = false;
    if constexpr (fwd_ksplit_fits(sizeof(E) == 4, Grp<G>::kOrder, NBUF, PERSIST)) {
      if (ks.nparts > 1 && ks.ws != nullptr) {
        const FwdKSplitPlan pl = fwd_ksplit_plan(tiles, (int)cdiv(kg, Traits<E>::kStageGroups),
                                                 fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF));
        if (pl.nparts != ks.nparts) return hipErrorInvalidValue;   // the caller's plan is another shape's
        ksplit = true;
        nparts = pl.nparts;
        nfull = tiles - pl.tail;
        grid = nfull + pl.tail * nparts;
        cnt = static_cast<uint32_t*>(ks.ws);
        slots = reinterpret_cast<float*>(static_cast<char*>(ks.ws) + kFwdKSplitCounterBytes);
      }
    }
    if constexpr (fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF)) {
      if (!ksplit && fwd_tail_split_enabled()) {
        nfull = fwd_full_tiles(tiles);
        grid = nfull + 2 * (tiles - nfull);
      }
    }
  }
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(64 * WM * WN), 0, s, static_cast<const E*>(in),
                     static_cast<const E*>(wp), static_cast<E*>(out), nrows, kg, mg, tiles_n,
                     static_cast<const E*>(bias), act, static_cast<const E*>(res), tiles, nfull, slots, cnt, nparts);
  return hipGetLastError();
}

// chunks > 1 (it divides nrows; chunks x mg and chunks x ng <= 64): the dw
// partials of the row-chunked product, rows_per_split counting chunked rows.
// width: the dw tile, 64 or (p4, chunks == 1) 128.
template <typename E, int G>
hipError_t launch_dw_t(const void* dy, const void* x, float* ws, float* dw, int64_t nrows, int mg, int ng,
                       int64_t rows_per_split, int nsplit, int chunks, int width, hipStream_t s) {
  const bool wide = G == 4 && width == 128 && chunks == 1;
  const int W = wide ? 128 : 64;
  const int tiles_m = (int)cdiv(chunks * mg, W), tiles_n = (int)cdiv(chunks * ng, W);
  if (nsplit > 0) {
    const int64_t grid = (int64_t)tiles_m * tiles_n * nsplit;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if constexpr (G == 4) {
      if (wide) {
        hipLaunchKernelGGL((dw_partial_kernel<E, G, 128>), dim3((unsigned)grid), dim3(DwShape<128>::kThreads), 0, s, static_cast<const E*>(dy),
                           static_cast<const E*>(x), ws, nrows, mg, ng, rows_per_split, tiles_m, tiles_n, mg, ng);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_dw_finalize<E, G>(ws, dw, mg, ng, nsplit, s);
      }
    }
    hipLaunchKernelGGL((dw_partial_kernel<E, G>), dim3((unsigned)grid), dim3(kThreads), 0, s, static_cast<const E*>(dy),
                       static_cast<const E*>(x), ws, nrows / chunks, chunks * mg, chunks * ng, rows_per_split, tiles_m,
                       tiles_n, mg, ng);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_dw_finalize<E, G>(ws, dw, mg, ng, nsplit, s);
}

template <typename E, int G>
hipError_t launch_bwd_fused_t(const void* dy, const void* x, const void* wb, void* dx, float* ws, float* dw,
                              int64_t nrows, int dg, int cg, int64_t rows_per_split, int nsplit, int chunks,
                              hipStream_t s) {
  const int dw_tiles_m = (int)cdiv(chunks * dg, 64), dw_tiles_n = (int)cdiv(chunks * cg, 64);
  const int64_t ndw = (int64_t)dw_tiles_m * dw_tiles_n * nsplit;
  const int64_t ndw_pad = cdiv(ndw, 8) * 8;
  const int dx_tiles_n = (int)cdiv(cg, 64);
  const int64_t ndx = cdiv(nrows, 64) * dx_tiles_n;
  int64_t ndx_full = ndx, grid = ndw_pad + ndx;
  if (fwd_tail_split_fits(sizeof(E) == 4, 1, 1, 2, 2, kBwdFwdBufs) && fwd_tail_split_enabled()) {
    ndx_full = fwd_full_tiles(ndx);
    grid = ndw_pad + ndx_full + 2 * (ndx - ndx_full);
  }
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (grid > 0) {
    hipLaunchKernelGGL((bwd_fused_kernel<E, G, 1>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       static_cast<const E*>(dy), static_cast<const E*>(x), static_cast<const E*>(wb),
                       static_cast<E*>(dx), ws, nrows, dg, cg, rows_per_split, dw_tiles_m, dw_tiles_n, ndw, ndw_pad,
                       dx_tiles_n, ndx_full, chunks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_dw_finalize<E, G>(ws, dw, dg, cg, nsplit, s);
}

template <typename E, int G>
hipError_t launch_prepare_t(const void* w, void* wf, void* wb, int mg, int ng, hipStream_t s) {
  constexpr int SG = Traits<E>::kStageGroups;
  const int64_t nf = (int64_t)mg * cdiv(ng, SG) * SG, nb = (int64_t)ng * cdiv(mg, SG) * SG;
  const int64_t nbf = cdiv(nf, kThreads), grid = nbf + cdiv(nb, kThreads);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prepare_kernel<E, G>), dim3((unsigned)grid), dim3(kThreads), 0, s, static_cast<const E*>(w),
                     static_cast<E*>(wf), static_cast<E*>(wb), mg, ng, nbf);
  return hipGetLastError();
}

}  // namespace eqlin
