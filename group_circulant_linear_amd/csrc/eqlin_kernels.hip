// HIP kernels of the p4 group-circulant linear layer for gfx950 (CDNA4).
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
//   * "Implementation": fused dataflow (no intermediate global writes), Fourier
//     fragments resident in registers / on-chip memory, shape-specialised
//     tiles on the matrix cores.
//
// Group DFT of one group z0..z3 (forward sign exp(-2 pi i k u / 4)):
//   F0 = (z0+z2)+(z1+z3)   F2 = (z0+z2)-(z1+z3)   Re F1 = z0-z2   Im F1 = z3-z1
// Inverse (F3 = conj F1):
//   z0 = (F0+F2)/4 + Re F1/2   z1 = (F0-F2)/4 - Im F1/2
//   z2 = (F0+F2)/4 - Re F1/2   z3 = (F0-F2)/4 + Im F1/2
//
// gfx950 mapping.  Work is expressed as one "complex-structured GEMM":
//   out_plane[m][n] = sum_k A_plane[m][k] (*) B_plane[n][k]
// where (*) is: f0*f0, f2*f2 and the complex product on (Re f1, Im f1).
// Both operands are staged per pipeline stage into LDS as four planes
// [plane][row][k] with k contiguous in 64-byte rows whose four 16-byte slots
// are XOR-swizzled (see swz_slot).  Every lane reads 16 bytes per plane per
// 32x32 fragment: 4 fp32 k-values (four 32x32x2 f32
// MFMAs) or 8 f16 k-values (one 32x32x16 f16 MFMA).  A workgroup has four
// 64-wide waves in a 2 x 2 arrangement; each wave owns FM x FN fragments of
// 32 x 32 for each of the four accumulator planes (f0, f2, Re f1, Im f1).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "eqlin_kernels.h"

namespace eqlin {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kNumXcd = 8;
#ifndef EQLIN_DW_BUFS
#define EQLIN_DW_BUFS 1
#endif
#ifndef EQLIN_BWD_FWD_BUFS
#define EQLIN_BWD_FWD_BUFS 1
#endif
// LDS stage buffers of the dw partial tiles and of the dX tiles inside the
// fused backward (1: smaller LDS, more resident workgroups per CU).
constexpr int kDwBufs = EQLIN_DW_BUFS;
constexpr int kBwdFwdBufs = EQLIN_BWD_FWD_BUFS;
#ifndef EQLIN_BWD_FWD_PREFETCH
#define EQLIN_BWD_FWD_PREFETCH 1
#endif
constexpr int kBwdFwdPrefetch = EQLIN_BWD_FWD_PREFETCH;

// LDS plane rows are 64 bytes (four 16-byte slots) with no padding; the slot
// index is XOR-swizzled with bits 2-3 of the row, which keeps both the
// 4-lanes-per-row stores and the 32-rows-per-wave fragment reads free of bank
// conflicts on gfx950 (checked with the LDS bank-conflict counter).
constexpr int kRowBytes = 64;
__device__ __forceinline__ int swz_slot(int row, int slot) { return slot ^ ((row >> 2) & 3); }

template <typename E> struct Traits;
template <> struct Traits<float> {
  static constexpr int kGroupsPerPiece = 1;   // one 16 B piece = one group of 4 floats
  static constexpr int kValsPerSlot = 4;      // k-values per lane per 16 B LDS read
};
template <> struct Traits<_Float16> {
  static constexpr int kGroupsPerPiece = 2;   // one 16 B piece = two groups of 4 halves
  static constexpr int kValsPerSlot = 8;
};

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

// GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt(2)))
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erf_as7126(x * 0.70710678118654752f)); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Buffer resource over [base, base + bytes): raw buffer loads at offsets past
// the range return zeros.  Ranges are clamped below 2^31 so that kOob is
// always out of range.
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7ffffff0ull ? 0x7ffffff0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Blocks are dispatched round-robin over the 8 XCDs.  Renumber so that
// consecutive logical tile ids land on the same XCD (and share its L2).
__device__ __forceinline__ int64_t xcd_logical_id(int64_t bid, int64_t nblocks) {
  const int64_t xcd = bid % kNumXcd;
  const int64_t per = nblocks / kNumXcd, rem = nblocks % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + bid / kNumXcd;
}

// Four 16 B pieces of one row (each 1 fp32 group or 2 f16 groups) -> four
// 16 B plane vectors (F0, F2, Re F1, Im F1), piece j filling slot j (fp32) or
// slots 2j, 2j+1 (f16).  kDft: the pieces hold raw groups (apply the group
// DFT); otherwise they already hold prepared spectra (F0, F2, Re F1, Im F1).
// kConj negates Im F1 (conjugate spectrum).
template <typename E, bool kDft, bool kConj>
__device__ __forceinline__ void pieces_to_planes(const u32x4 (&pc)[4], u32x4 (&pl)[4]);

template <>
__device__ __forceinline__ void pieces_to_planes<float, true, false>(const u32x4 (&pc)[4], u32x4 (&pl)[4]) {
  float v[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 x = __builtin_bit_cast(f32x4, pc[j]);
    dft4(x[0], x[1], x[2], x[3], v[j][0], v[j][1], v[j][2], v[j][3]);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) pl[p] = __builtin_bit_cast(u32x4, f32x4{v[0][p], v[1][p], v[2][p], v[3][p]});
}

template <>
__device__ __forceinline__ void pieces_to_planes<float, true, true>(const u32x4 (&pc)[4], u32x4 (&pl)[4]) {
  float v[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 x = __builtin_bit_cast(f32x4, pc[j]);
    dft4(x[0], x[1], x[2], x[3], v[j][0], v[j][1], v[j][2], v[j][3]);
    v[j][3] = -v[j][3];
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) pl[p] = __builtin_bit_cast(u32x4, f32x4{v[0][p], v[1][p], v[2][p], v[3][p]});
}

template <>
__device__ __forceinline__ void pieces_to_planes<float, false, false>(const u32x4 (&pc)[4], u32x4 (&pl)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) pl[p] = u32x4{pc[0][p], pc[1][p], pc[2][p], pc[3][p]};
}

// Group DFT of the two f16 groups of one 16-byte piece (registers lo01 =
// (z0, z1), hi23 = (z2, z3) of group 0 and lo45 / hi67 of group 1), written as
// packed f16 plane values: p0 = (F0_g0, F0_g1), p2 = (F2_g0, F2_g1),
// p1r = (Re F1_g0, Re F1_g1), p1i = (+-Im F1_g0, +-Im F1_g1).  The mixed
// precision FMA reads f16 halves directly, computes in f32 and rounds the
// result once (nearest-even) into the low or high half of the destination:
//   a = z0 + z2, b = z1 + z3 (f32);  F0 = a + b;  F2 = a - b;
//   Re F1 = z0 - z2;  Im F1 = z3 - z1 (negated when kConj).
template <bool kConj>
__device__ __forceinline__ void dft4_f16_pair(uint32_t z01, uint32_t z23, uint32_t z45, uint32_t z67,
                                              uint32_t& p0, uint32_t& p2, uint32_t& p1r, uint32_t& p1i) {
  float a0, b0, a1, b1;
  asm volatile(
      "v_fma_mix_f32 %0, %4, 1.0, %5 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mix_f32 %1, %4, 1.0, %5 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mix_f32 %2, %6, 1.0, %7 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mix_f32 %3, %6, 1.0, %7 op_sel:[1,0,1] op_sel_hi:[1,0,1]"
      : "=&v"(a0), "=&v"(b0), "=&v"(a1), "=&v"(b1)
      : "v"(z01), "v"(z23), "v"(z45), "v"(z67));
  asm volatile(
      "v_fma_mixlo_f16 %0, %2, 1.0, %3 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %4, 1.0, %5 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixlo_f16 %1, %2, 1.0, -%3 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %1, %4, 1.0, -%5 op_sel_hi:[0,0,0]"
      : "=&v"(p0), "=&v"(p2)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
  asm volatile(
      "v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %3, 1.0, -%4 op_sel:[0,0,0] op_sel_hi:[1,0,1]"
      : "=&v"(p1r)
      : "v"(z01), "v"(z23), "v"(z45), "v"(z67));
  if constexpr (!kConj) {
    asm volatile(
        "v_fma_mixlo_f16 %0, %2, 1.0, -%1 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mixhi_f16 %0, %4, 1.0, -%3 op_sel:[1,0,1] op_sel_hi:[1,0,1]"
        : "=&v"(p1i)
        : "v"(z01), "v"(z23), "v"(z45), "v"(z67));
  } else {
    asm volatile(
        "v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mixhi_f16 %0, %3, 1.0, -%4 op_sel:[1,0,1] op_sel_hi:[1,0,1]"
        : "=&v"(p1i)
        : "v"(z01), "v"(z23), "v"(z45), "v"(z67));
  }
}

template <bool kDft, bool kConj>
__device__ __forceinline__ void pieces_to_planes_f16(const u32x4 (&pc)[4], u32x4 (&pl)[4]) {
  if constexpr (kDft) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p0, p2, p1r, p1i;
      dft4_f16_pair<kConj>(pc[j][0], pc[j][1], pc[j][2], pc[j][3], p0, p2, p1r, p1i);
      pl[0][j] = p0;
      pl[1][j] = p2;
      pl[2][j] = p1r;
      pl[3][j] = p1i;
    }
    return;
  }
  _Float16 h[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x8 x = __builtin_bit_cast(f16x8, pc[j]);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if constexpr (kDft) {
        float f[4];
        dft4((float)x[4 * e + 0], (float)x[4 * e + 1], (float)x[4 * e + 2], (float)x[4 * e + 3],
             f[0], f[1], f[2], f[3]);
        if constexpr (kConj) f[3] = -f[3];
#pragma unroll
        for (int p = 0; p < 4; ++p) h[p][2 * j + e] = (_Float16)f[p];
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) h[p][2 * j + e] = x[4 * e + p];
        if constexpr (kConj) h[3][2 * j + e] = -h[3][2 * j + e];
      }
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    f16x8 o;
#pragma unroll
    for (int s = 0; s < 8; ++s) o[s] = h[p][s];
    pl[p] = __builtin_bit_cast(u32x4, o);
  }
}

template <>
__device__ __forceinline__ void pieces_to_planes<_Float16, true, false>(const u32x4 (&pc)[4], u32x4 (&pl)[4]) {
  pieces_to_planes_f16<true, false>(pc, pl);
}
template <>
__device__ __forceinline__ void pieces_to_planes<_Float16, true, true>(const u32x4 (&pc)[4], u32x4 (&pl)[4]) {
  pieces_to_planes_f16<true, true>(pc, pl);
}
template <>
__device__ __forceinline__ void pieces_to_planes<_Float16, false, false>(const u32x4 (&pc)[4], u32x4 (&pl)[4]) {
  pieces_to_planes_f16<false, false>(pc, pl);
}

// --------------------------------------------------------- MFMA complex core
//
// One 16-byte slot per operand plane and fragment: acc planes
//   0: f0 += A0 B0       1: f2 += A2 B2
//   2: Re f1 += A1r B1r - A1i B1i        3: Im f1 += A1r B1i + A1i B1r
template <typename E, int FM, int FN>
struct Core;

template <int FM, int FN>
struct Core<float, FM, FN> {
  __device__ __forceinline__ static void mma(f32x16 (&acc)[4][FM][FN], const u32x4 (&a)[4][FM],
                                             const u32x4 (&b)[4][FN]) {
    // bit-cast whole vectors, then index (a bit-cast of one vector element
    // would reinterpret the vector's first element)
    f32x4 af[4][FM], bf[4][FN];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) af[p][fm] = __builtin_bit_cast(f32x4, a[p][fm]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) bf[p][fn] = __builtin_bit_cast(f32x4, b[p][fn]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const float a0 = af[0][fm][j];
        const float a2 = af[1][fm][j];
        const float ar = af[2][fm][j];
        const float ai = af[3][fm][j];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const float b0 = bf[0][fn][j];
          const float b2 = bf[1][fn][j];
          const float br = bf[2][fn][j];
          const float bi = bf[3][fn][j];
          acc[0][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][fm][fn], 0, 0, 0);
          acc[2][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(ar, br, acc[2][fm][fn], 0, 0, 0);
          acc[1][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a2, b2, acc[1][fm][fn], 0, 0, 0);
          acc[3][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(ar, bi, acc[3][fm][fn], 0, 0, 0);
          acc[2][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(-ai, bi, acc[2][fm][fn], 0, 0, 0);
          acc[3][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(ai, br, acc[3][fm][fn], 0, 0, 0);
        }
      }
    }
  }
};

template <int FM, int FN>
struct Core<_Float16, FM, FN> {
  __device__ __forceinline__ static void mma(f32x16 (&acc)[4][FM][FN], const u32x4 (&a)[4][FM],
                                             const u32x4 (&b)[4][FN]) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const f16x8 a0 = __builtin_bit_cast(f16x8, a[0][fm]);
      const f16x8 a2 = __builtin_bit_cast(f16x8, a[1][fm]);
      const f16x8 ar = __builtin_bit_cast(f16x8, a[2][fm]);
      const f16x8 ai = __builtin_bit_cast(f16x8, a[3][fm]);
      const f16x8 nai = __builtin_bit_cast(f16x8, a[3][fm] ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const f16x8 b0 = __builtin_bit_cast(f16x8, b[0][fn]);
        const f16x8 b2 = __builtin_bit_cast(f16x8, b[1][fn]);
        const f16x8 br = __builtin_bit_cast(f16x8, b[2][fn]);
        const f16x8 bi = __builtin_bit_cast(f16x8, b[3][fn]);
        acc[0][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc[0][fm][fn], 0, 0, 0);
        acc[2][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ar, br, acc[2][fm][fn], 0, 0, 0);
        acc[1][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a2, b2, acc[1][fm][fn], 0, 0, 0);
        acc[3][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ar, bi, acc[3][fm][fn], 0, 0, 0);
        acc[2][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(nai, bi, acc[2][fm][fn], 0, 0, 0);
        acc[3][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ai, br, acc[3][fm][fn], 0, 0, 0);
      }
    }
  }
};

// Reads this lane's 16-byte operand slot of one chunk from every LDS plane
// and runs the complex core.  a_lds / b_lds point at the lane's slot in plane
// 0 of its first fragment row; plane p is p * a_plane further, fragment fm
// 32 rows further.
template <typename E, int FM, int FN>
__device__ __forceinline__ void mma_chunk(f32x16 (&acc)[4][FM][FN], const char* a_lds, int a_plane,
                                          const char* b_lds, int b_plane, int stride) {
  u32x4 a[4][FM], b[4][FN];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) a[p][fm] = ld16(a_lds + p * a_plane + fm * 32 * stride);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) b[p][fn] = ld16(b_lds + p * b_plane + fn * 32 * stride);
  }
  Core<E, FM, FN>::mma(acc, a, b);
}

// Instruction interleaving for one pipeline stage of fwd_kernel: spread the
// operand reads of the second chunk, the global loads two stages ahead, and
// the next stage's transform and LDS writes between the MFMAs, so that one
// wave keeps its matrix core busy while it prepares the next stage.
// Masks: 0x008 MFMA, 0x100 DS read, 0x200 DS write, 0x020 VMEM read, 0x002 VALU.
template <typename E, int FM, int FN, int PA, int PB>
__device__ __forceinline__ void interleave_schedule() {
  constexpr int kMfma = (sizeof(E) == 4 ? 4 : 1) * 6 * FM * FN * 2;
  constexpr int kDsRead = 2 * 4 * (FM + FN);
  constexpr int kVmem = 4 * (PA + PB);
  constexpr int kDsWrite = 4 * (PA + PB);
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
// out[n][4m + t] = IDFT_t( sum_k Ahat[n][k] (*) Bhat[m][k] )
// A = in [nrows][4 kg] (raw groups, transformed on the fly),
// B = prepared spectra in stage blocks (see prepare_kernel), out [nrows][4 mg].
// A stage covers 64 bytes of every plane row: SG = 16 fp32 or 32 f16 groups
// along k.  Thread t owns row t / 4 (+ NT/4 per pass) and 16-byte slot block
// q = t % 4 of that row: it loads the pieces q + 4j (j = 0..3) of the stage
// window (coalesced), transforms them and writes the contiguous LDS block q
// of each plane; the prepared weights are stored in that same slot order, so
// their 16-byte pieces are copied to LDS unchanged.  Global loads are buffer
// loads: addresses past the end of the tile's range (rows >= nrows) or
// flagged out of range (groups >= kg) return zeros without branches.
// LDS is double-buffered: one barrier per stage, and the loads of stage s+2
// are in flight while stage s is multiplied.
template <typename E, int FM, int FN, int WM, int WN, int NBUF>
constexpr int fwd_lds_bytes() {
  return NBUF * 4 * (32 * FM * WM + 32 * FN * WN) * kRowBytes;
}

// One forward (or dX) tile: workgroup-level logical tile id `lid`.  NBUF = 2
// double-buffers the LDS stages (one barrier per stage); NBUF = 1 halves the
// LDS footprint (two barriers per stage) so that more workgroups fit a CU.
// PF (1 or 2) is the number of stages whose global loads are in flight in
// registers ahead of the stage being transformed into LDS: with f16 a stage
// of MFMAs is short next to the memory latency, so two stages are needed.
template <typename E, int FM, int FN, int WM, int WN, int NBUF, int PF, int SCHED>
__device__ __forceinline__ void fwd_tile(char* lds, int64_t lid, const E* __restrict__ in,
                                         const E* __restrict__ wp, E* __restrict__ out, int64_t nrows, int kg,
                                         int mg, int tiles_n, const E* __restrict__ bias, int act) {
  constexpr int NT = 64 * WM * WN;
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  constexpr int GP = Traits<E>::kGroupsPerPiece;
  constexpr int SG = 16 * GP;              // groups per stage
  constexpr int STRIDE = kRowBytes;
  constexpr int A_PLANE = BM * STRIDE, B_PLANE = BN * STRIDE;
  constexpr int BUF = 4 * (A_PLANE + B_PLANE);
  constexpr int RPP = NT / 4;              // tile rows covered per load pass
  constexpr int PA = (BM + RPP - 1) / RPP, PB = (BN + RPP - 1) / RPP;
  static_assert(NBUF * BUF == fwd_lds_bytes<E, FM, FN, WM, WN, NBUF>(), "LDS size");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (lid / tiles_n) * BM;
  const int col0 = (int)(lid % tiles_n) * BN;
  const int ksteps = (kg + SG - 1) / SG;

  const uint32_t row_bytes = (uint32_t)kg * 4u * (uint32_t)sizeof(E);
  const __amdgpu_buffer_rsrc_t a_src =
      make_rsrc(in + row0 * 4 * (int64_t)kg, (uint64_t)(nrows - row0) * row_bytes);
  const __amdgpu_buffer_rsrc_t b_src =
      make_rsrc(wp + (int64_t)col0 * ksteps * SG * 4, (uint64_t)(mg - col0) * (uint64_t)ksteps * 256u);

  const int q = tid & 3, rl = tid >> 2;
  u32x4 ra[PF][PA][4], rb[PF][PB][4];   // register ring of PF stages of loads
  auto load = [&](int ks, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int ps = 0; ps < PA; ++ps) {
      const uint32_t r = (uint32_t)(ps * RPP + rl);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = ks * SG + (q + 4 * j) * GP;
        const uint32_t off = g < kg ? r * row_bytes + (uint32_t)g * 4u * (uint32_t)sizeof(E) : kOob;
        ra[sl][ps][j] = bload16(a_src, off);
      }
    }
#pragma unroll
    for (int ps = 0; ps < PB; ++ps) {
      const uint32_t m = (uint32_t)(ps * RPP + rl);
#pragma unroll
      for (int p = 0; p < 4; ++p)
        rb[sl][ps][p] =
            bload16(b_src, ks < ksteps ? (m * (uint32_t)ksteps + (uint32_t)ks) * 256u + p * 64 + q * 16 : kOob);
    }
  };
  auto store = [&](char* buf, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int ps = 0; ps < PA; ++ps) {
      const int r = ps * RPP + rl;
      if (BM % RPP == 0 || r < BM) {
        u32x4 pl[4];
        pieces_to_planes<E, true, false>(ra[sl][ps], pl);
#pragma unroll
        for (int p = 0; p < 4; ++p) st16(buf + p * A_PLANE + r * STRIDE + swz_slot(r, q) * 16, pl[p]);
      }
    }
#pragma unroll
    for (int ps = 0; ps < PB; ++ps) {
      const int m = ps * RPP + rl;
      if (BN % RPP == 0 || m < BN) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          st16(buf + 4 * A_PLANE + p * B_PLANE + m * STRIDE + swz_slot(m, q) * 16, rb[sl][ps][p]);
      }
    }
  };

  f32x16 acc[4][FM][FN];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[p][fm][fn] = f32x16{};

  const int wr = wave / WN, wc = wave % WN;
  const int li = lane & 31, lh = lane >> 5;
  // fragment rows differ from li by multiples of 32, so the swizzle of every
  // row this lane reads is that of li
  const int a_frag = (wr * 32 * FM + li) * STRIDE;
  const int b_frag = 4 * A_PLANE + (wc * 32 * FN + li) * STRIDE;
  const int c0 = swz_slot(li, lh) * 16, c1 = swz_slot(li, 2 + lh) * 16;

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, PF - 1>;
  // One pipeline step: multiply stage ks (LDS buffer of ks), then transform
  // the registers of stage ks + 1 into the other (or, single-buffered, the
  // same) buffer and issue the loads of stage ks + 1 + PF into the slot just
  // freed.  Past the last stage the loads read zeros (out of range) and the
  // stores fill an idle buffer, so the body is one basic block in which the
  // scheduler can interleave MFMAs with the transform, LDS writes and loads.
  auto step = [&](int ks, auto slot_next) {
    char* cur = lds + (NBUF == 2 ? (ks & 1) * BUF : 0);
    mma_chunk<E, FM, FN>(acc, cur + a_frag + c0, A_PLANE, cur + b_frag + c0, B_PLANE, STRIDE);
    mma_chunk<E, FM, FN>(acc, cur + a_frag + c1, A_PLANE, cur + b_frag + c1, B_PLANE, STRIDE);
    if constexpr (NBUF == 1) __syncthreads();   // every wave is done reading the only buffer
    store(lds + (NBUF == 2 ? ((ks + 1) & 1) * BUF : 0), slot_next);
    load(ks + 1 + PF, slot_next);
    if constexpr (SCHED == 1 && NBUF == 2) interleave_schedule<E, FM, FN, PA, PB>();
    __syncthreads();
  };

  load(0, S0{});
  store(lds, S0{});
  if constexpr (PF == 1) {
    load(1, S0{});
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) step(ks, S0{});
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

  // epilogue: inverse group DFT in registers, optional group-invariant bias
  // and GELU, one vector store per (row, group)
  const int64_t out_ld = 4 * (int64_t)mg;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int m = col0 + wc * 32 * FN + fn * 32 + li;
      const float bm = (bias != nullptr && m < mg) ? (float)bias[m] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + wr * 32 * FM + fm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < nrows && m < mg) {
          float y[4];
          idft4(acc[0][fm][fn][r], acc[1][fm][fn][r], acc[2][fm][fn][r], acc[3][fm][fn][r], y);
          if (bias != nullptr) {
#pragma unroll
            for (int t = 0; t < 4; ++t) y[t] += bm;
          }
          if (act == 1) {
#pragma unroll
            for (int t = 0; t < 4; ++t) y[t] = gelu_erf(y[t]);
          }
          E* dst = out + row * out_ld + 4 * (int64_t)m;
          if constexpr (sizeof(E) == 4) {
            st16(dst, __builtin_bit_cast(u32x4, f32x4{y[0], y[1], y[2], y[3]}));
          } else {
            const f16x4 h = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
            *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, h);
          }
        }
      }
    }
  }
}

// Two waves per SIMD (256 registers per lane) unless a wave holds 4+ fragments.
template <typename E, int FM, int FN, int WM, int WN, int NBUF, int PF, int SCHED>
__global__ void __launch_bounds__(64 * WM * WN, FM * FN >= 4 ? 1 : 2)
fwd_kernel(const E* __restrict__ in, const E* __restrict__ wp, E* __restrict__ out,
           int64_t nrows, int kg, int mg, int tiles_n, const E* __restrict__ bias, int act) {
  __shared__ __attribute__((aligned(16))) char lds[fwd_lds_bytes<E, FM, FN, WM, WN, NBUF>()];
  fwd_tile<E, FM, FN, WM, WN, NBUF, PF, SCHED>(lds, xcd_logical_id(blockIdx.x, gridDim.x), in, wp, out, nrows, kg, mg,
                                     tiles_n, bias, act);
}

// ============================================================ dw partials
//
// P_k[m][n] = sum_rows G_k[row][m] conj(Xhat_k[row][n])   (m = d', n = c')
// over the rows of one split; the four planes are written to
// ws[split][plane][mg][ng] (float32).  Tiles 64 x 64, one 32 x 32 fragment
// per wave and plane.  The k axis is the row axis: thread (piece column pc,
// row block rq) loads 4 consecutive rows of one 16 B piece (1 fp32 or 2 f16
// groups), transforms them and writes, per group and plane, the 4 rows as one
// contiguous LDS vector (16 B fp32, 8 B f16).  A stage is 64 bytes of every
// plane row (16 fp32 / 32 f16 rows); LDS is double-buffered as in fwd_kernel.
template <int NBUF>
constexpr int dw_lds_bytes() {
  return NBUF * 8 * 64 * kRowBytes;
}

template <typename E, int NBUF>
__device__ __forceinline__ void dw_tile(char* lds, int64_t lid, const E* __restrict__ dy, const E* __restrict__ x,
                                        float* __restrict__ ws, int64_t nrows, int mg, int ng,
                                        int64_t rows_per_split, int tiles_m, int tiles_n) {
  constexpr int GP = Traits<E>::kGroupsPerPiece;
  constexpr int KV = 4;                            // rows per thread per stage
  constexpr int PR = 64 / GP;                      // pieces per tile row (64 groups)
  constexpr int RB = kThreads / PR;                // row blocks per stage
  constexpr int SR = RB * KV;                      // rows per stage: 16 (fp32) / 32 (f16)
  constexpr int STRIDE = kRowBytes;
  constexpr int PLANE = 64 * STRIDE;
  constexpr int BUF = 8 * PLANE;
  static_assert(SR * (int)sizeof(E) == 64, "one stage is 64 bytes per plane row");
  static_assert(NBUF * BUF == dw_lds_bytes<NBUF>(), "LDS size");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = tiles_m * tiles_n;
  const int64_t split = lid / ntiles;
  const int tile = (int)(lid % ntiles);
  const int m0 = (tile / tiles_n) * 64, n0 = (tile % tiles_n) * 64;
  const int64_t rbeg = split * rows_per_split;
  const int64_t rend = (rbeg + rows_per_split < nrows) ? rbeg + rows_per_split : nrows;
  const int nstages = (int)((rend - rbeg + SR - 1) / SR);

  const uint32_t a_row = (uint32_t)mg * 4u * (uint32_t)sizeof(E);
  const uint32_t b_row = (uint32_t)ng * 4u * (uint32_t)sizeof(E);
  const __amdgpu_buffer_rsrc_t a_src = make_rsrc(dy + rbeg * 4 * (int64_t)mg, (uint64_t)(rend - rbeg) * a_row);
  const __amdgpu_buffer_rsrc_t b_src = make_rsrc(x + rbeg * 4 * (int64_t)ng, (uint64_t)(rend - rbeg) * b_row);

  const int pc = tid % PR, rq = tid / PR;
  const int ga = m0 + pc * GP, gb = n0 + pc * GP;
  const bool a_ok = ga < mg, b_ok = gb < ng;
  const uint32_t a_col = (uint32_t)ga * 4u * (uint32_t)sizeof(E);
  const uint32_t b_col = (uint32_t)gb * 4u * (uint32_t)sizeof(E);

  u32x4 ra[KV], rb[KV];
  auto load = [&](int st) {
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const uint32_t row = (uint32_t)(st * SR + rq * KV + v);
      ra[v] = bload16(a_src, a_ok ? row * a_row + a_col : kOob);
      rb[v] = bload16(b_src, b_ok ? row * b_row + b_col : kOob);
    }
  };
  auto store = [&](char* buf) {
    char* a_lds = buf;
    char* b_lds = buf + 4 * PLANE;
    if constexpr (sizeof(E) == 4) {
      u32x4 pa[4], pb[4];
      pieces_to_planes<float, true, false>(ra, pa);
      pieces_to_planes<float, true, true>(rb, pb);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        st16(a_lds + p * PLANE + pc * STRIDE + swz_slot(pc, rq) * 16, pa[p]);
        st16(b_lds + p * PLANE + pc * STRIDE + swz_slot(pc, rq) * 16, pb[p]);
      }
    } else {
      // 4 rows x 2 groups per operand: transform, gather 4 rows per (group, plane)
      f16x4 ha[2][4], hb[2][4];
#pragma unroll
      for (int v = 0; v < KV; ++v) {
        const f16x8 xa = __builtin_bit_cast(f16x8, ra[v]);
        const f16x8 xb = __builtin_bit_cast(f16x8, rb[v]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float f[4], g[4];
          dft4((float)xa[4 * e], (float)xa[4 * e + 1], (float)xa[4 * e + 2], (float)xa[4 * e + 3],
               f[0], f[1], f[2], f[3]);
          dft4((float)xb[4 * e], (float)xb[4 * e + 1], (float)xb[4 * e + 2], (float)xb[4 * e + 3],
               g[0], g[1], g[2], g[3]);
          g[3] = -g[3];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            ha[e][p][v] = (_Float16)f[p];
            hb[e][p][v] = (_Float16)g[p];
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int row = pc * 2 + e;
          const int off = row * STRIDE + swz_slot(row, rq >> 1) * 16 + (rq & 1) * 8;
          *reinterpret_cast<u32x2*>(a_lds + p * PLANE + off) = __builtin_bit_cast(u32x2, ha[e][p]);
          *reinterpret_cast<u32x2*>(b_lds + p * PLANE + off) = __builtin_bit_cast(u32x2, hb[e][p]);
        }
      }
    }
  };

  f32x16 acc[4][1][1];
#pragma unroll
  for (int p = 0; p < 4; ++p) acc[p][0][0] = f32x16{};

  const int wr = wave >> 1, wc = wave & 1;
  const int li = lane & 31, lh = lane >> 5;
  const int a_frag = (wr * 32 + li) * STRIDE;
  const int b_frag = 4 * PLANE + (wc * 32 + li) * STRIDE;
  const int c0 = swz_slot(li, lh) * 16, c1 = swz_slot(li, 2 + lh) * 16;

  if (nstages > 0) {
    load(0);
    store(lds);
    if (nstages > 1) load(1);
    __syncthreads();
  }
  for (int st = 0; st < nstages; ++st) {
    char* cur = lds + (NBUF == 2 ? (st & 1) * BUF : 0);
    mma_chunk<E, 1, 1>(acc, cur + a_frag + c0, PLANE, cur + b_frag + c0, PLANE, STRIDE);
    mma_chunk<E, 1, 1>(acc, cur + a_frag + c1, PLANE, cur + b_frag + c1, PLANE, STRIDE);
    if (st + 1 < nstages) {
      if constexpr (NBUF == 1) __syncthreads();   // every wave is done reading the only buffer
      store(lds + (NBUF == 2 ? ((st + 1) & 1) * BUF : 0));
      if (st + 2 < nstages) load(st + 2);
    }
    __syncthreads();
  }

  const int64_t plane_elems = (int64_t)mg * ng;
  float* dst = ws + split * 4 * plane_elems;
  const int n = n0 + wc * 32 + li;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wr * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
    if (m < mg && n < ng) {
#pragma unroll
      for (int p = 0; p < 4; ++p) dst[p * plane_elems + (int64_t)m * ng + n] = acc[p][0][0][r];
    }
  }
}

template <typename E>
__global__ void __launch_bounds__(kThreads, 2)
dw_partial_kernel(const E* __restrict__ dy, const E* __restrict__ x, float* __restrict__ ws,
                  int64_t nrows, int mg, int ng, int64_t rows_per_split, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[dw_lds_bytes<kDwBufs>()];
  dw_tile<E, kDwBufs>(lds, xcd_logical_id(blockIdx.x, gridDim.x), dy, x, ws, nrows, mg, ng, rows_per_split, tiles_m,
             tiles_n);
}

// Backward in one launch: the first ndw_pad workgroups are dw split partials,
// the rest are dX tiles (the forward structure on the transpose spectra).
// Both roles read dY; running them in one grid lets the dispatcher fill the
// tail of one role with work of the other.  ndw_pad is a multiple of 8, so
// each role keeps its own XCD-aware numbering.
template <typename E, int SCHED>
__global__ void __launch_bounds__(kThreads, 2)
bwd_fused_kernel(const E* __restrict__ dy, const E* __restrict__ x, const E* __restrict__ wb,
                 E* __restrict__ dx, float* __restrict__ ws, int64_t nrows, int dg, int cg,
                 int64_t rows_per_split, int dw_tiles_m, int dw_tiles_n, int64_t ndw, int64_t ndw_pad,
                 int dx_tiles_n) {
  constexpr int kLds = fwd_lds_bytes<E, 1, 1, 2, 2, kBwdFwdBufs>() > dw_lds_bytes<kDwBufs>()
                           ? fwd_lds_bytes<E, 1, 1, 2, 2, kBwdFwdBufs>()
                           : dw_lds_bytes<kDwBufs>();
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  const int64_t b = blockIdx.x;
  if (b < ndw_pad) {
    const int64_t lid = xcd_logical_id(b, ndw_pad);
    if (lid < ndw) dw_tile<E, kDwBufs>(lds, lid, dy, x, ws, nrows, dg, cg, rows_per_split, dw_tiles_m, dw_tiles_n);
  } else {
    const int64_t nb = gridDim.x - ndw_pad;
    fwd_tile<E, 1, 1, 2, 2, kBwdFwdBufs, kBwdFwdPrefetch, SCHED>(lds, xcd_logical_id(b - ndw_pad, nb), dy, wb, dx, nrows, dg, cg, dx_tiles_n,
                                   nullptr, 0);
  }
}

// Sum the split partials in split order (deterministic), inverse group DFT
// along u, write dw[m][n][0..3] (float32).  Thread (plane p, entry e) of a
// 256-thread block sums plane p of one of 64 consecutive entries; the four
// plane sums meet in LDS and one thread per entry applies the inverse DFT.
// nsplit == 0 writes zeros.
__global__ void __launch_bounds__(kThreads)
dw_finalize_kernel(const float* __restrict__ ws, float* __restrict__ dw, int mg, int ng, int nsplit) {
  __shared__ float part[4][64];
  const int64_t plane = (int64_t)mg * ng;
  const int e = threadIdx.x & 63, p = threadIdx.x >> 6;
  const int64_t idx = (int64_t)blockIdx.x * 64 + e;
  float acc = 0.f;
  if (idx < plane) {
    const float* src = ws + p * plane + idx;
    const int64_t step = 4 * plane;
    int s = 0;
    for (; s + 4 <= nsplit; s += 4) {
      const float v0 = src[(s + 0) * step], v1 = src[(s + 1) * step];
      const float v2 = src[(s + 2) * step], v3 = src[(s + 3) * step];
      acc += v0;
      acc += v1;
      acc += v2;
      acc += v3;
    }
    for (; s < nsplit; ++s) acc += src[s * step];
  }
  part[p][e] = acc;
  __syncthreads();
  if (p == 0 && idx < plane) {
    float y[4];
    idft4(part[0][e], part[1][e], part[2][e], part[3][e], y);
    st16(dw + idx * 4, __builtin_bit_cast(u32x4, f32x4{y[0], y[1], y[2], y[3]}));
  }
}

// ============================================================ prepare
//
// Weight spectra in the stage-block layout read by fwd_kernel:
//   dst[row][ks][plane][s]   (SG = 16 fp32 / 32 f16 slots per 64-byte block)
// where slot s of stage ks holds group channel ks * SG + slot_group(s) (the
// slot order fwd_kernel's loaders produce for the transformed input) and
// groups past the end are zero.
//   forward planes:   row = d', groups = c',  (F0, F2, Re F1,  Im F1) of w[d'][c']
//   transpose planes: row = c', groups = d',  (F0, F2, Re F1, -Im F1) of w[d'][c']
// The second set is the spectrum of the transposed, group-reversed weight
// (a conjugate), used by the dX pass.
template <typename E>
__host__ __device__ constexpr int slot_group(int s) {
  return sizeof(E) == 4 ? (s >> 2) + 4 * (s & 3) : 2 * ((s >> 3) + 4 * ((s >> 1) & 3)) + (s & 1);
}

template <typename E, bool kTranspose>
__global__ void __launch_bounds__(kThreads)
prepare_kernel(const E* __restrict__ w, E* __restrict__ dst, int mg, int ng) {
  constexpr int SG = 16 * Traits<E>::kGroupsPerPiece;
  const int rows = kTranspose ? ng : mg;
  const int kgr = kTranspose ? mg : ng;
  const int nks = (kgr + SG - 1) / SG;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)rows * nks * SG) return;
  const int s = (int)(idx % SG);
  const int64_t t = idx / SG;
  const int ks = (int)(t % nks);
  const int64_t row = t / nks;
  const int g = ks * SG + slot_group<E>(s);
  float f[4] = {0.f, 0.f, 0.f, 0.f};
  if (g < kgr) {
    const E* src = kTranspose ? w + ((int64_t)g * ng + row) * 4 : w + (row * ng + g) * 4;
    dft4((float)src[0], (float)src[1], (float)src[2], (float)src[3], f[0], f[1], f[2], f[3]);
    if (kTranspose) f[3] = -f[3];
  }
  E* o = dst + (row * nks + ks) * 4 * SG + s;
#pragma unroll
  for (int p = 0; p < 4; ++p) o[p * SG] = (E)f[p];
}

// ============================================================ launchers

namespace {
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

template <typename E, int FM, int FN, int WM, int WN, int NBUF, int PF, int SCHED>
hipError_t launch_fwd_s(const void* in, const void* wp, void* out, int64_t nrows, int kg, int mg,
                        const void* bias, int act, hipStream_t s) {
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  const int64_t tiles_m = cdiv(nrows, BM);
  const int tiles_n = (int)cdiv(mg, BN);
  const int64_t grid = tiles_m * tiles_n;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<E, FM, FN, WM, WN, NBUF, PF, SCHED>), dim3((unsigned)grid), dim3(64 * WM * WN), 0, s,
                     static_cast<const E*>(in), static_cast<const E*>(wp), static_cast<E*>(out), nrows, kg, mg,
                     tiles_n, static_cast<const E*>(bias), act);
  return hipGetLastError();
}

template <typename E, int FM, int FN, int WM, int WN, int NBUF, int PF>
hipError_t launch_fwd_t(const void* in, const void* wp, void* out, int64_t nrows, int kg, int mg, const void* bias,
                        int act, hipStream_t s) {
  static const int sched = [] {
    const char* e = getenv("EQLIN_SCHED");
    return e ? atoi(e) : 1;
  }();
  return sched == 1 ? launch_fwd_s<E, FM, FN, WM, WN, NBUF, PF, 1>(in, wp, out, nrows, kg, mg, bias, act, s)
                    : launch_fwd_s<E, FM, FN, WM, WN, NBUF, PF, 0>(in, wp, out, nrows, kg, mg, bias, act, s);
}

// compiled forward tiles, code = FM FN WM WN NBUF PF (decimal digits)
#define EQLIN_FWD_TILES(X)                                                                       \
  X(112221) X(111221) X(112121) X(222221) X(212421) X(112411) X(212211) X(122211) X(112211)      \
  X(112212) X(112412)

bool fwd_tile_known(int tile) {
  switch (tile) {
#define EQLIN_CASE(T) case T:
    EQLIN_FWD_TILES(EQLIN_CASE)
#undef EQLIN_CASE
    return true;
    default: return false;
  }
}

hipError_t launch_forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t nrows,
                          int kg, int mg, const void* bias, int act, hipStream_t s) {
#define EQLIN_CASE(T)                                                                                  \
  case T:                                                                                              \
    return dtype == 0 ? launch_fwd_t<float, T / 100000, (T / 10000) % 10, (T / 1000) % 10, (T / 100) % 10, \
                                     (T / 10) % 10, T % 10>(in, wp, out, nrows, kg, mg, bias, act, s)          \
                      : launch_fwd_t<_Float16, T / 100000, (T / 10000) % 10, (T / 1000) % 10, (T / 100) % 10,  \
                                     (T / 10) % 10, T % 10>(in, wp, out, nrows, kg, mg, bias, act, s);
  switch (tile) {
    EQLIN_FWD_TILES(EQLIN_CASE)
    default: return hipErrorInvalidValue;
  }
#undef EQLIN_CASE
}

int stage_groups(int dtype) { return dtype == 0 ? 16 : 32; }
int dw_rows_per_stage(int dtype) { return dtype == 0 ? 16 : 32; }

hipError_t launch_dw(int dtype, const void* dy, const void* x, float* ws, float* dw, int64_t nrows, int mg,
                     int ng, int64_t rows_per_split, int nsplit, hipStream_t s) {
  const int tiles_m = (int)cdiv(mg, 64), tiles_n = (int)cdiv(ng, 64);
  if (nsplit > 0) {
    const int64_t grid = (int64_t)tiles_m * tiles_n * nsplit;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (dtype == 0) {
      hipLaunchKernelGGL((dw_partial_kernel<float>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                         static_cast<const float*>(dy), static_cast<const float*>(x), ws, nrows, mg, ng,
                         rows_per_split, tiles_m, tiles_n);
    } else {
      hipLaunchKernelGGL((dw_partial_kernel<_Float16>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                         static_cast<const _Float16*>(dy), static_cast<const _Float16*>(x), ws, nrows, mg, ng,
                         rows_per_split, tiles_m, tiles_n);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t fgrid = cdiv((int64_t)mg * ng, 64);
  hipLaunchKernelGGL(dw_finalize_kernel, dim3((unsigned)fgrid), dim3(kThreads), 0, s, ws, dw, mg, ng, nsplit);
  return hipGetLastError();
}

hipError_t launch_bwd_fused(int dtype, const void* dy, const void* x, const void* wb, void* dx, float* ws,
                            float* dw, int64_t nrows, int dg, int cg, int64_t rows_per_split, int nsplit,
                            hipStream_t s) {
  const int dw_tiles_m = (int)cdiv(dg, 64), dw_tiles_n = (int)cdiv(cg, 64);
  const int64_t ndw = (int64_t)dw_tiles_m * dw_tiles_n * nsplit;
  const int64_t ndw_pad = cdiv(ndw, 8) * 8;
  const int dx_tiles_n = (int)cdiv(cg, 64);
  const int64_t ndx = cdiv(nrows, 64) * dx_tiles_n;
  const int64_t grid = ndw_pad + ndx;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (grid > 0) {
    if (dtype == 0) {
      hipLaunchKernelGGL((bwd_fused_kernel<float, 1>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                         static_cast<const float*>(dy), static_cast<const float*>(x),
                         static_cast<const float*>(wb), static_cast<float*>(dx), ws, nrows, dg, cg,
                         rows_per_split, dw_tiles_m, dw_tiles_n, ndw, ndw_pad, dx_tiles_n);
    } else {
      hipLaunchKernelGGL((bwd_fused_kernel<_Float16, 1>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                         static_cast<const _Float16*>(dy), static_cast<const _Float16*>(x),
                         static_cast<const _Float16*>(wb), static_cast<_Float16*>(dx), ws, nrows, dg, cg,
                         rows_per_split, dw_tiles_m, dw_tiles_n, ndw, ndw_pad, dx_tiles_n);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t fgrid = cdiv((int64_t)dg * cg, 64);
  hipLaunchKernelGGL(dw_finalize_kernel, dim3((unsigned)fgrid), dim3(kThreads), 0, s, ws, dw, dg, cg, nsplit);
  return hipGetLastError();
}

hipError_t launch_prepare(int dtype, const void* w, void* wf, void* wb, int mg, int ng, hipStream_t s) {
  const int sg = stage_groups(dtype);
  const int64_t nf = (int64_t)mg * cdiv(ng, sg) * sg, nb = (int64_t)ng * cdiv(mg, sg) * sg;
  if (dtype == 0) {
    hipLaunchKernelGGL((prepare_kernel<float, false>), dim3((unsigned)cdiv(nf, kThreads)), dim3(kThreads), 0, s,
                       static_cast<const float*>(w), static_cast<float*>(wf), mg, ng);
    hipLaunchKernelGGL((prepare_kernel<float, true>), dim3((unsigned)cdiv(nb, kThreads)), dim3(kThreads), 0, s,
                       static_cast<const float*>(w), static_cast<float*>(wb), mg, ng);
  } else {
    hipLaunchKernelGGL((prepare_kernel<_Float16, false>), dim3((unsigned)cdiv(nf, kThreads)), dim3(kThreads), 0,
                       s, static_cast<const _Float16*>(w), static_cast<_Float16*>(wf), mg, ng);
    hipLaunchKernelGGL((prepare_kernel<_Float16, true>), dim3((unsigned)cdiv(nb, kThreads)), dim3(kThreads), 0,
                       s, static_cast<const _Float16*>(w), static_cast<_Float16*>(wb), mg, ng);
  }
  return hipGetLastError();
}

}  // namespace eqlin
