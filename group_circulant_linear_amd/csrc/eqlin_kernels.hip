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
// [plane][row][k] with k contiguous (16 B padding per row keeps the 16-byte
// LDS reads of 32 consecutive rows on distinct banks).  Every lane reads 16
// bytes per plane per 32x32 fragment: 4 fp32 k-values (four 32x32x2 f32
// MFMAs) or 8 f16 k-values (one 32x32x16 f16 MFMA).  A workgroup has four
// 64-wide waves in a 2 x 2 arrangement; each wave owns FM x FN fragments of
// 32 x 32 for each of the four accumulator planes (f0, f2, Re f1, Im f1).
#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
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

template <bool kDft, bool kConj>
__device__ __forceinline__ void pieces_to_planes_f16(const u32x4 (&pc)[4], u32x4 (&pl)[4]) {
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

// Reads this lane's operand slots of chunk `c` from the LDS planes and runs
// the complex core.  Plane p of A starts at a_lds + p * a_plane; row r at
// r * stride; the lane reads 16 B at byte c * 32 + half * 16 of rows
// (wave_row + 32 fm + lane % 32).
template <typename E, int FM, int FN>
__device__ __forceinline__ void mma_chunk(f32x16 (&acc)[4][FM][FN], const char* a_lds, int a_plane,
                                          const char* b_lds, int b_plane, int stride, int c) {
  u32x4 a[4][FM], b[4][FN];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) a[p][fm] = ld16(a_lds + p * a_plane + fm * 32 * stride + c * 32);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) b[p][fn] = ld16(b_lds + p * b_plane + fn * 32 * stride + c * 32);
  }
  Core<E, FM, FN>::mma(acc, a, b);
}

// ============================================================ forward / dX
//
// out[n][4m + t] = IDFT_t( sum_k Ahat[n][k] (*) Bhat[m][k] )
// A = in [nrows][4 kg] (raw groups, transformed on the fly),
// B = prepared spectra wp [mg][kg][4], out [nrows][4 mg].
// Stage = 64 bytes per plane row (16 fp32 or 32 f16 groups along k).
// Thread t loads, for rows t/4 (+64 per pass), the 16 B pieces q + 4j
// (q = t % 4, j = 0..3) of the stage window: coalesced global reads, and the
// four pieces land in the contiguous LDS slots [16q, 16q+16) of each plane
// (a fixed permutation of k inside the stage, identical for A and B).
template <typename E, int FM, int FN>
__global__ void __launch_bounds__(kThreads)
fwd_kernel(const E* __restrict__ in, const E* __restrict__ wp, E* __restrict__ out,
           int64_t nrows, int kg, int mg, int tiles_n) {
  constexpr int BM = 64 * FM, BN = 64 * FN;
  constexpr int GP = Traits<E>::kGroupsPerPiece;
  constexpr int SG = 16 * GP;              // groups per stage
  constexpr int STRIDE = 80;               // 64 B + 16 B pad
  constexpr int A_PLANE = BM * STRIDE, B_PLANE = BN * STRIDE;
  __shared__ __attribute__((aligned(16))) char lds[4 * (A_PLANE + B_PLANE)];
  char* a_lds = lds;
  char* b_lds = lds + 4 * A_PLANE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int64_t tm = lid / tiles_n;
  const int tn = (int)(lid % tiles_n);
  const int64_t row0 = tm * BM;
  const int col0 = tn * BN;

  const int64_t in_ld = 4 * (int64_t)kg;    // elements per input row
  const int q = tid & 3, rl = tid >> 2;
  const int ksteps = (kg + SG - 1) / SG;

  // stage register buffers
  u32x4 ra[FM][4], rb[FN][4];
  auto load_stage = [&](int ks) {
#pragma unroll
    for (int ps = 0; ps < FM; ++ps) {
      const int64_t row = row0 + ps * 64 + rl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = ks * SG + (q + 4 * j) * GP;
        ra[ps][j] = (row < nrows && g < kg) ? ld16(in + row * in_ld + 4 * (int64_t)g) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int ps = 0; ps < FN; ++ps) {
      const int m = col0 + ps * 64 + rl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = ks * SG + (q + 4 * j) * GP;
        rb[ps][j] = (m < mg && g < kg) ? ld16(wp + ((int64_t)m * kg + g) * 4) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int ps = 0; ps < FM; ++ps) {
      u32x4 pl[4];
      pieces_to_planes<E, true, false>(ra[ps], pl);
#pragma unroll
      for (int p = 0; p < 4; ++p) st16(a_lds + p * A_PLANE + (ps * 64 + rl) * STRIDE + q * 16, pl[p]);
    }
#pragma unroll
    for (int ps = 0; ps < FN; ++ps) {
      u32x4 pl[4];
      pieces_to_planes<E, false, false>(rb[ps], pl);
#pragma unroll
      for (int p = 0; p < 4; ++p) st16(b_lds + p * B_PLANE + (ps * 64 + rl) * STRIDE + q * 16, pl[p]);
    }
  };

  f32x16 acc[4][FM][FN];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[p][fm][fn] = f32x16{};

  const int wr = wave >> 1, wc = wave & 1;
  const int li = lane & 31, lh = lane >> 5;
  const char* a_frag = a_lds + (wr * 32 * FM + li) * STRIDE + lh * 16;
  const char* b_frag = b_lds + (wc * 32 * FN + li) * STRIDE + lh * 16;

  load_stage(0);
  for (int ks = 0; ks < ksteps; ++ks) {
    store_stage();
    __syncthreads();
    if (ks + 1 < ksteps) load_stage(ks + 1);
    mma_chunk<E, FM, FN>(acc, a_frag, A_PLANE, b_frag, B_PLANE, STRIDE, 0);
    mma_chunk<E, FM, FN>(acc, a_frag, A_PLANE, b_frag, B_PLANE, STRIDE, 1);
    __syncthreads();
  }

  // epilogue: inverse group DFT in registers, one vector store per (row, group)
  const int64_t out_ld = 4 * (int64_t)mg;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int m = col0 + wc * 32 * FN + fn * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + wr * 32 * FM + fm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < nrows && m < mg) {
          float y[4];
          idft4(acc[0][fm][fn][r], acc[1][fm][fn][r], acc[2][fm][fn][r], acc[3][fm][fn][r], y);
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

// ============================================================ dw partials
//
// P_k[m][n] = sum_rows G_k[row][m] conj(Xhat_k[row][n])   (m = d', n = c')
// over the rows of one split; the four planes are written to
// ws[split][plane][mg][ng] (float32).  Tiles 64 x 64, one 32 x 32 fragment
// per wave and plane.  The k axis is the row axis: thread (piece column pc,
// row block rq) loads KV consecutive rows of one 16 B piece, so every LDS
// write is one 16 B vector of KV consecutive rows of one plane.
template <typename E>
__global__ void __launch_bounds__(kThreads)
dw_partial_kernel(const E* __restrict__ dy, const E* __restrict__ x, float* __restrict__ ws,
                  int64_t nrows, int mg, int ng, int64_t rows_per_split, int tiles_m, int tiles_n) {
  constexpr int GP = Traits<E>::kGroupsPerPiece;
  constexpr int KV = Traits<E>::kValsPerSlot;      // rows per thread (one 16 B slot)
  constexpr int PR = 64 / GP;                      // pieces per tile row (64 groups)
  constexpr int RB = kThreads / PR;                // row blocks per stage
  constexpr int SR = RB * KV;                      // rows per stage: 16 (fp32) / 64 (f16)
  constexpr int NCH = SR * (int)sizeof(E) / 32;    // 32-byte chunks per plane row
  constexpr int STRIDE = SR * (int)sizeof(E) + 16;
  constexpr int PLANE = 64 * STRIDE;
  __shared__ __attribute__((aligned(16))) char lds[8 * PLANE];
  char* a_lds = lds;
  char* b_lds = lds + 4 * PLANE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = tiles_m * tiles_n;
  const int64_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int64_t split = lid / ntiles;
  const int tile = (int)(lid % ntiles);
  const int m0 = (tile / tiles_n) * 64, n0 = (tile % tiles_n) * 64;
  const int64_t rbeg = split * rows_per_split;
  const int64_t rend = (rbeg + rows_per_split < nrows) ? rbeg + rows_per_split : nrows;

  const int pc = tid % PR, rq = tid / PR;
  const int64_t a_ld = 4 * (int64_t)mg, b_ld = 4 * (int64_t)ng;
  const int ga = m0 + pc * GP, gb = n0 + pc * GP;

  u32x4 ra[KV / 4][4], rb[KV / 4][4];
  auto load_stage = [&](int64_t r0) {
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int64_t row = r0 + rq * KV + v;
      const bool ok = row < rend;
      ra[v / 4][v % 4] = (ok && ga < mg) ? ld16(dy + row * a_ld + 4 * (int64_t)ga) : u32x4{0, 0, 0, 0};
      rb[v / 4][v % 4] = (ok && gb < ng) ? ld16(x + row * b_ld + 4 * (int64_t)gb) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_stage = [&]() {
    if constexpr (sizeof(E) == 4) {
      u32x4 pa[4], pb[4];
      pieces_to_planes<float, true, false>(ra[0], pa);
      pieces_to_planes<float, true, true>(rb[0], pb);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        st16(a_lds + p * PLANE + pc * STRIDE + rq * 16, pa[p]);
        st16(b_lds + p * PLANE + pc * STRIDE + rq * 16, pb[p]);
      }
    } else {
      // 8 rows x 2 groups per operand: transform, then gather per (group, plane)
      _Float16 ha[2][4][8], hb[2][4][8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const f16x8 xa = __builtin_bit_cast(f16x8, ra[v / 4][v % 4]);
        const f16x8 xb = __builtin_bit_cast(f16x8, rb[v / 4][v % 4]);
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
          f16x8 oa, ob;
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            oa[v] = ha[e][p][v];
            ob[v] = hb[e][p][v];
          }
          st16(a_lds + p * PLANE + (pc * 2 + e) * STRIDE + rq * 16, __builtin_bit_cast(u32x4, oa));
          st16(b_lds + p * PLANE + (pc * 2 + e) * STRIDE + rq * 16, __builtin_bit_cast(u32x4, ob));
        }
      }
    }
  };

  f32x16 acc[4][1][1];
#pragma unroll
  for (int p = 0; p < 4; ++p) acc[p][0][0] = f32x16{};

  const int wr = wave >> 1, wc = wave & 1;
  const int li = lane & 31, lh = lane >> 5;
  const char* a_frag = a_lds + (wr * 32 + li) * STRIDE + lh * 16;
  const char* b_frag = b_lds + (wc * 32 + li) * STRIDE + lh * 16;

  if (rbeg < rend) load_stage(rbeg);
  for (int64_t r0 = rbeg; r0 < rend; r0 += SR) {
    store_stage();
    __syncthreads();
    if (r0 + SR < rend) load_stage(r0 + SR);
#pragma unroll
    for (int c = 0; c < NCH; ++c) mma_chunk<E, 1, 1>(acc, a_frag, PLANE, b_frag, PLANE, STRIDE, c);
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

// Sum the split partials in split order (deterministic), inverse group DFT
// along u, write dw[m][n][0..3] (float32).  nsplit == 0 writes zeros.
__global__ void __launch_bounds__(kThreads)
dw_finalize_kernel(const float* __restrict__ ws, float* __restrict__ dw, int mg, int ng, int nsplit) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t plane = (int64_t)mg * ng;
  if (idx >= plane) return;
  float f[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float* src = ws + (int64_t)s * 4 * plane + idx;
#pragma unroll
    for (int p = 0; p < 4; ++p) f[p] += src[p * plane];
  }
  float y[4];
  idft4(f[0], f[1], f[2], f[3], y);
  st16(dw + idx * 4, __builtin_bit_cast(u32x4, f32x4{y[0], y[1], y[2], y[3]}));
}

// ============================================================ prepare
//
// w[m][n][0..3] -> wf[m][n] = (F0, F2, Re F1, Im F1) and the transposed,
// conjugated wb[n][m] = (F0, F2, Re F1, -Im F1) used by the dX pass.
template <typename E>
__global__ void __launch_bounds__(kThreads)
prepare_kernel(const E* __restrict__ w, E* __restrict__ wf, E* __restrict__ wb, int mg, int ng) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)mg * ng) return;
  const int m = (int)(idx / ng), n = (int)(idx % ng);
  float z[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) z[u] = (float)w[idx * 4 + u];
  float f[4];
  dft4(z[0], z[1], z[2], z[3], f[0], f[1], f[2], f[3]);
  E* pf = wf + idx * 4;
  E* pb = wb + ((int64_t)n * mg + m) * 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    pf[p] = (E)f[p];
    pb[p] = (E)(p == 3 ? -f[p] : f[p]);
  }
}

// ============================================================ launchers

namespace {
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

template <typename E, int FM, int FN>
hipError_t launch_fwd_t(const E* in, const E* wp, E* out, int64_t nrows, int kg, int mg, hipStream_t s) {
  const int64_t tiles_m = cdiv(nrows, 64 * FM);
  const int tiles_n = (int)cdiv(mg, 64 * FN);
  const int64_t grid = tiles_m * tiles_n;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<E, FM, FN>), dim3((unsigned)grid), dim3(kThreads), 0, s, in, wp, out, nrows,
                     kg, mg, tiles_n);
  return hipGetLastError();
}

hipError_t launch_forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t nrows,
                          int kg, int mg, hipStream_t s) {
  if (dtype == 0) {
    const float* i = static_cast<const float*>(in);
    const float* w = static_cast<const float*>(wp);
    float* o = static_cast<float*>(out);
    switch (tile) {
      case 11: return launch_fwd_t<float, 1, 1>(i, w, o, nrows, kg, mg, s);
      case 12: return launch_fwd_t<float, 1, 2>(i, w, o, nrows, kg, mg, s);
      case 22: return launch_fwd_t<float, 2, 2>(i, w, o, nrows, kg, mg, s);
      default: return launch_fwd_t<float, 2, 1>(i, w, o, nrows, kg, mg, s);
    }
  }
  const _Float16* i = static_cast<const _Float16*>(in);
  const _Float16* w = static_cast<const _Float16*>(wp);
  _Float16* o = static_cast<_Float16*>(out);
  switch (tile) {
    case 11: return launch_fwd_t<_Float16, 1, 1>(i, w, o, nrows, kg, mg, s);
    case 21: return launch_fwd_t<_Float16, 2, 1>(i, w, o, nrows, kg, mg, s);
    case 12: return launch_fwd_t<_Float16, 1, 2>(i, w, o, nrows, kg, mg, s);
    default: return launch_fwd_t<_Float16, 2, 2>(i, w, o, nrows, kg, mg, s);
  }
}

int dw_rows_per_stage(int dtype) { return dtype == 0 ? 16 : 64; }

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
  const int64_t fgrid = cdiv((int64_t)mg * ng, kThreads);
  hipLaunchKernelGGL(dw_finalize_kernel, dim3((unsigned)fgrid), dim3(kThreads), 0, s, ws, dw, mg, ng, nsplit);
  return hipGetLastError();
}

hipError_t launch_prepare(int dtype, const void* w, void* wf, void* wb, int mg, int ng, hipStream_t s) {
  const int64_t grid = cdiv((int64_t)mg * ng, kThreads);
  if (dtype == 0) {
    hipLaunchKernelGGL((prepare_kernel<float>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       static_cast<const float*>(w), static_cast<float*>(wf), static_cast<float*>(wb), mg, ng);
  } else {
    hipLaunchKernelGGL((prepare_kernel<_Float16>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       static_cast<const _Float16*>(w), static_cast<_Float16*>(wf), static_cast<_Float16*>(wb),
                       mg, ng);
  }
  return hipGetLastError();
}

}  // namespace eqlin
