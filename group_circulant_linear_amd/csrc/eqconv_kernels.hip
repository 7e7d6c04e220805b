// Kernels and launchers of the p4 group convolution.  The convolution is one
// group-circulant layer over a rotation-aware gather of each output pixel's
// K x K window (ConvGeom in eqlin_device.h):
//   - forward and dX: the forward tile of the linear layer with the gather
//     done by its A-side loads (no gathered copy in global memory);
//   - filter preparation: the group DFT of the gathered layer's weight, read
//     from the filter through the block decode (forward and adjoint sets);
//   - filter gradient: the linear layer's dw reduction (split partials, ordered
//     finalize) with the gather done by its loads, and a scatter of that
//     gradient onto the filter.
#include <stdlib.h>

#include "eqlin_device.h"
#include "eqlin_kernels.h"

namespace eqlin {

// compiled convolution tiles (the p4 tile table's candidates), code = FM FN WM WN NBUF PF
#define EQCONV_TILES(X) X(112211) X(112221) X(111211) X(212421) X(212431) X(112241) X(111221)

namespace {

template <typename E>
ConvGeom make_geom(int H, int W, int cpix, int K, int64_t npix) {
  constexpr int G = Units<E, 4>::kGroupsPerUnit;
  ConvGeom g;
  g.H = H;
  g.W = W;
  g.cpix = cpix;
  g.p = K / 2;
  g.ncb = cpix / (4 * G);
  g.bpo = cpix / G;
  g.nblk = cpix * K * K / (4 * G);
  g.inv_bpo = 1.0f / (float)g.bpo;
  g.inv_p1 = 1.0f / (float)(g.p + 1);
  g.in_bytes = (uint32_t)(npix * (int64_t)cpix * 4 * (int64_t)sizeof(E));
  // floor(n / d) = (n mul) >> shift for n < 2^31: shift = 31 + ceil(log2 d), mul = ceil(2^shift / d) < 2^32
  auto magic = [](int64_t d, uint32_t& mul, int& shift) {
    int l = 0;
    while ((int64_t(1) << l) < d) ++l;
    shift = 31 + l;
    mul = (uint32_t)(((uint64_t(1) << shift) + (uint64_t)d - 1) / (uint64_t)d);
  };
  magic(W > 0 ? W : 1, g.w_mul, g.w_shift);
  magic(H > 0 && W > 0 ? (int64_t)H * W : 1, g.hw_mul, g.hw_shift);
  return g;
}

// R^r (a, b) with R(a, b) = (-b, a)
__device__ __forceinline__ void turn_tap(int r, int& a, int& b) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (k < (r & 3)) {
      const int t = a;
      a = -b;
      b = t;
    }
  }
}

// Gathered-layer group channel g (of a row padded to whole stages) -> the
// filter entries of its weight w_lin[.][g][u], u = 0..3: input channel c,
// tap (ti, tj) and group offset v per u.  Centre: psi[., c, 0, u].  Orbit
// block with shift b = unit i: psi[., c, R^-u delta_o, (u - b) mod 4]
// (each filter entry feeds exactly one (g, u)).  Returns false for the
// padding of a partial last stage.
template <int G>
__device__ __forceinline__ bool conv_weight_source(int g, const ConvGeom& geo, int& c, int (&ti)[4], int (&tj)[4],
                                                   int (&v)[4]) {
  constexpr int SG = 16 * G;
  const int w = (g % SG) / G;  // unit position q + 4 i in the stage
  const int cb = (g / SG) * 4 + (w & 3), i = w >> 2, e = g % G;
  const ConvBlock k = conv_block<G>(cb, geo);
  c = k.centre ? k.ch0 + G * i + e : k.ch0 + e;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int mu = (4 - u) & 3;  // R^-u = R^(4 - u)
    ti[u] = k.di[mu];
    tj[u] = k.dj[mu];
    v[u] = k.centre ? u : ((u - i) & 3);
  }
  return k.live;
}

}  // namespace

// Forward (or dX) tile with the gather in its loads.
template <typename E, int FM, int FN, int WM, int WN, int NBUF, int PF>
__global__ void __launch_bounds__(64 * WM * WN, (fwd_waves_per_simd<E, 4, FM, FN>()))
conv_fwd_kernel(const E* __restrict__ in, const E* __restrict__ wp, E* __restrict__ out, int64_t npix, int kg,
                int mg, int tiles_n, const E* __restrict__ bias, int act, ConvGeom geo, int64_t nfull) {
  __shared__ __attribute__((aligned(16))) char lds[fwd_lds_bytes<E, 4, FM, FN, WM, WN, NBUF>()];
  // workgroups past nfull run the halves of the tail tiles (as fwd_kernel)
  const int64_t bid = blockIdx.x;
  if constexpr (fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF)) {
    if (bid >= nfull) {
      fwd_tile<E, 4, FM, FN, WM, WN, NBUF, PF, 1, true, true>(
          lds, 2 * nfull + xcd_logical_id(bid - nfull, (int64_t)gridDim.x - nfull), in, wp, out, npix, kg, mg,
          tiles_n, bias, act, nullptr, geo);
      return;
    }
  }
  fwd_tile<E, 4, FM, FN, WM, WN, NBUF, PF, 1, true>(lds, xcd_logical_id(bid, nfull), in, wp, out, npix, kg, mg,
                                                    tiles_n, bias, act, nullptr, geo);
}

// Prepared spectra of the gathered layer, in the stage-block layout of the
// linear layer (rows x stages x 4 planes x SG slots).  Forward (kAdj false):
// rows = D', w_lin[d'][g][u] = psi[d', c, tap, v] with (c, tap, v) from the
// block decode over C' input channels.  Adjoint (kAdj true, the dX pass is a
// convolution of dY): rows = C', the decode runs over D' channels, and the
// filter is psi'[c', d', delta, v] = psi[d', c', -R^v delta, -v mod 4].
// One launch writes both sets: blocks below nbf the forward set, the others
// the adjoint set.
template <typename E, bool kAdj>
__device__ __forceinline__ void conv_prepare_entry(const E* __restrict__ psi, E* __restrict__ dst, int rows, int kg,
                                                   int Cp, int K, const ConvGeom& geo, int64_t idx) {
  constexpr int SG = Traits<E>::kStageGroups, T = 4;
  constexpr int G = Units<E, T>::kGroupsPerUnit;
  const int nks = kg / SG;
  if (idx >= (int64_t)rows * nks * SG) return;
  const int s = (int)(idx % SG);
  const int64_t t = idx / SG;
  const int ks = (int)(t % nks);
  const int row = (int)(t / nks);
  const int g = ks * SG + slot_group<E, T>(s);
  float f[T] = {0.f, 0.f, 0.f, 0.f};
  int c, ti[4], tj[4], v[4];
  if (conv_weight_source<G>(g, geo, c, ti, tj, v)) {
    const int p = K / 2;
    float z[T];
#pragma unroll
    for (int u = 0; u < T; ++u) {
      int64_t src;
      if constexpr (!kAdj) {
        src = ((((int64_t)row * Cp + c) * K + ti[u] + p) * K + tj[u] + p) * 4 + v[u];
      } else {
        int a = ti[u], b = tj[u];
        turn_tap(v[u], a, b);
        src = ((((int64_t)c * Cp + row) * K + (p - a)) * K + (p - b)) * 4 + ((-v[u]) & 3);
      }
      z[u] = (float)psi[src];
    }
    Grp<4>::dft(z, f);
  }
  // f16: scaled into the operand range of the f16 products (Grp<4>::kF16Scale)
  E* o = dst + ((int64_t)row * nks + ks) * T * SG + s;
#pragma unroll
  for (int q = 0; q < T; ++q) o[q * SG] = (E)(sizeof(E) == 2 ? f[q] * Grp<4>::kF16Scale[q] : f[q]);
}

template <typename E>
__global__ void __launch_bounds__(kThreads)
conv_prepare_kernel(const E* __restrict__ psi, E* __restrict__ wf, E* __restrict__ wb, int Dp, int Cp, int kgf,
                    int kgb, int K, ConvGeom gf, ConvGeom gb, int64_t nbf) {
  const int64_t b = blockIdx.x;
  if (b < nbf)
    conv_prepare_entry<E, false>(psi, wf, Dp, kgf, Cp, K, gf, b * kThreads + threadIdx.x);
  else
    conv_prepare_entry<E, true>(psi, wb, Cp, kgb, Cp, K, gb, (b - nbf) * kThreads + threadIdx.x);
}

// Split partials of the gathered layer's dw, the gather done by the loads.
template <typename E>
__global__ void __launch_bounds__(kThreads, bwd_waves_per_simd<4>())
conv_dw_partial_kernel(const E* __restrict__ dy, const E* __restrict__ x, float* __restrict__ ws, int64_t npix,
                       int mg, int kg, int64_t rows_per_split, int tiles_m, int tiles_n, ConvGeom geo) {
  __shared__ __attribute__((aligned(16))) char lds[dw_lds_bytes<4, kDwBufs>()];
  dw_tile<E, 4, kDwBufs, true>(lds, xcd_logical_id(blockIdx.x, gridDim.x), dy, x, ws, npix, mg, kg, rows_per_split,
                               tiles_m, tiles_n, mg, kg, geo);
}

// Backward in one launch, as the linear layer's: the first ndw_pad
// workgroups are the dpsi split partials (gathered over the C' channels of
// X), the rest are dX tiles (the convolution of dY with the adjoint spectra,
// gathered over its D' channels).  Both read dY; one grid lets the dispatcher
// fill the tail of one role with work of the other.
template <typename E>
__global__ void __launch_bounds__(kThreads, bwd_waves_per_simd<4>())
conv_bwd_fused_kernel(const E* __restrict__ dy, const E* __restrict__ x, const E* __restrict__ wb,
                      E* __restrict__ dx, float* __restrict__ ws, int64_t npix, int Dp, int Cp, int kgw, int kgx,
                      int64_t rows_per_split, int dw_tiles_m, int dw_tiles_n, int64_t ndw, int64_t ndw_pad,
                      int dx_tiles_n, ConvGeom gw, ConvGeom gx, int64_t ndx_full) {
  constexpr int kFwd = fwd_lds_bytes<E, 4, 1, 1, 2, 2, kBwdFwdBufs>();
  constexpr int kDw = dw_lds_bytes<4, kDwBufs>();
  __shared__ __attribute__((aligned(16))) char lds[kFwd > kDw ? kFwd : kDw];
  const int64_t b = blockIdx.x;
  if (b < ndw_pad) {
    const int64_t lid = xcd_logical_id(b, ndw_pad);
    if (lid < ndw)
      dw_tile<E, 4, kDwBufs, true>(lds, lid, dy, x, ws, npix, Dp, kgw, rows_per_split, dw_tiles_m, dw_tiles_n, Dp,
                                   kgw, gw);
  } else {
    // dX tiles past ndx_full run as halves (the tail split of the forward)
    const int64_t bx = b - ndw_pad;
    if constexpr (fwd_tail_split_fits(sizeof(E) == 4, 1, 1, 2, 2, kBwdFwdBufs)) {
      if (bx >= ndx_full) {
        fwd_tile<E, 4, 1, 1, 2, 2, kBwdFwdBufs, kBwdFwdPrefetch, 1, true, true>(
            lds, 2 * ndx_full + xcd_logical_id(bx - ndx_full, (int64_t)gridDim.x - ndw_pad - ndx_full), dy, wb, dx,
            npix, kgx, Cp, dx_tiles_n, nullptr, 0, nullptr, gx);
        return;
      }
    }
    fwd_tile<E, 4, 1, 1, 2, 2, kBwdFwdBufs, kBwdFwdPrefetch, 1, true>(lds, xcd_logical_id(bx, ndx_full), dy, wb, dx,
                                                                       npix, kgx, Cp, dx_tiles_n, nullptr, 0, nullptr, gx);
  }
}

// Filter gradient from the gathered layer's dw: dpsi[d'][c][tap][v] =
// dwlin[d'][g][u] through the block decode (a permutation).
template <typename E>
__global__ void __launch_bounds__(kThreads)
conv_dw_scatter_kernel(const float* __restrict__ dwlin, float* __restrict__ dpsi, int Dp, int kg, int Cp, int K,
                       ConvGeom geo) {
  constexpr int G = Units<E, 4>::kGroupsPerUnit;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)Dp * kg) return;
  const int d = (int)(idx / kg), g = (int)(idx % kg);
  int c, ti[4], tj[4], v[4];
  if (!conv_weight_source<G>(g, geo, c, ti, tj, v)) return;
  const int p = K / 2;
  const f32x4 src = *reinterpret_cast<const f32x4*>(dwlin + idx * 4);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    dpsi[((((int64_t)d * Cp + c) * K + ti[u] + p) * K + tj[u] + p) * 4 + v[u]] = src[u];
}

namespace {

template <typename E, int FM, int FN, int WM, int WN, int NBUF, int PF>
hipError_t launch_conv_fwd(const void* in, const void* wp, void* out, int64_t npix, int H, int W, int cpix, int K,
                           int mg, const void* bias, int act, hipStream_t s) {
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  const int64_t tiles = cdiv(npix, BM) * cdiv(mg, BN);
  if (tiles <= 0) return hipSuccess;
  int64_t nfull = tiles, grid = tiles;
  if (fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF) && fwd_tail_split_enabled()) {
    nfull = fwd_full_tiles(tiles);
    grid = nfull + 2 * (tiles - nfull);
  }
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const ConvGeom g = make_geom<E>(H, W, cpix, K, npix);
  const int kg = conv_gathered_groups(cpix, K, sizeof(E) == 4 ? 0 : 1);
  hipLaunchKernelGGL((conv_fwd_kernel<E, FM, FN, WM, WN, NBUF, PF>), dim3((unsigned)grid), dim3(64 * WM * WN), 0, s,
                     static_cast<const E*>(in), static_cast<const E*>(wp), static_cast<E*>(out), npix, kg, mg,
                     (int)cdiv(mg, BN), static_cast<const E*>(bias), act, g, nfull);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_conv_prepare(const void* psi, void* wf, void* wb, int Dp, int Cp, int K, hipStream_t s) {
  const int dt = sizeof(E) == 4 ? 0 : 1;
  const int kgf = conv_gathered_groups(Cp, K, dt), kgb = conv_gathered_groups(Dp, K, dt);
  const ConvGeom gf = make_geom<E>(1, 1, Cp, K, 0), gb = make_geom<E>(1, 1, Dp, K, 0);
  const int64_t nf = (int64_t)Dp * kgf, nb = (int64_t)Cp * kgb;
  const int64_t nbf = cdiv(nf, kThreads), grid = nbf + cdiv(nb, kThreads);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((conv_prepare_kernel<E>), dim3((unsigned)grid), dim3(kThreads), 0, s, static_cast<const E*>(psi),
                     static_cast<E*>(wf), static_cast<E*>(wb), Dp, Cp, kgf, kgb, K, gf, gb, nbf);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_conv_dw(const void* dy, const void* x, float* ws, float* dwlin, int64_t npix, int H, int W, int Dp,
                          int Cp, int K, int64_t rows_per_split, int nsplit, hipStream_t s) {
  const int kg = conv_gathered_groups(Cp, K, sizeof(E) == 4 ? 0 : 1);
  const int tiles_m = (int)cdiv(Dp, 64), tiles_n = (int)cdiv(kg, 64);
  if (nsplit > 0) {
    const int64_t grid = (int64_t)tiles_m * tiles_n * nsplit;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((conv_dw_partial_kernel<E>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       static_cast<const E*>(dy), static_cast<const E*>(x), ws, npix, Dp, kg, rows_per_split, tiles_m,
                       tiles_n, make_geom<E>(H, W, Cp, K, npix));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_dw_finalize<E, 4>(ws, dwlin, Dp, kg, nsplit, s);
}

template <typename E>
hipError_t launch_conv_bwd_fused(const void* dy, const void* x, const void* wb, void* dx, float* ws, float* dwlin,
                                 int64_t npix, int H, int W, int Dp, int Cp, int K, int64_t rows_per_split, int nsplit,
                                 hipStream_t s) {
  const int dt = sizeof(E) == 4 ? 0 : 1;
  const int kgw = conv_gathered_groups(Cp, K, dt), kgx = conv_gathered_groups(Dp, K, dt);
  const int dw_tiles_m = (int)cdiv(Dp, 64), dw_tiles_n = (int)cdiv(kgw, 64);
  const int64_t ndw = (int64_t)dw_tiles_m * dw_tiles_n * nsplit;
  const int64_t ndw_pad = cdiv(ndw, 8) * 8;
  const int dx_tiles_n = (int)cdiv(Cp, 64);
  const int64_t ndx = cdiv(npix, 64) * dx_tiles_n;
  int64_t ndx_full = ndx, grid = ndw_pad + ndx;
  if (fwd_tail_split_fits(sizeof(E) == 4, 1, 1, 2, 2, kBwdFwdBufs) && fwd_tail_split_enabled()) {
    ndx_full = fwd_full_tiles(ndx);
    grid = ndw_pad + ndx_full + 2 * (ndx - ndx_full);
  }
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (grid > 0) {
    hipLaunchKernelGGL((conv_bwd_fused_kernel<E>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       static_cast<const E*>(dy), static_cast<const E*>(x), static_cast<const E*>(wb),
                       static_cast<E*>(dx), ws, npix, Dp, Cp, kgw, kgx, rows_per_split, dw_tiles_m, dw_tiles_n, ndw,
                       ndw_pad, dx_tiles_n, make_geom<E>(H, W, Cp, K, npix), make_geom<E>(H, W, Dp, K, npix), ndx_full);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_dw_finalize<E, 4>(ws, dwlin, Dp, kgw, nsplit, s);
}

template <typename E>
hipError_t launch_conv_dw_scatter(const float* dwlin, float* dpsi, int Dp, int Cp, int K, hipStream_t s) {
  const int kg = conv_gathered_groups(Cp, K, sizeof(E) == 4 ? 0 : 1);
  const int64_t n = (int64_t)Dp * kg;
  hipLaunchKernelGGL((conv_dw_scatter_kernel<E>), dim3((unsigned)cdiv(n, kThreads)), dim3(kThreads), 0, s, dwlin,
                     dpsi, Dp, kg, Cp, K, make_geom<E>(1, 1, Cp, K, 0));
  return hipGetLastError();
}

}  // namespace

bool ConvLaunch::tile_known(int tile) {
  switch (tile) {
#define EQCONV_CASE(C) case C:
    EQCONV_TILES(EQCONV_CASE)
#undef EQCONV_CASE
    return true;
    default: return false;
  }
}

hipError_t ConvLaunch::forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t npix, int H,
                               int W, int cpix, int K, int mg, const void* bias, int act, hipStream_t s) {
#define EQCONV_CASE(C)                                                                                         \
  case C:                                                                                                      \
    return dtype == 0 ? launch_conv_fwd<float, EQLIN_TILE_ARGS(C)>(in, wp, out, npix, H, W, cpix, K, mg, bias,  \
                                                                   act, s)                                     \
                      : launch_conv_fwd<_Float16, EQLIN_TILE_ARGS(C)>(in, wp, out, npix, H, W, cpix, K, mg,     \
                                                                      bias, act, s);
  switch (tile) {
    EQCONV_TILES(EQCONV_CASE)
    default: return hipErrorInvalidValue;
  }
#undef EQCONV_CASE
}

hipError_t ConvLaunch::prepare(int dtype, const void* psi, void* wf, void* wb, int Dp, int Cp, int K,
                               hipStream_t s) {
  return dtype == 0 ? launch_conv_prepare<float>(psi, wf, wb, Dp, Cp, K, s)
                    : launch_conv_prepare<_Float16>(psi, wf, wb, Dp, Cp, K, s);
}

hipError_t ConvLaunch::dw(int dtype, const void* dy, const void* x, float* ws, float* dwlin, int64_t npix, int H,
                          int W, int Dp, int Cp, int K, int64_t rows_per_split, int nsplit, hipStream_t s) {
  return dtype == 0 ? launch_conv_dw<float>(dy, x, ws, dwlin, npix, H, W, Dp, Cp, K, rows_per_split, nsplit, s)
                    : launch_conv_dw<_Float16>(dy, x, ws, dwlin, npix, H, W, Dp, Cp, K, rows_per_split, nsplit, s);
}

hipError_t ConvLaunch::bwd_fused(int dtype, const void* dy, const void* x, const void* wb, void* dx, float* ws,
                                 float* dwlin, int64_t npix, int H, int W, int Dp, int Cp, int K,
                                 int64_t rows_per_split, int nsplit, hipStream_t s) {
  return dtype == 0 ? launch_conv_bwd_fused<float>(dy, x, wb, dx, ws, dwlin, npix, H, W, Dp, Cp, K, rows_per_split,
                                                   nsplit, s)
                    : launch_conv_bwd_fused<_Float16>(dy, x, wb, dx, ws, dwlin, npix, H, W, Dp, Cp, K,
                                                      rows_per_split, nsplit, s);
}

hipError_t ConvLaunch::dw_scatter(int dtype, const float* dwlin, float* dpsi, int Dp, int Cp, int K, hipStream_t s) {
  return dtype == 0 ? launch_conv_dw_scatter<float>(dwlin, dpsi, Dp, Cp, K, s)
                    : launch_conv_dw_scatter<_Float16>(dwlin, dpsi, Dp, Cp, K, s);
}

}  // namespace eqlin
