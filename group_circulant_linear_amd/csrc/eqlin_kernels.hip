// Kernel instantiations and launchers of the p4 rotation group (T = 4).
// The kernels themselves are in eqlin_device.h.
#include <stdlib.h>

#include "eqlin_device.h"
#include "eqlin_kernels.h"

namespace eqlin {

// compiled forward tiles, code = FM FN WM WN NBUF PF [P] (decimal digits)
#define EQLIN_P4_TILES(X)                                                                                 \
  X(112221) X(111221) X(112121) X(222221) X(212421) X(212431) X(122241) X(112241) X(112411) X(212211)     \
  X(122211) X(112211) X(112212) X(112412) X(111211) X(2124211) X(1122111) X(1122211) X(1112111) X(112111) \
  X(1121111)

namespace {
// EQLIN_SCHED=0 drops the explicit MFMA / memory interleave of the
// double-buffered tiles (for comparisons).
template <typename E, int FM, int FN, int WM, int WN, int NBUF, int PF, int P>
hipError_t launch_fwd_p4(const void* in, const void* wp, void* out, int64_t nrows, int kg, int mg, const void* bias,
                         int act, const void* res, hipStream_t s, const FwdKSplit& ks) {
  static const int sched = [] {
    const char* e = getenv("EQLIN_SCHED");
    return e ? atoi(e) : 1;
  }();
  return sched == 1
             ? launch_fwd_s<E, 4, FM, FN, WM, WN, NBUF, PF, 1, P>(in, wp, out, nrows, kg, mg, bias, act, res, s, ks)
             : launch_fwd_s<E, 4, FM, FN, WM, WN, NBUF, PF, 0, P>(in, wp, out, nrows, kg, mg, bias, act, res, s, ks);
}
}  // namespace

template <>
bool Launch<4>::fwd_tile_known(int tile) {
  switch (tile) {
#define EQLIN_CASE(C) case C:
    EQLIN_P4_TILES(EQLIN_CASE)
#undef EQLIN_CASE
    return true;
    default: return false;
  }
}

template <>
hipError_t Launch<4>::forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t nrows, int kg,
                              int mg, const void* bias, int act, const void* res, hipStream_t s,
                              const FwdKSplit& ks) {
#define EQLIN_CASE(C)                                                                                       \
  case C:                                                                                                   \
    return dtype == 0                                                                                       \
               ? launch_fwd_p4<float, EQLIN_TILE_ARGS(C), EQLIN_TILE_PERSIST(C)>(in, wp, out, nrows, kg, mg, bias, \
                                                                                 act, res, s, ks)               \
               : launch_fwd_p4<_Float16, EQLIN_TILE_ARGS(C), EQLIN_TILE_PERSIST(C)>(in, wp, out, nrows, kg, mg,    \
                                                                                    bias, act, res, s, ks);
  switch (tile) {
    EQLIN_P4_TILES(EQLIN_CASE)
    default: return hipErrorInvalidValue;
  }
#undef EQLIN_CASE
}

template <>
hipError_t Launch<4>::dw(int dtype, const void* dy, const void* x, float* ws, float* dw, int64_t nrows, int mg,
                         int ng, int64_t rows_per_split, int nsplit, int chunks, int width, hipStream_t s) {
  return dtype == 0 ? launch_dw_t<float, 4>(dy, x, ws, dw, nrows, mg, ng, rows_per_split, nsplit, chunks, width, s)
                    : launch_dw_t<_Float16, 4>(dy, x, ws, dw, nrows, mg, ng, rows_per_split, nsplit, chunks, width, s);
}

template <>
hipError_t Launch<4>::bwd_fused(int dtype, const void* dy, const void* x, const void* wb, void* dx, float* ws,
                                float* dw, int64_t nrows, int dg, int cg, int64_t rows_per_split, int nsplit,
                                int chunks, hipStream_t s) {
  return dtype == 0 ? launch_bwd_fused_t<float, 4>(dy, x, wb, dx, ws, dw, nrows, dg, cg, rows_per_split, nsplit,
                                                     chunks, s)
                    : launch_bwd_fused_t<_Float16, 4>(dy, x, wb, dx, ws, dw, nrows, dg, cg, rows_per_split,
                                                        nsplit, chunks, s);
}

template <>
hipError_t Launch<4>::prepare(int dtype, const void* w, void* wf, void* wb, int mg, int ng, hipStream_t s) {
  return dtype == 0 ? launch_prepare_t<float, 4>(w, wf, wb, mg, ng, s)
                    : launch_prepare_t<_Float16, 4>(w, wf, wb, mg, ng, s);
}

}  // namespace eqlin
