// Kernel instantiations and launchers of the cyclic group C8 (T = 8).
// The kernels themselves are in eqlin_device.h.
#include "eqlin_device.h"
#include "eqlin_kernels.h"

namespace eqlin {

// compiled forward tiles, code = FM FN WM WN NBUF PF [P] (decimal digits)
// (the eight accumulators of a C8 tile rule out 8-wave workgroups with one
// fragment per wave: 512 threads leave 256 registers per lane)
#define EQLIN_C8_TILES(X) X(112211) X(112221) X(111221) X(212211) X(122211) X(1122111) X(1222111) X(2122111)

template <>
bool Launch<8>::fwd_tile_known(int tile) {
  switch (tile) {
#define EQLIN_CASE(C) case C:
    EQLIN_C8_TILES(EQLIN_CASE)
#undef EQLIN_CASE
    return true;
    default: return false;
  }
}

template <>
hipError_t Launch<8>::forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t nrows, int kg,
                              int mg, const void* bias, int act, const void* res, hipStream_t s) {
#define EQLIN_CASE(C)                                                                                      \
  case C:                                                                                                  \
    return dtype == 0 ? launch_fwd_s<float, 8, EQLIN_TILE_ARGS(C), 1, EQLIN_TILE_PERSIST(C)>(in, wp, out, nrows, kg,  \
                                                                                          mg, bias, act, res, s) \
                      : launch_fwd_s<_Float16, 8, EQLIN_TILE_ARGS(C), 1, EQLIN_TILE_PERSIST(C)>(in, wp, out, nrows,  \
                                                                                             kg, mg, bias, act, res, s);
  switch (tile) {
    EQLIN_C8_TILES(EQLIN_CASE)
    default: return hipErrorInvalidValue;
  }
#undef EQLIN_CASE
}

template <>
hipError_t Launch<8>::dw(int dtype, const void* dy, const void* x, float* ws, float* dw, int64_t nrows, int mg,
                         int ng, int64_t rows_per_split, int nsplit, int chunks, hipStream_t s) {
  return dtype == 0 ? launch_dw_t<float, 8>(dy, x, ws, dw, nrows, mg, ng, rows_per_split, nsplit, chunks, s)
                    : launch_dw_t<_Float16, 8>(dy, x, ws, dw, nrows, mg, ng, rows_per_split, nsplit, chunks, s);
}

template <>
hipError_t Launch<8>::bwd_fused(int dtype, const void* dy, const void* x, const void* wb, void* dx, float* ws,
                                float* dw, int64_t nrows, int dg, int cg, int64_t rows_per_split, int nsplit,
                                int chunks, hipStream_t s) {
  return dtype == 0 ? launch_bwd_fused_t<float, 8>(dy, x, wb, dx, ws, dw, nrows, dg, cg, rows_per_split, nsplit,
                                                     chunks, s)
                    : launch_bwd_fused_t<_Float16, 8>(dy, x, wb, dx, ws, dw, nrows, dg, cg, rows_per_split,
                                                        nsplit, chunks, s);
}

template <>
hipError_t Launch<8>::prepare(int dtype, const void* w, void* wf, void* wb, int mg, int ng, hipStream_t s) {
  return dtype == 0 ? launch_prepare_t<float, 8>(w, wf, wb, mg, ng, s)
                    : launch_prepare_t<_Float16, 8>(w, wf, wb, mg, ng, s);
}

}  // namespace eqlin
