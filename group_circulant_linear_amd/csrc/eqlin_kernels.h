// Internal launcher declarations shared by the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eqlin {

// Forward tile codes: six digits FM FN WM WN NBUF PF.  A workgroup has WM x WN
// waves; each wave owns FM x FN fragments of 32 x 32 per accumulator plane, so
// the workgroup tile is (32 FM WM) rows x (32 FN WN) output groups; NBUF (1 or
// 2) is the number of LDS stage buffers and PF (1 or 2) the number of stages
// of global loads in flight in registers.
bool fwd_tile_known(int tile);
// bias: nullable, one storage-dtype value per output group; act: 0 none, 1 GELU (erf)
hipError_t launch_forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t nrows,
                          int kg, int mg, const void* bias, int act, hipStream_t s);
hipError_t launch_dw(int dtype, const void* dy, const void* x, float* ws, float* dw, int64_t nrows, int mg,
                     int ng, int64_t rows_per_split, int nsplit, hipStream_t s);
// dX (forward structure on the transpose spectra wb, tile 1122) and the dw
// split partials in one launch, then the dw finalize.  nrows > 0.
hipError_t launch_bwd_fused(int dtype, const void* dy, const void* x, const void* wb, void* dx, float* ws,
                            float* dw, int64_t nrows, int dg, int cg, int64_t rows_per_split, int nsplit,
                            hipStream_t s);
hipError_t launch_prepare(int dtype, const void* w, void* wf, void* wb, int mg, int ng, hipStream_t s);
int stage_groups(int dtype);       // group channels per pipeline stage (16 fp32, 32 f16)
int dw_rows_per_stage(int dtype);  // rows per dw pipeline stage (16 fp32, 32 f16)

}  // namespace eqlin
