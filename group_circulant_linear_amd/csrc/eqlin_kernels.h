// Internal launcher declarations shared by the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eqlin {

// tile codes: 10 * FM + FN, workgroup tile (64 FM rows) x (64 FN output groups)
hipError_t launch_forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t nrows,
                          int kg, int mg, hipStream_t s);
hipError_t launch_dw(int dtype, const void* dy, const void* x, float* ws, float* dw, int64_t nrows, int mg,
                     int ng, int64_t rows_per_split, int nsplit, hipStream_t s);
hipError_t launch_prepare(int dtype, const void* w, void* wf, void* wb, int mg, int ng, hipStream_t s);
int dw_rows_per_stage(int dtype);

}  // namespace eqlin
