// Measured ceilings of the GPU the layer runs on, next to the published
// peaks: the rate of the two matrix-core products the kernels issue (fp32
// 32x32x2 and f16 32x32x16, every SIMD running independent back-to-back
// products), the rate of 16-byte LDS reads per compute unit (the operand
// reads of the product tiles), and the HBM rate of a device-to-device copy.
// Then the f16 product rate against the waves per SIMD and the independent
// accumulator chains per wave (how much issue parallelism the matrix core
// needs), and the rate of 16-byte global loads that hit the caches, in the
// shape of a forward stage (a 128-row x 256-byte window per workgroup, rows
// 2560 bytes apart, 64 or 256 contiguous bytes per row and instruction).  A standalone program (not part of the library); prints one JSON
// line of ceilings and one of the rate table.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                 \
      exit(1);                                                                        \
    }                                                                                 \
  } while (0)

constexpr int kChains = 4;   // independent accumulators per wave

// KIND 0: v_mfma_f32_32x32x2_f32 (4096 FLOP), KIND 1: v_mfma_f32_32x32x16_f16 (32768 FLOP).
// Operands come from the lane id, the sums are written once (one float per thread).
template <int KIND, int kChains = kChains>
__global__ void __launch_bounds__(256) mfma_loop(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  const float a = 1e-3f * (float)(lane + 1), b = 1e-3f * (float)(64 - lane);
  f16x8 ha, hb;
  for (int e = 0; e < 8; ++e) {
    ha[e] = (_Float16)(a * (float)(e + 1));
    hb[e] = (_Float16)(b * (float)(e + 1));
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (KIND == 0)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, hb, acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Every lane reads 16 bytes per LDS read from a 32 KiB buffer: lane l of a
// wave reads slot (l + i) mod 2048, so 64 consecutive lanes cover 1 KiB of
// consecutive addresses (no bank conflict).
__global__ void __launch_bounds__(256) lds_loop(float* out, int iters) {
  __shared__ f32x4 buf[2048];
  const int t = threadIdx.x;
  for (int i = t; i < 2048; i += 256) buf[i] = f32x4{(float)i, 1.f, 2.f, 3.f};
  __syncthreads();
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  int idx = t;
#pragma unroll 8
  for (int i = 0; i < iters; ++i) {
    const f32x4 v = buf[idx & 2047];
    s += v;
    idx += 64;
  }
  out[blockIdx.x * blockDim.x + t] = s[0] + s[1] + s[2] + s[3];
}

// Workgroup b reads 128 rows x 256 bytes of slab b % 64 per iteration,
// advancing 256 bytes per iteration over ten columns (a 21 MB array, rows
// 2560 bytes apart: an f16 ViT-H input): LPR lanes per row, each loading
// 16 / LPR 16-byte units of it.
template <int LPR>
__global__ void __launch_bounds__(512) load_loop(const char* __restrict__ src, int iters, unsigned* out) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  constexpr unsigned kRowBytes = 2560;
  constexpr int RPP = 512 / LPR, UPL = 16 / LPR;
  const int t = threadIdx.x, q = t % LPR, r = t / LPR;
  const unsigned slab = (blockIdx.x % 64) * 128u;
  u32x4 acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    const unsigned col = (unsigned)(it % 10) * 256u;
#pragma unroll
    for (int ps = 0; ps < 128 / RPP; ++ps)
#pragma unroll
      for (int u = 0; u < UPL; ++u)
        acc += *reinterpret_cast<const u32x4*>(src + (slab + ps * RPP + r) * kRowBytes + col +
                                               (unsigned)(q + LPR * u) * 16u);
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) out[0] = acc[0];   // keeps the loads
}

template <typename K>
double time_ms(K launch, int reps) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  launch();  // warm up and clock ramp
  launch();
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0, 0));
  for (int r = 0; r < reps; ++r) launch();
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return (double)ms / reps;
}

}  // namespace

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const int blocks = cus * 8;   // 8 workgroups of 4 waves per CU: 8 waves per SIMD
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)));

  const int iters = 4000;
  const double mf32 = time_ms([&] { hipLaunchKernelGGL(mfma_loop<0>, dim3(blocks), dim3(256), 0, 0, out, iters); }, 5);
  const double mf16 = time_ms([&] { hipLaunchKernelGGL(mfma_loop<1>, dim3(blocks), dim3(256), 0, 0, out, iters); }, 5);
  const double waves = (double)blocks * 4;
  const double f32_tflops = waves * iters * kChains * 4096.0 / (mf32 * 1e-3) / 1e12;
  const double f16_tflops = waves * iters * kChains * 32768.0 / (mf16 * 1e-3) / 1e12;

  const int liters = 20000;
  const double lms = time_ms([&] { hipLaunchKernelGGL(lds_loop, dim3(blocks), dim3(256), 0, 0, out, liters); }, 5);
  const double lds_bytes = (double)blocks * 256 * liters * 16.0;
  const double lds_tbs = lds_bytes / (lms * 1e-3) / 1e12;

  const size_t nbytes = (size_t)1 << 30;
  void *src = nullptr, *dst = nullptr;
  CHECK(hipMalloc(&src, nbytes));
  CHECK(hipMalloc(&dst, nbytes));
  CHECK(hipMemset(src, 1, nbytes));
  const double cms = time_ms([&] { CHECK(hipMemcpyAsync(dst, src, nbytes, hipMemcpyDeviceToDevice, 0)); }, 10);
  const double copy_gbs = 2.0 * (double)nbytes / (cms * 1e-3) / 1e9;
  CHECK(hipDeviceSynchronize());

  // f16 rate against waves per SIMD (1, 2, 4: 1, 2, 4 workgroups of four
  // waves per CU) and independent chains per wave (1, 2, 4, 8)
  printf("{\"f16_32x32x16_rate\": [");
  bool first = true;
  for (int wps : {1, 2, 4}) {
    const int nb = cus * wps;
    auto row = [&](auto chains_c) {
      constexpr int ch = decltype(chains_c)::value;
      const int it = 16000 / ch;
      const double ms =
          time_ms([&] { hipLaunchKernelGGL((mfma_loop<1, ch>), dim3(nb), dim3(256), 0, 0, out, it); }, 5);
      const double tf = (double)nb * 4 * it * ch * 32768.0 / (ms * 1e-3) / 1e12;
      printf("%s{\"waves_per_simd\": %d, \"chains_per_wave\": %d, \"tflops\": %.1f, \"cycles_per_mfma_at_peak_clock\": %.1f}",
             first ? "" : ", ", wps, ch, tf, (double)cus * 4 * (prop.clockRate * 1e3) * 32768.0 / (tf * 1e12));
      first = false;
    };
    row(std::integral_constant<int, 1>{});
    row(std::integral_constant<int, 2>{});
    row(std::integral_constant<int, 4>{});
    row(std::integral_constant<int, 8>{});
  }
  printf("]}\n");

  // cache-resident 16-byte loads in the shape of a forward stage
  {
    const size_t nsrc = (size_t)64 * 128 * 2560;
    char* src = nullptr;
    CHECK(hipMalloc(&src, nsrc));
    CHECK(hipMemset(src, 1, nsrc));
    const int lb = 1024, lit = 200;
    const double lbytes = (double)lb * lit * 128 * 256;
    const double l64 = time_ms([&] { hipLaunchKernelGGL(load_loop<4>, dim3(lb), dim3(512), 0, 0, src, lit, (unsigned*)out); }, 5);
    const double l256 = time_ms([&] { hipLaunchKernelGGL(load_loop<16>, dim3(lb), dim3(512), 0, 0, src, lit, (unsigned*)out); }, 5);
    printf("{\"cached_load_tb_per_s_64B_rows\": %.2f, \"cached_load_tb_per_s_256B_rows\": %.2f, "
           "\"cached_load_bytes_per_clk_per_cu_at_peak_clock\": %.1f}\n",
           lbytes / (l64 * 1e-3) / 1e12, lbytes / (l256 * 1e-3) / 1e12,
           lbytes / (l64 * 1e-3) / cus / (prop.clockRate * 1e3));
    CHECK(hipFree(src));
  }

  printf("{\"device\": \"%s\", \"compute_units\": %d, \"peak_clock_mhz\": %d, "
         "\"mfma_f32_32x32x2_tflops\": %.1f, \"mfma_f32_32x32x2_frac_of_157.3\": %.3f, "
         "\"mfma_f16_32x32x16_tflops\": %.1f, \"mfma_f16_32x32x16_frac_of_2516.6\": %.3f, "
         "\"lds_read_b128_tb_per_s\": %.2f, \"lds_read_bytes_per_clk_per_cu_at_peak_clock\": %.1f, "
         "\"hbm_copy_gb_per_s\": %.1f, \"hbm_copy_frac_of_8000\": %.3f}\n",
         prop.gcnArchName, cus, prop.clockRate / 1000, f32_tflops, f32_tflops / 157.3, f16_tflops,
         f16_tflops / 2516.6, lds_tbs, lds_tbs * 1e12 / cus / (prop.clockRate * 1e3), copy_gbs, copy_gbs / 8000.0);
  CHECK(hipFree(out));
  CHECK(hipFree(src));
  CHECK(hipFree(dst));
  return 0;
}
