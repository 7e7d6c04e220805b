// Check of the direct global-to-LDS load the f16 forward tiles use for their
// weight operand (dma16 in eqlin_device.h), on the GPU it runs on: a
// standalone diagnostic, not part of the library.  One workgroup of 256
// threads fills 4 KB of LDS with a marker, then each wave copies 64 lanes x
// 16 bytes with dma16, lane l reading the 16-byte source block (l ^ 5) + 64 w
// (w = wave); the source range ends 16 blocks early, so wave 3's lanes whose
// block is 240 or more read out of range.  After a full wait and a barrier the
// workgroup writes LDS back.  The host checks that lane l's bytes landed at
// LDS offset 1024 w + 16 l, that the out-of-range lanes wrote zeros, and
// prints one JSON line.  Every access is inside the buffers allocated here
// (the source allocation covers the out-of-range blocks too).
#include "eqlin_device.h"

#include <stdio.h>
#include <stdlib.h>

#include <vector>

using namespace eqlin;

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                 \
      exit(1);                                                                        \
    }                                                                                 \
  } while (0)

namespace {

constexpr int kBlocks = 256, kInRange = 240;
constexpr uint32_t kMarker = 0xdeadbeefu;

__global__ void __launch_bounds__(256) dma_kernel(const unsigned* __restrict__ src, unsigned* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned lds[1024];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < 1024; i += 256) lds[i] = kMarker;
  __syncthreads();
  const u32x4 words = rsrc_words(src, (uint64_t)kInRange * 16);
  const uint32_t off = (uint32_t)((lane ^ 5) + 64 * wave) * 16u;
  const uint32_t base = lds_address(reinterpret_cast<const char*>(lds)) + 1024u * (uint32_t)wave;
  dma16(words, (uint32_t)__builtin_amdgcn_readfirstlane((int)base), off, 0u, 0u);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int i = t; i < 1024; i += 256) out[i] = lds[i];
}

}  // namespace

int main() {
  std::vector<unsigned> h(kBlocks * 4);
  for (size_t i = 0; i < h.size(); ++i) h[i] = 1000000u + (unsigned)i;
  unsigned *src, *out;
  CHECK(hipMalloc(&src, h.size() * sizeof(unsigned)));
  CHECK(hipMalloc(&out, 1024 * sizeof(unsigned)));
  CHECK(hipMemcpy(src, h.data(), h.size() * sizeof(unsigned), hipMemcpyHostToDevice));
  hipLaunchKernelGGL(dma_kernel, dim3(1), dim3(256), 0, 0, src, out);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  std::vector<unsigned> r(1024);
  CHECK(hipMemcpy(r.data(), out, r.size() * sizeof(unsigned), hipMemcpyDeviceToHost));
  int mismatched = 0, oob_zero = 0, oob_other = 0;
  for (int w = 0; w < 4; ++w)
    for (int l = 0; l < 64; ++l) {
      const int blk = (l ^ 5) + 64 * w;
      for (int j = 0; j < 4; ++j) {
        const unsigned got = r[w * 256 + l * 4 + j];
        if (blk >= kInRange) {
          (got == 0 ? oob_zero : oob_other)++;
        } else if (got != h[blk * 4 + j]) {
          ++mismatched;
        }
      }
    }
  printf("{\"lanes\": 256, \"words_checked\": %d, \"mismatched\": %d, \"out_of_range_words\": %d, "
         "\"out_of_range_zero\": %d, \"out_of_range_other\": %d}\n",
         1024, mismatched, oob_zero + oob_other, oob_zero, oob_other);
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  return (mismatched == 0 && oob_other == 0) ? 0 : 2;
}
