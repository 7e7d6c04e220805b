// Stage timeline of the forward tile on the GPU it runs on: a standalone
// diagnostic (not part of the library).  Built with EQLIN_STAGE_TRACE, the
// forward tile writes the shader clock and the 100 MHz real-time counter of
// thread 0 of every workgroup at its start, after its prologue (first stage
// loaded into LDS), after its first and its last pipeline stage, after its
// epilogue's stores are issued and once they have completed.  For each layer
// shape the program times 100 launches (the hook present, its buffer unset),
// then traces one launch and prints one JSON line: the launch time, the
// shader clock, and per round of workgroups (or, for the tail-split halves,
// per kind) the medians of the prologue, of the first stage, of a later
// stage (the span from the first to the last stage over their count), of
// the epilogue and of the store drain.  The operands are synthetic (timing
// only; nothing is checked).
#define EQLIN_STAGE_TRACE 1
#include "eqlin_device.h"

#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
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

constexpr int kEvents = 64;
constexpr int64_t kMaxBlocks = 8192;

double median(std::vector<double> v) {
  if (v.empty()) return 0.0;
  std::sort(v.begin(), v.end());
  return v[v.size() / 2];
}

// one group of workgroups: medians in microseconds
void print_group(const char* label, const std::vector<int64_t>& ids, const std::vector<double>& rt, int nst,
                 bool first) {
  std::vector<double> pro, st0, st, epi, drain, start, end;
  for (int64_t b : ids) {
    const double* r = &rt[b * kEvents];
    pro.push_back(r[1] - r[0]);
    st0.push_back(r[2] - r[1]);
    if (nst > 1) st.push_back((r[3] - r[2]) / (nst - 1));
    epi.push_back(r[62] - r[3]);
    drain.push_back(r[63] - r[62]);
    start.push_back(r[0]);
    end.push_back(r[63]);
  }
  printf("%s{\"group\": \"%s\", \"workgroups\": %zu, \"start_us\": [%.1f, %.1f], \"end_us\": [%.1f, %.1f], "
         "\"prologue_us\": %.2f, \"first_stage_us\": %.2f, \"stage_us\": %.2f, \"epilogue_us\": %.2f, "
         "\"drain_us\": %.2f}",
         first ? "" : ", ", label, ids.size(), *std::min_element(start.begin(), start.end()),
         *std::max_element(start.begin(), start.end()), *std::min_element(end.begin(), end.end()),
         *std::max_element(end.begin(), end.end()), median(pro), median(st0), median(st), median(epi),
         median(drain));
}

template <typename E, int FM, int FN, int WM, int WN, int NBUF, int PF>
void run(const char* name, int64_t N, int C, int D) {
  constexpr int T = 4;
  constexpr int SG = Traits<E>::kStageGroups;
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  const int kg = C / T, mg = D / T;
  const int ksteps = (kg + SG - 1) / SG;
  const size_t xe = (size_t)N * C, we = (size_t)mg * ksteps * SG * T, oe = (size_t)N * D;
  E *x, *w, *o;
  CHECK(hipMalloc(&x, xe * sizeof(E)));
  CHECK(hipMalloc(&w, we * sizeof(E)));
  CHECK(hipMalloc(&o, oe * sizeof(E)));
  {
    std::vector<E> h(xe > we ? xe : we);
    for (size_t i = 0; i < h.size(); ++i) h[i] = (E)((float)((i * 2654435761u) % 1000) * 1e-3f - 0.5f);
    CHECK(hipMemcpy(x, h.data(), xe * sizeof(E), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(w, h.data(), we * sizeof(E), hipMemcpyHostToDevice));
  }
  const int64_t tiles_m = (N + BM - 1) / BM;
  const int tiles_n = (mg + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  int64_t grid = tiles, nfull = tiles;
  if constexpr (fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF)) {
    nfull = fwd_full_tiles(tiles);
    grid = nfull + 2 * (tiles - nfull);
  }
  if (grid > kMaxBlocks) {
    fprintf(stderr, "%s: %lld workgroups exceed the trace buffer\n", name, (long long)grid);
    exit(1);
  }
  unsigned long long* tr;
  const size_t tb = (size_t)kMaxBlocks * kEvents * 2 * sizeof(unsigned long long);
  CHECK(hipMalloc(&tr, tb));
  CHECK(hipMemset(tr, 0, tb));
  unsigned long long* none = nullptr;
  auto kernel = fwd_kernel<E, 4, FM, FN, WM, WN, NBUF, PF, 1, 0>;
  auto launch = [&] {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(64 * WM * WN), 0, 0, x, w, o, N, kg, mg, tiles_n,
                       (const E*)nullptr, 0, (const E*)nullptr, tiles, nfull, (float*)nullptr,
                       (uint32_t*)nullptr, 0);
  };
  CHECK(hipMemcpyToSymbol(HIP_SYMBOL(g_stage_trace), &none, sizeof(none)));
  for (int i = 0; i < 300; ++i) launch();   // settle the clocks
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0, 0));
  for (int i = 0; i < 100; ++i) launch();
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipMemcpyToSymbol(HIP_SYMBOL(g_stage_trace), &tr, sizeof(tr)));
  launch();
  CHECK(hipMemcpyToSymbol(HIP_SYMBOL(g_stage_trace), &none, sizeof(none)));
  CHECK(hipDeviceSynchronize());
  CHECK(hipGetLastError());
  std::vector<unsigned long long> raw((size_t)grid * kEvents * 2);
  CHECK(hipMemcpy(raw.data(), tr, raw.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));

  const int nst = ksteps;
  double r0 = 1e300;
  for (int64_t b = 0; b < grid; ++b)
    if (raw[(b * kEvents + 63) * 2] != 0) r0 = std::min(r0, (double)raw[(b * kEvents) * 2 + 1]);
  std::vector<double> rt((size_t)grid * kEvents, 0.0), clk;
  for (int64_t b = 0; b < grid; ++b) {
    for (int e = 0; e < kEvents; ++e) rt[b * kEvents + e] = ((double)raw[(b * kEvents + e) * 2 + 1] - r0) * 0.01;
    const double cyc = (double)raw[(b * kEvents + 63) * 2] - (double)raw[(b * kEvents) * 2];
    const double us = rt[b * kEvents + 63] - rt[b * kEvents];
    if (raw[(b * kEvents + 63) * 2] != 0 && us > 0) clk.push_back(cyc / us / 1e3);
  }
  printf("{\"layer\": \"%s\", \"dtype\": \"%s\", \"N\": %lld, \"C\": %d, \"D\": %d, \"tile\": \"%d%d%d%d%d%d\", "
         "\"tiles\": %lld, \"workgroups\": %lld, \"stages\": %d, \"launch_us\": %.2f, \"shader_clock_ghz\": %.2f, "
         "\"groups\": [",
         name, sizeof(E) == 4 ? "f32" : "f16", (long long)N, C, D, FM, FN, WM, WN, NBUF, PF, (long long)tiles,
         (long long)grid, ksteps, ms * 1e3 / 100, median(clk));
  // whole tiles by round (a new round starts where the start times jump by
  // more than 2 us), then the tail-split halves
  // (a workgroup that found no rows, a second half past the last row, left no events)
  std::vector<int64_t> whole, half;
  for (int64_t b = 0; b < grid; ++b)
    if (raw[(b * kEvents + 63) * 2] != 0) (b < nfull ? whole : half).push_back(b);
  std::sort(whole.begin(), whole.end(), [&](int64_t a, int64_t b) { return rt[a * kEvents] < rt[b * kEvents]; });
  bool first = true;
  int round = 0;
  for (size_t i = 0; i < whole.size();) {
    size_t j = i + 1;
    while (j < whole.size() && rt[whole[j] * kEvents] - rt[whole[j - 1] * kEvents] <= 2.0) ++j;
    char label[32];
    snprintf(label, sizeof label, "round %d", round++);
    print_group(label, std::vector<int64_t>(whole.begin() + i, whole.begin() + j), rt, nst, first);
    first = false;
    i = j;
  }
  if (!half.empty()) print_group("tail-split halves", half, rt, nst, first);
  printf("]}\n");
  fflush(stdout);
  CHECK(hipFree(x));
  CHECK(hipFree(w));
  CHECK(hipFree(o));
  CHECK(hipFree(tr));
}

}  // namespace

int main() {
  // f16: the 128 x 128 tile the forward picks at ViT widths (weight operand by
  // DMA); fp32: the 64 x 64 tile of the ViT-B attention projection, with its
  // tail split
  run<_Float16, 2, 1, 2, 4, 3, 1>("vith_fc1", 8224, 1280, 5120);
  run<_Float16, 2, 1, 2, 4, 3, 1>("vith_fc2", 8224, 5120, 1280);
  run<_Float16, 2, 1, 2, 4, 3, 1>("vitb_fc2", 12608, 3072, 768);
  run<float, 1, 1, 2, 2, 1, 1>("vitb_attn", 12608, 768, 768);
  return 0;
}
