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
// only; nothing is checked).  With the K split of the last round (fp32, as
// eqlin_forward_ws runs it) the parts form their own group: their stage
// time, when their stages end, and for the parts that arrive last the time
// of the reduction and epilogue; a placement summary counts the CUs by the
// parts and workgroups they hold (hardware and XCC ids of every workgroup).
#include <map>
#include <utility>
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
void run(const char* name, int64_t N, int C, int D, bool ksplit = false) {
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
  int nparts = 0;
  char* wsp = nullptr;
  if (ksplit) {
    // the K split as launch_fwd_s plans it (the counters zeroed once; every
    // launch leaves them zero)
    const FwdKSplitPlan pl = fwd_ksplit_plan(tiles, ksteps, fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF));
    if (pl.nparts < 2) {
      fprintf(stderr, "%s: no K split for this shape\n", name);
      exit(1);
    }
    nparts = pl.nparts;
    nfull = tiles - pl.tail;
    grid = nfull + pl.tail * nparts;
    const size_t wsb = kFwdKSplitCounterBytes + (size_t)pl.tail * nparts * kpiece_slot_bytes<4, FM, FN, 64 * WM * WN>();
    CHECK(hipMalloc(&wsp, wsb));
    CHECK(hipMemset(wsp, 0, wsb));
  } else if constexpr (fwd_tail_split_fits(sizeof(E) == 4, FM, FN, WM, WN, NBUF)) {
    nfull = fwd_full_tiles(tiles);
    grid = nfull + 2 * (tiles - nfull);
  }
  // part workgroups: dispatched first where each CU gets at most one (fwd_kernel)
  const int64_t nkp = grid - nfull;
  auto is_part = [&](int64_t b) { return nparts > 1 && (nkp <= kNumCu ? b < nkp : b >= nfull); };
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
                       (const E*)nullptr, 0, (const E*)nullptr, tiles, nfull,
                       wsp ? (float*)(wsp + kFwdKSplitCounterBytes) : (float*)nullptr, (uint32_t*)wsp, nparts);
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
    if (raw[(b * kEvents + 3) * 2] != 0) r0 = std::min(r0, (double)raw[(b * kEvents) * 2 + 1]);
  std::vector<double> rt((size_t)grid * kEvents, 0.0), clk;
  for (int64_t b = 0; b < grid; ++b) {
    for (int e = 0; e < kEvents; ++e) rt[b * kEvents + e] = ((double)raw[(b * kEvents + e) * 2 + 1] - r0) * 0.01;
    const double cyc = (double)raw[(b * kEvents + 63) * 2] - (double)raw[(b * kEvents) * 2];
    const double us = rt[b * kEvents + 63] - rt[b * kEvents];
    if (raw[(b * kEvents + 63) * 2] != 0 && us > 0) clk.push_back(cyc / us / 1e3);
  }
  printf("{\"layer\": \"%s\", \"dtype\": \"%s\", \"N\": %lld, \"C\": %d, \"D\": %d, \"tile\": \"%d%d%d%d%d%d\", "
         "\"tiles\": %lld, \"workgroups\": %lld, \"stages\": %d, \"ksplit_parts\": %d, \"launch_us\": %.2f, "
         "\"shader_clock_ghz\": %.2f, ",
         name, sizeof(E) == 4 ? "f32" : "f16", (long long)N, C, D, FM, FN, WM, WN, NBUF, PF, (long long)tiles,
         (long long)grid, ksteps, nparts, ms * 1e3 / 100, median(clk));
  // placement: CUs keyed by (XCC, hardware id bits of SE, SH and CU), counted by
  // (parts, workgroups) held over the launch; and whether XCC = workgroup id mod 8
  {
    std::map<std::pair<unsigned, unsigned>, std::pair<int, int>> cu;
    int64_t xcc_mod8 = 0, seen = 0;
    for (int64_t b = 0; b < grid; ++b) {
      if (raw[(b * kEvents + 3) * 2] == 0) continue;   // left no events (a half with no rows)
      const unsigned id = (unsigned)raw[(b * kEvents + 61) * 2], xcc = (unsigned)raw[(b * kEvents + 61) * 2 + 1];
      auto& c = cu[{xcc, (id >> 8) & 0xffu}];
      c.first += is_part(b) ? 1 : 0;
      c.second += 1;
      xcc_mod8 += xcc == (unsigned)(b % 8);
      ++seen;
    }
    std::map<std::pair<int, int>, int> hist;
    for (auto& kv : cu) hist[kv.second]++;
    printf("\"placement\": {\"cus\": %zu, \"xcc_is_workgroup_id_mod_8\": %s, \"cus_by_parts_and_workgroups\": {",
           cu.size(), xcc_mod8 == seen ? "true" : "false");
    bool f = true;
    for (auto& kv : hist) {
      printf("%s\"%d parts, %d workgroups\": %d", f ? "" : ", ", kv.first.first, kv.first.second, kv.second);
      f = false;
    }
    printf("}}, \"groups\": [");
  }
  // whole tiles by round (a new round starts where the start times jump by
  // more than 2 us), then the tail-split halves or the K-split parts
  // (a workgroup that found no rows, a second half past the last row, left no events)
  std::vector<int64_t> whole, half, parts;
  for (int64_t b = 0; b < grid; ++b) {
    if (is_part(b)) {
      parts.push_back(b);
    } else if (raw[(b * kEvents + 63) * 2] != 0) {
      // with the K split every other workgroup is a whole tile (its ids
      // shift past the parts where those are dispatched first)
      (nparts > 1 || b < nfull ? whole : half).push_back(b);
    }
  }
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
  if (!parts.empty()) {
    // every part: prologue, first stage, later stages (over its own stage
    // count), when its stages end; the parts that arrived last (events 62,
    // 63): reduction plus epilogue, and their end
    std::vector<double> pro, st0, st, sd, red, start, end;
    for (int64_t b : parts) {
      const double* r = &rt[b * kEvents];
      // the kernel's logical part id (xcd_logical_id, on the host)
      const int64_t pb = nkp <= kNumCu ? b : b - nfull, xcd = pb % kNumXcd, per = nkp / kNumXcd,
                    rem = nkp % kNumXcd;
      const int64_t lp = xcd * per + (xcd < rem ? xcd : rem) + pb / kNumXcd;
      const int part = (int)(lp % nparts);
      const int kn = (part + 1) * ksteps / nparts - part * ksteps / nparts;
      pro.push_back(r[1] - r[0]);
      st0.push_back(r[2] - r[1]);
      if (kn > 1) st.push_back((r[3] - r[2]) / (kn - 1));
      sd.push_back(r[3]);
      start.push_back(r[0]);
      if (raw[(b * kEvents + 63) * 2] != 0) {
        red.push_back(r[62] - r[3]);
        end.push_back(r[63]);
      }
    }
    if (end.empty()) end.push_back(0.0);
    printf("%s{\"group\": \"k-split parts\", \"workgroups\": %zu, \"last_parts\": %zu, \"start_us\": [%.1f, %.1f], "
           "\"stages_end_us\": [%.1f, %.1f], \"end_us\": [%.1f, %.1f], \"prologue_us\": %.2f, \"first_stage_us\": %.2f, "
           "\"stage_us\": %.2f, \"reduce_epilogue_us\": %.2f}",
           first ? "" : ", ", parts.size(), end.size(), *std::min_element(start.begin(), start.end()),
           *std::max_element(start.begin(), start.end()), *std::min_element(sd.begin(), sd.end()),
           *std::max_element(sd.begin(), sd.end()), *std::min_element(end.begin(), end.end()),
           *std::max_element(end.begin(), end.end()), median(pro), median(st0), median(st), median(red));
  }
  printf("]}\n");
  fflush(stdout);
  if (wsp) CHECK(hipFree(wsp));
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
  // fp32 with the K split of the last round: the parts dispatched first
  // (ViT-B attention, 79 tiles in 3 parts) and after the whole tiles (ViT-H
  // fc2, 133 tiles in 3 parts)
  run<float, 1, 1, 2, 2, 1, 1>("vitb_attn_ksplit", 12608, 768, 768, true);
  run<float, 1, 1, 2, 2, 1, 1>("vith_fc2_f32_ksplit", 8224, 5120, 1280, true);
  return 0;
}
