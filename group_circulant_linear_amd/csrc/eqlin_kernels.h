// Internal launcher declarations shared by the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace eqlin {

// Forward tile codes: six digits FM FN WM WN NBUF PF, optionally a seventh P.
// A workgroup has WM x WN waves; each wave owns FM x FN fragments of 32 x 32
// per accumulator plane, so the workgroup tile is (32 FM WM) rows x (32 FN WN)
// output groups; NBUF (1 or 2) is the number of LDS stage buffers, PF (1 or
// 2) the number of stages of global loads in flight in registers, and P = 1
// selects the persistent kernel (resident workgroups stream over the tiles).
#define EQLIN_TILE_BASE(C) ((C) >= 1000000 ? (C) / 10 : (C))
#define EQLIN_TILE_ARGS(C)                                                                                  \
  EQLIN_TILE_BASE(C) / 100000, (EQLIN_TILE_BASE(C) / 10000) % 10, (EQLIN_TILE_BASE(C) / 1000) % 10,         \
      (EQLIN_TILE_BASE(C) / 100) % 10, (EQLIN_TILE_BASE(C) / 10) % 10, EQLIN_TILE_BASE(C) % 10
#define EQLIN_TILE_PERSIST(C) ((C) >= 1000000 ? (C) % 10 : 0)

constexpr int kNumCu = 256;  // MI355X compute units (8 XCDs x 32)

// Tail split of a one-workgroup-per-tile forward launch.  Workgroups are
// spread evenly over the CUs, so a launch of `tiles` tiles costs each CU
// ceil(tiles / kNumCu) tiles.  When the last, partial round holds at most
// half the CUs' worth of tiles, each of those tiles runs as two workgroups
// of half its rows: the two wave rows of a half each multiply one of the two
// k chunks of every stage into the same fragments and add their partial sums
// through LDS at the end, so no CU runs more than half a tile beyond the
// whole rounds.  fp32 tiles with two wave rows, at most two fragments per
// wave (registers for the partial sums beside the accumulators) and LDS
// that holds the second row's accumulators run split.  The f16 tiles do not:
// they hold one or two workgroups per CU and their stages are bound by
// latency rather than by the matrix cores, so a half costs about as much as
// a whole tile (measured: no gain on the ViT-B and ViT-H layers).
constexpr bool fwd_tail_split_fits(bool f32, int FM, int FN, int WM, int WN, int NBUF) {
  return f32 && WM == 2 && NBUF < 3 && FM * FN <= 2 && 2 * WN * FM * FN <= NBUF * (2 * FM + FN * WN);
}
inline bool fwd_tail_split_fits_code(int code, bool f32) {
  const int c = EQLIN_TILE_BASE(code);
  return !EQLIN_TILE_PERSIST(code) &&
         fwd_tail_split_fits(f32, c / 100000, (c / 10000) % 10, (c / 1000) % 10, (c / 100) % 10, (c / 10) % 10);
}
// Tiles that run whole when `tiles` tiles are launched with the tail split
// (the rest run as halves); == tiles when the split does not pay.
inline int64_t fwd_full_tiles(int64_t tiles) {
  const int64_t r = tiles % kNumCu;
  return (tiles > kNumCu && 2 * r <= kNumCu) ? tiles - r : tiles;
}
// EQLIN_FWD_SPLIT=0 turns the tail split off (every tile whole); read at
// every launch, as the tile override is.
inline bool fwd_tail_split_enabled() {
  const char* e = getenv("EQLIN_FWD_SPLIT");
  return !(e && atoi(e) == 0);
}

// K split of the tail (float32 register-path tiles, one workgroup per tile):
// with a caller's workspace, the tiles of the last, partial round can each
// run as nparts workgroups over consecutive ranges of the k stages instead
// (see KPiece in eqlin_device.h), which caps the busiest CU's extra work at
// ceil(tail nparts / CUs) parts of ceil(stages / nparts) stages.  The plan
// takes the part count (2 .. kMaxKParts) that minimises that work, where it
// is at least 10% below what the tile's other choice costs (half a tile with
// the tail split, else a whole tile): the parts' sums make a round trip
// through memory.
constexpr int kMaxKParts = 4;
constexpr size_t kFwdKSplitCounterBytes = 1024;   // arrival counters of up to 256 tail tiles
// The order-8 groups do not take it: their parts' slots are twice as large
// and the fixup cost more than it saved (C8 ViT-B attention: 53.6 -> 68 us).
constexpr bool fwd_ksplit_fits(bool f32, int T, int NBUF, int PERSIST) {
  return f32 && T == 4 && NBUF < 3 && PERSIST == 0;
}
inline bool fwd_ksplit_fits_code(int code, bool f32, int T) {
  const int c = EQLIN_TILE_BASE(code);
  return fwd_ksplit_fits(f32, T, (c / 10) % 10, EQLIN_TILE_PERSIST(code));
}
struct FwdKSplitPlan {
  int64_t tail;   // tiles run in parts (the last tail tiles)
  int nparts;     // 0: no K split
};
inline FwdKSplitPlan fwd_ksplit_plan(int64_t tiles, int kst, bool halves_fit) {
  const int64_t r = tiles % kNumCu;
  FwdKSplitPlan best{0, 0};
  if (r == 0 || kst < 2) return best;
  double cost = (halves_fit && tiles > kNumCu && 2 * r <= kNumCu) ? 0.5 : 1.0;
  const double bar = 0.9 * cost;
  for (int sp = 2; sp <= kMaxKParts && sp <= kst; ++sp) {
    const double c = double((r * sp + kNumCu - 1) / kNumCu) * ((kst + sp - 1) / sp) / kst;
    if (c < bar && c < cost) {
      cost = c;
      best = {r, sp};
    }
  }
  return best;
}
// Bytes of one part's accumulators for tile code `code` and group order T
// (the tile's T planes of BM x BN float32 values).
inline size_t fwd_ksplit_slot_bytes(int code, int T) {
  const int c = EQLIN_TILE_BASE(code);
  return size_t(4096) * (c / 100000) * ((c / 10000) % 10) * ((c / 1000) % 10) * ((c / 100) % 10) * T;
}
// The caller's K-split workspace for one launch: counters (zero before the
// launch; the launch leaves them zero), then tail x nparts slots.
struct FwdKSplit {
  void* ws = nullptr;
  int nparts = 0;
};

//
// Group codes: 4 and 8 are the cyclic groups of that order (4: the p4
// rotation group), kP4M the dihedral group p4m of order 8.
constexpr int kP4M = 108;
inline int group_order(int g) { return g == kP4M ? 8 : g; }

// Launchers of group G, instantiated for G = 4, 8 and kP4M.  dtype 0 =
// float32, 1 = float16; kg / mg / dg / cg are group-channel counts
// (channels / group order).
template <int G>
struct Launch {
  static bool fwd_tile_known(int tile);
  // bias: nullable, one storage-dtype value per output group; act: 0 none, 1 GELU (erf);
  // res: nullable, a residual laid out as out, added after the activation
  // ks: the K split of the tail (FwdKSplit{}: none)
  static hipError_t forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t nrows, int kg,
                            int mg, const void* bias, int act, const void* res, hipStream_t s,
                            const FwdKSplit& ks = FwdKSplit{});
  // chunks (1, or a divisor of nrows with chunks x mg, chunks x ng <= 64): rows
  // read as rows of `chunks` consecutive rows (narrow layers), rows_per_split
  // counting those
  // width: dw tile 64, or 128 (p4 only; chunks == 1)
  static hipError_t dw(int dtype, const void* dy, const void* x, float* ws, float* dw, int64_t nrows, int mg, int ng,
                       int64_t rows_per_split, int nsplit, int chunks, int width, hipStream_t s);
  // dX (forward structure on the transpose spectra wb, 64 x 64 tiles) and the
  // dw split partials in one launch, then the dw finalize.  nrows > 0.
  static hipError_t bwd_fused(int dtype, const void* dy, const void* x, const void* wb, void* dx, float* ws,
                              float* dw, int64_t nrows, int dg, int cg, int64_t rows_per_split, int nsplit,
                              int chunks, hipStream_t s);
  static hipError_t prepare(int dtype, const void* w, void* wf, void* wb, int mg, int ng, hipStream_t s);
};

#define EQLIN_DECLARE_LAUNCH(T)                                                                                     \
  template <> bool Launch<T>::fwd_tile_known(int tile);                                                             \
  template <> hipError_t Launch<T>::forward(int, int, const void*, const void*, void*, int64_t, int, int,          \
                                            const void*, int, const void*, hipStream_t, const FwdKSplit&);         \
  template <> hipError_t Launch<T>::dw(int, const void*, const void*, float*, float*, int64_t, int, int, int64_t,   \
                                       int, int, int, hipStream_t);                                                \
  template <> hipError_t Launch<T>::bwd_fused(int, const void*, const void*, const void*, void*, float*, float*,   \
                                              int64_t, int, int, int64_t, int, int, hipStream_t);                  \
  template <> hipError_t Launch<T>::prepare(int, const void*, void*, void*, int, int, hipStream_t);
EQLIN_DECLARE_LAUNCH(4)
EQLIN_DECLARE_LAUNCH(8)
EQLIN_DECLARE_LAUNCH(kP4M)
#undef EQLIN_DECLARE_LAUNCH

inline int stage_groups(int dtype) { return dtype == 0 ? 16 : 32; }       // group channels per pipeline stage
inline int dw_rows_per_stage(int dtype) { return dtype == 0 ? 16 : 32; }  // rows per dw pipeline stage

// p4 group convolution (eqconv_kernels.hip): group channels of one gathered
// row (cpix K^2), padded to whole pipeline stages.
inline int conv_gathered_groups(int cpix, int K, int dtype) {
  const int sg = stage_groups(dtype);
  return (cpix * K * K + sg - 1) / sg * sg;
}

// Launchers of the p4 group convolution (T = 4).  cpix: group channels of the
// input map; mg: output group channels; K: odd filter width.
struct ConvLaunch {
  static bool tile_known(int tile);
  static hipError_t forward(int dtype, int tile, const void* in, const void* wp, void* out, int64_t npix, int H,
                            int W, int cpix, int K, int mg, const void* bias, int act, hipStream_t s);
  // forward set (rows D', gathered over C') into wf, adjoint set (rows C', gathered over D') into wb
  static hipError_t prepare(int dtype, const void* psi, void* wf, void* wb, int Dp, int Cp, int K, hipStream_t s);
  // split partials of the gathered layer's dw (the gather in the loads) and their ordered
  // finalize into dwlin [Dp][gathered groups][4]
  static hipError_t dw(int dtype, const void* dy, const void* x, float* ws, float* dwlin, int64_t npix, int H, int W,
                       int Dp, int Cp, int K, int64_t rows_per_split, int nsplit, hipStream_t s);
  // dX (64 x 64 tiles on the adjoint spectra wb) and the dw split partials in one launch,
  // then the finalize into dwlin.  npix > 0.
  static hipError_t bwd_fused(int dtype, const void* dy, const void* x, const void* wb, void* dx, float* ws,
                              float* dwlin, int64_t npix, int H, int W, int Dp, int Cp, int K, int64_t rows_per_split,
                              int nsplit, hipStream_t s);
  static hipError_t dw_scatter(int dtype, const float* dwlin, float* dpsi, int Dp, int Cp, int K, hipStream_t s);
};

}  // namespace eqlin
