// C ABI of the group-circulant linear layer (cyclic groups of order 4 and 8,
// the dihedral group p4m) and of the p4 group convolution built on it:
// argument validation, tile choice and kernel launches.  The contract of
// every entry point is stated in include/eqlin.h and include/eqconv.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "eqconv.h"
#include "eqlin.h"
#include "eqlin_kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int elem_bytes(int dtype) { return dtype == EQLIN_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape / dtype checks common to every entry point.  f16 rows of an odd
// number of 4-value groups would break the 16-byte alignment of the loads.
// T is the group code: 4, 8 (cyclic) or EQLIN_P4M (dihedral, order 8).
int check_shape(int64_t N, int C, int D, int T, int dtype) {
  static_assert(EQLIN_P4M == eqlin::kP4M, "group code");
  if (dtype != EQLIN_F32 && dtype != EQLIN_F16) return EQLIN_EINVAL;
  if (T != 4 && T != 8 && T != EQLIN_P4M) return EQLIN_ENOTSUP;
  const int O = eqlin::group_order(T);
  if (N < 0 || C <= 0 || D <= 0 || (C % O) != 0 || (D % O) != 0) return EQLIN_EINVAL;
  if (dtype == EQLIN_F16 && O == 4 && (((C / 4) % 2) != 0 || ((D / 4) % 2) != 0)) return EQLIN_ENOTSUP;
  return EQLIN_OK;
}

// Launchers of group T (a code accepted by check_shape).
#define EQLIN_BY_T(T, call) \
  ((T) == 4 ? eqlin::Launch<4>::call : (T) == 8 ? eqlin::Launch<8>::call : eqlin::Launch<eqlin::kP4M>::call)

int hip_status(hipError_t e) {
  if (e == hipSuccess) return EQLIN_OK;
  g_last_hip_error = static_cast<int>(e);
  return EQLIN_EHIP;
}

// Prepared planes of one direction: rows x ceil(groups / SG) stage blocks of
// 64 O bytes (O planes x 64 bytes; O = group order).
size_t plane_set_bytes(int rows, int groups, int O, int dtype) {
  const int sg = eqlin::stage_groups(dtype);
  return static_cast<size_t>(rows) * static_cast<size_t>(cdiv(groups, sg)) * 64u * static_cast<size_t>(O);
}

size_t transpose_offset(int C, int D, int O, int dtype) {
  return (plane_set_bytes(D / O, C / O, O, dtype) + 255u) & ~size_t(255);
}

// Buffer loads use 32-bit byte offsets inside one workgroup tile.
constexpr int64_t kMaxTileBytes = int64_t(1) << 30;

bool fwd_offsets_fit(int in_width, int O, int dtype) {
  const int64_t row_bytes = int64_t(in_width) * elem_bytes(dtype);
  const int64_t wrow_bytes = cdiv(in_width / O, eqlin::stage_groups(dtype)) * 64 * O;
  return 256 * row_bytes < kMaxTileBytes && 256 * wrow_bytes < kMaxTileBytes;
}

// The tile epilogue stores through 32-bit offsets within the tile's rows.
bool out_rows_fit(int out_width, int dtype) { return 256 * int64_t(out_width) * elem_bytes(dtype) < kMaxTileBytes; }

struct TileShape {
  int code, bm, bn;
  double eff;  // measured fraction of the MFMA peak on large shapes (MI355X, clocks settled)
};
// Forward tile candidates (code = FM FN WM WN NBUF PF, a seventh digit 1 for the
// persistent stream) with their measured efficiency on the ViT-B / ViT-H layer
// shapes.  For the order-8 groups in f16 the persistent stream wins on the
// long-K and wide layers (up to 15 % over the best one-tile-per-workgroup
// kernel): the tile epilogue, which dominates there, overlaps the next
// tile's loads and MFMAs.
// The last entry of each p4 table is the 64 x 32 tile of narrow layers (32 or
// fewer output groups), bound by HBM: its two-wave workgroups use half the
// LDS of 64 x 64 and six fit a CU, so more loads are in flight (C = D = 64 over
// 201728 rows: fp32 24.3 against 35.6 us, f16 persistent 14.3 against
// 25.1 us).  Its factor is set so that it wins only where 64 x 64 would leave
// at least a quarter of its columns empty.
constexpr TileShape kP4F32Tiles[] = {
    {112211, 64, 64, 0.745}, {112221, 64, 64, 0.70}, {111211, 32, 64, 0.59}, {112111, 64, 32, 0.55}};
// The f16 tiles copy their weight operand straight into LDS (NBUF 3 and 4):
// 5-14% faster than through registers (212421, 122211, 112211) at the ViT
// shapes and in the convolution.  The 64 x 128 tile fills the chip better
// than 128 x 128 where the larger tile leaves a CU one extra tile (ViT-B fc1:
// 37.6 against 43.1 us).
constexpr TileShape kP4F16Tiles[] = {{212431, 128, 128, 0.25},
                                     {122241, 64, 128, 0.24},
                                     {112241, 64, 64, 0.18},
                                     {111221, 32, 64, 0.12},
                                     {1121111, 64, 32, 0.12}};
// The p4 convolution in fp32: its gathered rows are 9x deeper than the linear
// layers' at K = 3, where the 128 x 128 tile's higher reuse per LDS byte pays
// once the pixel count leaves few tiles (28 x 28 and 14 x 14 maps, C = 512 and
// 1024: 7-8% faster than 64 x 64).
constexpr TileShape kConvF32Tiles[] = {{112211, 64, 64, 0.745}, {212421, 128, 128, 0.80}, {111211, 32, 64, 0.59}};
constexpr TileShape kConvF16Tiles[] = {{212431, 128, 128, 0.25}, {112241, 64, 64, 0.18}, {111221, 32, 64, 0.12}};
constexpr TileShape kC8F32Tiles[] = {{112211, 64, 64, 0.58}, {112221, 64, 64, 0.55}, {111221, 32, 64, 0.31}};
// The order-8 f16 64 x 128 tile with the weight DMA (122241, one workgroup
// per CU) runs ahead of the persistent register-path stream 1222111 or ties
// with it (C8 ViT-B attention 18.5 against 20.9 us, ViT-B fc2 43.8 against
// 46.5, ViT-H 2% faster); the 128 x 64 stream stays where it fills the chip
// better (ViT-H fc2).
constexpr TileShape kC8F16Tiles[] = {
    {122241, 64, 128, 0.145}, {2122111, 128, 64, 0.112}, {122211, 64, 128, 0.12}, {1122111, 64, 64, 0.105}};

// Forward tile choice: workgroups are spread round-robin over the CUs, so a
// CU's work is ceil(tiles / CUs) tiles, or the whole rounds plus half a tile
// where the launch splits its tail (eqlin::fwd_full_tiles); minimise that
// work divided by the tile's efficiency.  EQLIN_FWD_TILE overrides (any
// compiled tile code).
// kg, ksplit: with a K-split workspace (eqlin_forward_ws), the tail of a
// tile that takes the K split costs what fwd_ksplit_plan gives for kg input groups.
int choose_from_table(const TileShape* tiles, int ntiles, int64_t nrows, int mg, bool f32, bool split, int kg = 0,
                      bool ksplit = false);

int choose_fwd_tile(int T, int dtype, int64_t nrows, int mg, int kg = 0, bool ksplit = false) {
  if (const char* env = getenv("EQLIN_FWD_TILE")) {
    const int t = atoi(env);
    if (EQLIN_BY_T(T, fwd_tile_known(t))) return t;
  }
  const bool f32 = dtype == EQLIN_F32;
  // p4m has the same plane count and a similar product count as C8: same table
  const TileShape* tiles = T == 4 ? (f32 ? kP4F32Tiles : kP4F16Tiles) : (f32 ? kC8F32Tiles : kC8F16Tiles);
  const int ntiles = T == 4 ? (f32 ? int(sizeof(kP4F32Tiles) / sizeof(TileShape))
                                   : int(sizeof(kP4F16Tiles) / sizeof(TileShape)))
                            : (f32 ? int(sizeof(kC8F32Tiles) / sizeof(TileShape))
                                   : int(sizeof(kC8F16Tiles) / sizeof(TileShape)));
  return choose_from_table(tiles, ntiles, nrows, mg, f32, eqlin::fwd_tail_split_enabled(), kg, ksplit);
}

// The p4 convolution runs the p4 forward tiles (one workgroup per tile, with
// the fp32 tail split of the linear layer) with its own tables;
// EQCONV_FWD_TILE overrides the choice (any tile compiled for it).
int choose_conv_tile(int dtype, int64_t npix, int mg) {
  if (const char* env = getenv("EQCONV_FWD_TILE")) {
    const int t = atoi(env);
    if (eqlin::ConvLaunch::tile_known(t)) return t;
  }
  const bool split = eqlin::fwd_tail_split_enabled();
  return dtype == EQLIN_F32
             ? choose_from_table(kConvF32Tiles, int(sizeof(kConvF32Tiles) / sizeof(TileShape)), npix, mg, true, split)
             : choose_from_table(kConvF16Tiles, int(sizeof(kConvF16Tiles) / sizeof(TileShape)), npix, mg, false, split);
}

int choose_from_table(const TileShape* tiles, int ntiles, int64_t nrows, int mg, bool f32, bool split, int kg,
                      bool ksplit) {
  int best = tiles[0].code;
  double best_cost = 1e300;
  for (int i = 0; i < ntiles; ++i) {
    const TileShape& t = tiles[i];
    const int64_t n = cdiv(nrows, t.bm) * cdiv(mg, t.bn);
    const bool halves = split && eqlin::fwd_tail_split_fits_code(t.code, f32);
    const int64_t full = halves ? eqlin::fwd_full_tiles(n) : n;
    double rounds = full == n ? double(cdiv(n, eqlin::kNumCu)) : double(full / eqlin::kNumCu) + 0.5;
    if (split && ksplit && eqlin::fwd_ksplit_fits_code(t.code, f32, 4)) {
      const int kst = (int)cdiv(kg, eqlin::stage_groups(f32 ? EQLIN_F32 : EQLIN_F16));
      const eqlin::FwdKSplitPlan pl = eqlin::fwd_ksplit_plan(n, kst, halves);
      if (pl.nparts > 0)
        rounds = double(n / eqlin::kNumCu) +
                 double(cdiv(pl.tail * pl.nparts, eqlin::kNumCu)) * double(cdiv(kst, pl.nparts)) / kst;
    }
    const double cost = rounds * t.bm * t.bn / t.eff;
    if (cost < best_cost * 0.97) {  // keep the earlier (larger) tile unless clearly better
      best_cost = cost;
      best = t.code;
    }
  }
  return best;
}

// eqlin_backward with both outputs runs dX and the dw partials in one launch
// unless EQLIN_BWD_FUSED=0.
bool use_fused_backward() {
  static const bool fused = [] {
    const char* e = getenv("EQLIN_BWD_FUSED");
    return !(e && atoi(e) == 0);
  }();
  return fused;
}

// Row splits of the dw reduction: each split a whole number of pipeline
// stages and small enough for 32-bit offsets inside a split.  chunks > 1:
// rows_per_split counts rows of `chunks` consecutive rows (dw_chunks).
struct DwPlan {
  int64_t rows_per_split;
  int nsplit;
  int chunks;
  int width;   // dw partial tile: 64, or 128 (p4, whole rows)
};

// f16 p4 layers whose group-channel counts both reach 256 (the ViT-H MLP
// layers): the backward runs as separate launches, dX through the forward's
// tile choice (128 x 128 there, where the fused launch has 64 x 64) and dw
// alone with the 128-wide tile.  Measured (ViT-H f16, MI355X): fc1 159 ->
// 151 us, fc2 178 -> 155 us; the 128-wide dw alone 93 -> 88 us.  Smaller f16
// layers and fp32 keep the fused launch (ViT-B attention f16 34 against 40
// us separate, fp32 104 against 120 us).
bool wide_f16_layer(int O, int mg, int ng, int dtype) {
  return dtype == EQLIN_F16 && O == 4 && mg >= 256 && ng >= 256;
}

// Width of the stand-alone dw launch's tile: 64, or 128 for the wide f16 p4
// layers read in whole rows; EQLIN_DW_WIDTH=64|128 overrides for p4 (read at
// every call).
int dw_width(int O, int chunks, int mg, int ng, int dtype) {
  if (O != 4 || chunks != 1) return 64;
  if (const char* e = getenv("EQLIN_DW_WIDTH")) {
    const int w = atoi(e);
    if (w == 64 || w == 128) return w;
  }
  return wide_f16_layer(O, mg, ng, dtype) ? 128 : 64;
}

// Row chunks of the dw reduction of a narrow fp32 layer: when both
// group-channel counts are at most 16 (32), the rows are read as rows of 4
// (2) consecutive rows, so that the 64 x 64 dw tile holds 4 (2) row blocks
// side by side: every lane of its loads reads live data, and only its
// diagonal blocks are multiplied and summed (dw_tile).
// chunks divides N.  Measured (dw alone, 201728 rows): C = D = 64 fp32 96.5
// -> 38.2 us, C = D = 128 fp32 105 -> 68 us, C8 C = D = 128 over 100000 rows
// 132 -> 62 us.  f16 keeps whole rows: its MFMAs are cheap and its stage
// loop is bound by latency, and chunked it ran slower (C = D = 64 28.6 ->
// 33.0 us, C = D = 128 37.5 -> 44.6 us).
int dw_chunks(int64_t N, int mg, int ng, int dtype) {
  if (dtype != EQLIN_F32) return 1;
  const int w = mg > ng ? mg : ng;
  for (int c = 4; c > 1; c /= 2)
    if (c * w <= 64 && N % c == 0) return c;
  return 1;
}

DwPlan dw_plan_for(int64_t N, int C, int D, int dtype, int64_t want) {
  DwPlan p{0, 0, 1, 64};
  if (N <= 0) return p;
  const int64_t stage = eqlin::dw_rows_per_stage(dtype);
  const int64_t row_bytes = int64_t(C > D ? C : D) * elem_bytes(dtype);
  const int64_t max_split = cdiv(N, stage);
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  p.rows_per_split = cdiv(cdiv(N, want), stage) * stage;
  const int64_t cap = (kMaxTileBytes / row_bytes) / stage * stage;
  if (p.rows_per_split > cap) p.rows_per_split = cap > stage ? cap : stage;
  p.nsplit = static_cast<int>(cdiv(N, p.rows_per_split));
  return p;
}

// No cap on the number of dw row splits (the caller's workspace is sized by
// eqlin_backward_workspace_bytes).
constexpr int64_t kAnySplits = INT64_MAX;

// The dw launch (alone): a few 64 x 64 workgroups fit one CU; use two per CU
// in total.  The workspace holds this plan's splits, the most of the two.
// max_splits caps the splits asked for (a fixed-size scratch); the 32-bit
// offset cap inside a split can still ask for more, which the callers check.
// The 128-wide tile runs one workgroup per CU: one per CU in total.
// round_up: the split count rounded up instead of down (the fused fallback).
DwPlan plan_dw(int64_t N, int C, int D, int O, int dtype, bool chunked = false, int64_t max_splits = kAnySplits,
               int width = 64, bool round_up = false) {
  const int ch = chunked ? dw_chunks(N, D / O, C / O, dtype) : 1;
  const int W = ch == 1 ? width : 64;
  const int64_t tiles = cdiv(ch * D / O, W) * cdiv(ch * C / O, W);
  const int64_t slots = (W == 64 ? 2 : 1) * eqlin::kNumCu;
  const int64_t want = round_up ? cdiv(slots, tiles) : slots / tiles;
  DwPlan p = dw_plan_for(N / ch, ch * C, ch * D, dtype, want < max_splits ? want : max_splits);
  p.chunks = ch;
  p.width = W;
  return p;
}

// The stand-alone dw launch's plan.
DwPlan plan_dw_alone(int64_t N, int C, int D, int O, int dtype, int64_t max_splits = kAnySplits) {
  const int ch = dw_chunks(N, D / O, C / O, dtype);
  return plan_dw(N, C, D, O, dtype, true, max_splits, dw_width(O, ch, D / O, C / O, dtype));
}

// The fused backward launch: its dX tiles fill the chip besides the dw
// splits, so half as many splits (one dw workgroup per CU) pay, with less
// partial traffic and finalize work, unless one split grows long enough to
// set the launch's end: kept when a split's pipeline stages are at most 1.75
// times the launch's stages per resident workgroup (dw: tiles x row stages,
// dX: tiles x k stages; p4 fp32 three, p4 f16 two, order 8 one workgroup per
// CU), else two per CU as plan_dw.  Measured against two per CU: ViT-B
// attention fp32 113 -> 104 us and f16 -4%, ViT-H f16 and C8 -2% to -6%;
// the ViT-H fp32 layers (ratio 1.9) keep two per CU, where one per CU is 1%
// (fc1) and 9% (fc2) slower.  For p4 that fallback rounds its split count
// up: at ViT-H (100 dw tiles) 6 splits, not 5 (fp32 fused backward, fc1 744
// -> 655 us, fc2 646 -> 642 us; 3, 4 and 8 splits also beat 5 at fc1).
DwPlan plan_dw_fused(int64_t N, int C, int D, int O, int dtype, int64_t max_splits = kAnySplits) {
  const int ch = dw_chunks(N, D / O, C / O, dtype);
  const int64_t tiles = cdiv(ch * D / O, 64) * cdiv(ch * C / O, 64);
  const int64_t want = eqlin::kNumCu / tiles;
  DwPlan one = dw_plan_for(N / ch, ch * C, ch * D, dtype, want < max_splits ? want : max_splits);
  one.chunks = ch;
  if (one.nsplit > 0) {
    const int64_t split_stages = cdiv(one.rows_per_split, eqlin::dw_rows_per_stage(dtype));
    const int64_t dw_work = tiles * cdiv(N / ch, eqlin::dw_rows_per_stage(dtype));
    const int64_t dx_work = cdiv(N, 64) * cdiv(C / O, 64) * cdiv(D / O, eqlin::stage_groups(dtype));
    const int64_t per_cu = O == 4 ? (dtype == EQLIN_F32 ? 3 : 2) : 1;
    if (4 * split_stages * per_cu * eqlin::kNumCu <= 7 * (dw_work + dx_work)) return one;
  }
  return plan_dw(N, C, D, O, dtype, true, max_splits, 64, O == 4);
}

// Workspace bytes of the dw split partials (T planes of D' x C' float32 per
// split) for the plan of at most max_splits splits.  The fused plan never
// has more splits than this one (fewer splits asked for, the same offset cap).
size_t dw_split_bytes(int C, int D, int O) {
  return static_cast<size_t>(O) * static_cast<size_t>(C / O) * static_cast<size_t>(D / O) * sizeof(float);
}
size_t dw_workspace_need(int64_t N, int C, int D, int O, int dtype, int64_t max_splits) {
  // the most splits of any plan a call may run (the 64-wide stand-alone plan,
  // or the p4 fused fallback, which rounds its count up)
  const DwPlan a = plan_dw(N, C, D, O, dtype, true, max_splits);
  const DwPlan b = plan_dw_alone(N, C, D, O, dtype, max_splits);
  const DwPlan c = plan_dw_fused(N, C, D, O, dtype, max_splits);
  const int n = a.nsplit > b.nsplit ? (a.nsplit > c.nsplit ? a.nsplit : c.nsplit) : (b.nsplit > c.nsplit ? b.nsplit : c.nsplit);
  return static_cast<size_t>(n) * dw_split_bytes(C, D, O);
}

// ------------------------------------------------ p4 group convolution

int check_conv_shape(int64_t N, int H, int W, int C, int D, int K, int dtype) {
  if (dtype != EQLIN_F32 && dtype != EQLIN_F16) return EQLIN_EINVAL;
  if (N < 0 || H < 0 || W < 0 || C <= 0 || D <= 0 || (C % 4) != 0 || (D % 4) != 0) return EQLIN_EINVAL;
  if (K <= 0 || (K % 2) == 0) return EQLIN_EINVAL;
  if (K > 15) return EQLIN_ENOTSUP;
  // whole centre blocks: 4 group channels per 16-byte load group of 1 (f32) or 2 (f16)
  const int blk = dtype == EQLIN_F32 ? 4 : 8;
  if (((C / 4) % blk) != 0 || ((D / 4) % blk) != 0) return EQLIN_ENOTSUP;
  return EQLIN_OK;
}

// pixels of a batch, or -1 when N H W does not fit the 32-bit tile grid
int64_t conv_pixels(int64_t N, int H, int W) {
  if (N == 0 || H == 0 || W == 0) return 0;
  const int64_t hw = int64_t(H) * W;
  if (hw > (int64_t(1) << 31) || N > (int64_t(1) << 31) / hw) return -1;
  return N * hw;
}

size_t conv_set_bytes(int rows, int cpix, int K, int dtype) {
  return plane_set_bytes(rows, eqlin::conv_gathered_groups(cpix, K, dtype), 4, dtype);
}

size_t conv_adjoint_offset(int C, int D, int K, int dtype) {
  return (conv_set_bytes(D / 4, C / 4, K, dtype) + 255u) & ~size_t(255);
}

// the prepared rows of a launch must stay inside 32-bit buffer offsets of one workgroup tile
bool conv_weights_fit(int cpix, int K, int dtype) {
  const int64_t wrow = cdiv(eqlin::conv_gathered_groups(cpix, K, dtype), eqlin::stage_groups(dtype)) * 64 * 4;
  return 256 * wrow < kMaxTileBytes;
}

bool conv_map_fits(int64_t npix, int C, int dtype) { return npix * C * elem_bytes(dtype) < (int64_t(1) << 31); }

// Filter-gradient workspace: the gathered layer's dw, then its split partials.
struct ConvWs {
  size_t dwlin, split, total;
  DwPlan plan;
};

ConvWs conv_workspace(int64_t npix, int C, int D, int K, int dtype) {
  ConvWs w{};
  const int kg = eqlin::conv_gathered_groups(C / 4, K, dtype);
  w.plan = plan_dw(npix, 4 * kg, D, 4, dtype);
  w.dwlin = (static_cast<size_t>(D / 4) * kg * 4 * sizeof(float) + 255u) & ~size_t(255);
  w.split = static_cast<size_t>(w.plan.nsplit) * 4u * kg * static_cast<size_t>(D / 4) * sizeof(float);
  w.total = w.dwlin + w.split;
  return w;
}

// eqlin_forward_ws's launch for a shape: its tile, K-split plan and
// workspace bytes (0 where the plan has no K split).
struct FwdWsPlan {
  int tile;
  eqlin::FwdKSplitPlan ks;
  size_t bytes;
};

FwdWsPlan forward_ws_plan(int64_t N, int C, int D, int T, int dtype) {
  const int O = eqlin::group_order(T);
  const int kg = C / O, mg = D / O;
  const bool f32 = dtype == EQLIN_F32;
  FwdWsPlan p{choose_fwd_tile(T, dtype, N, mg, kg, O == 4), {0, 0}, 0};
  if (N == 0 || !eqlin::fwd_tail_split_enabled() || !eqlin::fwd_ksplit_fits_code(p.tile, f32, O)) return p;
  const int c = EQLIN_TILE_BASE(p.tile);
  const int bm = 32 * (c / 100000) * ((c / 1000) % 10), bn = 32 * ((c / 10000) % 10) * ((c / 100) % 10);
  p.ks = eqlin::fwd_ksplit_plan(cdiv(N, bm) * cdiv(mg, bn), (int)cdiv(kg, eqlin::stage_groups(dtype)),
                                eqlin::fwd_tail_split_fits_code(p.tile, f32));
  if (p.ks.nparts > 0)
    p.bytes = eqlin::kFwdKSplitCounterBytes +
              size_t(p.ks.tail) * size_t(p.ks.nparts) * eqlin::fwd_ksplit_slot_bytes(p.tile, O);
  return p;
}

}  // namespace

extern "C" {

int eqlin_version(void) { return 213; }

const char* eqlin_status_str(int status) {
  switch (status) {
    case EQLIN_OK: return "ok";
    case EQLIN_EINVAL: return "invalid argument";
    case EQLIN_ENOTSUP: return "unsupported configuration (T must be 4, 8 or EQLIN_P4M; f16 with T = 4 needs even group counts)";
    case EQLIN_EALIGN: return "data pointer not 16-byte aligned";
    case EQLIN_EWORKSPACE: return "workspace or prepared-weight buffer too small";
    case EQLIN_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int eqlin_last_hip_error(void) { return g_last_hip_error; }

size_t eqlin_prepared_weight_bytes(int C, int D, int T, int dtype) {
  if (check_shape(0, C, D, T, dtype) != EQLIN_OK) return 0;
  const int O = eqlin::group_order(T);
  return transpose_offset(C, D, O, dtype) + plane_set_bytes(C / O, D / O, O, dtype);
}

size_t eqlin_prepared_transpose_offset(int C, int D, int T, int dtype) {
  if (check_shape(0, C, D, T, dtype) != EQLIN_OK) return 0;
  const int O = eqlin::group_order(T);
  return transpose_offset(C, D, O, dtype);
}

int eqlin_prepare_weights(const void* w, int C, int D, int T, int dtype, void* W_hat, size_t W_hat_bytes,
                          void* stream) {
  int st = check_shape(0, C, D, T, dtype);
  if (st != EQLIN_OK) return st;
  const int O = eqlin::group_order(T);
  if (!w || !W_hat) return EQLIN_EINVAL;
  if (!aligned16(w) || !aligned16(W_hat)) return EQLIN_EALIGN;
  if (W_hat_bytes < eqlin_prepared_weight_bytes(C, D, T, dtype)) return EQLIN_EWORKSPACE;
  char* base = static_cast<char*>(W_hat);
  return hip_status(EQLIN_BY_T(T, prepare(dtype, w, base, base + transpose_offset(C, D, O, dtype), D / O, C / O,
                                          static_cast<hipStream_t>(stream))));
}

int eqlin_forward_plan(int64_t N, int C, int D, int T, int dtype, int* tile, int64_t* tiles, int64_t* whole) {
  const int st = check_shape(N, C, D, T, dtype);
  if (st != EQLIN_OK) return st;
  const int O = eqlin::group_order(T);
  // as eqlin_forward: an empty batch is accepted before the width checks
  if (N > 0 && (!fwd_offsets_fit(C, O, dtype) || !out_rows_fit(D, dtype))) return EQLIN_ENOTSUP;
  const int mg = D / O;
  const int code = choose_fwd_tile(T, dtype, N, mg);
  const int c = EQLIN_TILE_BASE(code);
  const int bm = 32 * (c / 100000) * ((c / 1000) % 10), bn = 32 * ((c / 10000) % 10) * ((c / 100) % 10);
  const int64_t n = cdiv(N, bm) * cdiv(mg, bn);
  const bool split = eqlin::fwd_tail_split_enabled() && eqlin::fwd_tail_split_fits_code(code, dtype == EQLIN_F32);
  if (tile) *tile = code;
  if (tiles) *tiles = n;
  if (whole) *whole = split ? eqlin::fwd_full_tiles(n) : n;
  return EQLIN_OK;
}

int eqlin_forward(const void* X, int64_t N, int C, int D, int T, const void* W_hat, void* Y, int dtype,
                  void* stream) {
  return eqlin_forward_ex(X, N, C, D, T, W_hat, nullptr, EQLIN_ACT_NONE, Y, dtype, stream);
}

int eqlin_forward_ex(const void* X, int64_t N, int C, int D, int T, const void* W_hat, const void* bias, int act,
                     void* Y, int dtype, void* stream) {
  return eqlin_forward_residual(X, N, C, D, T, W_hat, bias, act, nullptr, Y, dtype, stream);
}

int eqlin_forward_residual(const void* X, int64_t N, int C, int D, int T, const void* W_hat, const void* bias, int act,
                           const void* R, void* Y, int dtype, void* stream) {
  int st = check_shape(N, C, D, T, dtype);
  if (st != EQLIN_OK) return st;
  const int O = eqlin::group_order(T);
  if (act != EQLIN_ACT_NONE && act != EQLIN_ACT_GELU) return EQLIN_EINVAL;
  if (N == 0) return EQLIN_OK;
  if (!X || !W_hat || !Y) return EQLIN_EINVAL;
  if (!aligned16(X) || !aligned16(W_hat) || !aligned16(Y)) return EQLIN_EALIGN;
  if (R && !aligned16(R)) return EQLIN_EALIGN;
  if (bias && (reinterpret_cast<uintptr_t>(bias) % elem_bytes(dtype)) != 0) return EQLIN_EALIGN;
  if (!fwd_offsets_fit(C, O, dtype) || !out_rows_fit(D, dtype)) return EQLIN_ENOTSUP;
  const int tile = choose_fwd_tile(T, dtype, N, D / O);
  return hip_status(EQLIN_BY_T(T, forward(dtype, tile, X, W_hat, Y, N, C / O, D / O, bias, act, R,
                                          static_cast<hipStream_t>(stream))));
}

size_t eqlin_forward_workspace_bytes(int64_t N, int C, int D, int T, int dtype, int* parts) {
  if (parts) *parts = 0;
  if (check_shape(N, C, D, T, dtype) != EQLIN_OK) return 0;
  const int O = eqlin::group_order(T);
  if (N > 0 && (!fwd_offsets_fit(C, O, dtype) || !out_rows_fit(D, dtype))) return 0;
  const FwdWsPlan p = forward_ws_plan(N, C, D, T, dtype);
  if (parts) *parts = p.ks.nparts;
  return p.bytes;
}

int eqlin_forward_ws(const void* X, int64_t N, int C, int D, int T, const void* W_hat, const void* bias, int act,
                     const void* R, void* Y, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (!workspace) return eqlin_forward_residual(X, N, C, D, T, W_hat, bias, act, R, Y, dtype, stream);
  int st = check_shape(N, C, D, T, dtype);
  if (st != EQLIN_OK) return st;
  const int O = eqlin::group_order(T);
  if (act != EQLIN_ACT_NONE && act != EQLIN_ACT_GELU) return EQLIN_EINVAL;
  if (N == 0) return EQLIN_OK;
  if (!X || !W_hat || !Y) return EQLIN_EINVAL;
  if (!aligned16(X) || !aligned16(W_hat) || !aligned16(Y) || !aligned16(workspace)) return EQLIN_EALIGN;
  if (R && !aligned16(R)) return EQLIN_EALIGN;
  if (bias && (reinterpret_cast<uintptr_t>(bias) % elem_bytes(dtype)) != 0) return EQLIN_EALIGN;
  if (!fwd_offsets_fit(C, O, dtype) || !out_rows_fit(D, dtype)) return EQLIN_ENOTSUP;
  const FwdWsPlan p = forward_ws_plan(N, C, D, T, dtype);
  if (workspace_bytes < p.bytes) return EQLIN_EWORKSPACE;
  eqlin::FwdKSplit ks{};
  if (p.ks.nparts > 0) ks = eqlin::FwdKSplit{workspace, p.ks.nparts};
  return hip_status(EQLIN_BY_T(T, forward(dtype, p.tile, X, W_hat, Y, N, C / O, D / O, bias, act, R,
                                          static_cast<hipStream_t>(stream), ks)));
}

size_t eqlin_backward_workspace_bytes(int64_t N, int C, int D, int T, int dtype) {
  if (check_shape(N, C, D, T, dtype) != EQLIN_OK) return 0;
  return dw_workspace_need(N, C, D, eqlin::group_order(T), dtype, kAnySplits);
}

int eqlin_backward_dx(const void* dY, int64_t N, int C, int D, int T, const void* W_hat, void* dX, int dtype,
                      void* stream) {
  int st = check_shape(N, C, D, T, dtype);
  if (st != EQLIN_OK) return st;
  const int O = eqlin::group_order(T);
  if (N == 0) return EQLIN_OK;
  if (!dY || !W_hat || !dX) return EQLIN_EINVAL;
  if (!aligned16(dY) || !aligned16(W_hat) || !aligned16(dX)) return EQLIN_EALIGN;
  if (!fwd_offsets_fit(D, O, dtype) || !out_rows_fit(C, dtype)) return EQLIN_ENOTSUP;
  // dX = dY W: the forward kernel with the transposed, conjugated planes
  // (input groups D', output groups C').
  const char* wb = static_cast<const char*>(W_hat) + transpose_offset(C, D, O, dtype);
  const int tile = choose_fwd_tile(T, dtype, N, C / O);
  return hip_status(EQLIN_BY_T(T, forward(dtype, tile, dY, wb, dX, N, D / O, C / O, nullptr, 0, nullptr,
                                          static_cast<hipStream_t>(stream))));
}

}  // extern "C"

namespace {

// dw alone with at most max_splits row splits in the workspace.
int backward_dw_impl(const void* dY, const void* X, int64_t N, int C, int D, int T, float* dw, void* workspace,
                     size_t workspace_bytes, int dtype, void* stream, int64_t max_splits) {
  int st = check_shape(N, C, D, T, dtype);
  if (st != EQLIN_OK) return st;
  const int O = eqlin::group_order(T);
  if (!dw) return EQLIN_EINVAL;
  if (N > 0 && (!dY || !X || !workspace)) return EQLIN_EINVAL;
  if (!aligned16(dw)) return EQLIN_EALIGN;
  if (N > 0 && (!aligned16(dY) || !aligned16(X) || !aligned16(workspace))) return EQLIN_EALIGN;
  if (workspace_bytes < dw_workspace_need(N, C, D, O, dtype, max_splits)) return EQLIN_EWORKSPACE;
  const DwPlan p = plan_dw_alone(N, C, D, O, dtype, max_splits);
  return hip_status(EQLIN_BY_T(T, dw(dtype, dY, X, static_cast<float*>(workspace), dw, N, D / O, C / O,
                                     p.rows_per_split, p.nsplit, p.chunks, p.width,
                                     static_cast<hipStream_t>(stream))));
}

// eqlin_backward with the dw row splits capped at max_splits.
int backward_impl(const void* dY, const void* X, int64_t N, int C, int D, int T, const void* W_hat, void* dX,
                  float* dw, void* workspace, size_t workspace_bytes, int dtype, void* stream, int64_t max_splits) {
  int st = check_shape(N, C, D, T, dtype);
  if (st != EQLIN_OK) return st;
  const int O = eqlin::group_order(T);
  if (!dX && !dw) return EQLIN_EINVAL;
  // validate both halves before launching either
  if (dX && N > 0) {
    if (!dY || !W_hat) return EQLIN_EINVAL;
    if (!aligned16(dY) || !aligned16(W_hat) || !aligned16(dX)) return EQLIN_EALIGN;
    if (!fwd_offsets_fit(D, O, dtype) || !out_rows_fit(C, dtype)) return EQLIN_ENOTSUP;
  }
  if (dw) {
    if (N > 0 && (!dY || !X || !workspace)) return EQLIN_EINVAL;
    if (!aligned16(dw)) return EQLIN_EALIGN;
    if (N > 0 && (!aligned16(dY) || !aligned16(X) || !aligned16(workspace))) return EQLIN_EALIGN;
    if (workspace_bytes < dw_workspace_need(N, C, D, O, dtype, max_splits)) return EQLIN_EWORKSPACE;
  }
  // One fused launch for dX and the dw partials, except for f16 p4 layers of
  // 16 or fewer input groups (their dX runs faster as the forward's narrow
  // tile than as the fused launch's 64 x 64 one: C = D = 64 over 201728 rows,
  // 42.6 against 45.9 us; at 32 groups the fused launch still wins, 52.7
  // against 58.3 us), for the wide f16 p4 layers (wide_f16_layer) and for f16
  // p4 layers of 512 or more output groups, whose dX (an input-gradient of
  // that many k groups) runs on the forward's faster f16 tiles (ViT-B fc1:
  // 95.9 against 99.7 us fused; ViT-B attention and fc2, 192 output groups,
  // stay fused: 35.1 against 38.1 us, and a tie).
  const bool narrow_f16 = dtype == EQLIN_F16 && O == 4 && C / O <= 16;
  const bool wide_f16 = wide_f16_layer(O, D / O, C / O, dtype) || (dtype == EQLIN_F16 && O == 4 && D / O >= 512);
  if (dX && dw && N > 0 && use_fused_backward() && !narrow_f16 && !wide_f16) {
    // one launch for dX and the dw partials (they share dY), then the finalize
    const DwPlan p = plan_dw_fused(N, C, D, O, dtype, max_splits);
    const char* wb = static_cast<const char*>(W_hat) + transpose_offset(C, D, O, dtype);
    return hip_status(EQLIN_BY_T(T, bwd_fused(dtype, dY, X, wb, dX, static_cast<float*>(workspace), dw, N, D / O,
                                              C / O, p.rows_per_split, p.nsplit, p.chunks,
                                              static_cast<hipStream_t>(stream))));
  }
  if (dX) {
    st = eqlin_backward_dx(dY, N, C, D, T, W_hat, dX, dtype, stream);
    if (st != EQLIN_OK) return st;
  }
  if (dw) return backward_dw_impl(dY, X, N, C, D, T, dw, workspace, workspace_bytes, dtype, stream, max_splits);
  return EQLIN_OK;
}

}  // namespace

extern "C" {

int eqlin_backward_dw(const void* dY, const void* X, int64_t N, int C, int D, int T, float* dw, void* workspace,
                      size_t workspace_bytes, int dtype, void* stream) {
  return backward_dw_impl(dY, X, N, C, D, T, dw, workspace, workspace_bytes, dtype, stream, kAnySplits);
}

int eqlin_backward(const void* dY, const void* X, int64_t N, int C, int D, int T, const void* W_hat, void* dX,
                   float* dw, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  return backward_impl(dY, X, N, C, D, T, W_hat, dX, dw, workspace, workspace_bytes, dtype, stream, kAnySplits);
}

}  // extern "C"

// ------------------------------------------------ allocation-free backward
//
// The dw split partials of eqlin_backward_noalloc live in this file-scope
// device array: one copy per device, loaded with the library's code object
// and held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: the kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device (with that device
// current) and kept in g_scratch_addr.
static __device__ __align__(256) unsigned char scratch[EQLIN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
hipError_t scratch_address(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int eqlin_backward_noalloc(const void* dY, const void* X, int64_t N, int C, int D, int T, const void* W_hat,
                           void* dX, float* dw, int dtype, void* stream) {
  const int st = check_shape(N, C, D, T, dtype);
  if (st != EQLIN_OK) return st;
  if (!dw) return backward_impl(dY, X, N, C, D, T, W_hat, dX, dw, nullptr, 0, dtype, stream, kAnySplits);
  // The splits are capped to what the scratch holds; a layer whose one
  // split (T planes of D' x C' float32) does not fit is refused.
  const int O = eqlin::group_order(T);
  const int64_t max_splits = static_cast<int64_t>(EQLIN_NOALLOC_SCRATCH_BYTES / dw_split_bytes(C, D, O));
  if (max_splits < 1 || dw_workspace_need(N, C, D, O, dtype, max_splits) > EQLIN_NOALLOC_SCRATCH_BYTES)
    return EQLIN_EWORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_status(e);
  return backward_impl(dY, X, N, C, D, T, W_hat, dX, dw, ws, EQLIN_NOALLOC_SCRATCH_BYTES, dtype, stream,
                       max_splits);
}

// ------------------------------------------------ p4 group convolution

size_t eqconv_prepared_weight_bytes(int C, int D, int K, int dtype) {
  if (check_conv_shape(0, 0, 0, C, D, K, dtype) != EQLIN_OK) return 0;
  return conv_adjoint_offset(C, D, K, dtype) + conv_set_bytes(C / 4, D / 4, K, dtype);
}

size_t eqconv_prepared_adjoint_offset(int C, int D, int K, int dtype) {
  if (check_conv_shape(0, 0, 0, C, D, K, dtype) != EQLIN_OK) return 0;
  return conv_adjoint_offset(C, D, K, dtype);
}

int eqconv_prepare_weights(const void* psi, int C, int D, int K, int dtype, void* prepared, size_t prepared_bytes,
                           void* stream) {
  const int st = check_conv_shape(0, 0, 0, C, D, K, dtype);
  if (st != EQLIN_OK) return st;
  if (!psi || !prepared) return EQLIN_EINVAL;
  if (!aligned16(psi) || !aligned16(prepared)) return EQLIN_EALIGN;
  if (prepared_bytes < eqconv_prepared_weight_bytes(C, D, K, dtype)) return EQLIN_EWORKSPACE;
  char* base = static_cast<char*>(prepared);
  return hip_status(eqlin::ConvLaunch::prepare(dtype, psi, base, base + conv_adjoint_offset(C, D, K, dtype), D / 4,
                                               C / 4, K, static_cast<hipStream_t>(stream)));
}

int eqconv_forward(const void* X, int64_t N, int H, int W, int C, int D, int K, const void* prepared,
                   const void* bias, int act, void* Y, int dtype, void* stream) {
  const int st = check_conv_shape(N, H, W, C, D, K, dtype);
  if (st != EQLIN_OK) return st;
  if (act != EQLIN_ACT_NONE && act != EQLIN_ACT_GELU) return EQLIN_EINVAL;
  const int64_t npix = conv_pixels(N, H, W);
  if (npix < 0) return EQLIN_ENOTSUP;
  if (npix == 0) return EQLIN_OK;
  if (!X || !prepared || !Y) return EQLIN_EINVAL;
  if (!aligned16(X) || !aligned16(prepared) || !aligned16(Y)) return EQLIN_EALIGN;
  if (bias && (reinterpret_cast<uintptr_t>(bias) % elem_bytes(dtype)) != 0) return EQLIN_EALIGN;
  if (!conv_map_fits(npix, C, dtype) || !conv_weights_fit(C / 4, K, dtype) || !out_rows_fit(D, dtype))
    return EQLIN_ENOTSUP;
  const int tile = choose_conv_tile(dtype, npix, D / 4);
  return hip_status(eqlin::ConvLaunch::forward(dtype, tile, X, prepared, Y, npix, H, W, C / 4, K, D / 4, bias, act,
                                               static_cast<hipStream_t>(stream)));
}

size_t eqconv_backward_workspace_bytes(int64_t N, int H, int W, int C, int D, int K, int dtype) {
  if (check_conv_shape(N, H, W, C, D, K, dtype) != EQLIN_OK) return 0;
  const int64_t npix = conv_pixels(N, H, W);
  if (npix < 0) return 0;
  return conv_workspace(npix, C, D, K, dtype).total;
}

int eqconv_backward(const void* dY, const void* X, int64_t N, int H, int W, int C, int D, int K,
                    const void* prepared, void* dX, float* dpsi, void* workspace, size_t workspace_bytes, int dtype,
                    void* stream) {
  const int st = check_conv_shape(N, H, W, C, D, K, dtype);
  if (st != EQLIN_OK) return st;
  if (!dX && !dpsi) return EQLIN_EINVAL;
  const int64_t npix = conv_pixels(N, H, W);
  if (npix < 0) return EQLIN_ENOTSUP;
  // validate both halves before launching either
  if (dX && npix > 0) {
    if (!dY || !prepared) return EQLIN_EINVAL;
    if (!aligned16(dY) || !aligned16(prepared) || !aligned16(dX)) return EQLIN_EALIGN;
    if (!conv_map_fits(npix, D, dtype) || !conv_weights_fit(D / 4, K, dtype) || !out_rows_fit(C, dtype))
      return EQLIN_ENOTSUP;
  }
  ConvWs ws{};
  if (dpsi) {
    if (!workspace) return EQLIN_EINVAL;
    if (npix > 0 && (!dY || !X)) return EQLIN_EINVAL;
    if (!aligned16(dpsi) || !aligned16(workspace)) return EQLIN_EALIGN;
    if (npix > 0 && (!aligned16(dY) || !aligned16(X))) return EQLIN_EALIGN;
    // the gather reads X through 32-bit buffer offsets
    if (!conv_map_fits(npix, C, dtype)) return EQLIN_ENOTSUP;
    ws = conv_workspace(npix, C, D, K, dtype);
    if (workspace_bytes < ws.total) return EQLIN_EWORKSPACE;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dX && dpsi && npix > 0 && use_fused_backward()) {
    // one launch for dX and the dpsi partials (they share dY), the finalize, then onto the filter
    char* wsb = static_cast<char*>(workspace);
    const char* wb = static_cast<const char*>(prepared) + conv_adjoint_offset(C, D, K, dtype);
    int e = hip_status(eqlin::ConvLaunch::bwd_fused(dtype, dY, X, wb, dX, reinterpret_cast<float*>(wsb + ws.dwlin),
                                                    reinterpret_cast<float*>(wsb), npix, H, W, D / 4, C / 4, K,
                                                    ws.plan.rows_per_split, ws.plan.nsplit, s));
    if (e != EQLIN_OK) return e;
    return hip_status(eqlin::ConvLaunch::dw_scatter(dtype, reinterpret_cast<float*>(wsb), dpsi, D / 4, C / 4, K, s));
  }
  if (dX && npix > 0) {
    // dX: the convolution of dY with the adjoint filter (input D', output C')
    const char* wb = static_cast<const char*>(prepared) + conv_adjoint_offset(C, D, K, dtype);
    const int tile = choose_conv_tile(dtype, npix, C / 4);
    const int e = hip_status(eqlin::ConvLaunch::forward(dtype, tile, dY, wb, dX, npix, H, W, D / 4, K, C / 4, nullptr,
                                                        EQLIN_ACT_NONE, s));
    if (e != EQLIN_OK) return e;
  }
  if (dpsi) {
    char* wsb = static_cast<char*>(workspace);
    float* dwlin = reinterpret_cast<float*>(wsb);
    float* split = reinterpret_cast<float*>(wsb + ws.dwlin);
    // the gathered layer's dw (zeros for an empty batch), then onto the filter
    int e = hip_status(eqlin::ConvLaunch::dw(dtype, dY, X, split, dwlin, npix, H, W, D / 4, C / 4, K,
                                             ws.plan.rows_per_split, ws.plan.nsplit, s));
    if (e != EQLIN_OK) return e;
    e = hip_status(eqlin::ConvLaunch::dw_scatter(dtype, dwlin, dpsi, D / 4, C / 4, K, s));
    if (e != EQLIN_OK) return e;
  }
  return EQLIN_OK;
}

}  // extern "C"
