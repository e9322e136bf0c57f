// moe_api.cpp -- host side of the C ABI declared in include/moe.h:
// argument checks (host only, before any HIP call), the plan (block size,
// split of the down projection, workspace carve-up) and the launches of the
// six kernels on the caller's stream.  No device allocation, no
// synchronisation.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr size_t kAlign = 256;
constexpr int kBlockRows[] = {16, 32, 64, 128, 192};
constexpr int kMaxSplit = 8;
constexpr int kTargetDownWorkgroups = 1024;  // ~4 per CU on 256 CUs

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// 256-row blocks: only when asked, on the LDS-staged tiles (narrow gate/up,
// 256-column down).
constexpr int kLargeBlockRows = 256;
bool is_block_rows(int bm) {
  for (int b : kBlockRows)
    if (b == bm) return true;
  return bm == kLargeBlockRows;
}

// Checks that only depend on sizes.  dims: d and ffn are used.
int check_sizes(int T, int d, int ffn, int E, int k, bool dims) {
  if (T < 0 || E < 1) return MOE_ERR_SHAPE;
  if (dims && (d < 1 || ffn < 1)) return MOE_ERR_SHAPE;
  if (k < 1 || k > E) return MOE_ERR_TOPK;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (dims && (d % 64 != 0 || ffn % 64 != 0)) return MOE_ERR_ALIGN;
  if ((long long)T * k > MOE_MAX_ROWS) return MOE_ERR_UNSUPPORTED;
  // The GEMMs address one expert's weights with 32-bit buffer offsets
  // (including the rows of a partly filled last column tile).
  const long long lim = 1LL << 31;
  if (dims && ((2LL * ffn + 256) * d * 2 >= lim || (d + 256LL) * ffn * 2 >= lim))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Forced paths must fit their limits.
int check_paths(int T, int d, int E, int k, const moe_options* opt) {
  if (!opt) return MOE_OK;
  if (opt->routing_kernels == 1 && !small_routing_fits(T, E, k)) return MOE_ERR_UNSUPPORTED;
  if (opt->routing_kernels == 3 && !fused_reorder_fits(T * k, E)) return MOE_ERR_UNSUPPORTED;
  if (opt->gather_mode == 1 && (long long)T * d * 2 + 2LL * d >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  if (opt->gather_mode == 3 && ((long long)T * k + 16) * d * 2 >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_options(const moe_options* opt) {
  if (!opt) return MOE_OK;
  if (opt->block_rows != 0 && !is_block_rows(opt->block_rows)) return MOE_ERR_UNSUPPORTED;
  if (opt->split_k < 0 || opt->split_k > kMaxSplit) return MOE_ERR_UNSUPPORTED;
  if (opt->tile_variant < 0 || opt->rotate < 0 || opt->rotate > 4) return MOE_ERR_UNSUPPORTED;
  if (opt->routing_kernels < 0 || opt->routing_kernels > 3) return MOE_ERR_UNSUPPORTED;
  if (opt->gather_mode < 0 || opt->gather_mode > 3) return MOE_ERR_UNSUPPORTED;
  if (opt->unfused_swiglu < 0 || opt->unfused_swiglu > 1) return MOE_ERR_UNSUPPORTED;
  if (opt->xcd_order < 0 || opt->xcd_order > 3) return MOE_ERR_UNSUPPORTED;
  if (opt->fold_combine < 0 || opt->fold_combine > 2) return MOE_ERR_UNSUPPORTED;
  if (opt->fuse_down < 0 || opt->fuse_down > 2) return MOE_ERR_UNSUPPORTED;
  if (opt->schedule < 0 || opt->schedule > 3) return MOE_ERR_UNSUPPORTED;
  if (opt->down_variant < 0) return MOE_ERR_UNSUPPORTED;
  if (opt->down_variant > 0) {
    const int bm = opt->block_rows;
    if (bm == 0 || down_tile_cols(bm, opt->down_variant - 1) == 0) return MOE_ERR_UNSUPPORTED;
  }
  if (opt->tile_variant > 0) {
    const int bm = opt->block_rows;
    if (bm == 0 || gate_up_tile_cols(bm, opt->tile_variant - 1) == 0) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// Block size: at least kMinAutoBlockRows, and large enough that the mean
// rows per expert plus three standard deviations of a uniform router
// (binomial counts) fit one block, so that under near-uniform routing almost
// every expert is one block and its weights are streamed once.
//
// Why a floor: a block's cost is dominated by streaming its expert's
// weights, which is the same for any BM (the GEMMs skip the 16-row subtiles
// past a block's last row), while every extra block of an expert streams
// those weights again.  The host cannot see the routed counts, and under
// skewed routing the hot experts hold many times the mean; with the floor
// they take a few large blocks instead of many small ones.  Measured on the
// MoE workload shapes (uniform and skewed), BM = 128 was within a few
// percent of the best block size everywhere, and up to ~30% faster than
// sizing by the mean alone.
constexpr int kMinAutoBlockRows = 128;

int auto_block_rows(int A, int E) {
  const double mean = (double)A / E;
  const double want = std::max(mean + 3.0 * sqrt(mean) + 1.0, (double)kMinAutoBlockRows);
  for (int b : kBlockRows)
    if (b >= want) return b;
  return kBlockRows[sizeof(kBlockRows) / sizeof(kBlockRows[0]) - 1];
}

// Workgroups of a GEMM launch when every expert is active: blocks x tiles.
long long est_workgroups(int A, int E, int bm, int n_cols, int tile_cols) {
  const long long blocks = std::max<long long>((A + bm - 1) / bm, std::min(E, A));
  return std::max<long long>(blocks, 1) * ((n_cols + tile_cols - 1) / tile_cols);
}

// Split of the down projection's reduction.  Measured on the MoE workload
// shapes: one round of long-running workgroups (~one per CU) beats many
// short ones, so split only as far as needed to reach ~256 workgroups, and
// use two parts when a launch is small (< 640 workgroups).
int auto_split(int A, int E, int d, int ffn, int bm) {
  const int dcols = bm == kLargeBlockRows ? down_tile_cols(bm, kDownLdsVariant) : down_tile_cols(bm, 0);
  const long long wg = est_workgroups(A, E, bm, d, dcols > 0 ? dcols : 256);
  int s = (int)((256 + wg - 1) / wg);
  if (wg < 640 && s < 2) s = 2;
  const int max_by_k = ffn / (8 * 64);  // keep at least 8 K steps per part
  if (s > max_by_k) s = max_by_k;
  if (s > kMaxSplit) s = kMaxSplit;
  return s < 1 ? 1 : s;
}

// Fraction of a launch's workgroup slots doing work when `wg` workgroups run
// in rounds of `slots` (one resident workgroup per CU).
double round_balance(long long wg, long long slots) {
  const long long rounds = (wg + slots - 1) / slots;
  return rounds > 0 ? (double)wg / (double)(rounds * slots) : 1.0;
}

// Where the block-size rule gives 128 rows, 192-row blocks instead when the
// 224-column gate/up tile of BM = 192 then covers ffn exactly and its
// workgroups fill whole rounds of 256: with few experts each block holds
// one expert either way, and that tile's launch has no partial round where
// the narrow 128-column tile's has one (Mixtral-shaped T = 128 / 256, 8
// blocks: 512 workgroups against 896).  Measured, pass ms, interleaved,
// on two boxes: Mixtral T=128 0.4666 -> 0.4604 and 0.4664 -> 0.4660, T=256
// 0.4930 -> 0.4756 and 0.4925 -> 0.4876; the rule leaves
// Qwen2- and skewed-shaped workloads (ffn not a multiple of 224) at 128
// rows, where 192 measured slower (Qwen2 T=128 0.5744 -> 0.5775, skewed
// T=128 0.0798 -> 0.0860).
constexpr int kWideGateUpCols = 224;
bool prefer_192_rows(int A, int E, int ffn) {
  if (ffn <= 0 || ffn % kWideGateUpCols != 0) return false;
  return est_workgroups(A, E, 192, ffn, kWideGateUpCols) % kRoundWorkgroups == 0;
}

// Whether the LDS-staged gate/up tile (224 columns at BM = 192, 256 at
// BM = 128) can run: row-major activations (the last column tile may be
// partial).
bool gate_up_lds_fits(int bm, int ffn, bool x_tiled) {
  (void)ffn;
  return (bm == 128 || bm == 192) && gate_up_tile_cols(bm, kGateUpLdsVariant) > 0 && !x_tiled;
}

// Automatic use of a partial last LDS tile: at most this share of extra
// columns, and only for launches of at least two rounds (DeepSeek-V3 T=4096
// gate/up measured 3064 -> 2738 us with 2048 columns in 224-column tiles;
// skewed T=128/256, ~20 active blocks of 1408 columns in 256-column tiles,
// 42 -> 66 us: too few workgroups).
constexpr double kMaxLdsTileWaste = 0.1;
constexpr long long kPartialLdsMinWorkgroups = 512;


// Columns a launch of `tc`-column tiles covers beyond n, as a fraction of n
// (a partial last tile still reads its block's activation rows in full).
double tile_waste(int n, int tc) {
  return tc > 0 ? (double)((n + tc - 1) / tc * tc - n) / n : 1.0;
}

// Tile variant of the fused gate/up GEMM.  The LDS-staged tile (256
// columns at BM = 128, 224 at BM = 192) when its columns divide into whole
// tiles -- at BM = 128 only for launches of at least one round -- or nearly
// so on large launches (kMaxLdsTileWaste); measured faster on every such
// MoE workload shape (gate/up µs: Mixtral T=512 427.6 -> 334.9 with half
// the activation bytes per weight byte, DeepSeek-V3 T=512 2434 -> 2169,
// T=4096 3064 -> 2738, Mixtral T=128 355 -> 328, Qwen2 T=512 413 -> 393).
// Otherwise, BM = 64 and 128: the narrow variant when the wide one would
// give at most ~1.5 workgroups per CU; BM = 192: the 112-column variant
// when its tiles fill the rounds better than 128-column tiles do.
// At BM = 128 the narrow LDS-staged tile (8 waves x 16 columns, three
// stages): measured faster than both the 128-column register-ring tile and
// the 256-column LDS tile on every BM = 128 workload but one, gate/up us,
// former automatic choice -> narrow, interleaved in one process: Qwen2
// T=128/256/512 374 -> 353, 387 -> 363, 393 -> 372; Mixtral T=128/256 325
// -> 308, 333 -> 330; skewed T=128/512 41.9 -> 39.3, 79.0 -> 74.2;
// DeepSeek-V3 T=512 2164 -> 2156; skewed T=256 44.5 -> 47.1.
int auto_gu_variant(int A, int E, int ffn, int bm, bool x_tiled) {
  if (bm == kLargeBlockRows) return kGateUpLdsNarrowVariant;  // the only tile there
  if (bm == 128 && gate_up_lds_fits(bm, ffn, x_tiled)) return kGateUpLdsNarrowVariant;
  if ((bm == 128 || bm == 192) && gate_up_lds_fits(bm, ffn, x_tiled)) {
    const int tc = gate_up_tile_cols(bm, kGateUpLdsVariant);
    const double waste = tile_waste(ffn, tc);
    const long long wg = est_workgroups(A, E, bm, ffn, tc);
    if (waste == 0.0 ? (bm == 192 || wg >= 256)
                     : (waste <= kMaxLdsTileWaste && wg >= kPartialLdsMinWorkgroups))
      return kGateUpLdsVariant;
  }
  if (bm == 64 || bm == 128)
    return est_workgroups(A, E, bm, ffn, gate_up_tile_cols(bm, 0)) <= 384 ? 1 : 0;
  if (bm == 192) {
    const double b0 = round_balance(est_workgroups(A, E, bm, ffn, gate_up_tile_cols(192, 0)), 256);
    const double b1 = round_balance(est_workgroups(A, E, bm, ffn, gate_up_tile_cols(192, 1)), 256);
    const bool exact1 = ffn % gate_up_tile_cols(192, 1) == 0;  // no partial last tile
    return (exact1 && b1 > b0 + 0.05) ? 1 : 0;
  }
  return 0;
}

// XCD-grouped workgroup order: measured 1-2% faster when a launch has many
// schedule blocks (each XCD then streams its own range of experts and keeps
// their activation rows in its L2), and neutral to a few percent slower with
// few blocks (a few experts' weights then stream through one XCD each).
// Launching the blocks longest first when they are not grouped by XCD:
// measured no faster on the skewed workloads (the tail round of a launch is
// bound by each workgroup's own stream, not by which blocks run in it) and
// slower on some uniform ones, so automatic is off.
bool auto_longest_first(int A, int E, int bm) {
  (void)A, (void)E, (void)bm;
  return false;
}

// The stream-K schedule of the gate/up GEMM (see gemm_lds_sk_kernel):
// measured slower than one workgroup per unit of the same tile on every
// workload (gate/up us: skewed T=128 39.3 -> 251.4, Qwen2 T=128 353 -> 362,
// Mixtral T=128 308 -> 380, DeepSeek-V3 T=512 2156 -> 2203): the hand-off's
// agent-scope fences write back and invalidate whole L2s, and the units'
// activation rows are fetched once per workgroup sharing a unit.  Off.
bool auto_stream_k(int A, int E, int d, int ffn, int bm) {
  (void)A, (void)E, (void)d, (void)ffn, (void)bm;
  return false;
}

// The gate/up GEMM over the variable-size block table (launch_gate_up_var,
// VarRows): the routing kernels merge a hot expert's 128-row blocks into
// 256-row ones only when that takes the launch from more than one round of
// workgroups to one, and otherwise the table is the fixed one.  Built only
// where the routed counts can call for it: the most blocks the fixed table
// can have fill more than a round, and the fewest the merged one can have
// (every row in 256-row blocks) fit in one.  (Building it and deciding on the
// device cost the routing 0.2-0.6 us where it does not merge: Qwen2 T=512,
// whose 20 column tiles leave no merged table within one round, skips it.)
bool auto_var_rows(int A, int E, int d, int ffn) {
  (void)d;
  const long long tiles = (ffn + 127) / 128;
  const long long most = (A + 127) / 128 + std::min(E, A);
  const long long fewest = (A + 255) / 256;
  return most * tiles > kRoundWorkgroups && fewest * tiles <= kRoundWorkgroups;
}

bool auto_xcd_order(int A, int E, int bm) {
  const long long blocks = std::max<long long>((A + bm - 1) / bm, std::min(E, A));
  return blocks >= 128;
}

// Rotating the K start (see the GEMM kernel) was measured faster or equal on
// every MoE workload shape, so it is on unless the caller turns it off.  The
// key is the expert: with one block per expert (near-uniform routing) that
// is the per-block rotation; under skew, where a hot expert has several
// blocks, they then read the same weights at the same time (skewed routing,
// E = 64, top-4, T = 512: pass 146.0 -> 143.2 us, down GEMM 41.8 -> 39.0 us;
// all tokens on four experts 95.7 -> 93.5 us).
constexpr int kRotatePerExpert = 3;  // kernel value
int auto_rotate(int) { return kRotatePerExpert; }

// Whether the LDS-staged down tile (8 waves x 32 columns, BM = 128 or 192)
// can run: whole 256-column tiles, and the combination not folded into the
// down GEMM (the fold lives in the register-ring tiles).
bool down_lds_fits(int bm, int d, bool fold) {
  return (bm == 128 || bm == 192 || bm == kLargeBlockRows) &&
         d % down_tile_cols(bm, kDownLdsVariant) == 0 && !fold;
}

// Tile variant of the down GEMM.  The wide LDS-staged tile (64 columns per
// wave) when its columns divide into whole tiles or nearly so
// (kMaxLdsTileWaste), the launch, every expert active, has at least a round
// of workgroups, and each block has at least kWideDownMinTiles column tiles
// (skewed routing leaves most experts idle, and the host cannot see it: the
// launch must keep its workgroups through the columns).  Measured faster
// there (down GEMM, µs: Qwen2 T=128 215.6 -> 202.5, T=256 222.7 -> 204.6,
// T=512 231.6 -> 214.4, DeepSeek-V3 T=512 1255 -> 1237, T=4096
// 1688 -> 1662), slower on launches of a few long blocks (Mixtral T=512,
// 160-240 workgroups: 194 -> 206-262; T=128 144 -> 148-193) and on skewed
// routing with 4 tiles per block (T=128 25.4 -> 35.0, T=256 33.2 -> 36.5;
// T=512 42.6 -> 40.4).
// Else the 256-column LDS-staged tile wherever it fits -- measured faster
// or equal on every MoE workload shape than the register tiles (down GEMM,
// µs: skewed T=512 45.9 -> 39.5, Qwen2 T=512 267 -> 244, Mixtral T=512
// 205 -> 188, DeepSeek-V3 T=4096 1726 -> 1678, Mixtral T=128 162 -> 160) --
// else variant 0.
constexpr int kWideDownMinTiles = 6;

// At BM = 128 the wide tile comes in 8 waves (512 columns) and 7 (448): the
// 7-wave one where its whole tiles fill the last round of 256 workgroups
// better (Qwen2, d = 3584, 64 blocks: 7 x 64 = 448 workgroups, 1.75
// rounds, against 8 x 64 = 512, two whole rounds).  Measured, pass ms,
// interleaved: Qwen2 T=128/256/512 0.5751 -> 0.5667, 0.5886 -> 0.5825,
// 0.6142 -> 0.6117 (down 203 -> 194 us at T=128); the same bytes.
int auto_dn_variant(int A, int E, int bm, int d, int split, bool fold) {
  if (!fold && (bm == 128 || bm == 192)) {
    const int wc = down_tile_cols(bm, kDownLdsWideVariant);
    if (wc > 0 && tile_waste(d, wc) <= kMaxLdsTileWaste && (d + wc - 1) / wc >= kWideDownMinTiles &&
        est_workgroups(A, E, bm, d, wc) * split >= 256) {
      const int w7 = bm == 128 ? down_tile_cols(bm, kDownLdsWide7Variant) : 0;
      if (w7 > 0 && d % w7 == 0 &&
          round_balance(est_workgroups(A, E, bm, d, w7) * split, 256) >
              round_balance(est_workgroups(A, E, bm, d, wc) * split, 256) + 0.05)
        return kDownLdsWide7Variant;
      return kDownLdsWideVariant;
    }
  }
  return down_lds_fits(bm, d, fold) ? kDownLdsVariant : 0;
}

// The down projection fused into the gate/up GEMM: for launches of less
// than one round of workgroups, whose time is latency and launches, and
// only while the per-tile partials stay small (they are written and read
// once each).  Measured on the tiny workload: 28.4 -> 24.6 us per pass.
int auto_fuse_down(int A, int d, int ffn, int E, int bm, int tile_cols) {
  const long long parts = (ffn + tile_cols - 1) / tile_cols;
  const long long partial_bytes = parts * A * (long long)d * 4;
  return est_workgroups(A, E, bm, ffn, tile_cols) <= 256 && partial_bytes <= (8LL << 20);
}

// The weighted combination as its own kernel, or folded into the down GEMM.
// The separate kernel measured faster on every MoE workload shape (tiny to
// DeepSeek-V3): folded, the workgroups that finish last do the whole
// combination serially, and the partials go out as write-through stores.
int auto_fold(int T, int d, int E, int k) {
  (void)T, (void)d, (void)E, (void)k;
  return 0;
}

void make_plan(int T, int d, int ffn, int E, int k, const moe_options* opt, Plan* p) {
  memset(p, 0, sizeof(*p));
  p->T = T;
  p->d = d;
  p->ffn = ffn;
  p->E = E;
  p->k = k;
  p->A = T * k;
  const int A = p->A;
  // The stream-K and variable-size schedules run the 128-row tile: automatic
  // block rows are 128 then.
  const int sch = opt ? opt->schedule : 0;
  const bool sch128 = sch == 2 || sch == 3;
  p->bm = (opt && opt->block_rows) ? opt->block_rows
          : sch128                 ? 128
                                   : auto_block_rows(A > 0 ? A : 1, E);
  if (!(opt && opt->block_rows) && !sch128 && p->bm == 128 && prefer_192_rows(A, E, ffn))
    p->bm = 192;
  p->nb_max = (A + p->bm - 1) / p->bm + (E < A ? E : A);
  p->nchunks = (A + kChunk - 1) / kChunk;
  const int rk = opt ? opt->routing_kernels : 0;
  p->small_routing = rk == 1 || (rk == 0 && small_routing_fits(T, E, k) &&
                                  E <= kSmallRoutingAutoMaxExperts &&
                                  (long long)T * E * k <= kSmallRoutingAutoWork);
  // Otherwise two launches (route; histogram, scan, schedule and reorder in
  // one workgroup) where the per-group counts fit in LDS, else three.
  p->fused_reorder = !p->small_routing && (rk == 3 || (rk == 0 && fused_reorder_fits(A, E)));
  // The fused gate/up GEMM addresses x [T, d] with 32-bit buffer offsets.
  const int gm = opt ? opt->gather_mode : 0;
  const bool x_fits = (long long)T * d * 2 + 2LL * d < (1LL << 31);
  p->gather_in_gemm = gm == 1 || (gm == 0 && x_fits);
  p->x_tiled = gm == 3;
  p->unfused = opt ? opt->unfused_swiglu : 0;
  if (ffn > 0) {
    int s = (opt && opt->split_k) ? opt->split_k : auto_split(A, E, d, ffn, p->bm);
    const int ksteps = ffn / 64;
    const int per = (ksteps + s - 1) / s;
    p->ksplit = per * 64;
    p->split = (ksteps + per - 1) / per;  // every part has at least one K step
    p->gu_variant = (opt && opt->tile_variant) ? opt->tile_variant - 1
                                               : auto_gu_variant(A, E, ffn, p->bm, p->x_tiled);
    if ((p->bm == 128 || p->bm == 192) &&
        (p->gu_variant == kGateUpLdsVariant || p->gu_variant == kGateUpLdsNarrowVariant) &&
        !p->unfused &&
        !gate_up_lds_fits(p->bm, ffn, p->x_tiled))
      p->plan_error = MOE_ERR_UNSUPPORTED;  // forced where it cannot run
    const int fc = opt ? opt->fold_combine : 0;
    p->fold = fc == 0 ? auto_fold(T, d, E, k) : fc == 2;
    p->dn_variant = (opt && opt->down_variant) ? opt->down_variant - 1
                                               : auto_dn_variant(A, E, p->bm, d, p->split, p->fold);
    if (p->dn_variant == kDownLdsVariant && !down_lds_fits(p->bm, d, p->fold))
      p->plan_error = MOE_ERR_UNSUPPORTED;  // forced where it cannot run
    if ((p->dn_variant == kDownLdsWideVariant || p->dn_variant == kDownLdsWide7Variant) && p->fold)
      p->plan_error = MOE_ERR_UNSUPPORTED;  // the fold lives in the register-ring tiles
    // 256-row blocks run only the LDS-staged tiles: the narrow gate/up tile
    // and the 256-column down tile (d a multiple of 256); not the unfused
    // ablation, gather mode 3 or the folded combination.
    if (p->bm == kLargeBlockRows &&
        (p->gu_variant != kGateUpLdsNarrowVariant || p->dn_variant != kDownLdsVariant ||
         p->unfused || p->x_tiled || p->fold))
      p->plan_error = MOE_ERR_UNSUPPORTED;
    const int rot = opt ? opt->rotate : 0;
    // kernel values: 0 off, 1 per block, 2 per workgroup
    p->gu_rotate = rot == 0 ? auto_rotate(d) : rot - 1;
    p->dn_rotate = rot == 0 ? auto_rotate(ffn) : rot - 1;
    const int xo = opt ? opt->xcd_order : 0;
    // (an explicit variable-size schedule keeps the gate/up GEMM's blocks in
    // table order)
    p->dn_xcd = xo == 0 ? auto_xcd_order(A, E, p->bm) : xo == 2;
    p->gu_xcd = xo == 0 ? (sch != 3 && p->dn_xcd) : xo == 2;
    p->longest_first = xo == 3 || (xo == 0 && !p->gu_xcd && auto_longest_first(A, E, p->bm));
    const int dcols = down_tile_cols(p->bm, p->dn_variant);
    p->dn_tiles = dcols > 0 ? (d + dcols - 1) / dcols : 0;
    // The down projection inside the gate/up GEMM: one fp32 part per gate/up
    // column tile replaces the h buffer and the down GEMM.
    // At BM = 128 it takes the narrow tile unless the caller fixed one.
    const int fd = opt ? opt->fuse_down : 0;
    const bool gv_auto = !(opt && opt->tile_variant);
    const int fv = (p->bm == 128 && gv_auto) ? 1
                   : (p->bm == 192 && gv_auto && p->gu_variant == kGateUpLdsVariant) ? 0
                                                                                    : p->gu_variant;
    const int tc = gate_up_down_tile_cols(p->bm, fv);
    const bool fd_ok = tc > 0 && !p->unfused && (long long)d * ffn * 2 < (1LL << 31);
    if (fd == 2 && !fd_ok) p->plan_error = MOE_ERR_UNSUPPORTED;
    // (an explicit stream-K or variable-size schedule keeps the separate down GEMM)
    p->fused_down = fd == 2 ? fd_ok
                            : (fd == 0 && !sch128 && fd_ok && auto_fuse_down(A, d, ffn, E, p->bm, tc));
    if (p->fused_down) {
      p->gu_variant = fv;
      p->split = (ffn + tc - 1) / tc;
      p->fold = 0;
    }
    // An automatic split is an upper bound: the host's estimate assumes
    // every expert is active, and under skewed routing far fewer blocks
    // exist, so the down GEMM and the combination take the parts from the
    // routed block count on the device (device_down_split).  Measured
    // (us per pass, split 1 / 2 / 3 forced): skewed T=512 (30 blocks x 8
    // tiles) 136.9 / 143.7 / 152.7 -- one part; skewed T=128 (16 x 8)
    // 97.1 / 89.0 / 91.4 and Mixtral T=512 (8 x 16) 637.3 / 558.8 / 588.0 --
    // two; the device rule picks those.
    p->dyn_split = !(opt && opt->split_k) && !p->fold && !p->fused_down && p->split > 1;
    // The gate/up GEMM's schedule: one workgroup per (block, column tile),
    // or stream-K over the narrow LDS-staged tile at BM = 128.
    p->gu_sk = sch == 2 || (sch == 0 && auto_stream_k(A, E, d, ffn, p->bm));
    if (p->gu_sk) {
      const bool gv_ok = !(opt && opt->tile_variant) || p->gu_variant == kGateUpLdsNarrowVariant;
      const bool ok = p->bm == 128 && gv_ok && !p->unfused && !p->fused_down && !p->x_tiled;
      if (ok) {
        p->gu_variant = kGateUpLdsNarrowVariant;
        const int tc = gate_up_tile_cols(128, kGateUpLdsNarrowVariant);
        p->sk_units = p->nb_max * ((ffn + tc - 1) / tc);
      } else {
        if (sch == 2) p->plan_error = MOE_ERR_UNSUPPORTED;
        p->gu_sk = 0;
      }
    }
    // Or over the variable-size block table: the narrow LDS-staged tile at
    // 128 and 256 rows, the blocks in table order.
    const bool var_ok = p->bm == 128 && p->gu_variant == kGateUpLdsNarrowVariant && !p->unfused &&
                        !p->fused_down && !p->gu_sk && !p->x_tiled && !p->gu_xcd &&
                        !p->longest_first;
    if (sch == 3) {
      if (var_ok) p->gu_var = kVarRowsAlways;
      else p->plan_error = MOE_ERR_UNSUPPORTED;
    } else if (sch == 0 && var_ok && auto_var_rows(A, E, d, ffn)) {
      p->gu_var = kVarRowsAuto;
    }
  }
  size_t o = 0;
  auto seg = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t nck = (size_t)p->nchunks * E;
  p->o_ids = seg((size_t)A * 4);
  p->o_w = seg((size_t)A * 4);
  p->o_counts = seg((size_t)E * 4);
  p->o_offsets = seg((size_t)(E + 1) * 4);
  p->o_ccnt = seg(nck * 4);
  p->o_cbase = seg(nck * 4);
  p->o_perm = seg((size_t)A * 4);
  p->o_inv = seg((size_t)A * 4);
  p->o_blocks = seg((size_t)p->nb_max * 2 * 4);
  p->o_nb = seg(4);
  p->o_order = seg((size_t)p->nb_max * 4);
  p->route_bytes = o;
  p->o_xperm = seg(p->gather_in_gemm ? 0 : (size_t)(A + 15) / 16 * 16 * d * 2);
  p->o_h = seg(p->fused_down ? 0 : (size_t)A * ffn * 2);
  p->o_g = seg(p->unfused ? (size_t)A * ffn * 2 : 0);
  p->o_u = seg(p->unfused ? (size_t)A * ffn * 2 : 0);
  p->o_y = seg((size_t)p->split * A * d * 4);
  p->o_logits = seg((size_t)T * E * 4);
  p->router = plan_router(T, d > 0 ? d : 64, E);
  p->o_rparts = seg(p->router.parts > 1 ? (size_t)p->router.parts * T * E * 4 : 0);
  p->o_fold = seg(((p->fold ? (size_t)T * p->dn_tiles : 0) + (size_t)p->sk_units) * 4);
  p->o_skpart = seg(p->gu_sk ? 2 * (size_t)kRoundWorkgroups *
                                   gate_up_sk_slot_bytes(p->bm, p->gu_variant)
                             : 0);
  p->o_vblocks = seg(p->gu_var ? (size_t)p->nb_max * 3 * 4 : 0);
  p->o_vnb = seg(p->gu_var ? 4 : 0);
  p->total_bytes = o;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int record(const moe_options* opt, int i, hipStream_t s) {
  if (!opt || !opt->stage_events) return MOE_OK;
  hipEvent_t ev = static_cast<hipEvent_t>(opt->stage_events[i]);
  if (!ev) return MOE_OK;
  return hipEventRecord(ev, s) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

#define MOE_TRY_HIP(expr)                     \
  do {                                        \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)
#define MOE_TRY(expr)           \
  do {                          \
    const int rc_ = (expr);     \
    if (rc_ != MOE_OK) return rc_; \
  } while (0)

// K1..K3 into the workspace's routing section: one workgroup for small
// problems, else two launches where the reorder fits the histogram kernel,
// else three.
int run_routing(const LogitSrc& logits, const Plan& p, int renorm, int score, void* ws,
                const moe_options* opt, int32_t* order, ZeroRange zero, VarRows var,
                hipStream_t s) {
  int32_t* ids = at<int32_t>(ws, p.o_ids);
  float* w = at<float>(ws, p.o_w);
  int32_t* offsets = at<int32_t>(ws, p.o_offsets);
  MOE_TRY(record(opt, 0, s));
  if (p.small_routing) {
    MOE_TRY_HIP(launch_route_dispatch_small(logits, p.T, p.E, p.k, renorm, score, p.bm, ids, w,
                                            at<int32_t>(ws, p.o_counts), offsets,
                                            at<int32_t>(ws, p.o_perm), at<int32_t>(ws, p.o_inv),
                                            at<int32_t>(ws, p.o_blocks), at<int32_t>(ws, p.o_nb),
                                            order, zero, var, s));
    MOE_TRY(record(opt, 1, s));
    MOE_TRY(record(opt, 2, s));
    return MOE_OK;
  }
  MOE_TRY_HIP(launch_route(logits, p.T, p.E, p.k, renorm, score, ids, w, zero, s));
  MOE_TRY(record(opt, 1, s));
  int32_t* fperm = p.fused_reorder ? at<int32_t>(ws, p.o_perm) : nullptr;
  int32_t* finv = p.fused_reorder ? at<int32_t>(ws, p.o_inv) : nullptr;
  MOE_TRY_HIP(launch_hist_scan(ids, p.A, p.E, p.bm, p.nchunks, at<int32_t>(ws, p.o_counts),
                               offsets, at<int32_t>(ws, p.o_ccnt), at<int32_t>(ws, p.o_cbase),
                               at<int32_t>(ws, p.o_blocks), at<int32_t>(ws, p.o_nb), order, fperm,
                               finv, var, s));
  MOE_TRY(record(opt, 2, s));
  if (p.fused_reorder) return MOE_OK;
  MOE_TRY_HIP(launch_permute(ids, p.A, p.E, p.nchunks, offsets, at<int32_t>(ws, p.o_ccnt),
                             at<int32_t>(ws, p.o_cbase), at<int32_t>(ws, p.o_perm),
                             at<int32_t>(ws, p.o_inv), s));
  return MOE_OK;
}

// The forward pass from router scores already on the device (steps K1..K6).
int forward_from_logits(const uint16_t* x, const LogitSrc& router_logits, const uint16_t* W_gate_up,
                        const uint16_t* W_down, int top_k, int renorm, uint16_t* out, int score,
                        const Plan& p, const moe_options* opt, void* workspace, hipStream_t s) {
  const int T = p.T, d = p.d, ffn = p.ffn;
  // The routing kernels clear the arrival counters of the combination
  // folded into the down GEMM and the unit counters of the stream-K
  // gate/up GEMM (one range: the fold's, then stream-K's).
  const int n_fold = p.fold ? T * p.dn_tiles : 0;
  int32_t* counters = (p.fold || p.gu_sk) ? at<int32_t>(workspace, p.o_fold) : nullptr;
  int32_t* fold_cnt = p.fold ? counters : nullptr;
  int32_t* order = p.longest_first ? at<int32_t>(workspace, p.o_order) : nullptr;
  // The variable-size block table of the gate/up GEMM, when it runs over one.
  int32_t* vblocks = p.gu_var ? at<int32_t>(workspace, p.o_vblocks) : nullptr;
  int32_t* vnb = p.gu_var ? at<int32_t>(workspace, p.o_vnb) : nullptr;
  const int gu_tiles = p.gu_var ? (ffn + gate_up_tile_cols(128, kGateUpLdsNarrowVariant) - 1) /
                                      gate_up_tile_cols(128, kGateUpLdsNarrowVariant)
                                : 0;
  MOE_TRY(run_routing(router_logits, p, renorm, score, workspace, opt, order,
                      ZeroRange{counters, counters ? n_fold + p.sk_units : 0},
                      VarRows{vblocks, vnb, p.gu_var, gu_tiles}, s));
  const int32_t* perm = at<int32_t>(workspace, p.o_perm);
  const int32_t* blocks = at<int32_t>(workspace, p.o_blocks);
  const int32_t* nb = at<int32_t>(workspace, p.o_nb);
  const int32_t* offsets = at<int32_t>(workspace, p.o_offsets);
  uint16_t* x_perm = at<uint16_t>(workspace, p.o_xperm);
  uint16_t* h = at<uint16_t>(workspace, p.o_h);
  float* y = at<float>(workspace, p.o_y);
  if (p.x_tiled)
    MOE_TRY_HIP(launch_gather_tiled(x, perm, p.A, d, top_k, x_perm, s));
  else if (!p.gather_in_gemm)
    MOE_TRY_HIP(launch_gather(x, perm, p.A, d, top_k, x_perm, s));
  MOE_TRY(record(opt, 3, s));
  const uint16_t* X = p.gather_in_gemm ? x : x_perm;
  const int32_t* gperm = p.gather_in_gemm ? perm : nullptr;
  if (p.unfused) {
    // Ablation: the two projections each read the activation rows and write
    // a bf16 product; a third kernel applies SiLU and the product.
    uint16_t* g = at<uint16_t>(workspace, p.o_g);
    uint16_t* u = at<uint16_t>(workspace, p.o_u);
    const long long estride = 2LL * ffn * d;
    MOE_TRY_HIP(launch_proj_bf16(p.bm, X, gperm, top_k, T, W_gate_up, estride, blocks, nb,
                                 order, offsets, g, p.A, d, ffn, p.nb_max, p.gu_rotate, p.gu_xcd,
                                 p.x_tiled, s));
    MOE_TRY_HIP(launch_proj_bf16(p.bm, X, gperm, top_k, T, W_gate_up + (size_t)ffn * d, estride,
                                 blocks, nb, order, offsets, u, p.A, d, ffn, p.nb_max, p.gu_rotate,
                                 p.gu_xcd, p.x_tiled, s));
    MOE_TRY_HIP(launch_swiglu_act(g, u, h, (long long)p.A * ffn, s));
  } else if (p.fused_down) {
    MOE_TRY_HIP(launch_gate_up_down(p.bm, p.gu_variant, X, gperm, top_k, T, W_gate_up, W_down,
                                    blocks, nb, order, offsets, y, p.A, d, ffn, p.nb_max,
                                    p.gu_rotate, p.gu_xcd, p.x_tiled, s));
  } else if (p.gu_var) {
    MOE_TRY_HIP(launch_gate_up_var(X, gperm, top_k, T, W_gate_up, vblocks, vnb, blocks, nb,
                                   offsets, h, d, ffn, p.nb_max, p.gu_rotate, s));
  } else if (p.gu_sk) {
    MOE_TRY_HIP(launch_gate_up_sk(p.bm, p.gu_variant, X, gperm, top_k, T, W_gate_up, blocks, nb,
                                  offsets, h, d, ffn, p.gu_rotate,
                                  at<float>(workspace, p.o_skpart), counters + n_fold, s));
  } else {
    MOE_TRY_HIP(launch_gate_up(p.bm, p.gu_variant, X, gperm, top_k, T, W_gate_up, blocks, nb,
                               order, offsets, h, p.A, d, ffn, p.nb_max, p.gu_rotate, p.gu_xcd,
                               p.x_tiled, s));
  }
  MOE_TRY(record(opt, 4, s));
  const int32_t* inv = at<int32_t>(workspace, p.o_inv);
  const float* wts = at<float>(workspace, p.o_w);
  const FoldCombine fold{perm, inv, wts, top_k, fold_cnt, out};
  if (!p.fused_down)
    MOE_TRY_HIP(launch_down(p.bm, p.dn_variant, h, W_down, blocks, nb, order, offsets, y, p.A, d,
                            ffn, p.split, p.ksplit, p.nb_max, p.dn_rotate, p.dn_xcd,
                            p.fold ? fold : FoldCombine{}, s, p.dyn_split));
  MOE_TRY(record(opt, 5, s));
  if (!p.fold)
    MOE_TRY_HIP(launch_combine(y, p.split, p.A, d, inv, wts, top_k, T, out, s,
                               p.dyn_split ? DynSplit{nb, p.dn_tiles, ffn} : DynSplit{nullptr, 0, 0}));
  MOE_TRY(record(opt, 6, s));
  return MOE_OK;
}

// The workspace of moe_forward_static: a fixed device array, one per GPU
// (each device holds its own copy of a __device__ variable).  In host code
// `scratch` names a host-side stand-in, not device memory: kernels get the
// address hipGetSymbolAddress returns for the current device, kept per
// device below.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// Address of this device's array: looked up once per device, with that
// device current (restored afterwards).
int static_workspace(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[device]) {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return MOE_ERR_HIP;
    if (prev != device && hipSetDevice(device) != hipSuccess) return MOE_ERR_HIP;
    void* p = nullptr;
    const hipError_t rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != device) (void)hipSetDevice(prev);
    if (rc != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return MOE_OK;
}

// Size checks of the router scores alone (x [T, d], W_r [E, d]).
int check_router_sizes(int T, int d, int E) {
  if (T < 0 || d < 1 || E < 1) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS || T > MOE_MAX_ROWS) return MOE_ERR_UNSUPPORTED;
  if (d % 64 != 0) return MOE_ERR_ALIGN;
  // one 32-row tile of x or W_r is addressed with 32-bit buffer offsets
  if (32LL * d * 2 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid size";
    case MOE_ERR_TOPK: return "top_k must be in [1, E]";
    case MOE_ERR_ALIGN: return "d and ffn must be multiples of 64; pointers 16-byte aligned, workspace 256";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_UNSUPPORTED: return "outside the library's limits or an unsupported option";
    case MOE_ERR_HIP: return "a HIP call failed";
    case MOE_ERR_STATIC_LIMIT:
      return "the problem needs more workspace than the static array (MOE_STATIC_WORKSPACE_BYTES)";
    default: return "unknown status";
  }
}

int moe_workspace_size_ex(int T, int d, int ffn, int E, int top_k, const moe_options* opt,
                          size_t* bytes) {
  MOE_TRY(check_sizes(T, d, ffn, E, top_k, true));
  MOE_TRY(check_options(opt));
  MOE_TRY(check_paths(T, d, E, top_k, opt));
  if (!bytes) return MOE_ERR_NULL;
  if (T == 0) {
    *bytes = 0;
    return MOE_OK;
  }
  Plan p;
  make_plan(T, d, ffn, E, top_k, opt, &p);
  MOE_TRY(p.plan_error);
  *bytes = p.total_bytes;
  return MOE_OK;
}

int moe_workspace_size(int T, int d, int ffn, int E, int top_k, size_t* bytes) {
  return moe_workspace_size_ex(T, d, ffn, E, top_k, nullptr, bytes);
}

int moe_plan(int T, int d, int ffn, int E, int top_k, const moe_options* opt, int* block_rows,
             int* split_k, int* fused_down) {
  MOE_TRY(check_sizes(T, d, ffn, E, top_k, true));
  MOE_TRY(check_options(opt));
  MOE_TRY(check_paths(T, d, E, top_k, opt));
  Plan p;
  make_plan(T, d, ffn, E, top_k, opt, &p);
  MOE_TRY(p.plan_error);
  if (block_rows) *block_rows = p.bm;
  if (split_k) *split_k = p.split;
  if (fused_down) *fused_down = p.fused_down ? 1 : 0;
  return MOE_OK;
}

int moe_plan_ex(int T, int d, int ffn, int E, int top_k, const moe_options* opt,
                moe_plan_info* info) {
  MOE_TRY(check_sizes(T, d, ffn, E, top_k, true));
  MOE_TRY(check_options(opt));
  MOE_TRY(check_paths(T, d, E, top_k, opt));
  if (!info) return MOE_ERR_NULL;
  memset(info, 0, sizeof(*info));
  if (T == 0) return MOE_OK;
  Plan p;
  make_plan(T, d, ffn, E, top_k, opt, &p);
  MOE_TRY(p.plan_error);
  info->block_rows = p.bm;
  info->split_k = p.split;
  info->fused_down = p.fused_down ? 1 : 0;
  info->routing_launches = p.small_routing ? 1 : p.fused_reorder ? 2 : 3;
  info->gather_launch = p.gather_in_gemm ? 0 : 1;
  info->gate_up_variant = p.gu_variant;
  info->down_variant = p.fused_down ? -1 : p.dn_variant;
  info->unfused_swiglu = p.unfused ? 1 : 0;
  info->fold_combine = p.fold ? 1 : 0;
  info->xcd_grouped = p.gu_xcd ? 1 : 0;
  info->split_on_device = p.dyn_split ? 1 : 0;
  info->stream_k = p.gu_sk ? 1 : 0;
  info->variable_rows = p.gu_var;
  info->var_table_offset = p.gu_var ? (long long)p.o_vblocks : -1;
  info->var_count_offset = p.gu_var ? (long long)p.o_vnb : -1;
  info->launches = info->routing_launches + info->gather_launch + (p.unfused ? 3 : 1) +
                   (p.fused_down ? 0 : 1) + (p.fold ? 0 : 1);
  return MOE_OK;
}

int moe_route_workspace_size(int T, int E, int top_k, const moe_options* opt, size_t* bytes) {
  MOE_TRY(check_sizes(T, 0, 0, E, top_k, false));
  MOE_TRY(check_options(opt));
  MOE_TRY(check_paths(T, 0, E, top_k, opt));
  if (!bytes) return MOE_ERR_NULL;
  if (T == 0) {
    *bytes = 0;
    return MOE_OK;
  }
  Plan p;
  make_plan(T, 0, 0, E, top_k, opt, &p);
  *bytes = p.route_bytes;
  return MOE_OK;
}

int moe_forward_ex(const uint16_t* x, const float* router_logits, const uint16_t* W_gate_up,
                   const uint16_t* W_down, int top_k, int renormalize, uint16_t* out, int T, int d,
                   int ffn, int E, int score_func, const moe_options* opt, void* workspace,
                   size_t workspace_bytes, void* hip_stream) {
  MOE_TRY(check_sizes(T, d, ffn, E, top_k, true));
  MOE_TRY(check_options(opt));
  MOE_TRY(check_paths(T, d, E, top_k, opt));
  if (score_func != MOE_SCORE_SOFTMAX && score_func != MOE_SCORE_SIGMOID)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !router_logits || !W_gate_up || !W_down || !out || !workspace) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(router_logits, 16) || !aligned(W_gate_up, 16) ||
      !aligned(W_down, 16) || !aligned(out, 16) || !aligned(workspace, kAlign))
    return MOE_ERR_ALIGN;
  Plan p;
  make_plan(T, d, ffn, E, top_k, opt, &p);
  MOE_TRY(p.plan_error);
  if (workspace_bytes < p.total_bytes) return MOE_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  (void)hipGetLastError();  // report only this call's launches
  return forward_from_logits(x, LogitSrc{router_logits, 1, 0, nullptr}, W_gate_up, W_down, top_k,
                             renormalize ? 1 : 0, out, score_func, p, opt, workspace, s);
}

int moe_router_workspace_size(int T, int d, int E, size_t* bytes) {
  MOE_TRY(check_router_sizes(T, d, E));
  if (!bytes) return MOE_ERR_NULL;
  const RouterPlan rp = plan_router(T, d, E);
  *bytes = (T > 0 && rp.parts > 1) ? align_up((size_t)rp.parts * T * E * 4) : 0;
  return MOE_OK;
}

int moe_router_logits(const uint16_t* x, const uint16_t* W_router, float* logits, int T, int d,
                      int E, void* workspace, size_t workspace_bytes, void* hip_stream) {
  MOE_TRY(check_router_sizes(T, d, E));
  if (T == 0) return MOE_OK;
  if (!x || !W_router || !logits) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(W_router, 16) || !aligned(logits, 16)) return MOE_ERR_ALIGN;
  const RouterPlan rp = plan_router(T, d, E);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (rp.parts > 1) {
    if (!workspace) return MOE_ERR_NULL;
    if (!aligned(workspace, kAlign)) return MOE_ERR_ALIGN;
    if (workspace_bytes < (size_t)rp.parts * T * E * 4) return MOE_ERR_WORKSPACE;
  }
  (void)hipGetLastError();
  if (rp.parts == 1) {
    MOE_TRY_HIP(launch_router(x, W_router, T, d, E, rp, logits, s));
  } else {
    float* parts = static_cast<float*>(workspace);
    MOE_TRY_HIP(launch_router(x, W_router, T, d, E, rp, parts, s));
    MOE_TRY_HIP(launch_router_reduce(parts, rp.parts, (long long)T * E, logits, s));
  }
  return MOE_OK;
}

int moe_forward_router(const uint16_t* x, const uint16_t* W_router, const uint16_t* W_gate_up,
                       const uint16_t* W_down, int top_k, int renormalize, uint16_t* out,
                       float* logits_out, int T, int d, int ffn, int E, int score_func,
                       const moe_options* opt, void* workspace, size_t workspace_bytes,
                       void* hip_stream) {
  MOE_TRY(check_sizes(T, d, ffn, E, top_k, true));
  MOE_TRY(check_router_sizes(T, d, E));
  MOE_TRY(check_options(opt));
  MOE_TRY(check_paths(T, d, E, top_k, opt));
  if (score_func != MOE_SCORE_SOFTMAX && score_func != MOE_SCORE_SIGMOID)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !W_router || !W_gate_up || !W_down || !out || !workspace) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(W_router, 16) || !aligned(W_gate_up, 16) ||
      !aligned(W_down, 16) || !aligned(out, 16) || !aligned(workspace, kAlign) ||
      (logits_out && !aligned(logits_out, 16)))
    return MOE_ERR_ALIGN;
  Plan p;
  make_plan(T, d, ffn, E, top_k, opt, &p);
  MOE_TRY(p.plan_error);
  if (workspace_bytes < p.total_bytes) return MOE_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  (void)hipGetLastError();
  // One part: the router kernel writes the logits and routing reads them.
  // Several: it writes partial sums, which the routing kernel adds in part
  // order as it loads them (writing the sums to logits_out when given).
  LogitSrc src;
  if (p.router.parts == 1) {
    float* logits = logits_out ? logits_out : at<float>(workspace, p.o_logits);
    MOE_TRY_HIP(launch_router(x, W_router, T, d, E, p.router, logits, s));
    src = LogitSrc{logits, 1, 0, nullptr};
  } else {
    float* parts = at<float>(workspace, p.o_rparts);
    MOE_TRY_HIP(launch_router(x, W_router, T, d, E, p.router, parts, s));
    src = LogitSrc{parts, p.router.parts, (long long)T * E, logits_out};
  }
  return forward_from_logits(x, src, W_gate_up, W_down, top_k, renormalize ? 1 : 0, out,
                             score_func, p, opt, workspace, s);
}

int moe_forward(const uint16_t* x, const float* router_logits, const uint16_t* W_gate_up,
                const uint16_t* W_down, int top_k, int renormalize, uint16_t* out, int T, int d,
                int ffn, int E, int score_func, void* workspace, size_t workspace_bytes,
                void* hip_stream) {
  return moe_forward_ex(x, router_logits, W_gate_up, W_down, top_k, renormalize, out, T, d, ffn,
                        E, score_func, nullptr, workspace, workspace_bytes, hip_stream);
}

int moe_forward_static(const uint16_t* x, const float* router_logits, const uint16_t* W_gate_up,
                       const uint16_t* W_down, int top_k, int renormalize, uint16_t* out, int T,
                       int d, int ffn, int E, int score_func, void* hip_stream) {
  MOE_TRY(check_sizes(T, d, ffn, E, top_k, true));
  if (score_func != MOE_SCORE_SOFTMAX && score_func != MOE_SCORE_SIGMOID)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !router_logits || !W_gate_up || !W_down || !out) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(router_logits, 16) || !aligned(W_gate_up, 16) ||
      !aligned(W_down, 16) || !aligned(out, 16))
    return MOE_ERR_ALIGN;
  Plan p;
  make_plan(T, d, ffn, E, top_k, nullptr, &p);
  MOE_TRY(p.plan_error);
  if (p.total_bytes > (size_t)MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_STATIC_LIMIT;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  int device = -1;
  if (s ? hipStreamGetDevice(s, &device) != hipSuccess : hipGetDevice(&device) != hipSuccess)
    return MOE_ERR_HIP;
  void* ws = nullptr;
  MOE_TRY(static_workspace(device, &ws));
  (void)hipGetLastError();
  return forward_from_logits(x, LogitSrc{router_logits, 1, 0, nullptr}, W_gate_up, W_down, top_k,
                             renormalize ? 1 : 0, out, score_func, p, nullptr, ws, s);
}

int moe_route(const float* router_logits, int T, int E, int top_k, int renormalize,
              int score_func, const moe_options* opt, int32_t* topk_ids, float* topk_w,
              int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* blocks,
              int32_t* nb, int32_t* block_order, const uint16_t* x, int d, uint16_t* x_perm,
              int* bm_used, void* workspace, size_t workspace_bytes, void* hip_stream) {
  MOE_TRY(check_sizes(T, 0, 0, E, top_k, false));
  MOE_TRY(check_options(opt));
  MOE_TRY(check_paths(T, 0, E, top_k, opt));
  if (score_func != MOE_SCORE_SOFTMAX && score_func != MOE_SCORE_SIGMOID)
    return MOE_ERR_UNSUPPORTED;
  const bool gather = x && x_perm;
  if (gather && (d < 1)) return MOE_ERR_SHAPE;
  if (gather && d % 64 != 0) return MOE_ERR_ALIGN;
  Plan p;
  make_plan(T, 0, 0, E, top_k, opt, &p);
  if (bm_used) *bm_used = p.bm;
  if (T == 0) return MOE_OK;
  if (!router_logits || !workspace) return MOE_ERR_NULL;
  if (!aligned(router_logits, 16) || !aligned(workspace, kAlign)) return MOE_ERR_ALIGN;
  if (gather && (!aligned(x, 16) || !aligned(x_perm, 16))) return MOE_ERR_ALIGN;
  if (workspace_bytes < p.route_bytes) return MOE_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  (void)hipGetLastError();
  MOE_TRY(run_routing(LogitSrc{router_logits, 1, 0, nullptr}, p, renormalize ? 1 : 0, score_func,
                      workspace, opt, block_order ? at<int32_t>(workspace, p.o_order) : nullptr,
                      ZeroRange{nullptr, 0}, VarRows{nullptr, nullptr, 0, 0}, s));
  if (gather)
    MOE_TRY_HIP(launch_gather(x, at<int32_t>(workspace, p.o_perm), p.A, d, top_k, x_perm, s));
  MOE_TRY(record(opt, 3, s));
  const hipMemcpyKind dd = hipMemcpyDeviceToDevice;
  struct Copy {
    void* dst;
    size_t off, bytes;
  } copies[] = {
      {topk_ids, p.o_ids, (size_t)p.A * 4},          {topk_w, p.o_w, (size_t)p.A * 4},
      {counts, p.o_counts, (size_t)E * 4},           {offsets, p.o_offsets, (size_t)(E + 1) * 4},
      {perm, p.o_perm, (size_t)p.A * 4},             {inv, p.o_inv, (size_t)p.A * 4},
      {blocks, p.o_blocks, (size_t)p.nb_max * 2 * 4}, {nb, p.o_nb, 4},
      {block_order, p.o_order, (size_t)p.nb_max * 4},
  };
  for (const Copy& c : copies)
    if (c.dst) MOE_TRY_HIP(hipMemcpyAsync(c.dst, at<char>(workspace, c.off), c.bytes, dd, s));
  return MOE_OK;
}

int moe_timer_create(void** event) {
  if (!event) return MOE_ERR_NULL;
  hipEvent_t ev = nullptr;
  // Timing only: no system-scope fence (no L2 write-back) when recorded.
  if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess) return MOE_ERR_HIP;
  *event = ev;
  return MOE_OK;
}

int moe_timer_record(void* event, void* hip_stream) {
  if (!event) return MOE_ERR_NULL;
  return hipEventRecord(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(hip_stream)) ==
                 hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

int moe_timer_destroy(void* event) {
  if (!event) return MOE_ERR_NULL;
  return hipEventDestroy(static_cast<hipEvent_t>(event)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_timer_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return MOE_ERR_NULL;
  if (hipEventSynchronize(static_cast<hipEvent_t>(stop)) != hipSuccess) return MOE_ERR_HIP;
  return hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) ==
                 hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

}  // extern "C"
