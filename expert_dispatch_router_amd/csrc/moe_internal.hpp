// moe_internal.hpp -- shared definitions of the HIP library's translation
// units (device types, workspace plan, kernel launchers).  Internal: not part
// of the C ABI in include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Vector types of the gfx950 bf16 matrix instructions and 16-byte moves.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Router scores as the routing kernels read them: `nparts` fp32 partial
// sums [nparts][T][E], `part_stride` elements apart, added in part order
// (one part: the logits themselves).  When `out` is not null the summed
// logits are also written there ([T][E]).
struct LogitSrc {
  const float* p;
  int nparts;
  long long part_stride;
  float* out;
};

__device__ __forceinline__ float load_logit(const LogitSrc& s, size_t idx) {
  float v = s.p[idx];
  for (int q = 1; q < s.nparts; ++q) v += s.p[(size_t)q * s.part_stride + idx];
  if (s.out) s.out[idx] = v;
  return v;
}

// Flat routed rows handled by one reorder chunk; the histogram kernel keeps
// one count per (chunk, expert) so the reorder can start every chunk at its
// final position without a global sort.
constexpr int kChunk = 1024;

// Launch shape of the router scores kernel (see router.hip).
struct RouterPlan {
  int ts;     // 16-token subtiles per wave (1, 2 or 4)
  int nsub;   // 16-expert subtiles per wave (1, 2 or 4)
  int parts;  // split of the reduction over d (partial sums added in order)
  int lds;    // 1: the LDS-staged GEMM tile (launch_router_lds), ksplit d per part
  int ksplit;
};
RouterPlan plan_router(int T, int d, int E);

// Host-side plan of one call: sizes, tile choices and workspace carve-up.
struct Plan {
  RouterPlan router;
  int T, d, ffn, E, k;
  int A;          // routed rows T*k
  int bm;         // rows per schedule block (BLOCK_M)
  int nb_max;     // upper bound of the block count: ceil(A/bm) + min(E, A)
  int nchunks;    // ceil(A / kChunk)
  int split;      // split of the down projection's reduction
  int ksplit;     // reduction length of one split (multiple of 64)
  int gu_variant; // tile variant of the fused gate/up GEMM
  int dn_variant; // tile variant of the down GEMM
  int gu_rotate;  // rotate the K-step start per workgroup (fused gate/up GEMM)
  int gu_xcd, dn_xcd;  // group each block's workgroups on one XCD (see the GEMM kernel)
  int longest_first;   // else launch the blocks longest first (device-built order)
  int dn_rotate;  // same for the down GEMM
  int small_routing;  // one-workgroup routing kernel instead of three launches
  int fused_reorder;  // two launches: the histogram kernel also does the reorder
  int gather_in_gemm; // the fused gate/up GEMM reads token rows through perm
  int x_tiled;        // else x_perm is written in K-step tiles (gather mode 3)
  int unfused;        // SwiGLU as gate GEMM, up GEMM and activation (ablation)
  int fold;           // weighted combination in the down GEMM's epilogue
  int dn_tiles;       // column tiles of the down GEMM (d / its tile width)
  int fused_down;     // gate/up GEMM also does the down projection (split = its column tiles)
  int dyn_split;      // the down GEMM and the combination take the parts from the device
                      // (device_down_split, at most `split`)
  int gu_sk;          // the gate/up GEMM runs the stream-K schedule (launch_gate_up_sk)
  int sk_units;       // its counters: nb_max * column tiles
  int gu_var;         // the gate/up GEMM runs over the variable-size block table
                      // (launch_gate_up_var), built with VarRows mode gu_var
  int plan_error;     // an explicit option the plan cannot honour (MOE_ERR_*), else 0
  // byte offsets into the workspace (256-byte aligned)
  size_t o_ids, o_w, o_counts, o_offsets, o_ccnt, o_cbase, o_perm, o_inv, o_blocks, o_nb;
  size_t o_order;  // longest-first launch order of the blocks [nb_max]
  size_t o_vblocks, o_vnb;  // the variable-size block table [nb_max, 3] and its count
  size_t route_bytes;  // end of the routing section
  size_t o_xperm, o_h, o_y;
  size_t o_g, o_u;  // unfused gate and up products [A, ffn] bf16
  size_t o_logits;  // router scores [T, E] fp32 (moe_forward_router)
  size_t o_rparts;  // router partial sums [router.parts, T, E] fp32
  size_t o_fold;    // arrival counters of the folded combination [T, dn_tiles] int32,
                    // then the stream-K unit counters [sk_units] int32 (one cleared range)
  size_t o_skpart;  // stream-K partial sums [2 * kRoundWorkgroups slots]
  size_t total_bytes;
};

// Parts of the down projection's reduction in one call, decided on the
// device from the routed block count nb (the host sizes the partials buffer
// for split_max parts but cannot see the counts: under skewed routing far
// fewer blocks exist than its estimate assumes).  parts is the split whose
// workgroup count nb * n_tiles * parts is nearest to one round of
// kRoundWorkgroups, at least 1 and at most split_max; ksplit is the
// reduction length of one part (a multiple of 64), and every part has at
// least one 64-wide step.  The down GEMM and the combination both call it,
// so they agree on the parts.
constexpr int kRoundWorkgroups = 256;  // one workgroup per CU
struct DownSplit {
  int parts;
  int ksplit;
};
__host__ __device__ inline DownSplit device_down_split(int nb, int n_tiles, int split_max, int K) {
  const int wg = nb * n_tiles > 0 ? nb * n_tiles : 1;
  int s = (2 * kRoundWorkgroups + wg) / (2 * wg);  // round(kRoundWorkgroups / wg)
  s = s < 1 ? 1 : (s > split_max ? split_max : s);
  const int ksteps = K / 64;
  const int per = (ksteps + s - 1) / s;
  return DownSplit{(ksteps + per - 1) / per, per * 64};
}

// ---- launchers (enqueue on `s`, return the launch status) ----------------

// Router scores x . W_r^T (bf16 in, fp32 out): with rp.parts == 1 the
// logits [T, E] into `out`, else rp.parts partial sums [parts, T, E].
hipError_t launch_router(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                         const RouterPlan& rp, float* out, hipStream_t s);
// Router score parts [parts, T, E] by the LDS-staged GEMM tile (E % 16 == 0;
// part p sums d in [p * ksplit, (p + 1) * ksplit), ksplit a multiple of 64).
hipError_t launch_router_lds(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                             int parts, int ksplit, float* out, hipStream_t s);
// logits = the partial sums added in part order.
hipError_t launch_router_reduce(const float* parts, int nparts, long long n, float* logits,
                                hipStream_t s);

// An int32 range the routing kernels set to zero (p may be null): the
// arrival counters of the folded combination, cleared before the GEMMs run.
struct ZeroRange {
  int32_t* p;
  int n;
};

hipError_t launch_route(const LogitSrc& logits, int T, int E, int k, int renorm, int score,
                        int32_t* ids, float* w, ZeroRange zero, hipStream_t s);

// The gate/up GEMM's table of variable-size blocks, built by the routing
// kernels beside the fixed table (blocks null: not built): each expert
// with more than bm rows cut into blocks of 2 * bm rows and a last block of
// the rest, the others into blocks of bm rows as in the fixed table.  mode
// 1 merges when the fixed table needs more than one round of
// kRoundWorkgroups workgroups at `tiles` column tiles per block and the
// merged one needs at most one round; mode 2 always merges.  blocks [*, 3]
// = (expert, first row, rows) and nb[0] = their count when the table
// merges; else nb[0] = -1 and the table is not written (the GEMM takes the
// fixed table).
struct VarRows {
  int32_t* blocks;
  int32_t* nb;
  int mode;
  int tiles;
};
constexpr int kVarRowsAuto = 1;
constexpr int kVarRowsAlways = 2;

// Histogram, offsets and the block table; with `order` (may be null) also
// the longest-first launch order of the blocks (a stable sort by decreasing
// rows: the full blocks in block order, then the partial last blocks).
hipError_t launch_hist_scan(const int32_t* ids, int A, int E, int bm, int nchunks,
                            int32_t* counts, int32_t* offsets, int32_t* chunk_cnt,
                            int32_t* chunk_base, int32_t* blocks, int32_t* nb, int32_t* order,
                            int32_t* perm, int32_t* inv, VarRows var, hipStream_t s);
// Whether the histogram kernel can also do the reorder (perm, inv non-null):
// its per-64-row-group counts of every expert fit in LDS.
bool fused_reorder_fits(int A, int E);

hipError_t launch_permute(const int32_t* ids, int A, int E, int nchunks, const int32_t* offsets,
                          const int32_t* chunk_cnt, const int32_t* chunk_base, int32_t* perm,
                          int32_t* inv, hipStream_t s);

// Whole routing (route + histogram/scan/schedule + reorder) in one
// workgroup of 1024 threads, one token per thread.
constexpr int kSmallRoutingMaxTokens = 1024;
constexpr int kSmallRoutingMaxExperts = 64;
// The automatic choice also bounds T*E*k and E: the kernel's top-k runs on
// one CU (measured faster than the three launches at E = 8; at E = 64 slower
// than the two launches, pass us: skewed T=128/512 79.2 -> 90.9, 127.4 ->
// 144.6; Qwen2 T=128 576.5 -> 601.4).
constexpr long long kSmallRoutingAutoWork = 1 << 15;
constexpr int kSmallRoutingAutoMaxExperts = 32;
bool small_routing_fits(int T, int E, int k);
hipError_t launch_route_dispatch_small(const LogitSrc& logits, int T, int E, int k, int renorm,
                                       int score, int bm, int32_t* ids, float* w,
                                       int32_t* counts, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, int32_t* blocks, int32_t* nb,
                                       int32_t* order, ZeroRange zero, VarRows var,
                                       hipStream_t s);

hipError_t launch_gather(const uint16_t* x, const int32_t* perm, int A, int d, int k,
                         uint16_t* x_perm, hipStream_t s);

// x_perm in K-step tiles ([ceil(A/16)] groups x [d/64] steps x 16 rows x 64
// columns), the layout the GEMM reads with x_tiled.
hipError_t launch_gather_tiled(const uint16_t* x, const int32_t* perm, int A, int d, int k,
                               uint16_t* x_t, hipStream_t s);

// Fused gate/up SwiGLU grouped GEMM: h[A, F] = silu(X Wg^T) * (X Wu^T) per
// block.  X is x_perm [A, d] when gather_perm is null, else the token rows
// x [T, d] read through gather_perm (row p is x[gather_perm[p] / k]).
//
// Every GEMM launcher takes `order`: null = workgroups take the blocks in
// block order, else in the order listed there (longest first).
hipError_t launch_gate_up(int bm, int variant, const uint16_t* x, const int32_t* gather_perm,
                          int k, int T, const uint16_t* w_gate_up, const int32_t* blocks,
                          const int32_t* nb, const int32_t* order, const int32_t* offsets,
                          uint16_t* h, int A, int d,
                          int ffn, int nb_max, int rotate, int xcd_group, int x_tiled,
                          hipStream_t s);

// One projection of the unfused SwiGLU: out[A, ffn] = bf16(X w[e]^T) per
// block, w[e] = w + e * w_estride elements (ffn rows of d); X as for
// launch_gate_up.
hipError_t launch_proj_bf16(int bm, const uint16_t* x, const int32_t* gather_perm, int k, int T,
                            const uint16_t* w, long long w_estride, const int32_t* blocks,
                            const int32_t* nb, const int32_t* order, const int32_t* offsets,
                            uint16_t* out, int A, int d,
                            int ffn, int nb_max, int rotate, int xcd_group, int x_tiled,
                            hipStream_t s);

// h = bf16(silu(g) * u) over n elements (n % 8 == 0).
hipError_t launch_swiglu_act(const uint16_t* g, const uint16_t* u, uint16_t* h, long long n,
                             hipStream_t s);

// The weighted combination folded into the down GEMM (cnt null: not
// folded).  cnt [T, tiles] counts the partials written for each (token,
// column tile) and must be zero when the GEMM starts; the workgroup that
// writes the last of a token's k * split partials of a tile writes that
// token's output columns of the tile.
struct FoldCombine {
  const int32_t* perm;
  const int32_t* inv;
  const float* w;
  int k;
  int32_t* cnt;
  uint16_t* out;
};

// The fused gate/up GEMM on the stream-K schedule: kRoundWorkgroups
// persistent workgroups share the nb * ceil(ffn / tile) * (d / 64) K steps of
// all units evenly (see gemm_lds_sk_kernel).  part holds 2 * kRoundWorkgroups
// slots of gate_up_sk_slot_bytes; cnt [nb_max * ceil(ffn / tile)] must be
// zero when it starts.  Same arguments otherwise as launch_gate_up (row-major
// activations only: x_tiled is not supported).
size_t gate_up_sk_slot_bytes(int bm, int variant);  // 0: not compiled
hipError_t launch_gate_up_sk(int bm, int variant, const uint16_t* x, const int32_t* gather_perm,
                             int k, int T, const uint16_t* w_gate_up, const int32_t* blocks,
                             const int32_t* nb, const int32_t* offsets, uint16_t* h, int d,
                             int ffn, int rotate, float* part, int32_t* cnt, hipStream_t s);

// The fused gate/up GEMM over the variable-size block table (VarRows, bm
// 128), or over the fixed table (blocks, nb, offsets) when the routing
// kernels did not merge: blocks of up to 128 rows take the narrow
// LDS-staged tile, blocks of up to 256 rows the same tile at 256 rows, in
// one launch of nb_max * ceil(ffn / 128) workgroups (those past the table's
// count return at once).  Row-major activations only.
hipError_t launch_gate_up_var(const uint16_t* x, const int32_t* gather_perm, int k, int T,
                              const uint16_t* w_gate_up, const int32_t* vblocks,
                              const int32_t* vnb, const int32_t* blocks, const int32_t* nb,
                              const int32_t* offsets, uint16_t* h, int d, int ffn, int nb_max,
                              int rotate, hipStream_t s);

// Fused gate/up SwiGLU and down projection for small problems: each
// (block, column tile) workgroup keeps its h tile in LDS and writes
// y[tile, A, d] = h[:, tile cols] Wd[:, tile cols]^T (fp32, one part per
// column tile of gate_up_down_tile_cols columns), so no h buffer and no down
// GEMM launch; the combination adds the parts in tile order.
int gate_up_down_tile_cols(int bm, int variant);  // 0: not compiled
hipError_t launch_gate_up_down(int bm, int variant, const uint16_t* x, const int32_t* gather_perm,
                               int k, int T, const uint16_t* w_gate_up, const uint16_t* w_down,
                               const int32_t* blocks, const int32_t* nb, const int32_t* order,
                               const int32_t* offsets, float* y, int A, int d, int ffn,
                               int nb_max, int rotate, int xcd_group, int x_tiled,
                               hipStream_t s);

// Down grouped GEMM: y[split, A, d] = partial sums of h Wd^T per block, and
// with fold.cnt the weighted combination into fold.out.
// With dyn_split the launch covers split parts at most and the kernel uses
// device_down_split's parts (not with fold).
hipError_t launch_down(int bm, int variant, const uint16_t* h, const uint16_t* w_down,
                       const int32_t* blocks, const int32_t* nb, const int32_t* order,
                       const int32_t* offsets, float* y,
                       int A, int d, int ffn, int split, int ksplit, int nb_max, int rotate,
                       int xcd_group, const FoldCombine& fold, hipStream_t s, int dyn_split = 0);

// Weighted combination: out[t] = bf16(sum_j w[t,j] * sum_s y[s, inv[t*k+j]]).
// With dyn (non-null nb) the parts are device_down_split(*nb, dn_tiles,
// split, ffn).parts, as in the down GEMM of the same call.
struct DynSplit {
  const int32_t* nb;
  int dn_tiles;
  int ffn;
};
hipError_t launch_combine(const float* y, int split, int A, int d, const int32_t* inv,
                          const float* w, int k, int T, uint16_t* out, hipStream_t s,
                          DynSplit dyn = DynSplit{nullptr, 0, 0});

// Column tile widths (output columns per workgroup) of the two GEMMs for a
// block size; the planner uses them to size the grids.
int gate_up_tile_cols(int bm, int variant);
// Tile variant of the fused gate/up GEMM at BM = 192 that stages its weights in LDS
// (7 waves x 32 columns).
constexpr int kGateUpLdsVariant = 2;
// Tile variant of the fused gate/up GEMM at BM = 128 that stages its weights in LDS with
// one 16-column subtile per wave (8 waves x 16 columns) and three stages.
constexpr int kGateUpLdsNarrowVariant = 3;
// Tile variant of the down GEMM at BM = 192 that stages its weights in LDS (8 waves x 32
// columns).
constexpr int kDownLdsVariant = 2;
// Tile variant of the down GEMM at BM = 128 and 192 that stages its weights in LDS with 64
// columns per wave (8 waves, 512 columns at BM = 128; 7 waves, 448 at BM = 192).
constexpr int kDownLdsWideVariant = 3;
// The wide tile with 7 waves at BM = 128 (448 columns).
constexpr int kDownLdsWide7Variant = 4;
int down_tile_cols(int bm, int variant);

}  // namespace moe
