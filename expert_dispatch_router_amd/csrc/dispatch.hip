// dispatch.hip -- K2: expert histogram, LDS prefix scan and block schedule;
//                 K3: stable reorder of the routed rows and the row gather.
//
// [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in Triton".
// Tokens are reordered onto experts ("The reading"; abstract: token
// permutation) and fixed-size blocks of rows are mapped to (expert,
// token-offset) pairs (Algorithm 1, "What carries the argument"; BLOCK_M is
// fixed for one launch, "Assumptions & free parameters").  On the page the
// schedule is built on the host (Limitations (5) in the "Referee Report");
// here it is built on the device so the forward pass never waits for a
// device-to-host copy.
//
// Readings: rows of one expert keep ascending flat index i = t*k + j, which
// makes the reorder unique and deterministic; a block never spans two
// experts; an expert with no rows gets no block; the token-offset of a block
// is its first sorted row.
#include <type_traits>

#include "moe_internal.hpp"
#include "route_core.hpp"
#include "../../include/moe.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kAllChunkCounts = 16384;  // int counters of all (chunk, expert) pairs in LDS
static_assert(kScanThreads == kChunk, "one thread per row of a chunk");
static_assert(MOE_MAX_EXPERTS <= kScanThreads, "one thread per expert in the scans");

// Inclusive scan of v over the first MOE_MAX_EXPERTS threads; threads
// beyond contribute nothing and get 0.  Each wave scans its 64 values in
// registers (shuffles), the wave totals go through LDS (sh, at least
// MOE_MAX_EXPERTS / 64 ints): two barriers, the last one at the end.
// *total receives the sum of all values.
constexpr int kScanWaves = MOE_MAX_EXPERTS / 64;
__device__ int block_inclusive_scan(int v, int* sh, int* total = nullptr) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int x = tid < MOE_MAX_EXPERTS ? v : 0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63 && wave < kScanWaves) sh[wave] = x;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int q = 0; q < kScanWaves; ++q) {
    const int t = sh[q];
    base += q < wave ? t : 0;
    all += t;
  }
  if (total) *total = all;
  __syncthreads();  // sh is free again
  return tid < MOE_MAX_EXPERTS ? x + base : 0;
}

// block_inclusive_scan of two values at once (the same two barriers; sh
// holds at least 2 * kScanWaves ints): a and b are replaced by their
// inclusive scans, ta and tb receive the totals.
__device__ void block_inclusive_scan2(int& a, int& b, int* sh, int& ta, int& tb) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int x = tid < MOE_MAX_EXPERTS ? a : 0;
  int y = tid < MOE_MAX_EXPERTS ? b : 0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int xs = __shfl_up(x, off, 64);
    const int ys = __shfl_up(y, off, 64);
    if (lane >= off) {
      x += xs;
      y += ys;
    }
  }
  if (lane == 63 && wave < kScanWaves) {
    sh[wave] = x;
    sh[kScanWaves + wave] = y;
  }
  __syncthreads();
  int bx = 0, by = 0, ax = 0, ay = 0;
#pragma unroll
  for (int q = 0; q < kScanWaves; ++q) {
    const int tx = sh[q], ty = sh[kScanWaves + q];
    bx += q < wave ? tx : 0;
    by += q < wave ? ty : 0;
    ax += tx;
    ay += ty;
  }
  ta = ax;
  tb = ay;
  __syncthreads();  // sh is free again
  a = tid < MOE_MAX_EXPERTS ? x + bx : 0;
  b = tid < MOE_MAX_EXPERTS ? y + by : 0;
}

// Whether the variable-size table merges (see VarRows): nb_fixed and
// nb_merged are the block counts of the two cuttings.
__device__ __forceinline__ bool var_rows_merge(const VarRows& var, int nb_fixed, int nb_merged) {
  if (var.mode == kVarRowsAlways) return true;
  return (long long)nb_fixed * var.tiles > kRoundWorkgroups &&
         (long long)nb_merged * var.tiles <= kRoundWorkgroups;
}

// n blocks of expert e from table entry b0: `size` rows each from row0, the
// last holding the rest of the expert's cnt rows.
__device__ __forceinline__ void write_var_blocks(int32_t* vb, int b0, int n, int e, int row0,
                                                 int cnt, int size) {
  for (int r = 0; r < n; ++r) {
    vb[3 * (b0 + r)] = e;
    vb[3 * (b0 + r) + 1] = row0 + r * size;
    vb[3 * (b0 + r) + 2] = min(size, cnt - r * size);
  }
}

// One workgroup.  Per chunk c of kChunk flat rows: count each expert in LDS,
// record the count and the number of earlier rows of that expert.  Then the
// expert totals, their exclusive prefix (offsets), the number of blocks of
// each expert, their prefix, and the block table.  With `order`, also the
// longest-first launch order of the blocks: the full blocks in block order,
// then each expert's partial last block by rows descending, ties to the
// lower expert -- a stable sort of the blocks by decreasing row count.
// With `perm` (fused_reorder_fits), also the reorder: the counts are then
// kept per 64-row group in LDS instead of per chunk in memory, and each
// wave places the rows of its groups: the lanes of a group OR their bits
// into a per-expert mask in LDS, so each row lands at offsets[e] + (rows of
// e in earlier groups) + (lanes below it holding e) -- ascending flat order
// within the expert.
__global__ __launch_bounds__(kScanThreads) void hist_scan_kernel(
    const int32_t* __restrict__ ids, int A, int E, int bm, int nchunks,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ blocks, int32_t* __restrict__ nb,
    int32_t* __restrict__ order, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    VarRows var) {
  __shared__ int hist[MOE_MAX_EXPERTS];
  __shared__ int run[MOE_MAX_EXPERTS];
  __shared__ int sh[MOE_MAX_EXPERTS];
  __shared__ int chist[kAllChunkCounts];  // [chunk][expert], when they all fit
  // fused reorder: per wave and expert, the lanes of the current group that
  // hold the expert
  __shared__ unsigned long long lanes_of[(kScanThreads / 64) * MOE_MAX_EXPERTS];
  __shared__ int part[kScanThreads];  // fused reorder: slice totals of the group scan
  const int tid = threadIdx.x;
  const bool fused = perm != nullptr;  // uniform
  const int ngroups = fused ? (A + 63) >> 6 : nchunks;
  if (tid < E) run[tid] = 0;
  if (ngroups * E <= kAllChunkCounts) {  // uniform
    // every chunk's (group's) counts in one pass over the rows, then a scan
    // over the chunks per expert: no barrier per chunk
    for (int q = tid; q < ngroups * E; q += kScanThreads) chist[q] = 0;
    __syncthreads();
    for (int i = tid; i < A; i += kScanThreads)
      atomicAdd(&chist[(fused ? i >> 6 : i / kChunk) * E + ids[i]], 1);
    __syncthreads();
    if (fused) {
      // per expert, the exclusive prefix over the groups in two levels: S
      // slices of the groups per expert (thread e + E * s), each slice's
      // total, then each slice's base -- the same sums as one serial pass
      const int S = min(kScanThreads / E, ngroups);
      const int e = tid % E, sl = tid / E;
      const int g0 = sl * ngroups / S, g1 = (sl + 1) * ngroups / S;
      if (sl < S) {
        int r = 0;
        for (int c = g0; c < g1; ++c) r += chist[c * E + e];
        part[sl * E + e] = r;
      }
      __syncthreads();
      if (sl < S) {
        int r = 0;
        for (int q = 0; q < sl; ++q) r += part[q * E + e];
        for (int c = g0; c < g1; ++c) {
          const int h = chist[c * E + e];
          chist[c * E + e] = r;  // rows of this expert in earlier groups
          r += h;
        }
        if (sl == S - 1) run[e] = r;
      }
    } else if (tid < E) {
      int r = 0;
      for (int c = 0; c < ngroups; ++c) {
        const int h = chist[c * E + tid];
        chunk_cnt[(size_t)c * E + tid] = h;
        chunk_base[(size_t)c * E + tid] = r;
        r += h;
      }
      run[tid] = r;
    }
    __syncthreads();
  } else {
    for (int c = 0; c < nchunks; ++c) {
      if (tid < E) hist[tid] = 0;
      __syncthreads();
      const int i = c * kChunk + tid;
      if (i < A) atomicAdd(&hist[ids[i]], 1);
      __syncthreads();
      if (tid < E) {
        chunk_cnt[(size_t)c * E + tid] = hist[tid];
        chunk_base[(size_t)c * E + tid] = run[tid];
        run[tid] += hist[tid];
      }
      __syncthreads();
    }
  }
  const int cnt = tid < E ? run[tid] : 0;
  const int incl = block_inclusive_scan(cnt, sh);
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid + 1] = incl;
  }
  if (tid == 0) offsets[0] = 0;
  const int row0 = incl - cnt;
  const int nbk = (cnt + bm - 1) / bm;
  // blocks of the variable-size table's merged cutting (see VarRows)
  const int vbk = cnt > bm ? (cnt + 2 * bm - 1) / (2 * bm) : nbk;
  int bincl = nbk, vincl = vbk, btotal, vtotal;
  block_inclusive_scan2(bincl, vincl, sh, btotal, vtotal);
  if (tid < E) {
    const int b0 = bincl - nbk;
    for (int r = 0; r < nbk; ++r) {
      blocks[2 * (b0 + r)] = tid;
      blocks[2 * (b0 + r) + 1] = row0 + r * bm;
    }
  }
  if (tid == E - 1) nb[0] = bincl;
  if (var.blocks) {  // uniform
    const bool merge = var_rows_merge(var, btotal, vtotal);
    if (merge && tid < E)
      write_var_blocks(var.blocks, vincl - vbk, vbk, tid, row0, cnt, cnt > bm ? 2 * bm : bm);
    if (tid == 0) var.nb[0] = merge ? vtotal : -1;
  }
  if (order) {  // uniform
    const int nfull = cnt / bm;
    const int rem = cnt - nfull * bm;
    int ftotal;
    const int fincl = block_inclusive_scan(nfull, sh, &ftotal);
    if (tid < E) {
      const int b0 = bincl - nbk;
      for (int r = 0; r < nfull; ++r) order[fincl - nfull + r] = b0 + r;
      hist[tid] = rem;
    }
    __syncthreads();
    if (tid < E && rem > 0) {
      int rank = 0;
      for (int e = 0; e < E; ++e) {
        const int q = hist[e];
        rank += (q > rem) || (q == rem && e < tid);
      }
      order[ftotal + rank] = bincl - 1;
    }
  }
  if (fused) {  // uniform
    if (tid < E) run[tid] = row0;  // free: cnt was read before the scans
    __syncthreads();
    const int lane = tid & 63;
    const unsigned long long below = (1ull << lane) - 1ull;
    unsigned long long* wm = lanes_of + (tid >> 6) * E;  // this wave's masks, one per expert
    for (int e = lane; e < E; e += 64) wm[e] = 0ull;
    constexpr int kWaves = kScanThreads / 64;
    constexpr int kAhead = 4;  // groups whose ids one wave loads at once
    for (int g0 = tid >> 6; g0 < ngroups; g0 += kAhead * kWaves) {
      int ev[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        const int i = (g0 + u * kWaves) * 64 + lane;
        ev[u] = i < A ? ids[i] : 0;
      }
      int pos[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        const int g = g0 + u * kWaves;
        const int i = g * 64 + lane;
        const int e = ev[u];
        // the lanes of the group that hold each expert: OR is order-free, and
        // a wave's LDS operations complete in program order.  Every access to
        // the masks is atomic and any two may touch the same mask, so the
        // compiler keeps their order (a fence or a memory-clobbering asm
        // statement here would make it wait for every store in flight)
        pos[u] = 0;
        if (i < A) {
          atomicOr(&wm[e], 1ull << lane);
          const unsigned long long m =
              __hip_atomic_load(&wm[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
          pos[u] = run[e] + chist[g * E + e] + __popcll(m & below);
          // every lane that read it has read it
          __hip_atomic_store(&wm[e], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        }
      }
      // the stores after all the groups' LDS work: a store's registers are
      // not reused while it is in flight, so nothing waits for it
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        const int i = (g0 + u * kWaves) * 64 + lane;
        if (i < A) {
          perm[pos[u]] = i;
          inv[i] = pos[u];
        }
      }
    }
  }
}

// One wave per (chunk, expert).  The wave walks its chunk in order, 64 rows
// at a time; a ballot of "row goes to my expert" ranks the matching lanes,
// so rows land at consecutive sorted positions in ascending flat order.
__global__ __launch_bounds__(256) void permute_kernel(
    const int32_t* __restrict__ ids, int A, int E, int nchunks, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ chunk_cnt, const int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= E * nchunks) return;
  const int c = gw / E;
  const int e = gw - c * E;
  const int cnt = chunk_cnt[(size_t)c * E + e];
  if (cnt == 0) return;
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  int pos = offsets[e] + chunk_base[(size_t)c * E + e];
  const int end = pos + cnt;
  const int i0 = c * kChunk;
  for (int it = 0; it < kChunk / 64 && pos < end; ++it) {
    const int i = i0 + it * 64 + lane;
    const bool hit = i < A && ids[i] == e;
    const unsigned long long mask = __ballot(hit);
    if (hit) {
      const int p = pos + __popcll(mask & below);
      perm[p] = i;
      inv[i] = p;
    }
    pos += __popcll(mask);
  }
}

// x_perm[p] = x[perm[p] / k]: one workgroup per sorted row, 16-byte moves.
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ x,
                                                     const int32_t* __restrict__ perm, int d, int k,
                                                     uint16_t* __restrict__ x_perm) {
  const int p = blockIdx.x;
  const int src = perm[p] / k;
  const uint4* s = reinterpret_cast<const uint4*>(x + (size_t)src * d);
  uint4* o = reinterpret_cast<uint4*>(x_perm + (size_t)p * d);
  for (int c = threadIdx.x; c < d / 8; c += 256) o[c] = s[c];
}

// Tiled gather for the GEMM's activation loads: sorted row p of x_perm is
// x[perm[p] / k], stored in K-step tiles -- the 64 columns [64 s, 64 s + 64)
// of the 16 rows of group G = p / 16 are 2 KiB at (G * d/64 + s) * 2048,
// row p % 16 at +128 * (p % 16).  One step of a block then reads whole
// 2 KiB pieces instead of 128 bytes from rows 2*d bytes apart (which, for
// power-of-two d, all fall on the same memory channel).
__global__ __launch_bounds__(256) void gather_tiled_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ perm, int d,
                                                           int k, uint16_t* __restrict__ x_t) {
  const int p = blockIdx.x;
  const int src = perm[p] / k;
  const uint4* s = reinterpret_cast<const uint4*>(x + (size_t)src * d);
  const size_t g0 = (size_t)(p >> 4) * (d / 64) * 1024 + (p & 15) * 64;  // elements
  for (int c = threadIdx.x; c < d / 8; c += 256) {
    const int col = c * 8;
    *reinterpret_cast<uint4*>(x_t + g0 + (size_t)(col >> 6) * 1024 + (col & 63)) = s[c];
  }
}

// Small problems (T <= 1024 tokens, E <= 64 experts; automatic up to 32):
// the whole routing in one workgroup of 1024 threads, thread t = token t.
// Three launches (route, histogram+scan+schedule, reorder) cost more than
// this work.
//   1. route: up to 32 experts (LPT = 1), the token's E logits in registers,
//      k rounds of "best live candidate" in ascending expert order under the
//      same rank rule as the lane-group route (so the same experts, in the
//      same order); beyond, groups of LPT lanes per token run the lane-group
//      route itself and pass the k experts to thread t through LDS;
//   2. count: per expert and wave, the mask of lanes whose token chose e
//      (a ballot per expert, or with lane groups k LDS ORs per token); the
//      masks and their popcounts go to LDS;
//   3. one exclusive scan over the (expert, wave) counts in expert-major
//      order gives, for every wave, where its rows of expert e start; a
//      token has at most one row per expert, so ascending token order within
//      an expert is ascending flat index i = t*k + j, and a row's position is
//      that start plus the rank of its lane in the wave's mask;
//   4. counts, offsets, the block table and the block count.
// Identical results to the general path.
constexpr int kSmallWaves = kScanThreads / 64;

template <int EMAX, int LPT>
__global__ __launch_bounds__(kScanThreads) void route_dispatch_small_kernel(
    const LogitSrc logits, int T, int E, int k, int renorm, int score, int bm,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ blocks, int32_t* __restrict__ nb, int32_t* __restrict__ order,
    ZeroRange zero, VarRows var) {
  static_assert(EMAX <= 64 && EMAX * kSmallWaves <= kScanThreads, "one thread per (e, wave)");
  using Mask = typename std::conditional<(EMAX > 32), unsigned long long, unsigned>::type;
  constexpr int kMaskBits = 8 * sizeof(Mask);
  __shared__ unsigned long long wmask[EMAX * kSmallWaves];  // [e][wave] ballot of expert e
  __shared__ int start[EMAX * kSmallWaves];                 // [e][wave] first sorted position
  __shared__ int wave_sum[kSmallWaves];
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const bool ok = t < T;
  for (int i = t; i < zero.n; i += kScanThreads) zero.p[i] = 0;

  // 1. route
  int sel_e[MOE_MAX_TOPK];
  Mask chosen = 0;  // one thread per token: the token's experts as bits
  if constexpr (LPT == 1) {
    float v[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) v[e] = (ok && e < E) ? load_logit(logits, (size_t)t * E + e) : 0.0f;
    const Mask valid = ok ? (E >= kMaskBits ? ~Mask(0) : (Mask(1) << E) - Mask(1)) : Mask(0);
    Mask live = valid;
    float sel_v[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      sel_v[j] = 0.0f;
      sel_e[j] = -1;
    }
    // k rounds: a round past k (uniform over the launch) is skipped, not
    // computed and discarded (the empty volatile asm keeps the compiler from
    // speculating it)
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j < k) {
        asm volatile("");
        float bv = 0.0f;
        int be = -1;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
          if (((live >> e) & Mask(1)) && ranks_before(v[e], e, bv, be)) {
            bv = v[e];
            be = e;
          }
        if (be >= 0) live &= ~(Mask(1) << be);
        sel_v[j] = bv;
        sel_e[j] = be;
      }
    float z_all = 0.0f;
    if (score == MOE_SCORE_SOFTMAX && !renorm) {
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if ((valid >> e) & Mask(1)) z_all += expf(v[e] - sel_v[0]);
    }
    float wt[MOE_MAX_TOPK];
    topk_weights(sel_v, k, renorm, score, z_all, wt);
    if (ok) {
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j)
        if (j < k) {
          ids[(size_t)t * k + j] = sel_e[j];
          w[(size_t)t * k + j] = wt[j];
        }
    }
    chosen = valid & ~live;
  } else {
    // LPT lanes per token: the lane-group route of the general path (the
    // same experts and weights), T * LPT <= kScanThreads so every token in
    // one pass; then thread t takes token t's experts from an LDS copy
    static_assert(LPT <= 64 && (LPT & (LPT - 1)) == 0 && EMAX <= 256, "lane groups in a wave");
    __shared__ uint8_t sel[(kScanThreads / LPT) * MOE_MAX_TOPK];  // [token][j] expert
    if (t < EMAX * kSmallWaves) wmask[t] = 0ull;  // the count below ORs into it
    const int tt = t / LPT;
    route_token<LPT, (EMAX + LPT - 1) / LPT>(logits, tt, tt < T, t & (LPT - 1), E, k, renorm,
                                             score, ids, w, sel);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) sel_e[j] = (ok && j < k) ? (int)sel[t * k + j] : -1;
  }

  // 2. count (with lane groups: each lane ORs its bit into the masks of its
  // token's k experts instead of one ballot per expert)
  if constexpr (LPT == 1) {
    for (int e = 0; e < E; ++e) {
      const unsigned long long m = __ballot((int)((chosen >> e) & Mask(1)));
      if (lane == 0) wmask[e * kSmallWaves + wave] = m;
    }
  } else {
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (sel_e[j] >= 0) atomicOr(&wmask[sel_e[j] * kSmallWaves + wave], 1ull << lane);
  }
  __syncthreads();

  // 3. exclusive scan over (e, wave), e-major: a wave-level scan, then the
  // totals of the earlier waves.
  const int n = E * kSmallWaves;
  const int c = t < n ? __popcll(wmask[t]) : 0;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int q = 0; q < wave; ++q) before += wave_sum[q];
  if (t < n) start[t] = before + incl - c;
  __syncthreads();

  // positions of this token's rows
  if (ok) {
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j < k) {
        const int q = sel_e[j] * kSmallWaves + wave;
        const int p = start[q] + __popcll(wmask[q] & below);
        perm[p] = t * k + j;
        inv[t * k + j] = p;
      }
  }

  // 4. expert totals, offsets and the block table (wave 0, lane e)
  if (wave == 0) {
    int cnt = 0, first = 0;
    if (lane < E) {
      first = start[lane * kSmallWaves];
      const int last = lane * kSmallWaves + kSmallWaves - 1;
      cnt = start[last] + __popcll(wmask[last]) - first;
    }
    const int nbk = (cnt + bm - 1) / bm;
    int bincl = nbk;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(bincl, off, 64);
      if (lane >= off) bincl += o;
    }
    if (lane < E) {
      counts[lane] = cnt;
      offsets[lane] = first;
      if (lane == E - 1) {
        offsets[E] = first + cnt;
        nb[0] = bincl;
      }
      const int b0 = bincl - nbk;
      for (int r = 0; r < nbk; ++r) {
        blocks[2 * (b0 + r)] = lane;
        blocks[2 * (b0 + r) + 1] = first + r * bm;
      }
    }
    if (var.blocks) {  // uniform; lanes >= E have no rows
      const int vbk = cnt > bm ? (cnt + 2 * bm - 1) / (2 * bm) : nbk;
      int vincl = vbk;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(vincl, off, 64);
        if (lane >= off) vincl += o;
      }
      const int btotal = __shfl(bincl, 63, 64), vtotal = __shfl(vincl, 63, 64);
      const bool merge = var_rows_merge(var, btotal, vtotal);
      if (merge && lane < E)
        write_var_blocks(var.blocks, vincl - vbk, vbk, lane, first, cnt, cnt > bm ? 2 * bm : bm);
      if (lane == 0) var.nb[0] = merge ? vtotal : -1;
    }
    // longest-first launch order, as in hist_scan_kernel (lanes >= E have
    // no rows and take no part)
    if (order) {
      const int nfull = cnt / bm;
      const int rem = cnt - nfull * bm;
      int fincl = nfull;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(fincl, off, 64);
        if (lane >= off) fincl += o;
      }
      const int ftotal = __shfl(fincl, 63, 64);
      if (lane < E)
        for (int r = 0; r < nfull; ++r) order[fincl - nfull + r] = bincl - nbk + r;
      int rank = 0;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        const int q = __shfl(rem, e, 64);
        rank += (q > rem) || (q == rem && e < lane);
      }
      if (lane < E && rem > 0) order[ftotal + rank] = bincl - 1;
    }
  }
}

}  // namespace

bool fused_reorder_fits(int A, int E) {
  return (long long)((A + 63) / 64) * E <= kAllChunkCounts;
}

hipError_t launch_hist_scan(const int32_t* ids, int A, int E, int bm, int nchunks, int32_t* counts,
                            int32_t* offsets, int32_t* chunk_cnt, int32_t* chunk_base,
                            int32_t* blocks, int32_t* nb, int32_t* order, int32_t* perm,
                            int32_t* inv, VarRows var, hipStream_t s) {
  if ((perm != nullptr) != (inv != nullptr) || (perm && !fused_reorder_fits(A, E)))
    return hipErrorInvalidValue;
  if (var.blocks && (!var.nb || var.tiles < 1)) return hipErrorInvalidValue;
  hist_scan_kernel<<<1, kScanThreads, 0, s>>>(ids, A, E, bm, nchunks, counts, offsets, chunk_cnt,
                                              chunk_base, blocks, nb, order, perm, inv, var);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int A, int E, int nchunks, const int32_t* offsets,
                          const int32_t* chunk_cnt, const int32_t* chunk_base, int32_t* perm,
                          int32_t* inv, hipStream_t s) {
  const int waves = E * nchunks;
  permute_kernel<<<(waves + 3) / 4, 256, 0, s>>>(ids, A, E, nchunks, offsets, chunk_cnt,
                                                 chunk_base, perm, inv);
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* x, const int32_t* perm, int A, int d, int k,
                         uint16_t* x_perm, hipStream_t s) {
  gather_kernel<<<A, 256, 0, s>>>(x, perm, d, k, x_perm);
  return hipGetLastError();
}

hipError_t launch_gather_tiled(const uint16_t* x, const int32_t* perm, int A, int d, int k,
                               uint16_t* x_t, hipStream_t s) {
  if (A <= 0) return hipSuccess;
  gather_tiled_kernel<<<A, 256, 0, s>>>(x, perm, d, k, x_t);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

bool small_routing_fits(int T, int E, int k) {
  (void)k;
  return T <= kSmallRoutingMaxTokens && E <= kSmallRoutingMaxExperts;
}

hipError_t launch_route_dispatch_small(const LogitSrc& logits, int T, int E, int k, int renorm,
                                       int score, int bm, int32_t* ids, float* w,
                                       int32_t* counts, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, int32_t* blocks, int32_t* nb,
                                       int32_t* order, ZeroRange zero, VarRows var,
                                       hipStream_t s) {
  if (!small_routing_fits(T, E, k)) return hipErrorInvalidValue;
  if (var.blocks && (!var.nb || var.tiles < 1)) return hipErrorInvalidValue;
#define MOE_LAUNCH_SMALL(EMAX, LPT)                                                          \
  route_dispatch_small_kernel<EMAX, LPT><<<1, kScanThreads, 0, s>>>(                         \
      logits, T, E, k, renorm, score, bm, ids, w, counts, offsets, perm, inv, blocks, nb, order, \
      zero, var)
  // Up to 32 experts a thread routes its token alone; beyond, up to 256
  // tokens, the largest lane group per token that still covers every token
  // in one pass (with 2 lanes per token the kernel no longer fits its
  // registers, and it was no faster than one thread per token).
  if (E <= 8)
    MOE_LAUNCH_SMALL(8, 1);
  else if (E <= 16)
    MOE_LAUNCH_SMALL(16, 1);
  else if (E <= 32)
    MOE_LAUNCH_SMALL(32, 1);
  else if (T <= 16)
    MOE_LAUNCH_SMALL(64, 64);
  else if (T <= 32)
    MOE_LAUNCH_SMALL(64, 32);
  else if (T <= 64)
    MOE_LAUNCH_SMALL(64, 16);
  else if (T <= 128)
    MOE_LAUNCH_SMALL(64, 8);
  else if (T <= 256)
    MOE_LAUNCH_SMALL(64, 4);
  else
    MOE_LAUNCH_SMALL(64, 1);
#undef MOE_LAUNCH_SMALL
  return hipGetLastError();
}

}  // namespace moe
