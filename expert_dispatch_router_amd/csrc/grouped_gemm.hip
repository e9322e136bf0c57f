// grouped_gemm.hip -- K4: fused gate/up SwiGLU grouped GEMM; K5: down
// grouped GEMM.  bf16 inputs, fp32 accumulation on gfx950 MFMA
// (v_mfma_f32_16x16x32_bf16).
//
// [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in Triton".
// "What carries the argument": both SwiGLU projections are computed from one
// shared load of each input tile and SiLU is applied in registers, so the
// gate and up intermediates never reach global memory; the GEMMs are one
// launch over a block schedule whose blocks map to (expert, token-offset)
// pairs (Algorithm 1).  The down projection is the second expert GEMM of the
// SwiGLU FFN (abstract: expert GEMMs).
//
// Design on gfx950 (weights are K-contiguous, "NT"):
//   * One workgroup = one schedule block (expert e, up to BM sorted rows) x
//     one column tile; a wave owns NWT 16-column subtiles (for K4: NWT gate
//     subtiles and the NWT matching up subtiles) and all BM rows.
//   * The activation tile (BM rows x 64 of K) is staged once per K step in
//     LDS and shared by the workgroup's waves -- and, in K4, by the gate and
//     the up operand of every wave: this is the "one shared load of each
//     input tile" of the page, on LDS instead of L2.
//   * Weights are streamed from HBM straight into VGPRs in the MFMA operand
//     layout (16 bytes per lane per load), PF K steps ahead; the activation
//     loads ride in the same ring, so waiting for the oldest stage never
//     drains the younger prefetches.  Each weight element is read once per
//     block; only LDS is shared, so no weight byte goes through LDS.
//   * The MFMA's A operand is the weight (rows = output columns n), the B
//     operand the activation (columns = rows m): lane l then holds outputs
//     (n0 + 4*(l/16) + r, m0 + l%16), r = 0..3 -- four consecutive output
//     columns of one row, stored as one 8-byte (bf16) or 16-byte (fp32)
//     write.  Both operands take K elements [8*(l/16), 8*(l/16)+8) of each
//     32-wide chunk, so the contraction pairs them whatever the hardware's
//     internal K order.
//   * Blocks whose rows end early skip the 16-row subtiles past the end;
//     rows of the last partial subtile are masked at the store.  Subtiles
//     past the last column are skipped whole (N % 16 == 0).
//   * K5 may split its reduction into `split` contiguous parts, each written
//     as its own fp32 partial; the combination kernel adds them in order.
//   * K5 can also do the weighted combination itself (FoldCombine): after
//     writing its partials a workgroup counts them per (token, column tile);
//     the workgroup that writes the last of a token's k * split partials of
//     a tile computes that token's output columns there, in the same fixed
//     order as the combination kernel.  No waiting: every workgroup ends.
//   * The tiles above are the register-ring tiles.  The LDS-staged tiles
//     (gemm_lds_kernel, the default on most shapes) fetch weights and
//     activations by direct-to-LDS loads into a ring of two or three stages
//     instead, which frees the registers for wider tiles (224 columns at
//     BM = 192) or, with one subtile per wave, for a third stage (the narrow
//     tile of BM = 128).  gemm_lds_sk_kernel runs the same multiply loop on
//     a stream-K schedule (an option).
#include "buffer_load.hpp"
#include "combine_core.hpp"

namespace moe {
namespace {

constexpr int kBK = 64;               // K per pipeline step (two 32-wide MFMA chunks)
constexpr int kXcds = 8;              // accelerator complex dies of an MI355X
constexpr int kLdsStride = kBK + 8;   // bf16 per LDS row: 144 bytes, conflict-free reads

// Wait for this wave's LDS traffic, then a workgroup barrier.  Unlike
// __syncthreads() it does not wait for outstanding global loads, so the
// weight prefetches stay in flight across it.  The memory clobber keeps the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// Output of a launch: the fused SwiGLU h (bf16, gate and up rows from one
// activation tile), fp32 partial sums of one part of a split reduction, the
// plain product in bf16 (one projection of the unfused SwiGLU), or -- for
// small problems -- the down projection of the workgroup's own h columns:
// h stays in LDS and the workgroup writes the fp32 partial
// y[tile] = h[:, tile cols] . W_down[:, tile cols]^T, one part per column
// tile, which the combination adds in tile order.
enum {
  kOutSwiGLU = 0,
  kOutF32Parts = 1,
  kOutBF16 = 2,
  kOutSwiGLUDown = 3,
  kOutF32Wide = 4,
  kOutF32Dense = 5,
};

template <int BM, int NWT, int WAVES, int PF, int MODE>
struct Gemm {
  static constexpr int kMT = BM / 16;                        // 16-row subtiles
  static constexpr int kNG = (MODE == kOutSwiGLU || MODE == kOutSwiGLUDown) ? 2 : 1;  // gate, up
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kTileCols = WAVES * NWT * 16;         // output columns per workgroup
  static constexpr int kXChunks = BM * (kBK / 8);            // 16-byte chunks per activation tile
  static constexpr int kXPerThread = (kXChunks + kThreads - 1) / kThreads;
  // 4-wave, one-subtile tiles are sized for two workgroups per CU.
  static constexpr int kMinBlocks = (WAVES == 4 && NWT == 1) ? 2 : 1;
  static_assert(BM % 16 == 0, "BM is a multiple of 16");
};

// X: activations [A, K] (sorted rows).  W: weights [E, NG*N, K].
// out: K4 -> bf16 h [A, N];  K5 -> fp32 y [split, A, N].
template <int BM, int NWT, int WAVES, int PF, int MODE>
__global__ __launch_bounds__(WAVES * 64, (Gemm<BM, NWT, WAVES, PF, MODE>::kMinBlocks))
void grouped_gemm_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, long long w_estride,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ nb_dev,
    const int32_t* __restrict__ order, const int32_t* __restrict__ offsets,
    void* __restrict__ out, int A, int N, int K, int ksplit,
    int tiles_per_block, int rotate, const int32_t* __restrict__ gather_perm, int gather_k,
    int x_rows, int xcd_group, int x_tiled, FoldCombine fold, const uint16_t* __restrict__ W2,
    long long w2_estride, int N2, int dyn_split) {
  using G = Gemm<BM, NWT, WAVES, PF, MODE>;
  constexpr int MT = G::kMT, NG = G::kNG, XPT = G::kXPerThread;
  static_assert(PF >= 2, "the activation stage is issued PF-1 steps ahead");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kLdsStride];

  // The split of the reduction: as launched (tiles_per_block = column tiles
  // x parts, ksplit per part), or with dyn_split decided here from the
  // routed block count (device_down_split; at most the launched parts).
  const int n_tiles = (N + G::kTileCols - 1) / G::kTileCols;
  if (dyn_split) {
    const DownSplit ds = device_down_split(nb_dev[0], n_tiles, tiles_per_block / n_tiles, K);
    tiles_per_block = n_tiles * ds.parts;
    ksplit = ds.ksplit;
  }

  // Workgroup -> (block, tile).  Workgroups are dispatched to the XCDs
  // round-robin (workgroup i to XCD i % kXcds).  With xcd_group, the real
  // workgroups (nb * tiles_per_block of the device-built schedule, rounded
  // up to kXcds) are renumbered so that each XCD runs one contiguous range
  // of (block, tile) ids: the tiles of a block then share that XCD's L2 for
  // the block's activation rows instead of fetching them once per XCD.
  int wg = blockIdx.x;
  if (xcd_group) {
    const int r8 = (nb_dev[0] * tiles_per_block + kXcds - 1) / kXcds * kXcds;
    if (wg >= r8) return;
    wg = (wg % kXcds) * (r8 / kXcds) + wg / kXcds;
  }
  // Without XCD grouping the blocks may be taken longest first (`order`,
  // built on the device): the heavy blocks start in the first round and the
  // light ones fill the tail.  Results do not depend on the order.
  const int bi = wg / tiles_per_block;
  if (bi >= nb_dev[0]) return;  // beyond the schedule built on the device
  const int b = order ? order[bi] : bi;
  const int rem = wg - bi * tiles_per_block;
  const int e = blocks[2 * b];
  const int r0 = blocks[2 * b + 1];
  const int rows = min(BM, offsets[e + 1] - r0);
  const int mt_act = (rows + 15) >> 4;

  const int tile = rem % n_tiles;
  const int part = rem / n_tiles;
  const int kb = part * ksplit;
  const int nks = max(0, (min(K, kb + ksplit) - kb) / kBK);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: uniform branches
  const int n0 = tile * G::kTileCols + wave * (NWT * 16);
  const int lrow = lane & 15;
  const int lk = (lane >> 4) * 8;

  // Buffer resources: this expert's weights, and this block's rows of X.
  // Rows past the block's end are outside the X range and load as zeros;
  // column subtiles past N are never stored.  Every load below is
  // unconditional (K steps past the end reload the last step, an L2 hit),
  // so the compiler counts outstanding loads exactly and waits only for the
  // oldest ring stage.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (size_t)e * w_estride), (short)0, NG * N * K * 2, kRsrcWord3);
  // X rows: sorted rows r0 .. r0+rows-1 of X, or -- with gather_perm -- the
  // token rows x[perm[r0 + row] / gather_k] of the unsorted activations (the
  // reorder's row gather folded into this load), or -- with x_tiled -- the
  // sorted rows of X stored in K-step tiles: the 64-wide K step s of the
  // 16-row group G is 2 KiB at ((G * K/64) + s) * 2048, row p % 16 at
  // +128 * (p % 16).  Rows past the block's end get an offset outside the
  // descriptor's range and load as zeros.
  const __amdgpu_buffer_rsrc_t xres =
      (gather_perm || x_tiled)
          ? __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, x_rows * K * 2, kRsrcWord3)
          : __builtin_amdgcn_make_buffer_rsrc((void*)(X + (size_t)r0 * K), (short)0,
                                              rows * K * 2, kRsrcWord3);
  const int xstep = x_tiled ? 16 * kBK * 2 : kBK * 2;  // bytes between K steps of one row
  int woff[NG][NWT];
  bool jok[NWT];
#pragma unroll
  for (int j = 0; j < NWT; ++j) {
    jok[j] = n0 + 16 * j < N;
#pragma unroll
    for (int g = 0; g < NG; ++g) woff[g][j] = ((g * N + n0 + 16 * j + lrow) * K + kb + lk) * 2;
  }
  // Activation chunks this thread stages: chunk c -> (row c/8, 16-byte
  // column chunk c%8).  When the tile has fewer chunks than threads, extra
  // threads repeat a chunk (same data, same LDS slot).
  int xoff[XPT];
  int xdst[XPT];
#pragma unroll
  for (int q = 0; q < XPT; ++q) {
    const int c = (tid + q * G::kThreads) % G::kXChunks;
    const int row = c >> 3;
    if (x_tiled) {
      const int p = r0 + row;
      xoff[q] = row < rows ? ((p >> 4) * (K / kBK) + kb / kBK) * (16 * kBK * 2) + (p & 15) * kBK * 2 +
                                 (c & 7) * 16
                           : x_rows * K * 2;
    } else {
      int src_row = row;
      if (gather_perm) src_row = row < rows ? gather_perm[r0 + row] / gather_k : x_rows;
      xoff[q] = (src_row * K + kb + (c & 7) * 8) * 2;
    }
    xdst[q] = row * kLdsStride + (c & 7) * 8;
  }

  // Ring of PF slots.  Slot s = ks % PF carries the weights of step ks and
  // the activation tile of step ks - 1 (activation tiles are issued one step
  // later than weights, so only PF-1 of them are live at once).
  bf16x8 wr[PF][NG][NWT][2];
  u32x4 xr[PF][XPT];
  f32x4 acc[NG][MT][NWT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < NWT; ++j) acc[g][mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K-step order: with `rotate` (1: per block, 2: per workgroup, 3: per
  // expert), a workgroup starts its reduction at a step derived from its
  // block b (its own id, its expert e) and wraps around.  Workgroups walking
  // K in lockstep address the same memory channels at once -- weight rows
  // 2^n bytes apart share their low address bits -- and different starting
  // steps spread them.  Per block, the column tiles of one block still read
  // the same activation K-slice at the same time (shared in L2); per expert,
  // the blocks of one expert also read the same weights at the same time;
  // per workgroup spreads further.  The order is fixed by (block, tile):
  // results stay deterministic.
  const unsigned rkey = rotate == 2 ? (unsigned)wg : rotate == 3 ? (unsigned)e : (unsigned)b;
  const int shift = rotate ? (int)((rkey * 2654435761u) % (unsigned)max(nks, 1)) : 0;
  auto step_of = [&](int ks) {
    const int p = ks + shift;
    return p >= nks ? p - nks : p;
  };
  auto load_x = [&](u32x4(&dst)[XPT], int ks) {
    const int soff = step_of(ks) * xstep;
#pragma unroll
    for (int q = 0; q < XPT; ++q) dst[q] = buf_load16(xres, xoff[q], soff);
  };
  auto load_w = [&](bf16x8(&dst)[NG][NWT][2], int ks) {
    const int soff = step_of(ks) * kBK * 2;
#pragma unroll
    for (int j = 0; j < NWT; ++j)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        dst[g][j][0] = __builtin_bit_cast(bf16x8, buf_load16(wres, woff[g][j], soff));
        dst[g][j][1] = __builtin_bit_cast(bf16x8, buf_load16(wres, woff[g][j] + 64, soff));
      }
  };
  auto store_x = [&](int buf, const u32x4(&src)[XPT]) {
#pragma unroll
    for (int q = 0; q < XPT; ++q) *reinterpret_cast<u32x4*>(&xs[buf][xdst[q]]) = src[q];
  };
  // Multiply one K step.  Activation fragments are read from LDS one 16-row
  // subtile ahead of their MFMAs (rows past the block's end hold zeros, so
  // the read is always in bounds); the scheduling barriers keep the compiler
  // from hoisting every fragment read of the unrolled loop to the top.
  auto compute = [&](int buf, const bf16x8(&wv)[NG][NWT][2]) {
    const uint16_t* xb = &xs[buf][lrow * kLdsStride + lk];
    bf16x8 xa0 = *reinterpret_cast<const bf16x8*>(xb);
    bf16x8 xa1 = *reinterpret_cast<const bf16x8*>(xb + 32);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      bf16x8 xn0 = xa0, xn1 = xa1;
      if (mt + 1 < MT) {
        xn0 = *reinterpret_cast<const bf16x8*>(xb + (mt + 1) * 16 * kLdsStride);
        xn1 = *reinterpret_cast<const bf16x8*>(xb + (mt + 1) * 16 * kLdsStride + 32);
      }
      if (mt < mt_act) {
#pragma unroll
        for (int j = 0; j < NWT; ++j)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            acc[g][mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[g][j][0], xa0,
                                                                    acc[g][mt][j], 0, 0, 0);
            acc[g][mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[g][j][1], xa1,
                                                                    acc[g][mt][j], 0, 0, 0);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
      xa0 = xn0;
      xa1 = xn1;
    }
  };

  if (nks > 0) {
    const int last = nks - 1;
    // Prologue, in steady-state issue order: W(0); then X(i-1), W(i).
    // The barriers pin this order so the loop is entered with the same queue
    // of outstanding loads as every later iteration.
    load_w(wr[0], 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 1; i < PF; ++i) {
      load_x(xr[i], min(i - 1, last));
      __builtin_amdgcn_sched_barrier(0);
      load_w(wr[i], min(i, last));
      __builtin_amdgcn_sched_barrier(0);
    }
    // Step ks (slot s): stage X(ks) (slot s+1) in LDS, barrier, multiply with
    // W(ks), then refill slot s with X(ks+PF-1) and W(ks+PF), in that order
    // -- waiting for X(ks) never waits for W(ks+1..ks+PF-1).
    int ks0 = 0;
    for (; ks0 + PF <= nks; ks0 += PF) {
#pragma unroll
      for (int s = 0; s < PF; ++s) {
        const int ks = ks0 + s;
        const int buf = ks & 1;
        store_x(buf, xr[(s + 1) % PF]);
        lds_barrier();
        compute(buf, wr[s]);
        // Keep the refill after the multiplies: hoisting it would hold two
        // weight stages of this slot in registers at once.
        __builtin_amdgcn_sched_barrier(0);
        load_x(xr[s], min(ks + PF - 1, last));
        __builtin_amdgcn_sched_barrier(0);
        load_w(wr[s], min(ks + PF, last));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Remaining (< PF) steps: their stages are already in flight.
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int ks = ks0 + s;
      if (ks < nks) {
        const int buf = ks & 1;
        store_x(buf, xr[(s + 1) % PF]);
        lds_barrier();
        compute(buf, wr[s]);
      }
    }
  }

  if constexpr (MODE == kOutSwiGLUDown) {
    // h tile -> LDS (bf16, [BM][kTileCols + 8]) over the activation buffers;
    // rows past the block's end hold silu(0) * 0 = 0, subtiles past the
    // active ones are never read.
    constexpr int HS = G::kTileCols + 8;
    static_assert(BM * HS <= 2 * BM * kLdsStride, "h tile fits the staging buffers");
    static_assert(G::kTileCols % 32 == 0, "whole 32-wide K chunks");
    constexpr int KC = G::kTileCols / 32;
    uint16_t* hl = &xs[0][0];
    __syncthreads();  // every wave is done with the activation tiles
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_act) {
#pragma unroll
        for (int j = 0; j < NWT; ++j) {
          if (!jok[j]) continue;
          const f32x4 gv = acc[0][mt][j];
          const f32x4 uv = acc[1][mt][j];
          bf16x4 hv;
          hv[0] = (__bf16)(silu_f32(gv[0]) * uv[0]);
          hv[1] = (__bf16)(silu_f32(gv[1]) * uv[1]);
          hv[2] = (__bf16)(silu_f32(gv[2]) * uv[2]);
          hv[3] = (__bf16)(silu_f32(gv[3]) * uv[3]);
          *reinterpret_cast<bf16x4*>(hl + (mt * 16 + lrow) * HS + wave * (NWT * 16) + 16 * j +
                                     4 * (lane >> 4)) = hv;
        }
      }
    }
    lds_barrier();
    // y[tile][r0 + m][o] = sum over this tile's columns c of h[m][c] W2[o][c]:
    // W_down rows as the A operand (16 outputs o per subtile), h as B.
    const int c0 = tile * G::kTileCols;
    const int nkc = min(G::kTileCols, N - c0) / 32;
    const __amdgpu_buffer_rsrc_t w2res = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W2 + (size_t)e * w2_estride), (short)0, N2 * N * 2, kRsrcWord3);
    float* y = static_cast<float*>(out) + (size_t)tile * A * N2;
    for (int o0 = wave * 16; o0 < N2; o0 += WAVES * 16) {  // wave-uniform
      bf16x8 wa[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        if (kc < nkc)
          wa[kc] = __builtin_bit_cast(
              bf16x8, buf_load16(w2res, ((o0 + lrow) * N + c0 + kc * 32 + lk) * 2, 0));
      f32x4 acc2[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc2[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (kc < nkc) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if (mt < mt_act) {
              const bf16x8 hb =
                  *reinterpret_cast<const bf16x8*>(hl + (mt * 16 + lrow) * HS + kc * 32 + lk);
              acc2[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[kc], hb, acc2[mt], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);  // one operand read in flight per MFMA
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + lrow;
        if (mt < mt_act && m < rows)
          *reinterpret_cast<f32x4*>(y + (size_t)(r0 + m) * N2 + o0 + 4 * (lane >> 4)) = acc2[mt];
      }
    }
    return;
  }

  // Epilogue.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < mt_act) {
      const int m = mt * 16 + lrow;
      if (m < rows) {
        const size_t orow = (size_t)(r0 + m);
#pragma unroll
        for (int j = 0; j < NWT; ++j) {
          if (!jok[j]) continue;
          const int n = n0 + 16 * j + 4 * (lane >> 4);
          if constexpr (MODE == kOutSwiGLU) {
            const f32x4 gv = acc[0][mt][j];
            const f32x4 uv = acc[NG - 1][mt][j];
            bf16x4 hv;
            hv[0] = (__bf16)(silu_f32(gv[0]) * uv[0]);
            hv[1] = (__bf16)(silu_f32(gv[1]) * uv[1]);
            hv[2] = (__bf16)(silu_f32(gv[2]) * uv[2]);
            hv[3] = (__bf16)(silu_f32(gv[3]) * uv[3]);
            *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(out) + orow * N + n) = hv;
          } else if constexpr (MODE == kOutF32Parts) {
            float* y = static_cast<float*>(out) + ((size_t)part * A + orow) * N + n;
            if (fold.cnt) {
              // read by another workgroup of this launch: agent-scope stores
              // (written through to the device-coherent level)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                __hip_atomic_store(y + i, acc[0][mt][j][i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            } else {
              *reinterpret_cast<f32x4*>(y) = acc[0][mt][j];
            }
          } else {
            const f32x4 v = acc[0][mt][j];
            bf16x4 o;
            o[0] = (__bf16)v[0];
            o[1] = (__bf16)v[1];
            o[2] = (__bf16)v[2];
            o[3] = (__bf16)v[3];
            *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(out) + orow * N + n) = o;
          }
        }
      }
    }
  }

  if constexpr (MODE == kOutF32Parts) {
    if (fold.cnt) {
      // The partials went out as agent-scope stores.  After the barrier
      // (every thread's stores are ordered before it) each thread issues an
      // agent-scope release fence, then counts its rows' tokens for this
      // column tile with relaxed agent-scope increments: the counter's
      // modification order carries every earlier workgroup's release to the
      // workgroup whose increment completes a count, which acquires (agent
      // scope) before it owns that token's combination for the tile and
      // reads the partials with agent-scope loads.  The barrier below hands
      // the acquired view to the workgroup's other threads.
      __shared__ int n_last;
      __shared__ int last_tok[BM];
      if (tid == 0) n_last = 0;
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const int nsplit = tiles_per_block / n_tiles;
      const int need = fold.k * nsplit;  // k routed rows x split parts
      for (int m = tid; m < rows; m += G::kThreads) {
        const int t = fold.perm[r0 + m] / fold.k;
        if (__hip_atomic_fetch_add(&fold.cnt[(size_t)t * n_tiles + tile], 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) == need - 1) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          last_tok[atomicAdd(&n_last, 1)] = t;
        }
      }
      __syncthreads();
      const int nl = n_last;
      if (nl > 0) {
        const int c0 = tile * G::kTileCols;
        const int nq = min(G::kTileCols, N - c0) / 4;
        const float* y = static_cast<const float*>(out);
        for (int i = tid; i < nl * nq; i += G::kThreads)
          combine_quad(y, nsplit, A, N, fold.inv, fold.w, fold.k, last_tok[i / nq],
                       c0 + (i % nq) * 4, fold.out, AgentLoad{});
      }
    }
  }
}

template <int BM, int NWT, int WAVES, int PF, int MODE>
hipError_t launch_cfg(const uint16_t* X, const uint16_t* W, long long w_estride, const int32_t* blocks,
                      const int32_t* nb, const int32_t* order, const int32_t* offsets, void* out,
                      int A, int N, int K,
                      int split, int ksplit, int nb_max, int rotate, const int32_t* gather_perm,
                      int gather_k, int x_rows, int xcd_group, int x_tiled,
                      const FoldCombine& fold, hipStream_t s, const uint16_t* W2 = nullptr,
                      long long w2_estride = 0, int N2 = 0, int dyn_split = 0) {
  using G = Gemm<BM, NWT, WAVES, PF, MODE>;
  const int n_tiles = (N + G::kTileCols - 1) / G::kTileCols;
  const int tiles_per_block = n_tiles * split;
  // XCD grouping renumbers the real workgroups rounded up to kXcds: every
  // id below that must be launched
  const long long grid = xcd_group ? ((long long)tiles_per_block * nb_max + kXcds - 1) / kXcds * kXcds
                                   : (long long)tiles_per_block * nb_max;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  grouped_gemm_kernel<BM, NWT, WAVES, PF, MODE><<<(unsigned)grid, G::kThreads, 0, s>>>(
      X, W, w_estride, blocks, nb, order, offsets, out, A, N, K, ksplit, tiles_per_block, rotate,
      gather_perm, gather_k, x_rows, xcd_group, x_tiled, fold, W2, w2_estride, N2, dyn_split);
  return hipGetLastError();
}

// Tile shapes: (variant, BM, NWT, waves, PF).  NWT*16 output columns per wave
// (x2 rows for gate+up in K4), PF K steps of weight prefetch.  Chosen by
// measurement on the MoE workload shapes.  K4 variant 1 at BM=64 and 128 is
// the narrow tile for launches with few blocks; K4 variant 1 at BM=192 is a
// 7-wave, 112-column tile (two waves on three SIMDs) whose tile count
// divides evenly over the CUs where 128-column tiles leave a half-empty last
// round.
#define MOE_GU_CFGS(X) \
  X(0, 16, 4, 4, 2) X(0, 32, 4, 4, 2) X(0, 64, 4, 4, 3) X(1, 64, 2, 4, 4) X(0, 128, 1, 8, 3) \
  X(1, 128, 1, 4, 4) X(0, 192, 1, 8, 3) X(1, 192, 1, 7, 3)
#define MOE_DN_CFGS(X) \
  X(0, 16, 8, 4, 2) X(0, 32, 8, 4, 2) X(0, 64, 4, 4, 4) X(0, 128, 4, 4, 3) X(1, 128, 2, 8, 3) \
  X(0, 192, 2, 8, 3) X(1, 192, 4, 4, 3)


// ---------------------------------------------------------------------------
// Wide fused gate/up tile: weights staged in LDS.
//
// The tile above keeps each wave's weight ring in VGPRs, which leaves room
// for one 16-column subtile (x gate and up) per wave at BM = 192; every
// workgroup then streams its block's activation rows through the CU's
// vector-memory path once per 112 weight columns, ~0.57 activation bytes
// per weight byte at Mixtral's ~128 rows per block, and those reads share
// the path with the weight stream.  Here each wave owns SUB subtiles per
// operand -- two (WAVES * 32 columns per workgroup: half the activation
// bytes per weight byte; its 192 accumulator registers at BM = 192 fit only
// because the weight ring lives in LDS), or one (the narrow tile: WAVES * 16
// columns, smaller stages, so three of them fit) -- and weights and
// activations are fetched by direct-to-LDS buffer loads (no VGPRs), STAGES
// (two or three) stages of BK of K each.
//
// LDS stage: WAVES * kGPW weight groups (kGPW = NG operands -- or the wide
// mode's two column groups -- times SUB subtiles), then BM/16 activation
// groups; a group
// is 16 rows x (2 * BK) bytes, written by BK/32 loads of 64 lanes x 16
// bytes.  Load h of a group fetches rows [R*h, R*h + R) (R = 1024 / row
// bytes), whole rows of the step: with BK = 64 each load reads whole
// 128-byte lines (streaming half lines per step measured at ~60% of the
// whole-line rate).  The 16-byte slot s of row r holds K chunk
// s ^ swz(r), swz(r) = (r >> 2) & 3 (BK = 32) or (r >> 1) & 7 (BK = 64), so
// the MFMA fragment reads -- 16 rows at one K chunk per 16 lanes -- hit 64
// distinct banks.  Every wave issues the same number of loads per stage
// (kGPW weight groups, kXPerWave activation groups; surplus activation slots
// repeat a group: same bytes to the same place), so one immediate
// "vmcnt" waits for the wave's own loads of a stage; the barrier
// after it publishes the stage to all waves.
// MODE kOutSwiGLU: gate and up rows (NG = 2), bf16 h; kOutF32Parts: one
// operand (the down projection), fp32 partial sums of a split reduction;
// kOutF32Wide: the same output with 64 columns per wave, taken as two
// adjacent 32-column groups in the places of gate and up, so a stage holds
// twice the weight rows per activation row; kOutF32Dense: fp32 parts of one
// dense product (no schedule: block b is rows [b * BM, b * BM + BM) of X,
// all against W) -- the router scores.
template <int BM, int WAVES, int BK, int STAGES, int MODE = kOutSwiGLU, int SUB = 2>
struct LdsGemm {
  static_assert(BK == 32 || BK == 64, "K step of 32 or 64");
  static_assert(STAGES == 2 || STAGES == 3, "two or three stages");
  static_assert(SUB == 1 || SUB == 2, "one or two 16-column subtiles per wave and operand");
  static_assert(MODE == kOutSwiGLU || MODE == kOutF32Parts || MODE == kOutF32Wide ||
                    MODE == kOutF32Dense,
                "SwiGLU or fp32 parts");
  static constexpr bool kWide = MODE == kOutF32Wide;
  static_assert(!kWide || SUB == 2, "the wide tile takes two subtiles per column group");
  static constexpr int kNG = (MODE == kOutSwiGLU || kWide) ? 2 : 1;
  static constexpr int kSub = SUB;
  static constexpr int kWaveCols = kWide ? 64 : 16 * SUB;  // output columns of one wave
  static constexpr int kGPW = SUB * kNG;                   // 16-row weight groups per wave
  static constexpr int kMT = BM / 16;
  static constexpr int kKC = BK / 32;                 // MFMA K chunks per step
  static constexpr int kRowBytes = 2 * BK;
  static constexpr int kGroupBytes = 16 * kRowBytes;
  static constexpr int kLoadsPerGroup = kGroupBytes / 1024;
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kTileCols = WAVES * kWaveCols;
  static constexpr int kWBytes = WAVES * kGPW * kGroupBytes;
  static constexpr int kXGroups = BM / 16;
  static constexpr int kXPerWave = (kXGroups + WAVES - 1) / WAVES;
  static constexpr int kStageBytes = kWBytes + kXGroups * kGroupBytes;
  static constexpr int kLoadsPerStage = (kGPW + kXPerWave) * kLoadsPerGroup;
  // loads younger than a stage's activation loads when the wait for that
  // stage is full (see the main loop): STAGES - 2 whole stages and one
  // stage's weights
  static constexpr int kWaitAhead = (STAGES - 2) * kLoadsPerStage + kGPW * kLoadsPerGroup;
  static_assert(kWaitAhead <= 63, "immediate vmcnt");
  static_assert(kXPerWave * WAVES <= 2 * kXGroups, "a surplus slot repeats one group");
  static_assert(STAGES * kStageBytes <= 160 * 1024, "LDS of one CU");
  __device__ static int swz(int r) { return BK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16 bytes per lane from a buffer straight into LDS.  CPOL: cache-policy
// bits of the load (kCpolNT: non-temporal, for data read exactly once).
constexpr int kCpolNT = 2;
template <int CPOL = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, voff, soff, 0, CPOL);
}

template <int NG, int MT, int SUB>
__device__ __forceinline__ void lds_tile_zero(f32x4 (&acc)[NG][MT][SUB]) {
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < SUB; ++j) acc[g][mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// The multiplies of one (block, column tile, part) of the LDS-staged tile
// over K steps [s_first, s_first + s_count) of the part's step sequence: nks
// steps of BK from K offset kb, taken in the rotated order that starts at
// step `shift`.  Accumulates into acc (this wave's NG x MT x SUB fragments of
// columns n0 ..).  Every wave of the workgroup calls it together; on return
// the wave's loads have landed and its last LDS reads are done, but other
// waves may still read the ring: the caller synchronises before reusing it.
template <int BM, int WAVES, int BK, int STAGES, int MODE, int WCPOL, int SUB>
__device__ __forceinline__ void lds_tile_mma(
    uint8_t* lds, const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    long long w_estride, int e, int r0, int rows, int n0, int kb, int N, int K, int nks_all,
    int shift, int s_first, int s_count, const int32_t* __restrict__ gather_perm, int gather_k,
    int x_rows, f32x4 (&acc)[LdsGemm<BM, WAVES, BK, STAGES, MODE, SUB>::kNG][BM / 16][SUB]) {
  using G = LdsGemm<BM, WAVES, BK, STAGES, MODE, SUB>;
  constexpr int MT = G::kMT, KC = G::kKC, SB = G::kStageBytes, XPW = G::kXPerWave;
  constexpr int NG = G::kNG, GPW = G::kGPW;
  constexpr int LPG = G::kLoadsPerGroup, GB = G::kGroupBytes, RB = G::kRowBytes;
  const int mt_act = (rows + 15) >> 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  (void)tid;

  // loads: load h of a group, lane -> row h * (1024 / RB) + lane / (RB / 16),
  // slot lane % (RB / 16), which holds K chunk slot ^ swz(row)
  constexpr int SPR = RB / 16;  // 16-byte slots per row
  int lrow[LPG], lchk[LPG];
#pragma unroll
  for (int hh = 0; hh < LPG; ++hh) {
    lrow[hh] = hh * (1024 / RB) + lane / SPR;
    lchk[hh] = (lane % SPR) ^ G::swz(lrow[hh]);
  }
  // weight rows of the expert: NG operands of N rows (SwiGLU), else N rows
  constexpr int kWOps = G::kWide ? 1 : NG;
  const int wbytes = kWOps * N * K * 2;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (size_t)e * w_estride), (short)0, wbytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xres =
      gather_perm
          ? __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, x_rows * K * 2, kRsrcWord3)
          : __builtin_amdgcn_make_buffer_rsrc((void*)(X + (size_t)r0 * K), (short)0,
                                              rows * K * 2, kRsrcWord3);
  // weight groups of this wave: q = SUB * g + j -> operand g (gate, up), subtile j;
  // wide: column group g of the wave's 64 columns, subtile j.
  // Columns past N (a partial last tile) get an offset past the
  // descriptor's range: zeros, no memory request; their outputs are not
  // stored.
  int woff[GPW][LPG];
#pragma unroll
  for (int q = 0; q < GPW; ++q)
#pragma unroll
    for (int hh = 0; hh < LPG; ++hh) {
      const int col = n0 + (G::kWide ? 32 * (q / SUB) : 0) + 16 * (q % SUB) + lrow[hh];
      const int wrow = G::kWide ? col : (q / SUB) * N + col;
      woff[q][hh] = col < N ? (wrow * K + kb + lchk[hh] * 8) * 2 : wbytes;
    }
  int xoff[XPW][LPG];
  int xgrp[XPW];
#pragma unroll
  for (int q = 0; q < XPW; ++q) {
    const int gs = wave + q * WAVES;
    const int grp = gs < G::kXGroups ? gs : gs - G::kXGroups;  // surplus slots repeat a group
    xgrp[q] = grp;
#pragma unroll
    for (int hh = 0; hh < LPG; ++hh) {
      const int row = grp * 16 + lrow[hh];
      int src = row;
      if (gather_perm) src = row < rows ? gather_perm[r0 + row] / gather_k : x_rows;
      else if (row >= rows) src = rows;  // past the range: zeros, no memory request
      xoff[q][hh] = (src * K + kb + lchk[hh] * 8) * 2;
    }
  }

  auto soff_of = [&](int ks) {
    const int kk = ks + shift;
    return (kk >= nks_all ? kk - nks_all : kk) * (BK * 2);
  };
  // weights of stage ks into this wave's region of slot ks % STAGES
  auto issue_w = [&](int ks) {
    const int soff = soff_of(s_first + ks);
    uint8_t* st = lds + (ks % STAGES) * SB;
#pragma unroll
    for (int q = 0; q < GPW; ++q)
#pragma unroll
      for (int hh = 0; hh < LPG; ++hh)
        dma16<WCPOL>(wres, st + (wave * GPW + q) * GB + hh * 1024, woff[q][hh], soff);
  };
  // this wave's share of the activation tile of stage ks
  auto issue_x = [&](int ks) {
    const int soff = soff_of(s_first + ks);
    uint8_t* st = lds + (ks % STAGES) * SB;
#pragma unroll
    for (int q = 0; q < XPW; ++q)
#pragma unroll
      for (int hh = 0; hh < LPG; ++hh)
        dma16(xres, st + G::kWBytes + xgrp[q] * GB + hh * 1024, xoff[q][hh], soff);
  };

  // fragment reads: lane -> row (lane & 15), K chunk c * 4 + (lane >> 4) of
  // the step's chunk c
  const int rr = lane & 15;
  int roff[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) roff[c] = rr * RB + ((((lane >> 4) + 4 * c) ^ G::swz(rr)) * 16);
  constexpr int SL = G::kLoadsPerStage;
  const int nks = s_count;  // steps of this call, local indices 0 .. s_count - 1
  if (nks > 0) {
    // Each wave's weight region is its own: the wave refills it with stage
    // ks + STAGES right after its multiplies of stage ks, so its weight
    // stream keeps STAGES stages in flight without waiting for the other
    // waves.  The shared activation tile of stage ks + STAGES - 1 is issued
    // after the barrier of step ks, once every wave is done with stage
    // ks - 1, whose slot it takes.
    // Issue order per wave: W(0) X(0) ... W(S-2) X(S-2) W(S-1), then per step
    // ks: X(ks+S-1), W(ks+S) -- so the loads are W(j) X(j) in stage order,
    // and at the top of step ks the loads younger than X(ks) are those of
    // the stages issued beyond ks: S-2 whole stages and W(ks+S-1), or fewer
    // near the end of the reduction (whole stages only).
#pragma unroll
    for (int j = 0; j < STAGES - 1; ++j)
      if (j < nks) {
        issue_w(j);
        issue_x(j);
      }
    if (STAGES - 1 < nks) issue_w(STAGES - 1);
    for (int ks = 0; ks < nks; ++ks) {
      const int ahead = min(nks - 1 - ks, STAGES - 1);  // stages issued beyond ks
      if (ahead == STAGES - 1) wait_vmcnt<G::kWaitAhead>();
      else if (STAGES == 3 && ahead == 1) wait_vmcnt<(STAGES == 3 ? SL : 0)>();
      else wait_vmcnt<0>();
      lds_barrier();  // ... everyone's; and everyone is done with stage ks - 1
      if (ks + STAGES - 1 < nks) issue_x(ks + STAGES - 1);
      const uint8_t* st = lds + (ks % STAGES) * SB;
      const uint8_t* xb = st + G::kWBytes;
      // K chunk outermost: one chunk's weight fragments live at a time (each
      // output still sums its K chunks in ascending order)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        bf16x8 wa[GPW];
#pragma unroll
        for (int q = 0; q < GPW; ++q)
          wa[q] = *reinterpret_cast<const bf16x8*>(st + (wave * GPW + q) * GB + roff[c]);
        bf16x8 xa = *reinterpret_cast<const bf16x8*>(xb + roff[c]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          bf16x8 xn = xa;
          if (mt + 1 < MT) xn = *reinterpret_cast<const bf16x8*>(xb + (mt + 1) * GB + roff[c]);
          if (mt < mt_act) {
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
              for (int j = 0; j < SUB; ++j)
                acc[g][mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[SUB * g + j], xa,
                                                                        acc[g][mt][j], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          xa = xn;
        }
      }
      // this wave is done with its weights of stage ks
      if (ks + STAGES < nks) issue_w(ks + STAGES);
    }
  }
}

// Writes a tile's results: bf16 h = silu(gate) * up (SwiGLU) or fp32 parts
// [part, A, N].
template <int BM, int WAVES, int BK, int STAGES, int MODE, int SUB>
__device__ __forceinline__ void lds_tile_store(
    const f32x4 (&acc)[LdsGemm<BM, WAVES, BK, STAGES, MODE, SUB>::kNG][BM / 16][SUB], void* out,
    int A, int N, int r0, int rows, int n0, int part) {
  using G = LdsGemm<BM, WAVES, BK, STAGES, MODE, SUB>;
  constexpr int MT = G::kMT, NG = G::kNG;
  const int mt_act = (rows + 15) >> 4;
  const int lane = threadIdx.x & 63;
  const int rr = lane & 15;
  // epilogue: lane holds columns n0 + 16j + 4*(lane>>4) + 0..3 of row mt*16 + (lane & 15)
  // (wide: n0 + 32g + 16j + ...)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + rr;
    if constexpr (G::kWide) {
      if (mt < mt_act && m < rows) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int c0 = n0 + 32 * g + 16 * j;
            if (c0 >= N) continue;  // subtile past the last column (N % 16 == 0)
            const int n = c0 + 4 * (lane >> 4);
            *reinterpret_cast<f32x4*>(static_cast<float*>(out) +
                                      ((size_t)part * A + r0 + m) * N + n) = acc[g][mt][j];
          }
      }
      continue;
    }
    if (mt < mt_act && m < rows) {
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        if (n0 + 16 * j >= N) continue;  // subtile past the last column (N % 16 == 0)
        const int n = n0 + 16 * j + 4 * (lane >> 4);
        if constexpr (MODE == kOutSwiGLU) {
          const f32x4 gv = acc[0][mt][j];
          const f32x4 uv = acc[NG - 1][mt][j];
          bf16x4 hv;
          hv[0] = (__bf16)(silu_f32(gv[0]) * uv[0]);
          hv[1] = (__bf16)(silu_f32(gv[1]) * uv[1]);
          hv[2] = (__bf16)(silu_f32(gv[2]) * uv[2]);
          hv[3] = (__bf16)(silu_f32(gv[3]) * uv[3]);
          *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(out) + (size_t)(r0 + m) * N + n) = hv;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + ((size_t)part * A + r0 + m) * N + n) =
              acc[0][mt][j];
        }
      }
    }
  }
}

// One workgroup = one (block, column tile, part).  out: kOutSwiGLU -> bf16
// h [A, N]; kOutF32Parts, kOutF32Wide and kOutF32Dense -> fp32 y [split, A,
// N] (part p sums K steps [p * ksplit, (p + 1) * ksplit)).  kOutF32Dense
// reads no schedule (blocks, nb_dev, order and offsets may be null).
// BMS, BMS2 (0: none): a block of at most that many rows takes the same
// tile at that many rows, chosen per block (a shorter subtile loop; same
// columns, same K order, same bytes).
template <int BM, int WAVES, int BK, int STAGES, int MODE, int WCPOL, int SUB, int BMS = 0,
          int BMS2 = 0>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_lds_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, long long w_estride,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ nb_dev,
    const int32_t* __restrict__ order, const int32_t* __restrict__ offsets,
    void* __restrict__ out, int A, int N, int K, int ksplit, int tiles_per_block, int rotate,
    const int32_t* __restrict__ gather_perm, int gather_k, int x_rows, int xcd_group,
    int dyn_split) {
  using G = LdsGemm<BM, WAVES, BK, STAGES, MODE, SUB>;
  constexpr int MT = G::kMT, NG = G::kNG;
  __shared__ __attribute__((aligned(16))) uint8_t lds[STAGES * G::kStageBytes];

  // The split of the reduction: as launched, or with dyn_split decided here
  // from the routed block count (device_down_split; at most the launched
  // parts).
  const int n_tiles = (N + G::kTileCols - 1) / G::kTileCols;  // the last may be partial
  if (dyn_split) {
    const DownSplit ds = device_down_split(nb_dev[0], n_tiles, tiles_per_block / n_tiles, K);
    tiles_per_block = n_tiles * ds.parts;
    ksplit = ds.ksplit;
  }

  int wg = blockIdx.x;
  if (xcd_group) {
    const int r8 = (nb_dev[0] * tiles_per_block + kXcds - 1) / kXcds * kXcds;
    if (wg >= r8) return;
    wg = (wg % kXcds) * (r8 / kXcds) + wg / kXcds;
  }
  constexpr bool kDense = MODE == kOutF32Dense;
  const int bi = wg / tiles_per_block;
  if constexpr (kDense) {
    if (bi * BM >= A) return;
  } else {
    if (bi >= nb_dev[0]) return;
  }
  const int b = (!kDense && order) ? order[bi] : bi;
  const int rem = wg - bi * tiles_per_block;
  const int tile = rem % n_tiles;
  const int part = rem / n_tiles;
  const int kb = part * ksplit;
  const int e = kDense ? 0 : blocks[2 * b];
  const int r0 = kDense ? b * BM : blocks[2 * b + 1];
  const int rows = min(BM, (kDense ? A : offsets[e + 1]) - r0);
  const int nks = max(0, min(K - kb, ksplit) / BK);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = tile * G::kTileCols + wave * G::kWaveCols;
  const unsigned rkey = rotate == 2 ? (unsigned)wg : rotate == 3 ? (unsigned)e : (unsigned)b;
  const int shift = rotate ? (int)((rkey * 2654435761u) % (unsigned)max(nks, 1)) : 0;
  // a block of at most BMS2 (BMS) rows runs the same columns at BMS2 (BMS)
  // rows: fewer activation groups per stage and subtiles per wave, the same
  // K order
  if constexpr (BMS2 > 0) {
    using GS = LdsGemm<BMS2, WAVES, BK, STAGES, MODE, SUB>;
    static_assert(BMS2 < BMS && GS::kTileCols == G::kTileCols, "the smallest tile");
    if (rows <= BMS2) {
      f32x4 acc[NG][BMS2 / 16][SUB];
      lds_tile_zero<NG, BMS2 / 16, SUB>(acc);
      lds_tile_mma<BMS2, WAVES, BK, STAGES, MODE, WCPOL, SUB>(lds, X, W, w_estride, e, r0, rows,
                                                              n0, kb, N, K, nks, shift, 0, nks,
                                                              gather_perm, gather_k, x_rows, acc);
      lds_tile_store<BMS2, WAVES, BK, STAGES, MODE, SUB>(acc, out, A, N, r0, rows, n0, part);
      return;
    }
  }
  if constexpr (BMS > 0) {
    using GS = LdsGemm<BMS, WAVES, BK, STAGES, MODE, SUB>;
    static_assert(BMS < BM && GS::kTileCols == G::kTileCols && GS::kWaveCols == G::kWaveCols,
                  "the smaller tile covers the same columns");
    if (rows <= BMS) {
      f32x4 acc[NG][BMS / 16][SUB];
      lds_tile_zero<NG, BMS / 16, SUB>(acc);
      lds_tile_mma<BMS, WAVES, BK, STAGES, MODE, WCPOL, SUB>(lds, X, W, w_estride, e, r0, rows, n0,
                                                             kb, N, K, nks, shift, 0, nks,
                                                             gather_perm, gather_k, x_rows, acc);
      lds_tile_store<BMS, WAVES, BK, STAGES, MODE, SUB>(acc, out, A, N, r0, rows, n0, part);
      return;
    }
  }
  f32x4 acc[NG][MT][SUB];
  lds_tile_zero<NG, MT, SUB>(acc);
  lds_tile_mma<BM, WAVES, BK, STAGES, MODE, WCPOL, SUB>(lds, X, W, w_estride, e, r0, rows, n0, kb,
                                                        N, K, nks, shift, 0, nks, gather_perm,
                                                        gather_k, x_rows, acc);
  lds_tile_store<BM, WAVES, BK, STAGES, MODE, SUB>(acc, out, A, N, r0, rows, n0, part);
}

// The fused gate/up GEMM over a block table whose blocks hold up to 2 * BM
// rows (built on the device by the routing kernels, see VarRows): one
// workgroup per (block, column tile), and each block takes the tile of its
// size -- BM rows with SS stages, or 2 * BM rows with SL stages (the LDS of
// one CU holds three 48 KiB stages of the first or two 64 KiB stages of the
// second).  Both tiles are 8 waves x 16 columns, so a 2 * BM block reads its
// expert's weight tile once where two BM blocks would read it twice.  Each
// output sums the same 64-wide K steps in the same order whichever tile
// computes it; with the K start rotated per expert (or no rotation) the
// bytes equal those of the BM tile over the fixed-size table.
// vblocks: [*, 3] = (expert, first row, rows); vnb: their count, or -1:
// the fixed table of BM-row blocks (blocks, nb, offsets) instead.
template <int BM, int BK, int SS, int SL, int WCPOL>
__global__ __launch_bounds__(512, 1) void gemm_lds_var_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, long long w_estride,
    const int32_t* __restrict__ vblocks, const int32_t* __restrict__ vnb,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ nb_fixed,
    const int32_t* __restrict__ offsets, uint16_t* __restrict__ h, int N, int K, int rotate,
    const int32_t* __restrict__ gather_perm, int gather_k, int x_rows) {
  using GS = LdsGemm<BM, 8, BK, SS, kOutSwiGLU, 1>;
  using GL = LdsGemm<2 * BM, 8, BK, SL, kOutSwiGLU, 1>;
  static_assert(GS::kTileCols == GL::kTileCols && GS::kWaveCols == GL::kWaveCols,
                "one column tiling for both block sizes");
  constexpr int kSmallBytes = SS * GS::kStageBytes, kLargeBytes = SL * GL::kStageBytes;
  __shared__ __attribute__((aligned(16)))
      uint8_t lds[kSmallBytes > kLargeBytes ? kSmallBytes : kLargeBytes];

  const int n_tiles = (N + GS::kTileCols - 1) / GS::kTileCols;
  const int bi = blockIdx.x / n_tiles;
  const int nv = vnb[0], nf = nb_fixed[0];  // independent loads
  const bool merged = nv >= 0;
  if (bi >= (merged ? nv : nf)) return;
  const int tile = blockIdx.x - bi * n_tiles;
  int e, r0, rows;
  if (merged) {
    e = vblocks[3 * bi];
    r0 = vblocks[3 * bi + 1];
    rows = vblocks[3 * bi + 2];
  } else {
    e = blocks[2 * bi];
    r0 = blocks[2 * bi + 1];
    rows = min(BM, offsets[e + 1] - r0);
  }
  const int nks = K / BK;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = tile * GS::kTileCols + wave * GS::kWaveCols;
  const unsigned rkey = rotate == 2 ? (unsigned)blockIdx.x : rotate == 3 ? (unsigned)e : (unsigned)bi;
  const int shift = rotate ? (int)((rkey * 2654435761u) % (unsigned)max(nks, 1)) : 0;
  if (rows > BM) {
    f32x4 acc[2][2 * BM / 16][1];
    lds_tile_zero<2, 2 * BM / 16, 1>(acc);
    lds_tile_mma<2 * BM, 8, BK, SL, kOutSwiGLU, WCPOL, 1>(lds, X, W, w_estride, e, r0, rows, n0, 0,
                                                         N, K, nks, shift, 0, nks, gather_perm,
                                                         gather_k, x_rows, acc);
    lds_tile_store<2 * BM, 8, BK, SL, kOutSwiGLU, 1>(acc, h, 0, N, r0, rows, n0, 0);
  } else {
    f32x4 acc[2][BM / 16][1];
    lds_tile_zero<2, BM / 16, 1>(acc);
    lds_tile_mma<BM, 8, BK, SS, kOutSwiGLU, WCPOL, 1>(lds, X, W, w_estride, e, r0, rows, n0, 0, N,
                                                     K, nks, shift, 0, nks, gather_perm, gather_k,
                                                     x_rows, acc);
    lds_tile_store<BM, 8, BK, SS, kOutSwiGLU, 1>(acc, h, 0, N, r0, rows, n0, 0);
  }
}

// Stream-K schedule of the fused gate/up GEMM (one launch of persistent
// workgroups).  The work is every (block, column tile) unit of the schedule
// built on the device times its nks K steps: I = nb * n_tiles * nks
// iterations, of which workgroup g takes [g * I / NW, (g + 1) * I / NW) (NW =
// min(launched workgroups, I), so no range is empty).  So every workgroup
// streams the same number of weight steps whatever the routing, instead of
// one unit per workgroup in rounds of the CU count.  A workgroup
// runs the stretch of each unit its range covers; a unit covered whole is
// finished on the spot (SwiGLU, h written), a stretch of a split unit leaves
// its fp32 gate and up sums in a slot of `sk.part` (slot 2g for the first
// stretch of workgroup g, 2g + 1 for its last) and counts itself on the
// unit's counter.  The workgroup that completes the count adds the unit's
// stretches in K order (its own from registers), applies SwiGLU and writes
// h: the sum order is fixed by the unit's split points, not by which
// workgroup arrives last.  Nothing waits on another workgroup.  The routing
// kernels clear the counters on every call.
//
// Hand-off: the stretches are written with agent-scope stores, each thread
// then issues an agent-scope release fence, and after the barrier thread 0
// increments the counter (relaxed, agent scope); the workgroup whose
// increment completes the count acquires (agent scope, every thread) before
// reading the other stretches with agent-scope loads.
struct SkWork {
  float* part;   // [2 * launched workgroups] slots of NG * MT * SUB * threads f32x4
  int32_t* cnt;  // per unit, zero at entry
};

template <int BM, int WAVES, int BK, int STAGES, int WCPOL, int SUB>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_lds_sk_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, long long w_estride,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ nb_dev,
    const int32_t* __restrict__ offsets, uint16_t* __restrict__ h, int N, int K, int rotate,
    const int32_t* __restrict__ gather_perm, int gather_k, int x_rows, SkWork sk) {
  using G = LdsGemm<BM, WAVES, BK, STAGES, kOutSwiGLU, SUB>;
  constexpr int MT = G::kMT, NG = G::kNG;
  constexpr int kSlotF4 = NG * MT * SUB * G::kThreads;  // f32x4 of one slot
  __shared__ __attribute__((aligned(16))) uint8_t lds[STAGES * G::kStageBytes];
  __shared__ int completes;

  const int n_tiles = (N + G::kTileCols - 1) / G::kTileCols;
  const int nks = K / BK;
  const long long I = (long long)nb_dev[0] * n_tiles * nks;
  // With fewer iterations than workgroups only the first I take part, one
  // iteration each: every taking part workgroup has a non-empty range.
  const long long NW = min((long long)gridDim.x, I);
  const int wg = blockIdx.x;
  if (wg >= NW) return;
  const long long start = wg * I / NW, end = (wg + 1) * I / NW;
  // the workgroup whose range holds iteration i
  auto owner = [&](long long i) { return (int)(((i + 1) * NW - 1) / I); };
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  for (long long it = start; it < end;) {
    const int u = (int)(it / nks);
    const int k0 = (int)(it - (long long)u * nks);
    const int cnt = (int)min((long long)(nks - k0), end - it);
    const int b = u / n_tiles;
    const int tile = u - b * n_tiles;
    const int e = blocks[2 * b];
    const int r0 = blocks[2 * b + 1];
    const int rows = min(BM, offsets[e + 1] - r0);
    const int mt_act = (rows + 15) >> 4;
    const int n0 = tile * G::kTileCols + wave * G::kWaveCols;
    // rotation keys: per unit (in place of per workgroup), expert or block
    const unsigned rkey = rotate == 2 ? (unsigned)u : rotate == 3 ? (unsigned)e : (unsigned)b;
    const int shift = rotate ? (int)((rkey * 2654435761u) % (unsigned)nks) : 0;
    f32x4 acc[NG][MT][SUB];
    lds_tile_zero<NG, MT, SUB>(acc);
    __syncthreads();  // every wave is done with the ring of the previous stretch
    lds_tile_mma<BM, WAVES, BK, STAGES, kOutSwiGLU, WCPOL, SUB>(
        lds, X, W, w_estride, e, r0, rows, n0, 0, N, K, nks, shift, k0, cnt, gather_perm, gather_k,
        x_rows, acc);
    if (cnt == nks) {
      lds_tile_store<BM, WAVES, BK, STAGES, kOutSwiGLU, SUB>(acc, h, 0, N, r0, rows, n0, 0);
    } else {
      const int slot = 2 * wg + (it == start ? 0 : 1);
      float* ps = sk.part + (size_t)slot * kSlotF4 * 4;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (mt < mt_act) {
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
              float* q = ps + ((size_t)((g * MT + mt) * SUB + j) * G::kThreads + tid) * 4;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                __hip_atomic_store(q + i, acc[g][mt][j][i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
          }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      const long long u0 = (long long)u * nks;
      const int g_lo = owner(u0), g_hi = owner(u0 + nks - 1);
      if (tid == 0)
        completes = __hip_atomic_fetch_add(&sk.cnt[u], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == g_hi - g_lo;
      __syncthreads();
      if (completes) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        f32x4 tot[NG][MT][SUB];
        lds_tile_zero<NG, MT, SUB>(tot);
        for (int g = g_lo; g <= g_hi; ++g) {
          // the stretch of workgroup g: its first one if its range starts in this unit
          const int sl = 2 * g + ((long long)g * I / NW >= u0 ? 0 : 1);
          const float* src = sk.part + (size_t)sl * kSlotF4 * 4;
#pragma unroll
          for (int gg = 0; gg < NG; ++gg)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              if (mt < mt_act) {
#pragma unroll
                for (int j = 0; j < SUB; ++j) {
                  f32x4 v = acc[gg][mt][j];
                  if (g != wg)
                    v = AgentLoad{}(src + ((size_t)((gg * MT + mt) * SUB + j) * G::kThreads + tid) * 4);
                  tot[gg][mt][j] = g == g_lo ? v : tot[gg][mt][j] + v;
                }
              }
        }
        lds_tile_store<BM, WAVES, BK, STAGES, kOutSwiGLU, SUB>(tot, h, 0, N, r0, rows, n0, 0);
      }
    }
    it += cnt;
  }
}

constexpr int kLdsBK = 64;     // whole 128-byte lines of each weight row per step
constexpr int kLdsStages = 2;  // 2 x 80 KiB: the whole LDS of a CU at BM = 192, 7 waves
constexpr int kLdsNarrowStages = 3;  // 3 x 48 KiB at BM = 128 with one subtile per wave

// WCPOL: cache policy of the weight loads; STAGES, SUB as in LdsGemm.
template <int BM, int WAVES, int MODE, int WCPOL, int STAGES = kLdsStages, int SUB = 2, int BMS = 0,
          int BMS2 = 0>
hipError_t launch_lds_cfg(const uint16_t* X, const uint16_t* W, long long w_estride,
                          const int32_t* blocks, const int32_t* nb, const int32_t* order,
                          const int32_t* offsets, void* out, int A, int N, int K, int split,
                          int ksplit, int nb_max, int rotate, const int32_t* gather_perm,
                          int gather_k, int x_rows, int xcd_group, hipStream_t s,
                          int dyn_split = 0) {
  using G = LdsGemm<BM, WAVES, kLdsBK, STAGES, MODE, SUB>;
  // whole 16-column subtiles and whole K steps
  if (N % 16 != 0 || K % kLdsBK != 0 || ksplit % kLdsBK != 0 || split < 1)
    return hipErrorInvalidValue;
  const int tiles_per_block = (N + G::kTileCols - 1) / G::kTileCols * split;
  // XCD grouping renumbers the real workgroups rounded up to kXcds: every
  // id below that must be launched
  const long long grid = xcd_group ? ((long long)tiles_per_block * nb_max + kXcds - 1) / kXcds * kXcds
                                   : (long long)tiles_per_block * nb_max;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  gemm_lds_kernel<BM, WAVES, kLdsBK, STAGES, MODE, WCPOL, SUB, BMS, BMS2><<<(unsigned)grid, G::kThreads, 0, s>>>(
      X, W, w_estride, blocks, nb, order, offsets, out, A, N, K, ksplit, tiles_per_block, rotate,
      gather_perm, gather_k, x_rows, xcd_group, dyn_split);
  return hipGetLastError();
}

}  // namespace

int gate_up_tile_cols(int bm, int variant) {
#define X(V, BM, NWT, WV, PF) \
  if (bm == BM && variant == V) return Gemm<BM, NWT, WV, PF, kOutSwiGLU>::kTileCols;
  MOE_GU_CFGS(X)
#undef X
  if (bm == 192 && variant == kGateUpLdsVariant) return LdsGemm<192, 7, kLdsBK, kLdsStages>::kTileCols;
  if (bm == 128 && variant == kGateUpLdsVariant) return LdsGemm<128, 8, kLdsBK, kLdsStages>::kTileCols;
  if (bm == 128 && variant == kGateUpLdsNarrowVariant)
    return LdsGemm<128, 8, kLdsBK, kLdsNarrowStages, kOutSwiGLU, 1>::kTileCols;  // 128
  if (bm == 256 && variant == kGateUpLdsNarrowVariant)
    return LdsGemm<256, 8, kLdsBK, kLdsStages, kOutSwiGLU, 1>::kTileCols;  // 128
  return 0;
}

int down_tile_cols(int bm, int variant) {
#define X(V, BM, NWT, WV, PF) \
  if (bm == BM && V == variant) return Gemm<BM, NWT, WV, PF, kOutF32Parts>::kTileCols;
  MOE_DN_CFGS(X)
#undef X
  if ((bm == 192 || bm == 128 || bm == 256) && variant == kDownLdsVariant)
    return LdsGemm<192, 8, kLdsBK, kLdsStages, kOutF32Parts>::kTileCols;  // 256 at all three
  if (bm == 192 && variant == kDownLdsWideVariant)
    return LdsGemm<192, 7, kLdsBK, kLdsStages, kOutF32Wide>::kTileCols;  // 448
  if (bm == 128 && variant == kDownLdsWideVariant)
    return LdsGemm<128, 8, kLdsBK, kLdsStages, kOutF32Wide>::kTileCols;  // 512
  if (bm == 128 && variant == kDownLdsWide7Variant)
    return LdsGemm<128, 7, kLdsBK, kLdsStages, kOutF32Wide>::kTileCols;  // 448
  return 0;
}

hipError_t launch_gate_up(int bm, int variant, const uint16_t* x, const int32_t* gather_perm,
                          int k, int T, const uint16_t* w_gate_up, const int32_t* blocks,
                          const int32_t* nb, const int32_t* order, const int32_t* offsets,
                          uint16_t* h, int A, int d,
                          int ffn, int nb_max, int rotate, int xcd_group, int x_tiled,
                          hipStream_t s) {
  // The LDS-staged tiles read their weights once: non-temporal weight loads
  // (Mixtral T=512 gate/up measured 360.8 -> 334.9 us).
  if (bm == 192 && variant == kGateUpLdsVariant) {
    if (x_tiled) return hipErrorInvalidValue;  // row-major activations only
    return launch_lds_cfg<192, 7, kOutSwiGLU, kCpolNT, kLdsStages, 2, 128, 64>(x, w_gate_up, 2LL * ffn * d, blocks, nb, order,
                                              offsets, h, A, ffn, d, 1, d, nb_max, rotate,
                                              gather_perm, k, T, xcd_group, s);
  }
  // One 16-column subtile per wave and operand: 48 KiB stages, three of
  // them in LDS (more of the weight stream in flight per workgroup), and as
  // many workgroups as the register-ring tile of the same width.
  if (bm == 128 && variant == kGateUpLdsNarrowVariant) {
    if (x_tiled) return hipErrorInvalidValue;
    return launch_lds_cfg<128, 8, kOutSwiGLU, kCpolNT, kLdsNarrowStages, 1>(
        x, w_gate_up, 2LL * ffn * d, blocks, nb, order, offsets, h, A, ffn, d, 1, d, nb_max, rotate,
        gather_perm, k, T, xcd_group, s);
  }
  // At BM = 256 (asked for only): 8 waves x 16 columns, two 64 KiB stages.
  if (bm == 256 && variant == kGateUpLdsNarrowVariant) {
    if (x_tiled) return hipErrorInvalidValue;
    return launch_lds_cfg<256, 8, kOutSwiGLU, kCpolNT, kLdsStages, 1>(
        x, w_gate_up, 2LL * ffn * d, blocks, nb, order, offsets, h, A, ffn, d, 1, d, nb_max, rotate,
        gather_perm, k, T, xcd_group, s);
  }
  if (bm == 128 && variant == kGateUpLdsVariant) {
    if (x_tiled) return hipErrorInvalidValue;
    return launch_lds_cfg<128, 8, kOutSwiGLU, kCpolNT>(x, w_gate_up, 2LL * ffn * d, blocks, nb, order,
                                              offsets, h, A, ffn, d, 1, d, nb_max, rotate,
                                              gather_perm, k, T, xcd_group, s);
  }
#define X(V, BM, NWT, WV, PF)                                                                  \
  if (bm == BM && variant == V)                                                                \
    return launch_cfg<BM, NWT, WV, PF, kOutSwiGLU>(x, w_gate_up, 2LL * ffn * d, blocks, nb,      \
                                                   order, offsets, h, A, ffn, d, 1, d, nb_max, rotate,  \
                                                   gather_perm, k, x_tiled ? (A + 15) / 16 * 16 : T, \
                                                   xcd_group, x_tiled, FoldCombine{}, s);
  MOE_GU_CFGS(X)
#undef X
  return hipErrorInvalidValue;
}

size_t gate_up_sk_slot_bytes(int bm, int variant) {
  if (bm == 128 && variant == kGateUpLdsNarrowVariant) {
    using G = LdsGemm<128, 8, kLdsBK, kLdsNarrowStages, kOutSwiGLU, 1>;
    return (size_t)G::kNG * G::kMT * G::kSub * G::kThreads * 16;
  }
  return 0;
}

hipError_t launch_gate_up_sk(int bm, int variant, const uint16_t* x, const int32_t* gather_perm,
                             int k, int T, const uint16_t* w_gate_up, const int32_t* blocks,
                             const int32_t* nb, const int32_t* offsets, uint16_t* h, int d,
                             int ffn, int rotate, float* part, int32_t* cnt, hipStream_t s) {
  if (!(bm == 128 && variant == kGateUpLdsNarrowVariant)) return hipErrorInvalidValue;
  if (ffn % 16 != 0 || d % kLdsBK != 0 || d <= 0) return hipErrorInvalidValue;
  using G = LdsGemm<128, 8, kLdsBK, kLdsNarrowStages, kOutSwiGLU, 1>;
  gemm_lds_sk_kernel<128, 8, kLdsBK, kLdsNarrowStages, kCpolNT, 1>
      <<<kRoundWorkgroups, G::kThreads, 0, s>>>(x, w_gate_up, 2LL * ffn * d, blocks, nb, offsets,
                                                 h, ffn, d, rotate, gather_perm, k, T,
                                                 SkWork{part, cnt});
  return hipGetLastError();
}

hipError_t launch_gate_up_var(const uint16_t* x, const int32_t* gather_perm, int k, int T,
                              const uint16_t* w_gate_up, const int32_t* vblocks,
                              const int32_t* vnb, const int32_t* blocks, const int32_t* nb,
                              const int32_t* offsets, uint16_t* h, int d, int ffn, int nb_max,
                              int rotate, hipStream_t s) {
  if (ffn % 16 != 0 || d % kLdsBK != 0 || d <= 0 || nb_max < 0) return hipErrorInvalidValue;
  using G = LdsGemm<128, 8, kLdsBK, kLdsNarrowStages, kOutSwiGLU, 1>;
  const long long grid = (long long)(ffn + G::kTileCols - 1) / G::kTileCols * nb_max;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  gemm_lds_var_kernel<128, kLdsBK, kLdsNarrowStages, kLdsStages, kCpolNT>
      <<<(unsigned)grid, G::kThreads, 0, s>>>(x, w_gate_up, 2LL * ffn * d, vblocks, vnb, blocks,
                                             nb, offsets, h, ffn, d, rotate, gather_perm, k, T);
  return hipGetLastError();
}

// Fused gate/up SwiGLU and down projection (kOutSwiGLUDown): tiles whose
// column count is a multiple of 32 and whose h tile fits the staging LDS.
#define MOE_GUD_CFGS(X) X(1, 64, 2, 4, 4) X(1, 128, 1, 4, 4) X(0, 192, 1, 8, 3)

int gate_up_down_tile_cols(int bm, int variant) {
#define X(V, BM, NWT, WV, PF) \
  if (bm == BM && variant == V) return Gemm<BM, NWT, WV, PF, kOutSwiGLUDown>::kTileCols;
  MOE_GUD_CFGS(X)
#undef X
  return 0;
}

hipError_t launch_gate_up_down(int bm, int variant, const uint16_t* x, const int32_t* gather_perm,
                               int k, int T, const uint16_t* w_gate_up, const uint16_t* w_down,
                               const int32_t* blocks, const int32_t* nb, const int32_t* order,
                               const int32_t* offsets, float* y, int A, int d, int ffn,
                               int nb_max, int rotate, int xcd_group, int x_tiled,
                               hipStream_t s) {
#define X(V, BM, NWT, WV, PF)                                                                  \
  if (bm == BM && variant == V)                                                                \
    return launch_cfg<BM, NWT, WV, PF, kOutSwiGLUDown>(                                        \
        x, w_gate_up, 2LL * ffn * d, blocks, nb, order, offsets, y, A, ffn, d, 1, d, nb_max,    \
        rotate, gather_perm, k, x_tiled ? (A + 15) / 16 * 16 : T, xcd_group, x_tiled,          \
        FoldCombine{}, s, w_down, (long long)d * ffn, d);
  MOE_GUD_CFGS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_down(int bm, int variant, const uint16_t* h, const uint16_t* w_down,
                       const int32_t* blocks, const int32_t* nb, const int32_t* order,
                       const int32_t* offsets, float* y,
                       int A, int d, int ffn, int split, int ksplit, int nb_max, int rotate,
                       int xcd_group, const FoldCombine& fold, hipStream_t s, int dyn_split) {
  if (dyn_split && fold.cnt) return hipErrorInvalidValue;  // the fold counts parts as launched
  if ((bm == 192 || bm == 128 || bm == 256) && variant == kDownLdsVariant) {
    if (fold.cnt) return hipErrorInvalidValue;  // the fold runs in the register-ring tiles
    // Weights are read once.  Non-temporal weight loads measured faster on
    // every workload whose fp32 partials fit the 256 MiB MALL (down GEMM, µs:
    // Mixtral T=128 159 -> 143, Qwen2 T=512 245 -> 230, DeepSeek-V3 T=512
    // 1336 -> 1284) and slower where they do not (DeepSeek-V3 T=4096, 940 MB
    // of partials: down 1694 -> 1726, combination 188 -> 219).
    const bool nt = (long long)split * A * d * 4 <= (256LL << 20);
#define MOE_DOWN_LDS(BMV, CP, ST, BMS, BMS2)                                                     \
  return launch_lds_cfg<BMV, 8, kOutF32Parts, CP, ST, 2, BMS, BMS2>(h, w_down, (long long)d * ffn, blocks, nb, \
                                                  order, offsets, y, A, d, ffn, split, ksplit,    \
                                                  nb_max, rotate, nullptr, 1, A, xcd_group, s,    \
                                                  dyn_split)
    if (bm == 192) {
      if (nt) MOE_DOWN_LDS(192, kCpolNT, kLdsStages, 128, 64);
      MOE_DOWN_LDS(192, 0, kLdsStages, 128, 64);
    }
    if (bm == 256) {
      if (nt) MOE_DOWN_LDS(256, kCpolNT, kLdsStages, 0, 0);
      MOE_DOWN_LDS(256, 0, kLdsStages, 0, 0);
    }
    if (nt) MOE_DOWN_LDS(128, kCpolNT, kLdsStages, 0, 0);
    MOE_DOWN_LDS(128, 0, kLdsStages, 0, 0);
#undef MOE_DOWN_LDS
  }
  // The wide LDS-staged tile: 64 columns per wave (7 waves at BM = 192, 8 at
  // BM = 128), half the activation bytes per weight byte of the tile above;
  // the last column tile may be partial.  Non-temporal weight loads whatever
  // the size of the partials (DeepSeek-V3 T=4096, 940 MB of partials: down
  // 1663 -> 1603 us, combination 172.5 -> 185.6, pass 4603 -> 4556).
  if ((bm == 192 || bm == 128) && variant == kDownLdsWideVariant) {
    if (fold.cnt) return hipErrorInvalidValue;
    if (bm == 192)
      return launch_lds_cfg<192, 7, kOutF32Wide, kCpolNT, kLdsStages, 2, 128>(h, w_down, (long long)d * ffn, blocks, nb,
                                                         order, offsets, y, A, d, ffn, split, ksplit,
                                                         nb_max, rotate, nullptr, 1, A, xcd_group, s,
                                                         dyn_split);
    return launch_lds_cfg<128, 8, kOutF32Wide, kCpolNT>(h, w_down, (long long)d * ffn, blocks, nb,
                                                       order, offsets, y, A, d, ffn, split, ksplit,
                                                       nb_max, rotate, nullptr, 1, A, xcd_group, s,
                                                       dyn_split);
  }
  // The same tile with 7 waves at BM = 128 (448 columns)
  if (bm == 128 && variant == kDownLdsWide7Variant) {
    if (fold.cnt) return hipErrorInvalidValue;
    return launch_lds_cfg<128, 7, kOutF32Wide, kCpolNT>(h, w_down, (long long)d * ffn, blocks, nb,
                                                       order, offsets, y, A, d, ffn, split, ksplit,
                                                       nb_max, rotate, nullptr, 1, A, xcd_group, s,
                                                       dyn_split);
  }
#define X(V, BM, NWT, WV, PF)                                                                  \
  if (bm == BM && V == variant)                                                                      \
    return launch_cfg<BM, NWT, WV, PF, kOutF32Parts>(h, w_down, (long long)d * ffn, blocks, nb,  \
                                                     order, offsets, y, A, d, ffn, split, ksplit,       \
                                                     nb_max, rotate, nullptr, 1, A, xcd_group, 0,\
                                                     fold, s, nullptr, 0, 0, dyn_split);
  MOE_DN_CFGS(X)
#undef X
  return hipErrorInvalidValue;
}

// Router scores through the LDS-staged tile: logits parts [parts, T, E] of
// x [T, d] . W_r [E, d]^T, BM = 128 rows of x per block, 256 experts per
// column tile, part p over K steps [p * ksplit, (p + 1) * ksplit).
hipError_t launch_router_lds(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                             int parts, int ksplit, float* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (E % 16 != 0 || parts < 1 || (long long)(parts - 1) * ksplit >= d) return hipErrorInvalidValue;
  const int nb = (T + 127) / 128;
  return launch_lds_cfg<128, 8, kOutF32Dense, 0>(x, w_router, 0, nullptr, nullptr, nullptr, nullptr,
                                                 out, T, E, d, parts, ksplit, nb, 0, nullptr, 1, T,
                                                 0, s);
}

hipError_t launch_proj_bf16(int bm, const uint16_t* x, const int32_t* gather_perm, int k, int T,
                            const uint16_t* w, long long w_estride, const int32_t* blocks,
                            const int32_t* nb, const int32_t* order, const int32_t* offsets,
                            uint16_t* out, int A, int d,
                            int ffn, int nb_max, int rotate, int xcd_group, int x_tiled,
                            hipStream_t s) {
#define X(V, BM, NWT, WV, PF)                                                                   \
  if constexpr (V == 0) {                                                                       \
    if (bm == BM)                                                                               \
      return launch_cfg<BM, NWT, WV, PF, kOutBF16>(x, w, w_estride, blocks, nb, order, offsets,   \
                                                   out, A,                                     \
                                                   ffn, d, 1, d, nb_max, rotate, gather_perm, k, \
                                                   x_tiled ? (A + 15) / 16 * 16 : T, xcd_group,  \
                                                   x_tiled, FoldCombine{}, s);                  \
  }
  MOE_GU_CFGS(X)
#undef X
  return hipErrorInvalidValue;
}

namespace {

// h = bf16(silu(g) * u) elementwise from the bf16 gate and up products, 8
// values per thread.
__global__ __launch_bounds__(256) void swiglu_act_kernel(const uint16_t* __restrict__ g,
                                                         const uint16_t* __restrict__ u,
                                                         uint16_t* __restrict__ h, long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const bf16x8 gv = reinterpret_cast<const bf16x8*>(g)[i];
  const bf16x8 uv = reinterpret_cast<const bf16x8*>(u)[i];
  bf16x8 hv;
#pragma unroll
  for (int q = 0; q < 8; ++q) hv[q] = (__bf16)(silu_f32((float)gv[q]) * (float)uv[q]);
  reinterpret_cast<bf16x8*>(h)[i] = hv;
}

}  // namespace

hipError_t launch_swiglu_act(const uint16_t* g, const uint16_t* u, uint16_t* h, long long n,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long n8 = n / 8;
  const long long grid = (n8 + 255) / 256;
  if (n % 8 != 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  swiglu_act_kernel<<<(unsigned)grid, 256, 0, s>>>(g, u, h, n8);
  return hipGetLastError();
}

}  // namespace moe
