// router.hip -- router scores: logits[T, E] = x[T, d] . W_r[E, d]^T, bf16
// inputs, fp32 accumulation and output; the step before routing.
//
// [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in Triton".
// Tokens are scored before they are routed ("The reading"); the router of
// Eq. (1)-(4) ("Assumptions & free parameters") is the standard linear map
// from a token's hidden state to one score per expert.
//
// Design: a skinny GEMM (E <= 512 columns, K = d) whose cost is reading x
// and W_r; with a few hundred tokens there are too few (token, expert)
// tiles to fill the chip, so the reduction over d is split into `parts`
// contiguous ranges (bounded so the partial sums move fewer bytes than x).
// One wave computes a tile of 16*TS tokens x 16*NSUB experts over one range
// with v_mfma_f32_16x16x32_bf16 (W_r as the A operand, x as B: lane l holds
// experts e0 + 4*(l/16) + r of token t0 + l%16 in each 16x16 subtile),
// streaming its range through a ring of RING chunks; each x fragment serves
// NSUB MFMAs and each W_r fragment TS.  The reads of x and W_r beyond the
// first come from L2 (x once per expert tile, W_r once per token tile), so
// large problems take the 64 x 64 tile (4 x 4 subtiles, a 2-deep ring to
// stay within two waves per SIMD).  A workgroup's 4 waves are 2
// token tiles x 2 expert tiles (4 token tiles when E fits one expert tile),
// so waves sharing rows read them together.  With one part the wave writes
// the logits; otherwise it writes its partial sums [part][T][E], which the
// routing kernels (or launch_router_reduce) add in part order -- the result
// does not depend on timing.  Rows past T or E load as zeros (the buffer
// range ends there) and are not stored.  Large problems (T >= 1024,
// E >= 128) instead run the expert GEMMs' LDS-staged tile in its dense
// mode (plan_router below).
#include "buffer_load.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kRouterWaves = 4;      // waves per workgroup: 2 token tiles x 2 expert tiles
constexpr int kRouterTargetWaves = 1024;

template <int TS, int NSUB, int RING>  // RING: 64-wide K chunks in flight per wave
__global__ __launch_bounds__(kRouterWaves * 64) void router_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    int parts, int wg_e, float* __restrict__ out) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  // wg_e expert tiles x (4 / wg_e) token tiles per workgroup: waves that
  // share a token tile (or an expert tile) read the same rows together.
  const int wg_t = kRouterWaves / wg_e;
  const int t0 = (blockIdx.x * wg_t + wave / wg_e) * (16 * TS);
  const int e0 = (blockIdx.y * wg_e + wave % wg_e) * (16 * NSUB);
  if (t0 >= T || e0 >= E) return;  // wave-uniform; no barrier below
  const int part = blockIdx.z;
  const int nch = d / 64;
  const int c0 = (int)((long long)part * nch / parts);
  const int c1 = (int)((long long)(part + 1) * nch / parts);
  const int nt = min(16 * TS, T - t0);
  const int ne = min(16 * NSUB, E - e0);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)t0 * d), (short)0, nt * d * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wr + (size_t)e0 * d), (short)0, ne * d * 2, kRsrcWord3);
  // Lane l reads row l%16 of each 16-row subtile at K offset 8*(l/16) of
  // each 32-wide half-chunk.
  const int off = ((lane & 15) * d + (lane >> 4) * 8) * 2;
  const int sub = 16 * d * 2;  // bytes between 16-row subtiles
  f32x4 acc[TS][NSUB];
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Ring of RING chunks; chunk c lives in slot (c - c0) % RING.
  // Every reload is unconditional (clamped to the last chunk), so the
  // compiler's wait before a slot's MFMAs covers exactly that slot.
  bf16x8 rb[RING][TS][2], ra[RING][NSUB][2];
  auto load = [&](int u, int c) {
    const int soff = min(c, c1 - 1) * 128;
#pragma unroll
    for (int i = 0; i < TS; ++i) {
      rb[u][i][0] = __builtin_bit_cast(bf16x8, buf_load16(xres, off + i * sub, soff));
      rb[u][i][1] = __builtin_bit_cast(bf16x8, buf_load16(xres, off + i * sub + 64, soff));
    }
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      ra[u][j][0] = __builtin_bit_cast(bf16x8, buf_load16(wres, off + j * sub, soff));
      ra[u][j][1] = __builtin_bit_cast(bf16x8, buf_load16(wres, off + j * sub + 64, soff));
    }
  };
#pragma unroll
  for (int u = 0; u < RING; ++u) load(u, c0 + u);
  for (int cb = c0; cb < c1; cb += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      if (cb + u < c1) {  // wave-uniform
#pragma unroll
        for (int i = 0; i < TS; ++i)
#pragma unroll
          for (int j = 0; j < NSUB; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[u][j][0], rb[u][i][0],
                                                                acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[u][j][1], rb[u][i][1],
                                                                acc[i][j], 0, 0, 0);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
      load(u, cb + u + RING);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float* dst = out + (size_t)part * T * E;
#pragma unroll
  for (int i = 0; i < TS; ++i) {
    const int t = t0 + i * 16 + (lane & 15);
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      const int eb = e0 + j * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (eb + r < E) dst[(size_t)t * E + eb + r] = acc[i][j][r];
    }
  }
}

// logits[i] = sum over parts of parts[q][i], in part order.
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ parts,
                                                            int nparts, long long n,
                                                            float* __restrict__ logits) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = parts[i];
  for (int q = 1; q < nparts; ++q) v += parts[(size_t)q * n + i];
  logits[i] = v;
}

}  // namespace

// Large problems (T >= 1024, E >= 128, E a multiple of 16) take the
// LDS-staged GEMM tile of the expert GEMMs in its dense mode: a workgroup
// stages 128 rows of x and 256 rows of W_r per K step in LDS, so x is read
// once per 256 experts and W_r once per 128 tokens (the wave tiles above
// read them once per 64).  The split over d is sized for about one round of
// workgroups, under the same bounds as above.
constexpr int kRouterLdsRows = 128;
constexpr int kRouterLdsCols = 256;

RouterPlan plan_router(int T, int d, int E) {
  RouterPlan rp;
  rp.lds = 0;
  rp.ksplit = 0;
  const bool lds_ok = T >= 1024 && E >= 128 && E % 16 == 0 && d % 64 == 0 &&
                      (long long)(E + kRouterLdsCols) * d * 2 < (1LL << 31) &&
                      (long long)kRouterLdsRows * d * 2 < (1LL << 31);
  if (lds_ok) {
    const int nch = d / 64;
    const long long wgs = (long long)((T + kRouterLdsRows - 1) / kRouterLdsRows) *
                          ((E + kRouterLdsCols - 1) / kRouterLdsCols);
    long long parts = (256 + wgs - 1) / wgs;
    parts = std::min<long long>(parts, std::max(1, nch / 4));
    parts = std::min<long long>(parts, std::max(1, d / (4 * E)));
    parts = std::max<long long>(parts, 1);
    const int per = (int)((nch + parts - 1) / parts);  // K steps per part
    rp.lds = 1;
    rp.ts = rp.nsub = 0;
    rp.parts = (nch + per - 1) / per;  // every part has at least one K step
    rp.ksplit = per * 64;
    return rp;
  }
  // 64-row tiles of x and W_r need 64*d*2 bytes within a 32-bit buffer range
  const bool wide_ok = 128LL * d < (1LL << 31);
  rp.ts = (T >= 1024 && wide_ok) ? 4 : T >= 64 ? 2 : 1;
  rp.nsub = (E >= 128 && rp.ts == 4) ? 4 : E <= 16 ? 1 : 2;
  const long long tiles = (long long)((T + 16 * rp.ts - 1) / (16 * rp.ts)) *
                          ((E + 16 * rp.nsub - 1) / (16 * rp.nsub));
  const int nch = d / 64;
  long long parts = tiles > 0 ? (kRouterTargetWaves + tiles - 1) / tiles : 1;
  // at least 4 chunks per part, and partial sums (written and read once)
  // of no more bytes than x itself: parts * 8*T*E <= 2*T*d
  parts = std::min<long long>(parts, std::max(1, nch / 4));
  parts = std::min<long long>(parts, std::max(1, d / (4 * E)));
  rp.parts = (int)std::max<long long>(parts, 1);
  return rp;
}

hipError_t launch_router(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                         const RouterPlan& rp, float* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (rp.lds) return launch_router_lds(x, w_router, T, d, E, rp.parts, rp.ksplit, out, s);
  const int e_tiles = (E + 16 * rp.nsub - 1) / (16 * rp.nsub);
  const int wg_e = e_tiles >= 2 ? 2 : 1;
  const int wg_t = kRouterWaves / wg_e;
  const int t_tiles = (T + 16 * rp.ts - 1) / (16 * rp.ts);
  const dim3 grid((t_tiles + wg_t - 1) / wg_t, (e_tiles + wg_e - 1) / wg_e, rp.parts);
#define MOE_ROUTER(TS, NSUB, RING)                                                             \
  if (rp.ts == TS && rp.nsub == NSUB) {                                                        \
    router_kernel<TS, NSUB, RING><<<grid, kRouterWaves * 64, 0, s>>>(x, w_router, T, d, E,      \
                                                                     rp.parts, wg_e, out);     \
    return hipGetLastError();                                                                  \
  }
  MOE_ROUTER(1, 1, 4) MOE_ROUTER(1, 2, 4) MOE_ROUTER(2, 1, 4) MOE_ROUTER(2, 2, 4)
  MOE_ROUTER(4, 1, 2) MOE_ROUTER(4, 2, 2) MOE_ROUTER(4, 4, 2)
#undef MOE_ROUTER
  return hipErrorInvalidValue;
}

hipError_t launch_router_reduce(const float* parts, int nparts, long long n, float* logits,
                                hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long grid = (n + 255) / 256;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  router_reduce_kernel<<<(unsigned)grid, 256, 0, s>>>(parts, nparts, n, logits);
  return hipGetLastError();
}

}  // namespace moe
