// router.hip -- router scores: logits[T, E] = x[T, d] . W_r[E, d]^T, bf16
// inputs, fp32 accumulation and output; the step before routing.
//
// [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in Triton".
// Tokens are scored before they are routed ("The reading"); the router of
// Eq. (1)-(4) ("Assumptions & free parameters") is the standard linear map
// from a token's hidden state to one score per expert.
//
// Design: a skinny GEMM (E <= 512 columns, K = d) whose cost is reading x
// once.  One workgroup of 16 waves per tile of 16 tokens x 16 experts; the
// waves split K (wave w takes the 64-wide chunks w, w+16, ...) and each
// accumulates the whole 16x16 tile with v_mfma_f32_16x16x32_bf16 (W_r as the
// A operand, x as B: lane l holds experts e0 + 4*(l/16) + r of token
// t0 + l%16).  The 16 partial tiles are added in wave order through LDS, so
// the result does not depend on timing.  Rows past T or E load as zeros (the
// buffer range ends there) and are not stored.
#include "buffer_load.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kRouterWaves = 16;
constexpr int kRouterUnroll = 4;  // chunks in flight per wave

__global__ __launch_bounds__(kRouterWaves * 64) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    float* __restrict__ logits) {
  __shared__ f32x4 part[kRouterWaves][64];
  const int t0 = blockIdx.x * 16;
  const int e0 = blockIdx.y * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nt = min(16, T - t0);
  const int ne = min(16, E - e0);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)t0 * d), (short)0, nt * d * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wr + (size_t)e0 * d), (short)0, ne * d * 2, kRsrcWord3);
  // Lane l reads row l%16 at K offset 8*(l/16) of each 32-wide half-chunk.
  const int off = ((lane & 15) * d + (lane >> 4) * 8) * 2;
  const int nch = d / 64;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = wave; c0 < nch; c0 += kRouterUnroll * kRouterWaves) {
    bf16x8 a[kRouterUnroll][2], b[kRouterUnroll][2];
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) {
      const int soff = min(c0 + u * kRouterWaves, nch - 1) * 128;  // clamped: loads stay in range
      a[u][0] = __builtin_bit_cast(bf16x8, buf_load16(wres, off, soff));
      a[u][1] = __builtin_bit_cast(bf16x8, buf_load16(wres, off + 64, soff));
      b[u][0] = __builtin_bit_cast(bf16x8, buf_load16(xres, off, soff));
      b[u][1] = __builtin_bit_cast(bf16x8, buf_load16(xres, off + 64, soff));
    }
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) {
      if (c0 + u * kRouterWaves < nch) {  // wave-uniform
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][0], b[u][0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][1], b[u][1], acc, 0, 0, 0);
      }
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 s = part[0][lane];
    for (int w = 1; w < kRouterWaves; ++w) {
      const f32x4 q = part[w][lane];
      s[0] += q[0];
      s[1] += q[1];
      s[2] += q[2];
      s[3] += q[3];
    }
    const int t = t0 + (lane & 15);
    const int eb = e0 + 4 * (lane >> 4);
    if (t < T) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (eb + r < E) logits[(size_t)t * E + eb + r] = s[r];
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                                float* logits, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((T + 15) / 16, (E + 15) / 16);
  router_logits_kernel<<<grid, kRouterWaves * 64, 0, s>>>(x, w_router, T, d, E, logits);
  return hipGetLastError();
}

}  // namespace moe
