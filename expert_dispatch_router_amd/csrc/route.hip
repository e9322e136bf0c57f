// route.hip -- K1: router top-k and routing weights, one lane group per token.
//
// [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in Triton".
// Tokens are scored and their top-k experts chosen ("The reading"); the
// score is a softmax or a sigmoid of the router logits ("Assumptions & free
// parameters", paper Eq. (1)-(4)).
//
// Selection key: the raw fp32 logit (softmax and sigmoid are increasing, so
// the chosen set is the same; comparing logits keeps equal-score cases that
// rounding would create, e.g. saturated sigmoids, ordered).  Equal logits --
// IEEE equality, so -0 == +0 -- rank the lower expert first.  The order of
// the k results is descending key.
//
// Mapping: a group of LPT lanes (a power of two, LPT = min(64, E rounded up))
// owns one token; lane `sub` of the group holds experts sub, sub+LPT, ...
// (EPL of them).  Each of the k rounds takes each lane's best unselected
// candidate and reduces it over the group with xor-butterfly shuffles; the
// group agrees on the winner because the rank order is total.
#include "moe_internal.hpp"
#include "../../include/moe.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;

// a ranks before b; an index < 0 means "no candidate" and ranks last.
__device__ __forceinline__ bool ranks_before(float va, int ea, float vb, int eb) {
  if (ea < 0) return false;
  if (eb < 0) return true;
  return va > vb || (va == vb && ea < eb);
}

template <int LPT, int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ logits,
                                                              int T, int E, int k, int renorm,
                                                              int score, int32_t* __restrict__ ids,
                                                              float* __restrict__ w) {
  constexpr int kTokPerBlock = kRouteThreads / LPT;
  const int sub = threadIdx.x & (LPT - 1);
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / LPT;
  const bool tok_ok = t < T;

  float v[EPL];
  unsigned live = 0;  // bit i set: expert sub + i*LPT exists and is not yet chosen
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = sub + i * LPT;
    const bool ok = tok_ok && e < E;
    v[i] = ok ? logits[(size_t)t * E + e] : 0.0f;
    live |= ok ? (1u << i) : 0u;
  }

  float sel_v[MOE_MAX_TOPK];
  int sel_e[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    sel_v[j] = 0.0f;
    sel_e[j] = -1;
    if (j < k) {
      float bv = 0.0f;
      int be = -1;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = sub + i * LPT;
        if (((live >> i) & 1u) && ranks_before(v[i], e, bv, be)) {
          bv = v[i];
          be = e;
        }
      }
#pragma unroll
      for (int off = LPT / 2; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oe = __shfl_xor(be, off, 64);
        if (ranks_before(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      sel_v[j] = bv;
      sel_e[j] = be;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (sub + i * LPT == be) live &= ~(1u << i);
    }
  }

  // Routing weights of the selected experts (fp32).
  float wt[MOE_MAX_TOPK];
  if (score == MOE_SCORE_SOFTMAX) {
    const float m = sel_v[0];  // the largest logit of the token
    float z = 0.0f;
    if (renorm) {
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j)
        if (j < k) z += expf(sel_v[j] - m);
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = sub + i * LPT;
        if (tok_ok && e < E) z += expf(v[i] - m);
      }
#pragma unroll
      for (int off = LPT / 2; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) wt[j] = (j < k) ? expf(sel_v[j] - m) / z : 0.0f;
  } else {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      wt[j] = (j < k) ? 1.0f / (1.0f + expf(-sel_v[j])) : 0.0f;
      s += wt[j];
    }
    if (renorm) {
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j) wt[j] = wt[j] / s;
    }
  }

  if (tok_ok) {
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && sub == j) {
        ids[(size_t)t * k + j] = sel_e[j];
        w[(size_t)t * k + j] = wt[j];
      }
    }
  }
}

template <int LPT, int EPL>
hipError_t launch(const float* logits, int T, int E, int k, int renorm, int score, int32_t* ids,
                  float* w, hipStream_t s) {
  constexpr int kTokPerBlock = kRouteThreads / LPT;
  const int grid = (T + kTokPerBlock - 1) / kTokPerBlock;
  route_kernel<LPT, EPL><<<grid, kRouteThreads, 0, s>>>(logits, T, E, k, renorm, score, ids, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int renorm, int score,
                        int32_t* ids, float* w, hipStream_t s) {
  // Every lane of a group must hold at least one candidate whenever k <= E:
  // k <= 16 <= LPT for E > 16, and k <= E <= LPT otherwise.
  if (E <= 8) return launch<8, 1>(logits, T, E, k, renorm, score, ids, w, s);
  if (E <= 16) return launch<16, 1>(logits, T, E, k, renorm, score, ids, w, s);
  if (E <= 32) return launch<32, 1>(logits, T, E, k, renorm, score, ids, w, s);
  if (E <= 64) return launch<64, 1>(logits, T, E, k, renorm, score, ids, w, s);
  if (E <= 128) return launch<64, 2>(logits, T, E, k, renorm, score, ids, w, s);
  if (E <= 256) return launch<64, 4>(logits, T, E, k, renorm, score, ids, w, s);
  return launch<64, 8>(logits, T, E, k, renorm, score, ids, w, s);
}

}  // namespace moe
