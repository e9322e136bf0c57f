// route_core.hpp -- the per-token router top-k and weights, shared by the
// routing kernels: the rank order of candidates, the weights of a selection,
// and one token routed by a group of LPT lanes.
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
// Mapping: a group of LPT lanes (a power of two up to 64; the many-workgroup
// route takes E rounded up, the one-workgroup kernel fewer) owns one token;
// lane `sub` of the group holds experts sub, sub+LPT, ... (EPL of them).  Each of the k rounds takes each lane's best unselected
// candidate and reduces it over the group with xor-butterfly shuffles; the
// group agrees on the winner because the rank order is total.
#pragma once

#include "moe_internal.hpp"
#include "../../include/moe.h"

namespace moe {

// a ranks before b; an index < 0 means "no candidate" and ranks last.
__device__ __forceinline__ bool ranks_before(float va, int ea, float vb, int eb) {
  if (ea < 0) return false;
  if (eb < 0) return true;
  return va > vb || (va == vb && ea < eb);
}

// Weights of the k selected logits sel_v (descending): softmax over the
// selection (renorm), softmax over all experts with denominator z_all
// (computed by the caller as the sum of exp(logit - sel_v[0])), or sigmoid,
// optionally divided by the sum of the k sigmoids.
__device__ __forceinline__ void topk_weights(const float* sel_v, int k, int renorm, int score,
                                             float z_all, float* wt) {
  // Entries past k (uniform over the launch) are not computed: each block
  // below holds an empty volatile asm statement, which the compiler may not
  // speculate, so it stays a branch on k instead of becoming a computed
  // exponential and a select.  Entries past k stay 0 and are never used; the
  // sums and quotients are the same operations in the same order.
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) wt[j] = 0.0f;
  if (score == MOE_SCORE_SOFTMAX) {
    const float m = sel_v[0];  // the largest logit of the token
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j < k) {
        asm volatile("");
        wt[j] = expf(sel_v[j] - m);
      }
    float z = z_all;
    if (renorm) {
      z = 0.0f;
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j)
        if (j < k) z += wt[j];
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j < k) {
        asm volatile("");
        wt[j] = wt[j] / z;
      }
  } else {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j < k) {
        asm volatile("");
        wt[j] = 1.0f / (1.0f + expf(-sel_v[j]));
        s += wt[j];
      }
    if (renorm) {
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j)
        if (j < k) {
          asm volatile("");
          wt[j] = wt[j] / s;
        }
    }
  }
}

// Routes token t (all LPT lanes of its group call this; tok_ok is false for
// padding groups past the last token).  The whole group ends with all k
// results; lane j mod LPT writes entry j: ids[t*k + j] and w[t*k + j].
// sel, if given: the ids also go to sel[t*k + j] (an LDS copy for the
// one-workgroup kernel).
template <int LPT, int EPL>
__device__ __forceinline__ void route_token(const LogitSrc& logits, int t, bool tok_ok,
                                            int sub, int E, int k, int renorm, int score,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            uint8_t* sel = nullptr) {
  float v[EPL];
  unsigned live = 0;  // bit i set: expert sub + i*LPT exists and is not yet chosen
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = sub + i * LPT;
    const bool ok = tok_ok && e < E;
    v[i] = ok ? load_logit(logits, (size_t)t * E + e) : 0.0f;
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
  float z_all = 0.0f;  // full softmax denominator, only without renormalisation
  if (score == MOE_SCORE_SOFTMAX && !renorm) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = sub + i * LPT;
      if (tok_ok && e < E) z_all += expf(v[i] - sel_v[0]);
    }
#pragma unroll
    for (int off = LPT / 2; off >= 1; off >>= 1) z_all += __shfl_xor(z_all, off, 64);
  }
  float wt[MOE_MAX_TOPK];
  topk_weights(sel_v, k, renorm, score, z_all, wt);

  if (tok_ok) {
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && (j & (LPT - 1)) == sub) {
        ids[(size_t)t * k + j] = sel_e[j];
        w[(size_t)t * k + j] = wt[j];
        if (sel) sel[t * k + j] = (uint8_t)sel_e[j];
      }
    }
  }
}

// Expands CALL(LPT, EPL) for the lane-group shape of E experts used by the
// many-workgroup route: LPT = E rounded up to a power of two, between 8 and
// 64; EPL = the experts per lane.
#define MOE_ROUTE_SHAPES(E, CALL) \
  do {                            \
    if ((E) <= 8) {               \
      CALL(8, 1);                 \
    } else if ((E) <= 16) {       \
      CALL(16, 1);                \
    } else if ((E) <= 32) {       \
      CALL(32, 1);                \
    } else if ((E) <= 64) {       \
      CALL(64, 1);                \
    } else if ((E) <= 128) {      \
      CALL(64, 2);                \
    } else if ((E) <= 256) {      \
      CALL(64, 4);                \
    } else {                      \
      CALL(64, 8);                \
    }                             \
  } while (0)

}  // namespace moe
