// combine_core.hpp -- one output quad of the weighted combination, shared by
// the combination kernel and the down GEMM's folded epilogue so that both
// produce the same bytes.
//
// [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in Triton".
// The expert results are scattered back to token order, each scaled by its
// routing weight and summed ("The reading"; abstract: weighted output
// combination): out[t] = sum_j w[t,j] * y[inv[t*k+j]], where y of a routed
// row is the sum of its split partials.  The order is fixed -- split parts
// ascending inside each routed row, then j ascending -- so the result does
// not depend on which thread or workgroup computes it.
#pragma once
#include "moe_internal.hpp"

namespace moe {

// Loads of y: plain (after a kernel boundary; non-temporal, since every
// partial is read exactly once -- DeepSeek-V3 T=4096's combination measured
// 189.9 -> 173.9 us), or agent-scope atomic loads, which read the
// device-coherent value written by another workgroup of the same kernel
// without touching this XCD's L2 contents.
struct PlainLoad {
  __device__ __forceinline__ f32x4 operator()(const float* p) const {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  }
};
struct AgentLoad {
  __device__ __forceinline__ f32x4 operator()(const float* p) const {
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
  }
};

// out[t, c .. c+3] from y [split, A, d] fp32.
template <class Load>
__device__ __forceinline__ void combine_quad(const float* __restrict__ y, int split, int A,
                                             int d, const int32_t* __restrict__ inv,
                                             const float* __restrict__ w, int k, int t, int c,
                                             uint16_t* __restrict__ out, Load load) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const size_t row = (size_t)inv[(size_t)t * k + j];
    const float wj = w[(size_t)t * k + j];
    f32x4 v = load(y + row * d + c);
    for (int s = 1; s < split; ++s) v += load(y + ((size_t)s * A + row) * d + c);
    acc += wj * v;
  }
  bf16x4 o;
  o[0] = (__bf16)acc[0];
  o[1] = (__bf16)acc[1];
  o[2] = (__bf16)acc[2];
  o[3] = (__bf16)acc[3];
  *reinterpret_cast<bf16x4*>(out + (size_t)t * d + c) = o;
}

}  // namespace moe
