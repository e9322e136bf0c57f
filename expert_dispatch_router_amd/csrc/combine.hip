// combine.hip -- K6: weighted combination of the expert outputs.
//
// [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in Triton".
// The expert results are scattered back to token order, each scaled by its
// routing weight and summed ("The reading"; abstract: weighted output
// combination).  Reading: the weight multiplies the down projection's
// output, i.e. out[t] = sum_j w[t,j] * y[inv[t*k+j]].
//
// Deterministic by construction: each output element is owned by one thread
// that adds the split partials of a routed row in split order and the k
// routed rows in j order -- no atomics, so repeated runs are bitwise equal.
// Workgroups cover 1024 columns of one token, 4 consecutive columns per thread.
#include "moe_internal.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int split,
                                                      int A, int d,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int k,
                                                      int col_blocks, uint16_t* __restrict__ out) {
  const int t = blockIdx.x / col_blocks;
  const int cb = blockIdx.x - t * col_blocks;
  const int c = (cb * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const size_t row = (size_t)inv[(size_t)t * k + j];
    const float wj = w[(size_t)t * k + j];
    f32x4 v = *reinterpret_cast<const f32x4*>(y + row * d + c);
    for (int s = 1; s < split; ++s)
      v += *reinterpret_cast<const f32x4*>(y + ((size_t)s * A + row) * d + c);
    acc += wj * v;
  }
  bf16x4 o;
  o[0] = (__bf16)acc[0];
  o[1] = (__bf16)acc[1];
  o[2] = (__bf16)acc[2];
  o[3] = (__bf16)acc[3];
  *reinterpret_cast<bf16x4*>(out + (size_t)t * d + c) = o;
}

}  // namespace

hipError_t launch_combine(const float* y, int split, int A, int d, const int32_t* inv,
                          const float* w, int k, int T, uint16_t* out, hipStream_t s) {
  const int col_blocks = (d / 4 + 255) / 256;
  const long long grid = (long long)col_blocks * T;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  combine_kernel<<<(unsigned)grid, 256, 0, s>>>(y, split, A, d, inv, w, k, col_blocks, out);
  return hipGetLastError();
}

}  // namespace moe
