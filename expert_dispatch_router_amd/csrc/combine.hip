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
// routed rows in j order (combine_quad) -- no atomics, so repeated runs are
// bitwise equal.  Workgroups cover 1024 columns of one token, 4 consecutive
// columns per thread.  The down GEMM can do the same work in its epilogue
// instead (moe_options.fold_combine).
#include "combine_core.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int split,
                                                      int A, int d,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int k,
                                                      int col_blocks, uint16_t* __restrict__ out,
                                                      DynSplit dyn) {
  const int t = blockIdx.x / col_blocks;
  const int cb = blockIdx.x - t * col_blocks;
  const int c = (cb * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  // the parts the down GEMM of this call wrote (decided there from nb)
  const int parts = dyn.nb ? device_down_split(dyn.nb[0], dyn.dn_tiles, split, dyn.ffn).parts
                           : split;
  combine_quad(y, parts, A, d, inv, w, k, t, c, out, PlainLoad{});
}

}  // namespace

hipError_t launch_combine(const float* y, int split, int A, int d, const int32_t* inv,
                          const float* w, int k, int T, uint16_t* out, hipStream_t s,
                          DynSplit dyn) {
  const int col_blocks = (d / 4 + 255) / 256;
  const long long grid = (long long)col_blocks * T;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  combine_kernel<<<(unsigned)grid, 256, 0, s>>>(y, split, A, d, inv, w, k, col_blocks, out, dyn);
  return hipGetLastError();
}

}  // namespace moe
