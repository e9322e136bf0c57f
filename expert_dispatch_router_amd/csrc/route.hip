// route.hip -- K1: router top-k and routing weights, one lane group per
// token (the per-token logic is in route_core.hpp).
#include "route_core.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;

template <int LPT, int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const LogitSrc logits,
                                                              int T, int E, int k, int renorm,
                                                              int score, int32_t* __restrict__ ids,
                                                              float* __restrict__ w,
                                                              ZeroRange zero) {
  constexpr int kTokPerBlock = kRouteThreads / LPT;
  for (int i = blockIdx.x * kRouteThreads + threadIdx.x; i < zero.n; i += gridDim.x * kRouteThreads)
    zero.p[i] = 0;
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / LPT;
  route_token<LPT, EPL>(logits, t, t < T, threadIdx.x & (LPT - 1), E, k, renorm, score, ids, w);
}

}  // namespace

hipError_t launch_route(const LogitSrc& logits, int T, int E, int k, int renorm, int score,
                        int32_t* ids, float* w, ZeroRange zero, hipStream_t s) {
#define MOE_LAUNCH_ROUTE(LPT, EPL)                                                        \
  {                                                                                       \
    constexpr int kTokPerBlock = kRouteThreads / LPT;                                     \
    route_kernel<LPT, EPL><<<(T + kTokPerBlock - 1) / kTokPerBlock, kRouteThreads, 0, s>>>( \
        logits, T, E, k, renorm, score, ids, w, zero);                                    \
  }
  MOE_ROUTE_SHAPES(E, MOE_LAUNCH_ROUTE);
#undef MOE_LAUNCH_ROUTE
  return hipGetLastError();
}

}  // namespace moe
