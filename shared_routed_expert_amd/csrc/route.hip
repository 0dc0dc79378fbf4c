// Router top-K with the shared expert appended in the last slot.
//
// One wavefront per token (4 per workgroup); see route_token_wave. The shared expert is written as id E in slot K with the
// caller's coefficient (intelliparadigm, GLM4-MoE production optimisation,
// section 2.1: the shared expert becomes routed expert E+1 and every token
// takes top-(K+1); Optimizing GLM4-MoE for production, section 1: it always
// takes the last position).
#include "front_dev.hpp"

namespace srmoe {

__global__ void __launch_bounds__(256) route_topk_plus_shared_kernel(
    const LogitSrc logits, int T, int E, int K, float shared_weight,
    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole wavefronts leave together
  route_token_wave(logits, t, E, K, shared_weight, ids, w, nullptr);
}

// The routed-only router of the unfused layer (the shared expert computed apart, as in
// the pages' unfused formulation): K entries per token, no shared slot.
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int K, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token_wave(LogitSrc{logits, nullptr, 0, 0}, t, E, K, 0.f, ids, w, nullptr, false);
}

hipError_t launch_route(const LogitSrc& logits, int T, int E, int K, float shared_weight, int32_t* ids,
                        float* w, hipStream_t stream) {
  hipLaunchKernelGGL(route_topk_plus_shared_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits,
                     T, E, K, shared_weight, ids, w);
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                             hipStream_t stream) {
  hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, K, ids, w);
  return hipGetLastError();
}

}  // namespace srmoe
