// Router top-K with the shared expert appended in the last slot.
//
// One wavefront per token. Each lane holds up to 4 of the E <= 255 routed
// logits; K rounds of a 64-lane max-reduction pick the experts in the order
// (logit descending, id ascending). The shared expert is then written as id E
// in slot K with the caller's coefficient (intelliparadigm, GLM4-MoE production
// optimisation, section 2.1: the shared expert becomes routed expert E+1 and
// every token takes top-(K+1); Optimizing GLM4-MoE for production, section 1:
// it always takes the last position).
#include "common.hpp"

namespace srmoe {

// Order-preserving map of a finite float to uint32 (-0 is folded into +0, so
// equal values compare equal and the id decides).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ void __launch_bounds__(256) route_topk_plus_shared_kernel(
    const float* __restrict__ logits, int T, int E, int K, float shared_weight,
    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int K1 = K + 1;
  // 64-bit keys: high word = ordered logit, low word = 255 - id (lower id wins ties).
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? ((uint64_t)ordered_key(logits[(size_t)t * E + e]) << 32) | (uint32_t)(255 - e)
                     : 0ull;
  }
  int sel_id[16];
  float sel_val[16];
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    if (k < K) {
      uint64_t best = key[0];
#pragma unroll
      for (int j = 1; j < 4; ++j) best = key[j] > best ? key[j] : best;
      best = wave_max_u64(best);
      const int e = 255 - (int)(best & 0xFFu);
      sel_id[k] = e;
      sel_val[k] = key_to_float((uint32_t)(best >> 32));
      if ((e & 63) == lane) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e >> 6 == j) key[j] = 0ull;   // taken: below every finite logit
      }
    }
  }
  // Renormalised softmax over the selected logits: p_k / sum_j p_j with the full
  // softmax denominator cancelling; exponents are taken relative to the top logit.
  // Lane k < K takes the exponent of slot k; the denominator is summed in slot order.
  float mine = 0.0f, denom = 0.0f;
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    if (k < K) {
      const float p = expf(sel_val[k] - sel_val[0]);
      denom += p;
      if (lane == k) mine = p;
    }
  }
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    if (k < K && lane == k) {
      ids[(size_t)t * K1 + k] = sel_id[k];
      w[(size_t)t * K1 + k] = __fdiv_rn(mine, denom);
    }
  }
  if (lane == K) {
    ids[(size_t)t * K1 + K] = E;
    w[(size_t)t * K1 + K] = shared_weight;
  }
}

hipError_t launch_route(const float* logits, int T, int E, int K, float shared_weight, int32_t* ids,
                        float* w, hipStream_t stream) {
  const int grid = (T + 3) / 4;
  hipLaunchKernelGGL(route_topk_plus_shared_kernel, dim3(grid), dim3(256), 0, stream, logits, T, E,
                     K, shared_weight, ids, w);
  return hipGetLastError();
}

}  // namespace srmoe
