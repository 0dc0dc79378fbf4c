// First launch of moe_layer_forward.
//
// Routing and the FP8 quantisation of x do not depend on each other, so one
// launch covers both: workgroups 0 .. ceil(T/4)-1 route 4 tokens each (one
// wavefront per token, as in the routing call), the remaining T workgroups
// each quantise one token of x (as in the quantisation stage). The results are
// the same bits the separate kernels produce.
#include "front_dev.hpp"

namespace srmoe {

template <bool kBlock>
__global__ void __launch_bounds__(256) layer_front_kernel(
    const LogitSrc logits, int T, int E, int K, float shared_weight,
    int32_t* __restrict__ ids, float* __restrict__ w, const uint16_t* __restrict__ x, int H,
    uint8_t* __restrict__ xq, float* __restrict__ sx) {
  __shared__ float red[4];
  const int route_blocks = (T + 3) / 4;
  if ((int)blockIdx.x < route_blocks) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < T) route_token_wave(logits, t, E, K, shared_weight, ids, w, nullptr);
    return;
  }
  quant_x_token<kBlock>(x, blockIdx.x - route_blocks, true, H, xq, sx, threadIdx.x, red);
}

hipError_t launch_layer_front(const LogitSrc& logits, int T, int E, int K, float shared_weight,
                              int32_t* ids, float* w, const uint16_t* x, int H, bool block,
                              uint8_t* xq, float* sx, hipStream_t stream) {
  const dim3 grid((T + 3) / 4 + T);
  if (block)
    hipLaunchKernelGGL(layer_front_kernel<true>, grid, dim3(256), 0, stream, logits, T, E, K,
                       shared_weight, ids, w, x, H, xq, sx);
  else
    hipLaunchKernelGGL(layer_front_kernel<false>, grid, dim3(256), 0, stream, logits, T, E, K,
                       shared_weight, ids, w, x, H, xq, sx);
  return hipGetLastError();
}

}  // namespace srmoe
