// FP8 activation quantisation: x per token before the gate/up GEMM, and the
// SwiGLU product `a` per sorted row before the down GEMM. Scale = amax / 448
// (1 when amax == 0), code = E4M3FN(v / scale) with round-to-nearest-even and
// saturation; the whole decision is taken in float32. Per-channel mode uses
// one scale per row; block mode one per row and 128-column group. (The pages
// run the layer in FP8 E4M3: intelliparadigm section 3.1; Optimizing GLM4-MoE
// for production, benchmark configuration.)
#include "front_dev.hpp"

namespace srmoe {

// x [T,H] bf16 -> xq [T,H] e4m3, sx [T] or [T,H/128]: one 256-thread workgroup per token.
template <bool kBlock>
__global__ void __launch_bounds__(256) quant_x_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                      uint8_t* __restrict__ xq, float* __restrict__ sx) {
  __shared__ float red[4];
  quant_x_token<kBlock>(x, blockIdx.x, true, H, xq, sx, threadIdx.x, red);
}

// a [P,I] float32 -> aq [P,I] e4m3, sa [P] or [P,I/128].
// It also writes each sorted row's output scale for the down GEMM: the row's
// routing weight topk_w[s] (0 for padding rows), times the row's FP8 scale in
// per-channel mode. One 256-thread workgroup per 16 rows, 16 threads (one DPP
// row) per sorted row; each thread takes 4 consecutive values per 64-wide stripe.
template <bool kBlock>
__global__ void __launch_bounds__(256) quant_a_kernel(const float* __restrict__ a, int I,
                                                      const int32_t* __restrict__ sorted,
                                                      const float* __restrict__ topk_w, int sentinel,
                                                      const int32_t* __restrict__ num_padded,
                                                      uint8_t* __restrict__ aq, float* __restrict__ sa,
                                                      float* __restrict__ row_scale) {
  // Rows past the used blocks (a multiple of 16 rows) are skipped: no GEMM reads them.
  if ((int)blockIdx.x * 16 >= num_padded[0]) return;
  const int p = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  const float* row = a + (size_t)p * I;
  uint8_t* qrow = aq + (size_t)p * I;
  float wgt = 0.f;
  if (part == 0) {
    const int s = sorted[p];
    if (s < sentinel) wgt = topk_w[s];
  }
  if (!kBlock) {
    // one pass for I <= 512 (8 stripes of 4 values per thread), else two
    constexpr int kMaxStripes = 8;
    float4 v[kMaxStripes];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxStripes; ++j) {
      const int i = j * 64 + part * 4;
      v[j] = i < I ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    }
    for (int i = kMaxStripes * 64 + part * 4; i < I; i += 64) {
      const float4 w = *reinterpret_cast<const float4*>(row + i);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w))));
    }
    const float scale = fp8_scale(row16_max(amax));
    if (part == 0) {
      sa[p] = scale;
      row_scale[p] = wgt * scale;
    }
    const ScaleDiv q = scale_div(scale);
#pragma unroll
    for (int j = 0; j < kMaxStripes; ++j) {
      const int i = j * 64 + part * 4;
      if (i < I)
        *reinterpret_cast<uint32_t*>(qrow + i) = quant2(q, v[j].x, v[j].y) | (quant2(q, v[j].z, v[j].w) << 16);
    }
    for (int i = kMaxStripes * 64 + part * 4; i < I; i += 64) {
      const float4 w = *reinterpret_cast<const float4*>(row + i);
      *reinterpret_cast<uint32_t*>(qrow + i) = quant2(q, w.x, w.y) | (quant2(q, w.z, w.w) << 16);
    }
  } else {
    if (part == 0) row_scale[p] = wgt;
    // 128-column groups in batches of 4, every load of a batch issued before any is used;
    // a group is the row's 16 threads x 2 float4 (columns g + 4 part + 64 j)
    constexpr int kBatch = 4;
    for (int g0 = 0; g0 < I; g0 += kBatch * kGroup) {
      float4 v[kBatch][2];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int g = g0 + b * kGroup;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          v[b][j] = g < I ? *reinterpret_cast<const float4*>(row + g + part * 4 + 64 * j)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int g = g0 + b * kGroup;
        if (g >= I) break;
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[b][j].x), fabsf(v[b][j].y)), fmaxf(fabsf(v[b][j].z), fabsf(v[b][j].w))));
        const float scale = fp8_scale(row16_max(amax));
        if (part == 0) sa[(size_t)p * (I / kGroup) + g / kGroup] = scale;
        const ScaleDiv q = scale_div(scale);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          *reinterpret_cast<uint32_t*>(qrow + g + part * 4 + 64 * j) =
              quant2(q, v[b][j].x, v[b][j].y) | (quant2(q, v[b][j].z, v[b][j].w) << 16);
      }
    }
  }
}

hipError_t launch_quant_x(const uint16_t* x, int T, int H, bool block, uint8_t* xq, float* sx,
                          hipStream_t stream) {
  const dim3 grid(T), blk(256);
  if (block)
    hipLaunchKernelGGL(quant_x_kernel<true>, grid, blk, 0, stream, x, T, H, xq, sx);
  else
    hipLaunchKernelGGL(quant_x_kernel<false>, grid, blk, 0, stream, x, T, H, xq, sx);
  return hipGetLastError();
}

hipError_t launch_quant_a(const float* a, int P_max, int I, bool block, const int32_t* sorted,
                          const float* topk_w, int sentinel, const int32_t* num_padded, uint8_t* aq,
                          float* sa, float* row_scale, hipStream_t stream) {
  const dim3 grid(P_max / 16), blk(256);
  if (block)
    hipLaunchKernelGGL(quant_a_kernel<true>, grid, blk, 0, stream, a, I, sorted, topk_w, sentinel, num_padded, aq, sa, row_scale);
  else
    hipLaunchKernelGGL(quant_a_kernel<false>, grid, blk, 0, stream, a, I, sorted, topk_w, sentinel, num_padded, aq, sa, row_scale);
  return hipGetLastError();
}

}  // namespace srmoe
