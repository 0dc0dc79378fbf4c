// Grouped expert GEMMs of the fused MoE layer on the gfx950 fp8 matrix cores.
//
// After the align step every block of block_m sorted rows belongs to a single
// expert (the shared expert included: it is just expert E with T rows), so
// both GEMMs run as one grid over (row block, output tile) -- the one grouped
// pass over all K+1 slots that the fusion asks for (Optimizing GLM4-MoE for
// production, section 1: shared and routed experts have the same shapes and
// compute flow, so one structure serves both).
//
// gate_up: a[p, i] = silu(g) * u, g/u = dequantised x_q[t] . w13[e] rows i / I+i
// down:    slot_out[s, h] = bf16( w[s] * dequantised a_q[p] . w2[e] row h )
//
// Each wavefront owns 16 output columns per MFMA tile and all block_m/16 row
// tiles of its block; operands are loaded straight from global memory in the
// MFMA's register layout (lane: row/column l & 15, 32 K-bytes at 32 * (l >> 4)).
#include "common.hpp"

namespace srmoe {

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Decode-shaped gate_up (block_m == 16): the weights stream from HBM once and each
// byte feeds a single MFMA, so the kernel is organised for memory-level
// parallelism. grid: (P_max / 16, I / 16); one workgroup per (row block, 16
// intermediate columns), its 4 wavefronts splitting K = H four ways, each
// issuing kPrefetch K-steps of loads ahead of its MFMAs. The partial tiles are
// summed through LDS in a fixed order, then scaled, passed through SiLU * up
// and stored as float32.
template <bool kBlock>
__global__ void __launch_bounds__(256) gate_up_skinny_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ sx, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ a_out, int T, int H, int I, int K1) {
  constexpr int kPrefetch = 4;
  __shared__ float red[4][2][16][17];
  const int b = blockIdx.x;
  if (b * 16 >= *num_padded) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int col0 = blockIdx.y * 16;
  const int e = block_expert[b];
  const int sentinel = T * K1;
  const int HB = H / kGroup;
  const int nsteps = H / kGroup;
  const int s0 = wv * nsteps / 4, s1 = (wv + 1) * nsteps / 4;

  const int s_in = sorted[b * 16 + r16];
  const bool avalid = s_in < sentinel;
  const uint8_t* arow = xq + (size_t)(avalid ? s_in / K1 : 0) * H + kq * 32;
  const uint8_t* gp = w13 + ((size_t)e * 2 * I + col0 + r16) * H + kq * 32;
  const uint8_t* upp = gp + (size_t)I * H;
  int otok[4];
  if (kBlock) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = sorted[b * 16 + 4 * kq + j];
      otok[j] = s < sentinel ? s / K1 : -1;
    }
  }
  const size_t sg_base = ((size_t)e * (2 * I / kGroup) + col0 / kGroup) * HB;
  const size_t su_base = ((size_t)e * (2 * I / kGroup) + (I + col0) / kGroup) * HB;

  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f accg = zero4, accu = zero4;
  for (int st = s0; st < s1; st += kPrefetch) {
    v8i A[kPrefetch], G[kPrefetch], U[kPrefetch];
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      const bool ok = st + j < s1;
      const size_t k = (size_t)(st + j) * kGroup;
      A[j] = (ok && avalid) ? load32(arow + k) : zero8;
      G[j] = ok ? load32(gp + k) : zero8;
      U[j] = ok ? load32(upp + k) : zero8;
    }
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      if (!kBlock) {
        accg = mfma_16x16x128_fp8(A[j], G[j], accg);
        accu = mfma_16x16x128_fp8(A[j], U[j], accu);
      } else if (st + j < s1) {
        const int kb = st + j;
        const v4f tg = mfma_16x16x128_fp8(A[j], G[j], zero4);
        const v4f tu = mfma_16x16x128_fp8(A[j], U[j], zero4);
        const float swg = s13[sg_base + kb], swu = s13[su_base + kb];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sxv = otok[q] >= 0 ? sx[(size_t)otok[q] * HB + kb] : 0.f;
          accg[q] += tg[q] * (sxv * swg);
          accu[q] += tu[q] * (sxv * swu);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    red[wv][0][4 * kq + q][r16] = accg[q];
    red[wv][1][4 * kq + q][r16] = accu[q];
  }
  __syncthreads();
  const int row = threadIdx.x >> 4, c = threadIdx.x & 15;
  float g = red[0][0][row][c], u = red[0][1][row][c];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    g += red[w][0][row][c];
    u += red[w][1][row][c];
  }
  const int p = b * 16 + row;
  const int s = sorted[p];
  float av = 0.f;
  if (s < sentinel) {
    if (!kBlock) {
      const float sxv = sx[s / K1];
      g = g * sxv * s13[(size_t)e * 2 * I + col0 + c];
      u = u * sxv * s13[(size_t)e * 2 * I + I + col0 + c];
    }
    av = silu(g) * u;
  }
  a_out[(size_t)p * I + col0 + c] = av;
}

// grid: (P_max / block_m, ceil(I / 64)); 4 wavefronts, each 16 intermediate columns
// (one gate tile and the matching up tile).
template <int MT, bool kBlock>
__global__ void __launch_bounds__(256) gate_up_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ sx, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ a_out, int T, int H, int I, int K1) {
  constexpr int BM = MT * 16;
  const int b = blockIdx.x;
  if (b * BM >= *num_padded) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = blockIdx.y * 64 + wv * 16;
  if (col0 >= I) return;
  const int e = block_expert[b];
  const int r16 = lane & 15, kq = lane >> 4;
  const int sentinel = T * K1;
  const int HB = H / kGroup;

  const uint8_t* arow[MT];
  bool avalid[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int s = sorted[b * BM + m * 16 + r16];
    avalid[m] = s < sentinel;
    arow[m] = xq + (size_t)(avalid[m] ? s / K1 : 0) * H + kq * 32;
  }
  // output rows of this lane: 4 * kq + j in every row tile
  int otok[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = sorted[b * BM + m * 16 + 4 * kq + j];
      otok[m][j] = s < sentinel ? s / K1 : -1;
    }
  const uint8_t* gptr = w13 + ((size_t)e * 2 * I + col0 + r16) * H + kq * 32;
  const uint8_t* uptr = gptr + (size_t)I * H;

  v4f accg[MT], accu[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    accg[m] = v4f{0.f, 0.f, 0.f, 0.f};
    accu[m] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < H; k += kGroup) {
    const v8i bg = load32(gptr + k);
    const v8i bu = load32(uptr + k);
    float swg = 0.f, swu = 0.f;
    if (kBlock) {
      const int kb = k / kGroup;
      swg = s13[((size_t)e * (2 * I / kGroup) + col0 / kGroup) * HB + kb];
      swu = s13[((size_t)e * (2 * I / kGroup) + (I + col0) / kGroup) * HB + kb];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const v8i a = avalid[m] ? load32(arow[m] + k) : zero8;
      if (!kBlock) {
        accg[m] = mfma_16x16x128_fp8(a, bg, accg[m]);
        accu[m] = mfma_16x16x128_fp8(a, bu, accu[m]);
      } else {
        const v4f tg = mfma_16x16x128_fp8(a, bg, zero4);
        const v4f tu = mfma_16x16x128_fp8(a, bu, zero4);
        const int kb = k / kGroup;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float s = otok[m][j] >= 0 ? sx[(size_t)otok[m][j] * HB + kb] : 0.f;
          accg[m][j] += tg[j] * (s * swg);
          accu[m][j] += tu[j] * (s * swu);
        }
      }
    }
  }
  const int col = col0 + r16;
  float sg = 1.f, su = 1.f;
  if (!kBlock) {
    sg = s13[(size_t)e * 2 * I + col];
    su = s13[(size_t)e * 2 * I + I + col];
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = b * BM + m * 16 + 4 * kq + j;
      float av = 0.f;
      if (otok[m][j] >= 0) {
        float g = accg[m][j], u = accu[m][j];
        if (!kBlock) {
          const float s = sx[otok[m][j]];
          g = g * s * sg;
          u = u * s * su;
        }
        av = silu(g) * u;
      }
      a_out[(size_t)p * I + col] = av;
    }
}

// grid: (P_max / block_m, ceil(H / 256)); 4 wavefronts, each 64 output columns
// (4 tiles of 16). All loads of a pair of K-steps are issued before its MFMAs.
template <int MT, bool kBlock>
__global__ void __launch_bounds__(256) down_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ sa, const uint8_t* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    const float* __restrict__ topk_w, uint16_t* __restrict__ slot_out, int T, int H, int I,
    int K1) {
  constexpr int BM = MT * 16;
  constexpr int NT = 4;
  constexpr int KU = 2;   // K-steps per load batch
  const int b = blockIdx.x;
  if (b * BM >= *num_padded) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h0 = blockIdx.y * 256 + wv * 64;
  if (h0 >= H) return;
  const int e = block_expert[b];
  const int r16 = lane & 15, kq = lane >> 4;
  const int sentinel = T * K1;
  const int IB = I / kGroup;

  v4f acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* wrow = w2 + ((size_t)e * H + h0 + r16) * I + kq * 32;
  const uint8_t* arow = aq + (size_t)(b * BM + r16) * I + kq * 32;
  for (int k0 = 0; k0 < I; k0 += KU * kGroup) {
    v8i bw[KU][NT], av[KU][MT];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int k = k0 + u * kGroup;
      const bool in = k + kq * 32 < I;   // I % 32 == 0: a lane's 32 K-bytes are all in or all out
#pragma unroll
      for (int n = 0; n < NT; ++n) bw[u][n] = in ? load32(wrow + (size_t)n * 16 * I + k) : zero8;
#pragma unroll
      for (int m = 0; m < MT; ++m) av[u][m] = in ? load32(arow + (size_t)m * 16 * I + k) : zero8;
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int k = k0 + u * kGroup;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (!kBlock) {
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[m][n] = mfma_16x16x128_fp8(av[u][m], bw[u][n], acc[m][n]);
        } else if (k < I) {
          const int kb = k / kGroup;
          float sr[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) sr[j] = sa[(size_t)(b * BM + m * 16 + 4 * kq + j) * IB + kb];
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const float sw = s2[((size_t)e * (H / kGroup) + (h0 + n * 16) / kGroup) * IB + kb];
            const v4f t = mfma_16x16x128_fp8(av[u][m], bw[u][n], zero4);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[m][n][j] += t[j] * (sr[j] * sw);
          }
        }
      }
    }
  }
  float sw[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) sw[n] = kBlock ? 1.f : s2[(size_t)e * H + h0 + n * 16 + r16];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = b * BM + m * 16 + 4 * kq + j;
      const int s = sorted[p];
      if (s >= sentinel) continue;
      const float rs = (kBlock ? 1.f : sa[p]);
      const float wgt = topk_w[s];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float y = acc[m][n][j] * rs * sw[n];
        slot_out[(size_t)s * H + h0 + n * 16 + r16] = f32_to_bf16(y * wgt);
      }
    }
}

template <bool kBlock>
static hipError_t launch_gate_up_t(int block_m, dim3 grid, hipStream_t st, const uint8_t* xq,
                                   const float* sx, const uint8_t* w13, const float* s13,
                                   const int32_t* sorted, const int32_t* be, const int32_t* np,
                                   float* a, int T, int H, int I, int K1) {
  switch (block_m) {
    case 16: hipLaunchKernelGGL((gate_up_kernel<1, kBlock>), grid, dim3(256), 0, st, xq, sx, w13, s13, sorted, be, np, a, T, H, I, K1); break;
    case 32: hipLaunchKernelGGL((gate_up_kernel<2, kBlock>), grid, dim3(256), 0, st, xq, sx, w13, s13, sorted, be, np, a, T, H, I, K1); break;
    case 64: hipLaunchKernelGGL((gate_up_kernel<4, kBlock>), grid, dim3(256), 0, st, xq, sx, w13, s13, sorted, be, np, a, T, H, I, K1); break;
    default: hipLaunchKernelGGL((gate_up_kernel<8, kBlock>), grid, dim3(256), 0, st, xq, sx, w13, s13, sorted, be, np, a, T, H, I, K1); break;
  }
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint8_t* xq, const float* sx, const uint8_t* w13, const float* s13,
                          bool block, const int32_t* sorted, const int32_t* block_expert,
                          const int32_t* num_padded, float* a, int T, int H, int I, int E1, int K1,
                          int block_m, hipStream_t stream) {
  const int P_max = (int)sorted_capacity(T, K1, E1, block_m);
  if (block_m == 16) {
    const dim3 grid(P_max / 16, I / 16);
    if (block)
      hipLaunchKernelGGL(gate_up_skinny_kernel<true>, grid, dim3(256), 0, stream, xq, sx, w13, s13,
                         sorted, block_expert, num_padded, a, T, H, I, K1);
    else
      hipLaunchKernelGGL(gate_up_skinny_kernel<false>, grid, dim3(256), 0, stream, xq, sx, w13, s13,
                         sorted, block_expert, num_padded, a, T, H, I, K1);
    return hipGetLastError();
  }
  const dim3 grid(P_max / block_m, (I + 63) / 64);
  return block ? launch_gate_up_t<true>(block_m, grid, stream, xq, sx, w13, s13, sorted, block_expert, num_padded, a, T, H, I, K1)
               : launch_gate_up_t<false>(block_m, grid, stream, xq, sx, w13, s13, sorted, block_expert, num_padded, a, T, H, I, K1);
}

template <bool kBlock>
static hipError_t launch_down_t(int block_m, dim3 grid, hipStream_t st, const uint8_t* aq,
                                const float* sa, const uint8_t* w2, const float* s2,
                                const int32_t* sorted, const int32_t* be, const int32_t* np,
                                const float* tw, uint16_t* so, int T, int H, int I, int K1) {
  switch (block_m) {
    case 16: hipLaunchKernelGGL((down_kernel<1, kBlock>), grid, dim3(256), 0, st, aq, sa, w2, s2, sorted, be, np, tw, so, T, H, I, K1); break;
    case 32: hipLaunchKernelGGL((down_kernel<2, kBlock>), grid, dim3(256), 0, st, aq, sa, w2, s2, sorted, be, np, tw, so, T, H, I, K1); break;
    case 64: hipLaunchKernelGGL((down_kernel<4, kBlock>), grid, dim3(256), 0, st, aq, sa, w2, s2, sorted, be, np, tw, so, T, H, I, K1); break;
    default: hipLaunchKernelGGL((down_kernel<8, kBlock>), grid, dim3(256), 0, st, aq, sa, w2, s2, sorted, be, np, tw, so, T, H, I, K1); break;
  }
  return hipGetLastError();
}

hipError_t launch_down(const uint8_t* aq, const float* sa, const uint8_t* w2, const float* s2,
                       bool block, const int32_t* sorted, const int32_t* block_expert,
                       const int32_t* num_padded, const float* topk_w, uint16_t* slot_out, int T,
                       int H, int I, int E1, int K1, int block_m, hipStream_t stream) {
  const int P_max = (int)sorted_capacity(T, K1, E1, block_m);
  const dim3 grid(P_max / block_m, (H + 255) / 256);
  return block ? launch_down_t<true>(block_m, grid, stream, aq, sa, w2, s2, sorted, block_expert, num_padded, topk_w, slot_out, T, H, I, K1)
               : launch_down_t<false>(block_m, grid, stream, aq, sa, w2, s2, sorted, block_expert, num_padded, topk_w, slot_out, T, H, I, K1);
}

// out[t, :] = bf16( sum_k slot_out[t*K1 + k, :] ), float32 in slot order. 8 columns per thread.
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ slot_out, int T,
                                                      int K1, int H, uint16_t* __restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int n8 = H / 8;
  const size_t t = idx / n8;
  if (t >= (size_t)T) return;
  const int h = (int)(idx % n8) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K1; ++k) {
    const uint4 v = *reinterpret_cast<const uint4*>(slot_out + (t * K1 + k) * H + h);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_to_f32(w[j] & 0xFFFFu);
      acc[2 * j + 1] += bf16_to_f32(w[j] >> 16);
    }
  }
  uint4 o;
  o.x = f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
  o.y = f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
  o.z = f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
  o.w = f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + t * H + h) = o;
}

hipError_t launch_combine(const uint16_t* slot_out, int T, int K1, int H, uint16_t* out,
                          hipStream_t stream) {
  const size_t n = (size_t)T * (H / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, slot_out,
                     T, K1, H, out);
  return hipGetLastError();
}

}  // namespace srmoe
