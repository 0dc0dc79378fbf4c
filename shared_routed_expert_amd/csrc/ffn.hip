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
// down:    slot_out[s, h] = bf16( w[s] * dequantised a_q[p] . w2[e] row h ), with the
//          routing weight (times the row's FP8 scale in per-channel mode) taken from
//          the per-row output scale the quantisation of a writes
//
// These kernels serve row blocks of 32..128 (block_m == 16 has its own
// decode-shaped kernels in ffn_decode.hip). Each wavefront owns 16 output
// columns per MFMA tile and all block_m/16 row tiles of its block; operands are
// loaded straight from global memory in the MFMA's register layout (lane:
// row/column l & 15, 32 K-bytes at 32 * (l >> 4)).
#include "common.hpp"

namespace srmoe {

// grid: (P_max / block_m, ceil(I / 64)); 4 wavefronts, each 16 intermediate columns
// (one gate tile and the matching up tile).
template <int MT, bool kBlock>
__global__ void __launch_bounds__(256) gate_up_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ sx, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, float* __restrict__ a_out, int T, int H, int I,
    int K1) {
  constexpr int BM = MT * 16;
  const int b = blockIdx.x;
  const int e = block_expert[b];   // -1 past the used rows
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = blockIdx.y * 64 + wv * 16;
  if (e < 0 || col0 >= I) return;
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

// grid: (P_max / block_m, ceil(H / 256)); 4 wavefronts, each 64 output columns as
// four 16-row MFMA tiles. The weights are the MFMA's A operand (16 rows of w2[e])
// and the block's quantised a rows its B operand, so D holds [column][token].
// Inside a wavefront's 64 columns, tile n row r holds column
// h0 + (r / 4) * 16 + 4 * n + r % 4: then lane (r16, kq) ends with the 16
// consecutive columns h0 + 16 * kq .. + 15 of token r16 and writes them with two
// 16-byte stores. All loads of a pair of K-steps are issued ahead of its MFMAs;
// loads are never predicated per lane (a lane whose K bytes fall past I reads a
// clamped, valid address and zeroes its B operand), so the compiler's memory
// waits stay exact; for small row blocks the per-row epilogue data (slot and
// output scale) is fetched at the start to hide under the weight stream.
template <int MT, bool kBlock>
__global__ void __launch_bounds__(256) down_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ sa, const uint8_t* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const float* __restrict__ row_scale,
    uint16_t* __restrict__ slot_out, int T, int H, int I, int K1) {
  constexpr int BM = MT * 16;
  constexpr int NT = 4;
  constexpr int KU = 2;   // K-steps per load batch
  constexpr bool kHoist = MT <= 2;
  const int b = blockIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int h0 = blockIdx.y * 256 + wv * 64;
  const int e = block_expert[b];   // -1 past the used rows
  int srow[MT];
  float rsc[MT];
  if (kHoist) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      srow[m] = sorted[b * BM + m * 16 + r16];
      rsc[m] = row_scale[b * BM + m * 16 + r16];
    }
  }
  if (e < 0 || h0 >= H) return;
  const int sentinel = T * K1;
  const int IB = I / kGroup;

  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* wbase = w2 + ((size_t)e * H + h0 + (r16 >> 2) * 16 + (r16 & 3)) * I;
  const uint8_t* abase = aq + (size_t)(b * BM + r16) * I;
  v8i bw[KU][NT], av[KU][MT];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int koff = k0 + u * kGroup + kq * 32;
      const bool in = koff < I;          // I % 32 == 0: a lane's 32 K-bytes are all in or all out
      const int kc = in ? koff : I - 32; // clamped, always inside the row
#pragma unroll
      for (int n = 0; n < NT; ++n) bw[u][n] = load32(wbase + (size_t)(4 * n) * I + kc);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const v8i t = load32(abase + (size_t)m * 16 * I + kc);
        av[u][m] = in ? t : zero8;       // a zero operand removes the clamped lane's product
      }
    }
  };
  load(0);
  float sw[16];   // per-channel scales of this lane's 16 output columns
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
    const float4 v = kBlock ? make_float4(1.f, 1.f, 1.f, 1.f)
                            : *reinterpret_cast<const float4*>(s2 + (size_t)e * H + h0 + kq * 16 + c);
    sw[c] = v.x; sw[c + 1] = v.y; sw[c + 2] = v.z; sw[c + 3] = v.w;
  }

  v4f acc[NT][MT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[n][m] = zero4;
  for (int k0 = 0; k0 < I; k0 += KU * kGroup) {
    if (k0 > 0) load(k0);
    __builtin_amdgcn_sched_barrier(0);   // all loads of the batch ahead of its MFMAs
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int k = k0 + u * kGroup;
      if (!kBlock) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[n][m] = mfma_16x16x128_fp8(bw[u][n], av[u][m], acc[n][m]);
      } else if (k < I) {
        const int kb = k / kGroup;
        // a wavefront's 64 columns lie in one 128-column block of w2's scales
        const float swb = s2[((size_t)e * (H / kGroup) + h0 / kGroup) * IB + kb];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float sr = sa[(size_t)(b * BM + m * 16 + r16) * IB + kb] * swb;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const v4f t = mfma_16x16x128_fp8(bw[u][n], av[u][m], zero4);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[n][m][j] += t[j] * sr;
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int p = b * BM + m * 16 + r16;
    const int s = kHoist ? srow[m] : sorted[p];
    if (s >= sentinel) continue;
    const float r = kHoist ? rsc[m] : row_scale[p];
    uint32_t packed[8];
#pragma unroll
    for (int c = 0; c < 16; c += 2) {
      // column c = 4 * n + j of this lane's 16
      const float y0 = acc[c >> 2][m][c & 3] * sw[c] * r;
      const float y1 = acc[(c + 1) >> 2][m][(c + 1) & 3] * sw[c + 1] * r;
      packed[c >> 1] = pack_bf16x2(y0, y1);
    }
    uint4* dst = reinterpret_cast<uint4*>(slot_out + (size_t)s * H + h0 + kq * 16);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  }
}

template <bool kBlock>
static hipError_t launch_gate_up_t(int block_m, dim3 grid, hipStream_t st, const uint8_t* xq,
                                   const float* sx, const uint8_t* w13, const float* s13,
                                   const int32_t* sorted, const int32_t* be, float* a, int T, int H,
                                   int I, int K1) {
  switch (block_m) {
    case 32: hipLaunchKernelGGL((gate_up_kernel<2, kBlock>), grid, dim3(256), 0, st, xq, sx, w13, s13, sorted, be, a, T, H, I, K1); break;
    case 64: hipLaunchKernelGGL((gate_up_kernel<4, kBlock>), grid, dim3(256), 0, st, xq, sx, w13, s13, sorted, be, a, T, H, I, K1); break;
    default: hipLaunchKernelGGL((gate_up_kernel<8, kBlock>), grid, dim3(256), 0, st, xq, sx, w13, s13, sorted, be, a, T, H, I, K1); break;
  }
  return hipGetLastError();
}

hipError_t launch_gate_up_tile(const uint8_t*, const float*, const uint8_t*, const float*, bool,
                               const int32_t*, const int32_t*, const int32_t*, const int32_t*, float*, int,
                               int, int, int, int, hipStream_t);

// block_m 32..128 (block_m 16 uses launch_gate_up_decode; 128 the LDS-tiled kernel).
// expert_offsets (block_m 128; may be null): group the tiles of one expert (grouped_tile).
hipError_t launch_gate_up(const uint8_t* xq, const float* sx, const uint8_t* w13, const float* s13,
                          bool block, const int32_t* sorted, const int32_t* block_expert,
                          const int32_t* num_padded, const int32_t* expert_offsets, float* a, int T, int H,
                          int I, int E1, int K1, int block_m, hipStream_t stream) {
  if (block_m == 128)
    return launch_gate_up_tile(xq, sx, w13, s13, block, sorted, block_expert, num_padded, expert_offsets, a, T,
                               H, I, E1, K1, stream);
  const int P_max = (int)sorted_capacity(T, K1, E1, block_m);
  const dim3 grid(P_max / block_m, (I + 63) / 64);
  return block ? launch_gate_up_t<true>(block_m, grid, stream, xq, sx, w13, s13, sorted, block_expert, a, T, H, I, K1)
               : launch_gate_up_t<false>(block_m, grid, stream, xq, sx, w13, s13, sorted, block_expert, a, T, H, I, K1);
}

template <bool kBlock>
static hipError_t launch_down_t(int block_m, dim3 grid, hipStream_t st, const uint8_t* aq,
                                const float* sa, const uint8_t* w2, const float* s2,
                                const int32_t* sorted, const int32_t* be, const float* rs,
                                uint16_t* so, int T, int H, int I, int K1) {
  switch (block_m) {
    case 16: hipLaunchKernelGGL((down_kernel<1, kBlock>), grid, dim3(256), 0, st, aq, sa, w2, s2, sorted, be, rs, so, T, H, I, K1); break;
    case 32: hipLaunchKernelGGL((down_kernel<2, kBlock>), grid, dim3(256), 0, st, aq, sa, w2, s2, sorted, be, rs, so, T, H, I, K1); break;
    case 64: hipLaunchKernelGGL((down_kernel<4, kBlock>), grid, dim3(256), 0, st, aq, sa, w2, s2, sorted, be, rs, so, T, H, I, K1); break;
    default: hipLaunchKernelGGL((down_kernel<8, kBlock>), grid, dim3(256), 0, st, aq, sa, w2, s2, sorted, be, rs, so, T, H, I, K1); break;
  }
  return hipGetLastError();
}

hipError_t launch_down_tile(const uint8_t*, const float*, const uint8_t*, const float*, bool,
                            const int32_t*, const int32_t*, const int32_t*, const int32_t*, const float*,
                            uint16_t*, int, int, int, int, int, hipStream_t);

bool down_decode_supported(int I);
hipError_t launch_down_decode(const uint8_t*, const float*, const uint8_t*, const float*, bool,
                              const int32_t*, const int32_t*, const float*, uint16_t*, int, int,
                              int, int, int, hipStream_t);

hipError_t launch_down(const uint8_t* aq, const float* sa, const uint8_t* w2, const float* s2,
                       bool block, const int32_t* sorted, const int32_t* block_expert,
                       const int32_t* num_padded, const int32_t* expert_offsets, const float* row_scale,
                       uint16_t* slot_out, int T, int H, int I, int E1, int K1, int block_m, hipStream_t stream) {
  if (block_m == 128)
    return launch_down_tile(aq, sa, w2, s2, block, sorted, block_expert, num_padded, expert_offsets, row_scale,
                            slot_out, T, H, I, E1, K1, stream);
  if (block_m == 16 && down_decode_supported(I))
    return launch_down_decode(aq, sa, w2, s2, block, sorted, block_expert, row_scale, slot_out, T,
                              H, I, E1, K1, stream);
  const int P_max = (int)sorted_capacity(T, K1, E1, block_m);
  const dim3 grid(P_max / block_m, (H + 255) / 256);
  return block ? launch_down_t<true>(block_m, grid, stream, aq, sa, w2, s2, sorted, block_expert, row_scale, slot_out, T, H, I, K1)
               : launch_down_t<false>(block_m, grid, stream, aq, sa, w2, s2, sorted, block_expert, row_scale, slot_out, T, H, I, K1);
}

// out[t, :] = bf16( sum_k slot_out[t*K1 + k, :] (+ extra[t, :]) ), float32 in slot order,
// extra (the separately computed shared expert of the unfused layer, or null) last.
// 8 columns per thread. K1 is a template parameter so that all K1 row loads are issued
// before the first add (with a runtime trip count they go out one at a time, each
// waiting for memory).
template <int K1, bool kExtra>
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ slot_out,
                                                      const uint16_t* __restrict__ extra, int T,
                                                      int H, uint16_t* __restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int n8 = H / 8;
  const size_t t = idx / n8;
  if (t >= (size_t)T) return;
  const int h = (int)(idx % n8) * 8;
  uint4 v[K1 + 1];
#pragma unroll
  for (int k = 0; k < K1; ++k) v[k] = *reinterpret_cast<const uint4*>(slot_out + (t * K1 + k) * H + h);
  if (kExtra) v[K1] = *reinterpret_cast<const uint4*>(extra + t * H + h);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < K1 + (kExtra ? 1 : 0); ++k) {
    const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_to_f32(w[j] & 0xFFFFu);
      acc[2 * j + 1] += bf16_to_f32(w[j] >> 16);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + t * H + h) = o;
}

hipError_t launch_combine(const uint16_t* slot_out, const uint16_t* extra, int T, int K1, int H,
                          uint16_t* out, hipStream_t stream) {
  const size_t n = (size_t)T * (H / 8);
  const dim3 grid((unsigned)((n + 255) / 256)), blk(256);
  switch (K1) {
#define SRMOE_COMBINE(K)                                                                             \
    case K:                                                                                          \
      if (extra)                                                                                     \
        hipLaunchKernelGGL((combine_kernel<K, true>), grid, blk, 0, stream, slot_out, extra, T, H, out); \
      else                                                                                           \
        hipLaunchKernelGGL((combine_kernel<K, false>), grid, blk, 0, stream, slot_out, extra, T, H, out); \
      break;
    SRMOE_COMBINE(1) SRMOE_COMBINE(2) SRMOE_COMBINE(3) SRMOE_COMBINE(4) SRMOE_COMBINE(5)
    SRMOE_COMBINE(6) SRMOE_COMBINE(7) SRMOE_COMBINE(8) SRMOE_COMBINE(9) SRMOE_COMBINE(10)
    SRMOE_COMBINE(11) SRMOE_COMBINE(12) SRMOE_COMBINE(13) SRMOE_COMBINE(14) SRMOE_COMBINE(15)
    SRMOE_COMBINE(16)
#undef SRMOE_COMBINE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace srmoe
