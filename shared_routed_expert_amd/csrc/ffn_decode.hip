// Decode-shaped expert GEMMs (block_m == 16) of the fused MoE layer.
//
// With few tokens per expert every weight byte feeds one MFMA, so these
// kernels are organised around streaming the expert weights from HBM: many
// short workgroups with several K steps of loads in flight per wavefront.
//
// Operand layout as everywhere here: lane l takes row/column l & 15 and the 32
// K-bytes at 32 * (l >> 4) of each 128-byte K step (one K step per MFMA).
// (Giving each lane a longer contiguous run of K was measured slower: every
// load instruction then touches four times as many cache lines.)
//
// gate_up: grid (P_max/16, I/16); the 4 wavefronts take contiguous quarters of
//          K = H and issue kPrefetch steps of loads ahead of their MFMAs; the
//          partial tiles are summed through LDS in a fixed order; a = silu(g)*u
//          as float32. The epilogue's row data is fetched at the start so its
//          latency hides under the weight stream.
// (The down GEMM for these blocks is the generic kernel in ffn.hip with one row
// tile; quantising a inside its prologue was measured slower than one separate
// quantisation pass, because every column tile then repeats the work.)
#include "common.hpp"

namespace srmoe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool kBlock>
__global__ void __launch_bounds__(256) gate_up_decode_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ sx, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, float* __restrict__ a_out, int T, int H, int I,
    int K1) {
  constexpr int kPrefetch = 5;
  constexpr int kRS = kGroup + 16;   // LDS row stride of a staged K step (conflict-free fragment reads)
  __shared__ float red[4][2][16][17];
  // per wavefront, one K step of its 48 rows: x rows 0..15, gate rows 16..31, up rows 32..47
  __shared__ __align__(16) uint8_t stage[4][48 * kRS];
  const int b = blockIdx.x;
  const int e = block_expert[b];   // -1 past the used rows
  const int erow = threadIdx.x >> 4, ec = threadIdx.x & 15;   // epilogue element of this thread
  const int s_epi = sorted[b * 16 + erow];
  if (e < 0) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int col0 = blockIdx.y * 16;
  const int sentinel = T * K1;
  const int HB = H / kGroup;
  const int nsteps = H / kGroup;
  const int s0 = wv * nsteps / 4, s1 = (wv + 1) * nsteps / 4;

  // Loads are whole 128-byte lines: load instruction i of a K step covers rows
  // 8 i .. 8 i + 7 of the 48 (lane l: row 8 i + l / 8, bytes 16 (l % 8) .. +15),
  // 21% faster to stream than loading the MFMA fragments directly (16 rows x 64
  // bytes per instruction). Each step then passes through the wavefront's LDS
  // buffer into the fragment layout. No load is predicated per lane, so the
  // compiler's memory waits stay exact: padding rows read token 0 (their outputs
  // are discarded) and the unused slots of the last batch re-read the last step.
  const uint8_t* rowp[6];
  const int r8 = lane >> 3;
#pragma unroll
  for (int i = 0; i < 2; ++i) {   // x rows of the block's tokens
    const int s_in = sorted[b * 16 + 8 * i + r8];
    const uint32_t t = (uint32_t)s_in / (uint32_t)K1;
    rowp[i] = xq + (size_t)(s_in < sentinel ? t : 0u) * H + (lane & 7) * 16;
  }
  const uint8_t* wrow = w13 + ((size_t)e * 2 * I + col0 + r8) * H + (lane & 7) * 16;
  rowp[2] = wrow;                              // gate rows col0 .. col0 + 7
  rowp[3] = wrow + (size_t)8 * H;              // gate rows col0 + 8 .. + 15
  rowp[4] = wrow + (size_t)I * H;              // up rows
  rowp[5] = wrow + (size_t)(I + 8) * H;
  uint8_t* stg = stage[wv];
  int otok[4] = {0, 0, 0, 0};
  bool oval[4] = {false, false, false, false};
  if (kBlock) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s = sorted[b * 16 + 4 * kq + q];
      oval[q] = s < sentinel;
      otok[q] = oval[q] ? s / K1 : 0;
    }
  }
  const size_t sg_base = ((size_t)e * (2 * I / kGroup) + col0 / kGroup) * HB;
  const size_t su_base = ((size_t)e * (2 * I / kGroup) + (I + col0) / kGroup) * HB;
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f accg = zero4, accu = zero4;
  float e_sx = 0.f, e_sg = 1.f, e_su = 1.f;
  if (!kBlock) {
    e_sg = s13[(size_t)e * 2 * I + col0 + ec];
    e_su = s13[(size_t)e * 2 * I + I + col0 + ec];
    e_sx = sx[s_epi < sentinel ? s_epi / K1 : 0];
  }

  for (int st = s0; st < s1; st += kPrefetch) {
    u32x4 L[kPrefetch][6];
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      const size_t k = (size_t)min(st + j, s1 - 1) * kGroup;
#pragma unroll
      for (int i = 0; i < 6; ++i) L[j][i] = *reinterpret_cast<const u32x4*>(rowp[i] + k);
    }
    // keep every load of the batch ahead of its MFMAs (the scheduler would otherwise
    // interleave them and wait on each step in turn)
    __builtin_amdgcn_sched_barrier(0);
    const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      // one K step through LDS: rows in, fragments out (a wavefront's LDS
      // operations complete in order, so the buffer is reused without a barrier)
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        // opaque to the optimiser: a plain load-then-store pair is merged into one
        // global-to-LDS copy at the store, which would move the load behind the barrier
        asm volatile("" : "+v"(L[j][i]));
        *reinterpret_cast<u32x4*>(stg + (8 * i + r8) * kRS + (lane & 7) * 16) = L[j][i];
      }
      const v8i At = load32(stg + r16 * kRS + kq * 32);
      const v8i A = st + j < s1 ? At : zero8;   // a repeated step contributes nothing
      const v8i G = load32(stg + (16 + r16) * kRS + kq * 32);
      const v8i U = load32(stg + (32 + r16) * kRS + kq * 32);
      if (!kBlock) {
        accg = mfma_16x16x128_fp8(A, G, accg);
        accu = mfma_16x16x128_fp8(A, U, accu);
      } else if (st + j < s1) {
        const int kb = st + j;
        const v4f tg = mfma_16x16x128_fp8(A, G, zero4);
        const v4f tu = mfma_16x16x128_fp8(A, U, zero4);
        const float swg = s13[sg_base + kb], swu = s13[su_base + kb];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sxl = sx[(size_t)otok[q] * HB + kb];
          const float sxv = oval[q] ? sxl : 0.f;
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
  float g = red[0][0][erow][ec], u = red[0][1][erow][ec];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    g += red[w][0][erow][ec];
    u += red[w][1][erow][ec];
  }
  float av = 0.f;
  if (s_epi < sentinel) {
    if (!kBlock) {
      g = g * e_sx * e_sg;
      u = u * e_sx * e_su;
    }
    av = silu(g) * u;
  }
  a_out[(size_t)(b * 16 + erow) * I + col0 + ec] = av;
}

// down for 16-row blocks and I <= 256: one 256-thread workgroup per (block, 256
// output columns) like the generic kernel (row tile of 16, the weights as the
// MFMA A operand, lane (r16, kq) ending with 16 consecutive columns of row r16),
// but each wavefront's 64 weight rows -- 64 * I contiguous bytes -- are loaded as
// whole 1 KB runs and passed through a per-wavefront LDS buffer into the
// fragment layout. Column c of the wavefront's 64 goes to LDS row
// 16 ((c / 4) % 4) + 4 (c / 16) + c % 4, so MFMA tile n reads rows 16 n .. 16 n + 15
// in lane order; with a row stride of I + 16 bytes those reads are bank-conflict
// free. Both K steps run, the second (or its tail) with a zeroed a_q operand and
// clamped weight offsets, as in the generic kernel.
template <bool kBlock, int NI>   // NI = I / 16: 1 KB load runs per wavefront
__global__ void __launch_bounds__(256) down_decode_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ sa, const uint8_t* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const float* __restrict__ row_scale,
    uint16_t* __restrict__ slot_out, int T, int H, int K1) {
  constexpr int I = NI * 16;
  constexpr int kRS = I + 16;
  __shared__ __align__(16) uint8_t stage[4][64 * kRS];
  const int b = blockIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int h0 = blockIdx.y * 256 + wv * 64;
  const int e = block_expert[b];   // -1 past the used rows
  const int srow = sorted[b * 16 + r16];
  const float rsc = row_scale[b * 16 + r16];
  if (e < 0 || h0 >= H) return;
  const int sentinel = T * K1;
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};

  // the wavefront's 64 rows of w2[e]: 64 * I contiguous bytes, 1 KB per load
  const uint8_t* wsrc = w2 + ((size_t)e * H + h0) * I + lane * 16;
  u32x4 L[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) L[i] = *reinterpret_cast<const u32x4*>(wsrc + i * 1024);
  uint32_t kc[2];
  v8i av[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int koff = u * kGroup + kq * 32;
    const bool in = koff < I;
    kc[u] = in ? koff : I - 32;
    const v8i t = load32(aq + (size_t)(b * 16 + r16) * I + kc[u]);
    av[u] = in ? t : zero8;
  }
  float sw[16];
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
    const float4 v = kBlock ? make_float4(1.f, 1.f, 1.f, 1.f)
                            : *reinterpret_cast<const float4*>(s2 + (size_t)e * H + h0 + kq * 16 + c);
    sw[c] = v.x; sw[c + 1] = v.y; sw[c + 2] = v.z; sw[c + 3] = v.w;
  }
  __builtin_amdgcn_sched_barrier(0);
  uint8_t* stg = stage[wv];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int o = i * 1024 + lane * 16;
    const int c = o / I, byte = o - c * I;
    const int lr = 16 * ((c >> 2) & 3) + 4 * (c >> 4) + (c & 3);
    asm volatile("" : "+v"(L[i]));   // keeps the load ahead of the barrier (see gate_up)
    *reinterpret_cast<u32x4*>(stg + lr * kRS + byte) = L[i];
  }
  v4f acc[4] = {zero4, zero4, zero4, zero4};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    v8i bw[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) bw[n] = load32(stg + (16 * n + r16) * kRS + kc[u]);
    if (!kBlock) {
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[n] = mfma_16x16x128_fp8(bw[n], av[u], acc[n]);
    } else if (u * kGroup < I) {
      const int kb = u;
      // a wavefront's 64 columns lie in one 128-column block of w2's scales
      const float swb = s2[((size_t)e * (H / kGroup) + h0 / kGroup) * (I / kGroup) + kb];
      const float sr = sa[(size_t)(b * 16 + r16) * (I / kGroup) + kb] * swb;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const v4f t = mfma_16x16x128_fp8(bw[n], av[u], zero4);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[n][j] += t[j] * sr;
      }
    }
  }
  // the MFMAs read their scale operands across the whole wavefront: keep them ahead of the
  // per-row exit below, under a full exec mask
#pragma unroll
  for (int n = 0; n < 4; ++n) asm volatile("" : "+v"(acc[n]));
  if (srow >= sentinel) return;
  uint32_t packed[8];
#pragma unroll
  for (int c = 0; c < 16; c += 2) {   // column c = 4 * n + j of this lane's 16
    const float y0 = acc[c >> 2][c & 3] * sw[c] * rsc;
    const float y1 = acc[(c + 1) >> 2][(c + 1) & 3] * sw[c + 1] * rsc;
    packed[c >> 1] = pack_bf16x2(y0, y1);
  }
  uint4* dst = reinterpret_cast<uint4*>(slot_out + (size_t)srow * H + h0 + kq * 16);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

bool down_decode_supported(int I) { return I >= 32 && I <= 2 * kGroup && I % 32 == 0; }

hipError_t launch_down_decode(const uint8_t* aq, const float* sa, const uint8_t* w2,
                              const float* s2, bool block, const int32_t* sorted,
                              const int32_t* block_expert, const float* row_scale,
                              uint16_t* slot_out, int T, int H, int I, int E1, int K1,
                              hipStream_t stream) {
  const int P_max = (int)sorted_capacity(T, K1, E1, 16);
  const dim3 grid(P_max / 16, (H + 255) / 256), blk(256);
#define SRMOE_DD(B, N)                                                                            \
  hipLaunchKernelGGL((down_decode_kernel<B, N>), grid, blk, 0, stream, aq, sa, w2, s2, sorted,    \
                     block_expert, row_scale, slot_out, T, H, K1)
#define SRMOE_DD2(N) if (block) SRMOE_DD(true, N); else SRMOE_DD(false, N); break;
  switch (I / 16) {
    case 2: SRMOE_DD2(2)
    case 4: SRMOE_DD2(4)
    case 6: SRMOE_DD2(6)
    case 8: SRMOE_DD2(8)
    case 10: SRMOE_DD2(10)
    case 12: SRMOE_DD2(12)
    case 14: SRMOE_DD2(14)
    default: SRMOE_DD2(16)
  }
#undef SRMOE_DD2
#undef SRMOE_DD
  return hipGetLastError();
}

hipError_t launch_gate_up_decode(const uint8_t* xq, const float* sx, const uint8_t* w13,
                                 const float* s13, bool block, const int32_t* sorted,
                                 const int32_t* block_expert, float* a, int T, int H, int I, int E1,
                                 int K1, hipStream_t stream) {
  const int P_max = (int)sorted_capacity(T, K1, E1, 16);
  const dim3 grid(P_max / 16, I / 16);
  if (block)
    hipLaunchKernelGGL(gate_up_decode_kernel<true>, grid, dim3(256), 0, stream, xq, sx, w13, s13,
                       sorted, block_expert, a, T, H, I, K1);
  else
    hipLaunchKernelGGL(gate_up_decode_kernel<false>, grid, dim3(256), 0, stream, xq, sx, w13, s13,
                       sorted, block_expert, a, T, H, I, K1);
  return hipGetLastError();
}

}  // namespace srmoe
