// Per-head RMS norm of q and k fused with the rotary position embedding, in place on
// the bf16 output of the qkv projection (intelliparadigm, GLM4-MoE production
// optimisation, section 2.2; Optimizing GLM4-MoE for production, section 2: both
// steps work on one attention head at a time, so one kernel does both, and GLM4-MoE
// rotates only part of each head's dimensions).
//
// Layout of one token's row of qkv: Hq q heads, then Hkv k heads, then Hkv v heads,
// D values each. Only the q and k heads are touched.
//   norm:     y = x / sqrt(mean(x^2) + eps) * w      (w: q_norm_w for q, k_norm_w for k)
//   rotation: the first rd dims of y, rotated by angle(pos, i) = pos * theta^(-2i/rd),
//             i < rd/2; the pair of frequency i is (i, i + rd/2) in the rotate-half
//             ("neox") arrangement, (2i, 2i+1) in the interleaved one. cos/sin come from
//             a table [max_pos][rd] (rd/2 cosines, then rd/2 sines) built by
//             rope_table_kernel. Dims >= rd keep the normalised value.
//
// Work split: D/8 lanes per head, each lane one 16-byte load of 8 consecutive bf16
// values (64/(D/8) heads per wavefront, a coalesced 1-2 KB per load instruction). The
// sum of squares is a butterfly over the head's lanes (every lane gets the identical
// sum); a rotate-half partner sits rd/16 lanes away, so it is one lane swap per value;
// interleaved partners are in the same lane. Arithmetic in float32, one rounding to
// bf16 at the store. The unfused form runs the norm and the rotation as two passes,
// with the normalised heads stored as bf16 in between.
#include "common.hpp"

namespace srmoe {

template <int LPH>
__device__ __forceinline__ float head_sum(float v) {
#pragma unroll
  for (int m = 1; m < LPH; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// LPH = D / 8 lanes per head. kNorm / kRope select the fused kernel (both) or one of the
// two passes of the unfused form.
template <int LPH, bool kNorm, bool kRope, bool kNeox>
__global__ void __launch_bounds__(256) qk_norm_rope_kernel(
    uint16_t* __restrict__ qkv, int T, int Hq, int Hkv, int rd, const float* __restrict__ qw,
    const float* __restrict__ kw, float eps, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int max_pos) {
  constexpr int D = 8 * LPH;
  constexpr int kHeadsPerWave = kWave / LPH;
  const int lane = threadIdx.x & 63;
  const int nqk = Hq + Hkv;
  const long total = (long)T * nqk;
  const long g = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * kHeadsPerWave + lane / LPH;
  const bool valid = g < total;
  // lanes past the last head work on the last head and store nothing, so every lane of a
  // head group takes part in the exchanges
  const long gc = valid ? g : total - 1;
  const int t = (int)(gc / nqk), h = (int)(gc % nqk);
  const int j = lane % LPH;   // dims 8j .. 8j+7 of the head
  uint16_t* p = qkv + (size_t)t * (nqk + Hkv) * D + (size_t)h * D + 8 * j;
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_f32(r[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(r[i] >> 16);
  }
  if (kNorm) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
    ss = head_sum<LPH>(ss);
    const float inv = rsqrtf(ss * (1.0f / D) + eps);
    const float* w = (h < Hq ? qw : kw) + 8 * j;
    const float4 w0 = *reinterpret_cast<const float4*>(w);
    const float4 w1 = *reinterpret_cast<const float4*>(w + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = x[i] * inv * wv[i];
  }
  if (kRope) {
    const int half = rd >> 1;
    int pos = positions[t];
    pos = pos < 0 ? 0 : (pos >= max_pos ? max_pos - 1 : pos);
    const float* cs = cos_sin + (size_t)pos * rd;
    const bool rotated = 8 * j < rd;
    if (kNeox) {
      // partner of dim d is d + half (d < half) or d - half: lane j ^ (half / 8)
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = __shfl_xor(x[i], half >> 3, kWave);
      if (rotated) {
        const bool first = 8 * j < half;
        const int f0 = first ? 8 * j : 8 * j - half;   // frequency index of x[0]
        const float4 c0 = *reinterpret_cast<const float4*>(cs + f0);
        const float4 c1 = *reinterpret_cast<const float4*>(cs + f0 + 4);
        const float4 s0 = *reinterpret_cast<const float4*>(cs + half + f0);
        const float4 s1 = *reinterpret_cast<const float4*>(cs + half + f0 + 4);
        const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = first ? x[i] * c[i] - y[i] * s[i] : x[i] * c[i] + y[i] * s[i];
      }
    } else if (rotated) {
      const int f0 = 4 * j;   // pairs (8j + 2q, 8j + 2q + 1) have frequency 4j + q
      const float4 c = *reinterpret_cast<const float4*>(cs + f0);
      const float4 s = *reinterpret_cast<const float4*>(cs + half + f0);
      const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = x[2 * q], b = x[2 * q + 1];
        x[2 * q] = a * cc[q] - b * ss[q];
        x[2 * q + 1] = b * cc[q] + a * ss[q];
      }
    }
  }
  if (!valid) return;
  uint4 o;
  o.x = pack_bf16x2(x[0], x[1]);
  o.y = pack_bf16x2(x[2], x[3]);
  o.z = pack_bf16x2(x[4], x[5]);
  o.w = pack_bf16x2(x[6], x[7]);
  *reinterpret_cast<uint4*>(p) = o;
}

// cos_sin[pos][i] = cos(pos * theta^(-2i/rd)), cos_sin[pos][rd/2 + i] = sin(...), i < rd/2:
// angles, cosines and sines in float64, stored as float32.
__global__ void __launch_bounds__(256) rope_table_kernel(float* __restrict__ cos_sin, int max_pos,
                                                         int rd, double theta) {
  const int half = rd >> 1;
  const long n = (long)max_pos * half;
  for (long k = (long)blockIdx.x * 256 + threadIdx.x; k < n; k += (long)gridDim.x * 256) {
    const int pos = (int)(k / half), i = (int)(k % half);
    const double ang = (double)pos * pow(theta, -2.0 * i / rd);
    cos_sin[(size_t)pos * rd + i] = (float)cos(ang);
    cos_sin[(size_t)pos * rd + half + i] = (float)sin(ang);
  }
}

template <int LPH, bool kNorm, bool kRope>
static void launch_pass(bool neox, dim3 grid, hipStream_t stream, uint16_t* qkv, int T, int Hq, int Hkv,
                        int rd, const float* qw, const float* kw, float eps, const int32_t* positions,
                        const float* cos_sin, int max_pos) {
  if (neox)
    hipLaunchKernelGGL((qk_norm_rope_kernel<LPH, kNorm, kRope, true>), grid, dim3(256), 0, stream, qkv, T,
                       Hq, Hkv, rd, qw, kw, eps, positions, cos_sin, max_pos);
  else
    hipLaunchKernelGGL((qk_norm_rope_kernel<LPH, kNorm, kRope, false>), grid, dim3(256), 0, stream, qkv, T,
                       Hq, Hkv, rd, qw, kw, eps, positions, cos_sin, max_pos);
}

template <int LPH>
static hipError_t launch_qk(uint16_t* qkv, int T, int Hq, int Hkv, int rd, bool neox, const float* qw,
                            const float* kw, float eps, const int32_t* positions, const float* cos_sin,
                            int max_pos, bool fused, hipStream_t stream) {
  const long heads = (long)T * (Hq + Hkv);
  const long per_block = 4L * (kWave / LPH);
  const dim3 grid((unsigned)((heads + per_block - 1) / per_block));
  if (fused) {
    launch_pass<LPH, true, true>(neox, grid, stream, qkv, T, Hq, Hkv, rd, qw, kw, eps, positions, cos_sin,
                                 max_pos);
  } else {
    launch_pass<LPH, true, false>(neox, grid, stream, qkv, T, Hq, Hkv, rd, qw, kw, eps, positions, cos_sin,
                                  max_pos);
    launch_pass<LPH, false, true>(neox, grid, stream, qkv, T, Hq, Hkv, rd, qw, kw, eps, positions, cos_sin,
                                  max_pos);
  }
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(uint16_t* qkv, int T, int Hq, int Hkv, int D, int rd, bool neox,
                               const float* qw, const float* kw, float eps, const int32_t* positions,
                               const float* cos_sin, int max_pos, bool fused, hipStream_t stream) {
  switch (D) {
    case 64:
      return launch_qk<8>(qkv, T, Hq, Hkv, rd, neox, qw, kw, eps, positions, cos_sin, max_pos, fused, stream);
    case 128:
      return launch_qk<16>(qkv, T, Hq, Hkv, rd, neox, qw, kw, eps, positions, cos_sin, max_pos, fused, stream);
    default:
      return launch_qk<32>(qkv, T, Hq, Hkv, rd, neox, qw, kw, eps, positions, cos_sin, max_pos, fused, stream);
  }
}

hipError_t launch_rope_table(float* cos_sin, int max_pos, int rd, double theta, hipStream_t stream) {
  const long n = (long)max_pos * (rd / 2);
  long blocks = (n + 255) / 256;
  blocks = blocks > 4096 ? 4096 : blocks;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, cos_sin, max_pos, rd,
                     theta);
  return hipGetLastError();
}

}  // namespace srmoe
