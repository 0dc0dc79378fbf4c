// Router gate: logits[t, e] = sum_h x[t, h] * W_r[e, h] + bias[e] for the E routed
// experts (the linear router upstream of the top-K; each token scores the 160 routed
// experts: Optimizing GLM4-MoE for production, section 1). x is bf16 [T, H], W_r
// float32 [E, H].
//
// Matrix cores, float32 accuracy: every fp32 weight w is split into three bf16 parts,
// hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid), which together carry its
// 24 significand bits. x is exactly bf16, so each product x * part is exact in float32
// and three 16x16x32 bf16 MFMAs per K step accumulate x * w in float32 -- the bf16
// matrix-core rate instead of the float32 one. Workgroup tile: four wavefronts of 16
// (small batches) or 64 tokens x 32 experts over a chunk of K; when the tiles alone
// cannot fill the GPU K is split over workgroups and a second pass sums the partial
// tiles in chunk order (deterministic).
#include "common.hpp"

namespace srmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kRExp = 32;   // experts per workgroup (two 16-column tiles)

// Lane l of a 16x16x32 bf16 MFMA supplies row/column l & 15 and the 8 K elements at
// 8 * (l >> 4) of the K step; A and B use the same K mapping.
__device__ __forceinline__ v4f mfma_16x16x32_bf16(const bf16x8& a, const bf16x8& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 float32 weights -> their hi / mid / lo bf16 parts (each remainder is exact in float32)
__device__ __forceinline__ void split3(const float4& w0, const float4& w1, bf16x8& hi, bf16x8& mid,
                                       bf16x8& lo) {
  const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  u16x8 h, m, l;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint16_t a = f32_to_bf16(w[j]);
    const float r1 = w[j] - bf16_to_f32(a);
    const uint16_t b = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(b);
    h[j] = a;
    m[j] = b;
    l[j] = f32_to_bf16(r2);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  mid = __builtin_bit_cast(bf16x8, m);
  lo = __builtin_bit_cast(bf16x8, l);
}

// One K step: the wavefront's MT token fragments against both expert tiles.
template <int MT>
__device__ __forceinline__ void router_step(const uint4 (&xa)[MT], const float4 (&wf)[4], v4f (&acc)[MT][2]) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    bf16x8 h, m, l;
    split3(wf[2 * n], wf[2 * n + 1], h, m, l);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const bf16x8 A = __builtin_bit_cast(bf16x8, xa[t]);
      acc[t][n] = mfma_16x16x32_bf16(A, h, acc[t][n]);
      acc[t][n] = mfma_16x16x32_bf16(A, m, acc[t][n]);
      acc[t][n] = mfma_16x16x32_bf16(A, l, acc[t][n]);
    }
  }
}

// grid (ceil(T / (64 MT)), ceil(E / 32), KS); wavefront w takes tokens 64 MT bx + 16 (MT w + t)
// for t < MT. NS > 0: a K chunk of exactly NS steps whose loads are all issued before the
// first MFMA (small batches: one memory round trip per workgroup); NS == 0: any chunk,
// streamed with the next step's loads in flight. direct: write logits (+ bias); else the
// partial tile of K chunk blockIdx.z to part[KS][T][E].
template <int MT, int NS>
__global__ void __launch_bounds__(256) router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ bias, int T,
                                                          int H, int E, int kchunk, int direct,
                                                          float* __restrict__ out) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * 64 * MT + wv * 16 * MT;
  const int e0 = blockIdx.y * kRExp;
  const int kb = blockIdx.z * kchunk, ke = min(H, kb + kchunk);
  // rows past T / E read the last valid row; their results are not stored
  const uint16_t* xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xr[t] = x + (size_t)min(t0 + 16 * t + r16, T - 1) * H + 8 * kq;
  const float* wr0 = w + (size_t)min(e0 + r16, E - 1) * H + 8 * kq;
  const float* wr1 = w + (size_t)min(e0 + 16 + r16, E - 1) * H + 8 * kq;
  auto load = [&](int k, uint4 (&xa)[MT], float4 (&wf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < MT; ++t) xa[t] = *reinterpret_cast<const uint4*>(xr[t] + k);
    wf[0] = *reinterpret_cast<const float4*>(wr0 + k);
    wf[1] = *reinterpret_cast<const float4*>(wr0 + k + 4);
    wf[2] = *reinterpret_cast<const float4*>(wr1 + k);
    wf[3] = *reinterpret_cast<const float4*>(wr1 + k + 4);
  };
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f acc[MT][2];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t][0] = acc[t][1] = zero4;
  if (NS > 0) {
    uint4 xa[NS > 0 ? NS : 1][MT];
    float4 wf[NS > 0 ? NS : 1][4];
#pragma unroll
    for (int s = 0; s < NS; ++s) load(kb + 32 * s, xa[s], wf[s]);
#pragma unroll
    for (int s = 0; s < NS; ++s) router_step<MT>(xa[s], wf[s], acc);
  } else {
    uint4 xa[MT], xn[MT];
    float4 wf[4], wn[4];
    load(kb, xa, wf);
    for (int k = kb; k < ke; k += 32) {
      load(min(k + 32, ke - 32), xn, wn);   // the last step re-reads itself (never used)
      router_step<MT>(xa, wf, acc);
#pragma unroll
      for (int t = 0; t < MT; ++t) xa[t] = xn[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[i] = wn[i];
    }
  }
  // element j of acc[t][n] in lane (r16, kq): token t0 + 16 t + 4 kq + j, expert e0 + 16 n + r16
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int e = e0 + 16 * n + r16;
    if (e >= E) continue;
    const float be = direct && bias ? bias[e] : 0.f;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = t0 + 16 * t + 4 * kq + j;
        if (tok >= T) continue;
        if (direct)
          out[(size_t)tok * E + e] = acc[t][n][j] + be;
        else
          out[((size_t)blockIdx.z * T + tok) * E + e] = acc[t][n][j];
      }
  }
}

// logits[t, e] = (sum over chunks c, in order, of part[c][t][e]) + bias[e]
__global__ void __launch_bounds__(256) router_reduce_kernel(const float* __restrict__ part,
                                                            const float* __restrict__ bias, int T,
                                                            int E, int KS,
                                                            float* __restrict__ logits) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n = (size_t)T * E;
  if (i >= n) return;
  float s = 0.f;
#pragma unroll 4
  for (int c = 0; c < KS; ++c) s += part[c * n + i];
  logits[i] = s + (bias ? bias[i % E] : 0.f);
}

// Small batches (T <= 256): one 16-token fragment per wavefront and K chunks of 256
// (8 steps, all loads up front). Larger: four fragments per wavefront (each split
// weight fragment feeds four token tiles) and K split so that the workgroups spread
// evenly over the CUs.
constexpr int kRSmallT = 256;
struct RouterPlan {
  int mt, ks, kchunk;
};
static RouterPlan router_plan(int T, int H, int E) {
  RouterPlan p;
  if (T <= kRSmallT) {
    p.mt = 1;
    p.kchunk = 256;
  } else {
    p.mt = 4;
    // K splits: the smallest k minimising ceil(tiles k / 256) / k, the number of workgroups
    // each of the 256 CUs runs times the work of one (a split count that leaves a few CUs
    // with one workgroup more than the rest costs a whole extra round)
    const int tiles = ((T + 255) / 256) * ((E + kRExp - 1) / kRExp);
    // (at most 8 splits, or as many as fill the GPU with one round when the tiles are few;
    // each split adds a [T, E] float32 partial tile to write and sum)
    int kmax = 256 / tiles > 8 ? 256 / tiles : 8;
    kmax = kmax > H / 256 ? H / 256 : kmax;
    kmax = kmax < 1 ? 1 : kmax;
    int k = 1;
    long best_num = (tiles + 255) / 256, best_den = 1;
    for (int c = 2; c <= kmax; ++c) {
      const long num = ((long)tiles * c + 255) / 256;
      if (num * best_den < best_num * c) {
        best_num = num;
        best_den = c;
        k = c;
      }
    }
    p.kchunk = ((H + k - 1) / k + 31) / 32 * 32;
  }
  p.ks = (H + p.kchunk - 1) / p.kchunk;
  return p;
}

size_t router_workspace_bytes(int T, int H, int E) {
  const RouterPlan p = router_plan(T, H, E);
  return p.ks > 1 ? (size_t)p.ks * T * E * sizeof(float) : 0;
}

int router_splits(int T, int H, int E) { return router_plan(T, H, E).ks; }

// The GEMM pass alone: with one K chunk it writes the logits (bias included) to dst,
// otherwise the partial tiles [ks][T][E] (summed by router_reduce_kernel, or by the
// routing kernels through LogitSrc).
hipError_t launch_router_gemm(const uint16_t* x, const float* w, const float* bias, int T, int H, int E,
                              float* dst, hipStream_t stream) {
  const RouterPlan p = router_plan(T, H, E);
  const int direct = p.ks == 1;
  const dim3 grid((T + 64 * p.mt - 1) / (64 * p.mt), (E + kRExp - 1) / kRExp, p.ks);
  // H % 128 == 0, so a 256-element chunk is whole except possibly the last one of H % 256 == 128:
  // that one runs the streaming kernel
  if (p.mt == 1 && H % 256 == 0)
    hipLaunchKernelGGL((router_gemm_kernel<1, 8>), grid, dim3(256), 0, stream, x, w, bias, T, H, E,
                       p.kchunk, direct, dst);
  else if (p.mt == 1)
    hipLaunchKernelGGL((router_gemm_kernel<1, 0>), grid, dim3(256), 0, stream, x, w, bias, T, H, E,
                       p.kchunk, direct, dst);
  else
    hipLaunchKernelGGL((router_gemm_kernel<4, 0>), grid, dim3(256), 0, stream, x, w, bias, T, H, E,
                       p.kchunk, direct, dst);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const float* w, const float* bias, int T, int H, int E,
                         float* logits, float* part, hipStream_t stream) {
  const RouterPlan p = router_plan(T, H, E);
  if (p.ks == 1) return launch_router_gemm(x, w, bias, T, H, E, logits, stream);
  const hipError_t e = launch_router_gemm(x, w, bias, T, H, E, part, stream);
  if (e != hipSuccess) return e;
  const size_t n = (size_t)T * E;
  hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     part, bias, T, E, p.ks, logits);
  return hipGetLastError();
}

}  // namespace srmoe
