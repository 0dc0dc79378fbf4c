// Device code shared by the routing, align and x-quantisation kernels and by the
// fused front of moe_layer_forward.
#pragma once
#include "common.hpp"

namespace srmoe {

// ----------------------------------------------------------------------------- routing
// Order-preserving map of a finite float to uint32 (-0 is folded into +0, so
// equal values compare equal and the id decides).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Where the router logits of a token come from: a [T,E] float32 array (ks == 0), or the
// router gate's K-split partial tiles part[c][T][E], c < ks, summed in chunk order and
// then offset by the bias -- the same float32 operations, in the same order, as the
// gate's own reduction pass, so both give the same logits bit for bit.
struct LogitSrc {
  const float* p;
  const float* bias;   // with ks > 0 (may be null)
  int ks;
  size_t stride;       // T * E: distance between partial tiles
};
__device__ __forceinline__ float logit_at(const LogitSrc& s, int t, int E, int e) {
  const size_t i = (size_t)t * E + e;
  if (s.ks == 0) return s.p[i];
  // 16 partial loads in flight at a time, summed in chunk order
  float v = 0.f;
  for (int c0 = 0; c0 < s.ks; c0 += 16) {
    float t[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) t[c] = c0 + c < s.ks ? s.p[(size_t)(c0 + c) * s.stride + i] : 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c)
      if (c0 + c < s.ks) v += t[c];
  }
  return v + (s.bias ? s.bias[e] : 0.f);
}

// Route token t with the 64 lanes of the caller's wavefront: the K routed experts
// with the largest logits in the order (logit desc, id asc), weights
// p_k / sum_{j in top-K} p_j (the full softmax denominator cancels; exponents are
// taken relative to the top logit), then the shared expert E in slot K with
// coefficient shared_weight. Each lane holds the logits of experts lane, lane+64,
// ... (E <= 255); each of the K rounds is a local max and a DPP wave reduction of a
// 64-bit key (ordered logit, 255 - id). ids/w are written to global memory;
// lds_ids (if not null) gets a copy of the ids. With append_shared false the rows
// have K entries and no shared slot (the routed-only router of the unfused layer).
__device__ __forceinline__ void route_token_wave(const LogitSrc& logits, int t, int E, int K,
                                                 float shared_weight, int32_t* __restrict__ ids,
                                                 float* __restrict__ w, int* lds_ids,
                                                 bool append_shared = true) {
  const int lane = threadIdx.x & 63;
  const int K1 = K + (append_shared ? 1 : 0);
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? ((uint64_t)ordered_key(logit_at(logits, t, E, e)) << 32) | (uint32_t)(255 - e)
                     : 0ull;
  }
  int sel_id[15];
  float sel_val[15];
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    sel_id[k] = 0;
    sel_val[k] = 0.f;
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
  // lane k < K takes slot k's exponent; the denominator is summed in slot order
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
      if (lds_ids) lds_ids[t * K1 + k] = sel_id[k];
    }
  }
  if (append_shared && lane == K) {
    ids[(size_t)t * K1 + K] = E;
    w[(size_t)t * K1 + K] = shared_weight;
    if (lds_ids) lds_ids[t * K1 + K] = E;
  }
}

// ----------------------------------------------------------------------------- x quantisation
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d, const ScaleDiv& q) {
  return quant2(q, a, b) | (quant2(q, c, d) << 16);
}

__device__ __forceinline__ float4 load_bf16x4(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                     bf16_to_f32(v.y >> 16));
}

__device__ __forceinline__ float amax4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// 8 bf16 values, low half of each word first
__device__ __forceinline__ float4 bf16x4_lo(const uint4& v) {
  return make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                     bf16_to_f32(v.y >> 16));
}
__device__ __forceinline__ float4 bf16x4_hi(const uint4& v) {
  return make_float4(bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xFFFFu),
                     bf16_to_f32(v.w >> 16));
}
__device__ __forceinline__ float amax_bf16x8(const uint4& v) {
  return fmaxf(amax4(bf16x4_lo(v)), amax4(bf16x4_hi(v)));
}
__device__ __forceinline__ uint2 encode_bf16x8(const uint4& v, const ScaleDiv& q) {
  const float4 a = bf16x4_lo(v), b = bf16x4_hi(v);
  return make_uint2(encode4(a.x, a.y, a.z, a.w, q), encode4(b.x, b.y, b.z, b.w, q));
}

// FP8 quantisation of token t's row of x by a group of 256 threads (tid 0..255);
// red points at 4 LDS floats owned by the group. Per-channel: one scale for the row
// (one pass while H <= 8192); block mode: one scale per 128 columns. Contains
// __syncthreads(), so every thread of the workgroup must call it (valid = false
// for groups without a token).
template <bool kBlock>
__device__ __forceinline__ void quant_x_token(const uint16_t* __restrict__ x, int t, bool valid, int H,
                                              uint8_t* __restrict__ xq, float* __restrict__ sx,
                                              int tid, float* red) {
  const int lane = tid & 63, wv = tid >> 6;
  const uint16_t* row = x + (size_t)t * H;
  uint8_t* qrow = xq + (size_t)t * H;
  if (!kBlock) {
    // 8 values (16 bytes) per thread and stripe: up to 4 stripes of 2048 values stay in
    // registers between the absmax and the encode (one pass while H <= 8192)
    constexpr int kMaxStripes = 4;
    uint4 v[kMaxStripes];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxStripes; ++i) {
      const int h = i * 2048 + tid * 8;
      v[i] = (valid && h < H) ? *reinterpret_cast<const uint4*>(row + h) : make_uint4(0u, 0u, 0u, 0u);
      amax = fmaxf(amax, amax_bf16x8(v[i]));
    }
    if (valid)
      for (int h = kMaxStripes * 2048 + tid * 8; h < H; h += 2048)
        amax = fmaxf(amax, amax_bf16x8(*reinterpret_cast<const uint4*>(row + h)));
    amax = wave_max(amax);
    if (lane == 0) red[wv] = amax;
    __syncthreads();
    const float scale = fp8_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    if (!valid) return;
    if (tid == 0) sx[t] = scale;
    const ScaleDiv q = scale_div(scale);
#pragma unroll
    for (int i = 0; i < kMaxStripes; ++i) {
      const int h = i * 2048 + tid * 8;
      if (h < H) *reinterpret_cast<uint2*>(qrow + h) = encode_bf16x8(v[i], q);
    }
    for (int h = kMaxStripes * 2048 + tid * 8; h < H; h += 2048)
      *reinterpret_cast<uint2*>(qrow + h) = encode_bf16x8(*reinterpret_cast<const uint4*>(row + h), q);
  } else {
    if (!valid) return;
    // 128-wide groups are 32 consecutive threads; H % 128 == 0 keeps every group whole.
    for (int h0 = 0; h0 < H; h0 += 1024) {
      const int h = h0 + tid * 4;
      const bool in = h < H;
      const float4 v = in ? load_bf16x4(row + h) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float scale = fp8_scale(group_max(amax4(v), 32));
      if (in && (tid & 31) == 0) sx[(size_t)t * (H / kGroup) + h / kGroup] = scale;
      if (in) *reinterpret_cast<uint32_t*>(qrow + h) = encode4(v.x, v.y, v.z, v.w, scale_div(scale));
    }
  }
}

// ----------------------------------------------------------------------------- align
// Stable counting sort of the flat (token, slot) entries by expert. A wavefront's chunk
// is an entry range [start, end) of at most 64 * kPer entries; lanes holding the same
// expert find each other with 8 ballots over the bits of the expert id; a lane's rank
// among them is the popcount of the lower lanes in that set, and the lowest lane
// advances the chunk's running count for that expert.
constexpr int kMaxE1 = 256;

__device__ __forceinline__ uint64_t lanes_with_same_expert(int e, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t set = __ballot(valid && bit);
    m &= bit ? set : ~set;
  }
  return m;
}

// entry start + 64*i + lane -> ev[i] (-1 past end); all loads issued together.
// ids may point to global memory or to LDS.
template <int kPer>
__device__ __forceinline__ void load_chunk(const int32_t* ids, int start, int end, int (&ev)[kPer]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = start + i * kWave + lane;
    ev[i] = s < end ? ids[s] : -1;
  }
}

// Count one chunk into cnt[0..E1) (LDS, zeroed by the caller).
template <int kPer>
__device__ __forceinline__ void count_chunk(const int (&ev)[kPer], int start, int end, int* cnt) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (start + i * kWave >= end) break;
    const bool valid = ev[i] >= 0;
    const int e = valid ? ev[i] : 0;
    const uint64_t m = lanes_with_same_expert(e, valid);
    if (valid && lane == __ffsll((unsigned long long)m) - 1) cnt[e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

// Scatter one chunk: run[e] (LDS) starts at the chunk's first output position for e.
template <int kPer>
__device__ __forceinline__ void scatter_chunk(const int (&ev)[kPer], int start, int end, int* run,
                                              int32_t* __restrict__ sorted) {
  const int lane = threadIdx.x & 63;
  const uint64_t lower = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (start + i * kWave >= end) break;
    const int s = start + i * kWave + lane;
    const bool valid = ev[i] >= 0;
    const int e = valid ? ev[i] : 0;
    const uint64_t m = lanes_with_same_expert(e, valid);
    int base = 0;
    if (valid) base = run[e];
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      sorted[base + __popcll(m & lower)] = s;
      if (lane == __ffsll((unsigned long long)m) - 1) run[e] = base + __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Exclusive scan of one value per thread over the workgroup (<= 16 wavefronts);
// wsum holds 16 ints of LDS. Returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* excl, int* wsum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int pre = 0, total = 0;
  for (int j = 0; j < nw; ++j) {
    if (j < wv) pre += wsum[j];
    total += wsum[j];
  }
  *excl = pre + inc - v;
  __syncthreads();
  return total;
}

// Expert totals -> padded offsets and the outputs. Thread e owns expert e (< E1 <= 256).
// off[e] (LDS) receives expert e's first row. `sorted` and `block_expert` must already
// hold the sentinel / -1 everywhere (fill_layout): only the used blocks' experts are
// written here, the entries by the scatter.
__device__ __forceinline__ void finish_layout(int e, int E1, int block_m, int total_e, int sentinel,
                                              int P_max, int* off, int* wsum,
                                              int32_t* __restrict__ sorted,
                                              int32_t* __restrict__ block_expert,
                                              int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ num_padded) {
  const int padded = (e < E1) ? (total_e + block_m - 1) / block_m * block_m : 0;
  int excl;
  const int total = block_exclusive_scan(padded, &excl, wsum);
  if (e < E1) {
    off[e] = excl;
    counts[e] = total_e;
    offsets[e] = excl;
    for (int b = excl / block_m; b < (excl + padded) / block_m; ++b) block_expert[b] = e;
  }
  if (threadIdx.x == 0) {
    offsets[E1] = total;
    num_padded[0] = total;
  }
}

// Every row of `sorted` := sentinel, every entry of `block_expert` := -1, with coalesced
// stores by `nthreads` threads numbered i (the padding rows and unused blocks keep these
// values; the align writes the rest afterwards).
__device__ __forceinline__ void fill_layout(int i, int nthreads, int sentinel, int block_m, int P_max,
                                            int32_t* __restrict__ sorted,
                                            int32_t* __restrict__ block_expert) {
  for (int r = i; r < P_max; r += nthreads) sorted[r] = sentinel;
  for (int b = i; b < P_max / block_m; b += nthreads) block_expert[b] = -1;
}

// Whole align of N <= 64 * kPer * (blockDim/64) entries inside one workgroup: the
// wavefronts take consecutive ranges of the entries (in whole 64s), count them into
// cnt[wave][E1], lay the experts out, then scatter stably. ids may be global or LDS;
// cnt holds (blockDim/64) x kMaxE1 ints of LDS, off kMaxE1, wsum 16.
template <int kPer>
__device__ __forceinline__ void align_in_workgroup(const int32_t* ids, int N, int E1, int block_m,
                                                   int P_max, int (*cnt)[kMaxE1], int* off, int* wsum,
                                                   int32_t* __restrict__ sorted,
                                                   int32_t* __restrict__ block_expert,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ num_padded) {
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int per = ((N + nw * kWave - 1) / (nw * kWave)) * kWave;
  const int start = min(wv * per, N), end = min(start + per, N);
  int ev[kPer];
  load_chunk<kPer>(ids, start, end, ev);
  fill_layout(threadIdx.x, blockDim.x, N, block_m, P_max, sorted, block_expert);
  for (int i = threadIdx.x; i < nw * kMaxE1; i += blockDim.x) (&cnt[0][0])[i] = 0;
  __syncthreads();
  count_chunk<kPer>(ev, start, end, cnt[wv]);
  __syncthreads();
  const int e = threadIdx.x;
  int total_e = 0;
  if (e < E1)
    for (int c = 0; c < nw; ++c) total_e += cnt[c][e];
  finish_layout(e, E1, block_m, total_e, N, P_max, off, wsum, sorted, block_expert, counts, offsets,
                num_padded);
  __syncthreads();
  if (e < E1) {   // per-wavefront first positions: expert offset + earlier wavefronts' counts
    int run = off[e];
    for (int c = 0; c < nw; ++c) {
      const int n = cnt[c][e];
      cnt[c][e] = run;
      run += n;
    }
  }
  __syncthreads();
  scatter_chunk<kPer>(ev, start, end, cnt[wv], sorted);
}

}  // namespace srmoe
