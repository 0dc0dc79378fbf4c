// Align / sort / pad of the (token, slot) entries by expert: a stable counting sort.
//
// The T*K1 flat entries s = t*K1 + k are cut into chunks of 1024, one
// wavefront per chunk. Inside a chunk, 64 entries at a time, lanes holding the
// same expert find each other with 8 ballots over the bits of the expert id;
// a lane's rank among them is the popcount of the lower lanes in that set, and
// the lowest lane advances the chunk's running count for the expert. Chunks
// are processed in entry order, experts are laid out in ascending id and each
// expert's segment is padded to the MFMA row block (block_m) with the
// sentinel T*K1. Nothing depends on atomics or scheduling, so the output is
// the unique stable order.
//
// Small inputs (<= 4 chunks) run as one workgroup whose 4 wavefronts take
// consecutive quarters of the entries; larger ones as count -> scan -> scatter.
#include "common.hpp"

namespace srmoe {

constexpr int kChunk = 1024;
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

constexpr int kPerLane = kChunk / kWave;   // 16 entries of a chunk per lane

// A wavefront's chunk is the entry range [start, end), at most kChunk long.
// Load its expert ids into registers: entry start + 64*i + lane -> ev[i] (-1 past end).
// All loads are issued together, so a chunk costs one memory round trip.
__device__ __forceinline__ void load_chunk(const int32_t* __restrict__ ids, int start, int end,
                                           int (&ev)[kPerLane]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int s = start + i * kWave + lane;
    ev[i] = s < end ? ids[s] : -1;
  }
}

// Count the entries of one chunk into cnt[0..E1) (LDS, zeroed by the caller).
__device__ __forceinline__ void count_chunk(const int (&ev)[kPerLane], int start, int end, int* cnt) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    if (start + i * kWave >= end) break;
    const bool valid = ev[i] >= 0;
    const int e = valid ? ev[i] : 0;
    const uint64_t m = lanes_with_same_expert(e, valid);
    if (valid && lane == __ffsll((unsigned long long)m) - 1) cnt[e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

// Scatter one chunk: run[e] (LDS) starts at the chunk's first output position for e.
__device__ __forceinline__ void scatter_chunk(const int (&ev)[kPerLane], int start, int end, int* run,
                                              int32_t* __restrict__ sorted) {
  const int lane = threadIdx.x & 63;
  const uint64_t lower = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
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

// Exclusive scan of one value per thread over a 256-thread workgroup; returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* excl, int* lds4) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == 63) lds4[wv] = inc;
  __syncthreads();
  int pre = 0;
  for (int j = 0; j < wv; ++j) pre += lds4[j];
  const int total = lds4[0] + lds4[1] + lds4[2] + lds4[3];
  *excl = pre + inc - v;
  __syncthreads();
  return total;
}

// Expert totals -> padded offsets, outputs, and the padding/tail fills. Thread e
// owns expert e. Returns through LDS: off[e] = expert e's first row.
__device__ void finish_layout(int e, int E1, int block_m, int total_e, int sentinel, int P_max,
                              int* off, int* lds4, int32_t* __restrict__ sorted,
                              int32_t* __restrict__ block_expert, int32_t* __restrict__ counts,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded) {
  const int padded = (e < E1) ? (total_e + block_m - 1) / block_m * block_m : 0;
  int excl;
  const int total = block_exclusive_scan(padded, &excl, lds4);
  if (e < E1) {
    off[e] = excl;
    counts[e] = total_e;
    offsets[e] = excl;
    for (int r = excl + total_e; r < excl + padded; ++r) sorted[r] = sentinel;
    for (int b = excl / block_m; b < (excl + padded) / block_m; ++b) block_expert[b] = e;
  }
  if (threadIdx.x == 0) {
    offsets[E1] = total;
    num_padded[0] = total;
  }
  for (int r = total + threadIdx.x; r < P_max; r += blockDim.x) sorted[r] = sentinel;
  for (int b = total / block_m + threadIdx.x; b < P_max / block_m; b += blockDim.x) block_expert[b] = -1;
}

__global__ void __launch_bounds__(256) align_small_kernel(
    const int32_t* __restrict__ ids, int N, int E1, int block_m, int P_max,
    int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded) {
  __shared__ int cnt[4][kMaxE1];
  __shared__ int off[kMaxE1];
  __shared__ int lds4[4];
  const int wv = threadIdx.x >> 6;
  // the N <= 4*kChunk entries are split over the 4 wavefronts in order, in whole 64s
  const int per = ((N + 4 * kWave - 1) / (4 * kWave)) * kWave;
  const int start = min(wv * per, N), end = min(start + per, N);
  int ev[kPerLane];
  load_chunk(ids, start, end, ev);
  for (int i = threadIdx.x; i < 4 * kMaxE1; i += blockDim.x) (&cnt[0][0])[i] = 0;
  __syncthreads();
  count_chunk(ev, start, end, cnt[wv]);
  __syncthreads();
  const int e = threadIdx.x;
  int total_e = 0;
  if (e < E1) total_e = cnt[0][e] + cnt[1][e] + cnt[2][e] + cnt[3][e];
  finish_layout(e, E1, block_m, total_e, N, P_max, off, lds4, sorted, block_expert, counts, offsets,
                num_padded);
  __syncthreads();
  if (e < E1) {  // per-chunk first positions: expert offset + earlier chunks' counts
    int run = off[e];
    for (int c = 0; c < 4; ++c) {
      const int n = cnt[c][e];
      cnt[c][e] = run;
      run += n;
    }
  }
  __syncthreads();
  scatter_chunk(ev, start, end, cnt[wv], sorted);
}

// Large inputs. Pass 1: per-chunk counts -> chunk_counts[chunk][E1].
__global__ void __launch_bounds__(256) align_count_kernel(const int32_t* __restrict__ ids, int N,
                                                          int E1, int32_t* __restrict__ chunk_counts) {
  __shared__ int cnt[4][kMaxE1];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + wv;
  const int nchunks = (N + kChunk - 1) / kChunk;
  for (int i = lane; i < kMaxE1; i += kWave) cnt[wv][i] = 0;
  __builtin_amdgcn_wave_barrier();
  if (chunk >= nchunks) return;
  const int start = chunk * kChunk, end = min(start + kChunk, N);
  int ev[kPerLane];
  load_chunk(ids, start, end, ev);
  count_chunk(ev, start, end, cnt[wv]);
  __builtin_amdgcn_wave_barrier();
  for (int i = lane; i < E1; i += kWave) chunk_counts[(size_t)chunk * E1 + i] = cnt[wv][i];
}

// Pass 2 (one workgroup): totals, padded offsets, outputs, fills; chunk_counts
// becomes each chunk's first output position per expert.
__global__ void __launch_bounds__(256) align_scan_kernel(
    int N, int E1, int block_m, int P_max, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded) {
  __shared__ int off[kMaxE1];
  __shared__ int lds4[4];
  const int nchunks = (N + kChunk - 1) / kChunk;
  const int e = threadIdx.x;
  int total_e = 0;
  if (e < E1)
    for (int c = 0; c < nchunks; ++c) total_e += chunk_counts[(size_t)c * E1 + e];
  finish_layout(e, E1, block_m, total_e, N, P_max, off, lds4, sorted, block_expert, counts, offsets,
                num_padded);
  __syncthreads();
  if (e < E1) {
    int run = off[e];
    for (int c = 0; c < nchunks; ++c) {
      const int n = chunk_counts[(size_t)c * E1 + e];
      chunk_counts[(size_t)c * E1 + e] = run;
      run += n;
    }
  }
}

// Pass 3: stable scatter of every chunk.
__global__ void __launch_bounds__(256) align_scatter_kernel(const int32_t* __restrict__ ids, int N,
                                                            int E1,
                                                            const int32_t* __restrict__ chunk_base,
                                                            int32_t* __restrict__ sorted) {
  __shared__ int run[4][kMaxE1];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + wv;
  const int nchunks = (N + kChunk - 1) / kChunk;
  if (chunk >= nchunks) return;
  const int start = chunk * kChunk, end = min(start + kChunk, N);
  int ev[kPerLane];
  load_chunk(ids, start, end, ev);
  for (int i = lane; i < E1; i += kWave) run[wv][i] = chunk_base[(size_t)chunk * E1 + i];
  __builtin_amdgcn_wave_barrier();
  scatter_chunk(ev, start, end, run[wv], sorted);
}

size_t align_workspace_bytes(int T, int K1, int E1) {
  const size_t N = (size_t)T * K1;
  const size_t nchunks = (N + kChunk - 1) / kChunk;
  return (nchunks * E1 * sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_align(const int32_t* ids, int T, int K1, int E1, int block_m, int32_t* sorted,
                        int32_t* block_expert, int32_t* counts, int32_t* offsets,
                        int32_t* num_padded, void* ws, hipStream_t stream) {
  const int N = T * K1;
  const int P_max = (int)sorted_capacity(T, K1, E1, block_m);
  const int nchunks = (N + kChunk - 1) / kChunk;
  if (nchunks <= 4) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(256), 0, stream, ids, N, E1, block_m, P_max,
                       sorted, block_expert, counts, offsets, num_padded);
    return hipGetLastError();
  }
  int32_t* chunk_counts = static_cast<int32_t*>(ws);
  const int grid = (nchunks + 3) / 4;
  hipLaunchKernelGGL(align_count_kernel, dim3(grid), dim3(256), 0, stream, ids, N, E1, chunk_counts);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(256), 0, stream, N, E1, block_m, P_max,
                     chunk_counts, sorted, block_expert, counts, offsets, num_padded);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(grid), dim3(256), 0, stream, ids, N, E1, chunk_counts,
                     sorted);
  return hipGetLastError();
}

}  // namespace srmoe
