// Align / sort / pad of the (token, slot) entries by expert: a stable counting sort.
//
// The T*K1 flat entries s = t*K1 + k are cut into chunks of 256, one
// wavefront per chunk. Inside a chunk, 64 entries at a time, lanes holding the
// same expert find each other with 8 ballots over the bits of the expert id;
// a lane's rank among them is the popcount of the lower lanes in that set, and
// the lowest lane advances the chunk's running count for the expert. Chunks
// are processed in entry order, experts are laid out in ascending id and each
// expert's segment is padded to the MFMA row block (block_m) with the
// sentinel T*K1. Nothing depends on atomics or scheduling, so the output is
// the unique stable order.
//
// Small inputs (<= 4096 entries) run as one workgroup whose 4 wavefronts take
// consecutive quarters of the entries; larger ones as count -> scan -> scatter.
#include "front_dev.hpp"

namespace srmoe {

constexpr int kSmallMax = 4096;                 // entries handled by the one-workgroup path
constexpr int kSmallPerLane = kSmallMax / 256;   // 16 per lane there
constexpr int kChunk = 256;                      // entries per wavefront chunk in the large path
constexpr int kPerLane = kChunk / kWave;         // 4 entries of a chunk per lane

__global__ void __launch_bounds__(256) align_small_kernel(
    const int32_t* __restrict__ ids, int N, int E1, int block_m, int P_max,
    int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded) {
  __shared__ int cnt[4][kMaxE1];
  __shared__ int off[kMaxE1];
  __shared__ int wsum[16];
  align_in_workgroup<kSmallPerLane>(ids, N, E1, block_m, P_max, cnt, off, wsum, sorted,
                                    block_expert, counts, offsets, num_padded);
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
  load_chunk<kPerLane>(ids, start, end, ev);
  count_chunk<kPerLane>(ev, start, end, cnt[wv]);
  __builtin_amdgcn_wave_barrier();
  for (int i = lane; i < E1; i += kWave) chunk_counts[(size_t)chunk * E1 + i] = cnt[wv][i];
}

// Pass 2 (one workgroup): totals, padded offsets, outputs, fills; chunk_counts
// becomes each chunk's first output position per expert. Thread e walks expert e's
// column of chunk_counts kScanU chunks at a time, all of a group's loads issued before
// they are used (one load per iteration would wait on memory once per chunk).
constexpr int kScanU = 16;

__global__ void __launch_bounds__(256) align_scan_kernel(
    int N, int E1, int block_m, int P_max, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded) {
  __shared__ int off[kMaxE1];
  __shared__ int wsum[16];
  const int nchunks = (N + kChunk - 1) / kChunk;
  const int e = threadIdx.x;
  int total_e = 0;
  if (e < E1)
    for (int c0 = 0; c0 < nchunks; c0 += kScanU) {
      int v[kScanU];
#pragma unroll
      for (int u = 0; u < kScanU; ++u) v[u] = c0 + u < nchunks ? chunk_counts[(size_t)(c0 + u) * E1 + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanU; ++u) total_e += v[u];
    }
  finish_layout(e, E1, block_m, total_e, N, P_max, off, wsum, sorted, block_expert, counts, offsets,
                num_padded);
  __syncthreads();
  if (e < E1) {
    int run = off[e];
    for (int c0 = 0; c0 < nchunks; c0 += kScanU) {
      int v[kScanU];
#pragma unroll
      for (int u = 0; u < kScanU; ++u) v[u] = c0 + u < nchunks ? chunk_counts[(size_t)(c0 + u) * E1 + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        if (c0 + u < nchunks) chunk_counts[(size_t)(c0 + u) * E1 + e] = run;
        run += v[u];
      }
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
  load_chunk<kPerLane>(ids, start, end, ev);
  for (int i = lane; i < E1; i += kWave) run[wv][i] = chunk_base[(size_t)chunk * E1 + i];
  __builtin_amdgcn_wave_barrier();
  scatter_chunk<kPerLane>(ev, start, end, run[wv], sorted);
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
  if (N <= kSmallMax) {
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
