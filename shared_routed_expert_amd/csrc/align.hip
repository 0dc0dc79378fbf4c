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
// consecutive quarters of the entries; larger ones as count -> per-expert column scan
// -> scatter.
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

// Large inputs. Pass 1: per-chunk counts -> chunk_counts[chunk][E1]; the grid also
// fills sorted / block_expert with the sentinel / -1 (the later passes overwrite the
// used entries).
__global__ void __launch_bounds__(256) align_count_kernel(const int32_t* __restrict__ ids, int N,
                                                          int E1, int block_m, int P_max,
                                                          int32_t* __restrict__ chunk_counts,
                                                          int32_t* __restrict__ sorted,
                                                          int32_t* __restrict__ block_expert) {
  __shared__ int cnt[4][kMaxE1];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + wv;
  const int nchunks = (N + kChunk - 1) / kChunk;
  fill_layout(blockIdx.x * 256 + threadIdx.x, gridDim.x * 256, N, block_m, P_max, sorted, block_expert);
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

// Pass 2, one workgroup per expert e: expert e's column of chunk_counts becomes its
// exclusive prefix over the chunks (in chunk order), and e's total goes to totals[e]
// and counts[e]. 256 chunks per round of a workgroup-wide scan.
__global__ void __launch_bounds__(256) align_colscan_kernel(int N, int E1,
                                                            int32_t* __restrict__ chunk_counts,
                                                            int32_t* __restrict__ totals,
                                                            int32_t* __restrict__ counts) {
  __shared__ int wsum[16];
  const int e = blockIdx.x;
  const int nchunks = (N + kChunk - 1) / kChunk;
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int v = c < nchunks ? chunk_counts[(size_t)c * E1 + e] : 0;
    int excl;
    const int tot = block_exclusive_scan(v, &excl, wsum);
    if (c < nchunks) chunk_counts[(size_t)c * E1 + e] = carry + excl;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    totals[e] = carry;
    counts[e] = carry;
  }
}

// Pass 3: every workgroup lays the experts out from the totals (thread e owns expert e:
// padded segment, exclusive scan); workgroup 0 writes offsets and num_padded, workgroup
// g the block_expert entries of the experts e with e % gridDim == g. Then each
// wavefront scatters one chunk stably from position offset[e] + chunk prefix[e].
__global__ void __launch_bounds__(256) align_scatter_kernel(
    const int32_t* __restrict__ ids, int N, int E1, int block_m,
    const int32_t* __restrict__ chunk_prefix, const int32_t* __restrict__ totals,
    int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded) {
  __shared__ int run[4][kMaxE1];
  __shared__ int off[kMaxE1];
  __shared__ int wsum[16];
  const int e = threadIdx.x;
  const int total_e = e < E1 ? totals[e] : 0;
  const int padded = (total_e + block_m - 1) / block_m * block_m;
  int excl;
  const int total = block_exclusive_scan(padded, &excl, wsum);
  if (e < E1) {
    off[e] = excl;
    if (blockIdx.x == 0) offsets[e] = excl;
    if (e % (int)gridDim.x == (int)blockIdx.x)
      for (int b = excl / block_m; b < (excl + padded) / block_m; ++b) block_expert[b] = e;
  }
  if (blockIdx.x == 0 && e == 0) {
    offsets[E1] = total;
    num_padded[0] = total;
  }
  __syncthreads();
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + wv;
  const int nchunks = (N + kChunk - 1) / kChunk;
  if (chunk >= nchunks) return;
  const int start = chunk * kChunk, end = min(start + kChunk, N);
  int ev[kPerLane];
  load_chunk<kPerLane>(ids, start, end, ev);
  for (int i = lane; i < E1; i += kWave) run[wv][i] = off[i] + chunk_prefix[(size_t)chunk * E1 + i];
  __builtin_amdgcn_wave_barrier();
  scatter_chunk<kPerLane>(ev, start, end, run[wv], sorted);
}

// workspace: chunk_counts [nchunks][E1], then the expert totals [E1]
static size_t chunk_table_bytes(size_t N, int E1) {
  const size_t nchunks = (N + kChunk - 1) / kChunk;
  return (nchunks * E1 * sizeof(int32_t) + 255) / 256 * 256;
}

size_t align_workspace_bytes(int T, int K1, int E1) {
  return chunk_table_bytes((size_t)T * K1, E1) + ((size_t)E1 * sizeof(int32_t) + 255) / 256 * 256;
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
  int32_t* totals = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + chunk_table_bytes(N, E1));
  const int grid = (nchunks + 3) / 4;
  hipLaunchKernelGGL(align_count_kernel, dim3(grid), dim3(256), 0, stream, ids, N, E1, block_m, P_max,
                     chunk_counts, sorted, block_expert);
  hipLaunchKernelGGL(align_colscan_kernel, dim3(E1), dim3(256), 0, stream, N, E1, chunk_counts, totals,
                     counts);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(grid), dim3(256), 0, stream, ids, N, E1, block_m,
                     chunk_counts, totals, sorted, block_expert, offsets, num_padded);
  return hipGetLastError();
}

}  // namespace srmoe
