// Both expert GEMMs of a 16-row block in one workgroup (decode-shaped batches).
//
// A block is 16 sorted rows of one expert e. One 512-thread workgroup per block:
//
//  phase 1  gate/up: the block's 16 token rows of x_q go to LDS once; each of
//           the 8 wavefronts owns NT = I / 64 tiles of 16 rows of w13[e] and
//           streams them tile after tile in batches of 16 rows x 1 KB of K,
//           one load instruction per row (1 KB contiguous: HBM streams runs
//           like these faster than the same bytes as 8 rows x 128 B). A batch
//           passes through the wavefront's LDS buffer in two 512-byte halves
//           into the MFMA fragment layout (x is the A operand, the weight rows
//           the B operand). Two batches are in flight per wavefront: while one
//           is multiplied the next is loading.
//  phase 2  g, u -> a = silu(g) * u -> FP8 a_q with the row (or row x 128-column
//           group) absmax scale, in LDS; the row's output scale is its routing
//           weight (times the FP8 scale per channel). a itself (float32) is also
//           stored to the workspace, where the split kernels keep it, when a_out
//           is given.
//  phase 3  down: each wavefront takes every eighth group of 64 output columns;
//           a group's 64 rows of w2[e] are 64 * I contiguous bytes, loaded as
//           1 KB runs and passed through LDS into the swap-AB fragment layout
//           (weights as the A operand, a_q as B), the next group loading while
//           one is multiplied. The weighted bf16 rows pass through LDS once more so
//           that every store writes whole 128-byte row pieces to slot_out.
//
// The split kernels stream the same weights but pass a through HBM, quantise it in
// a pass of their own and re-read it; here the down GEMM takes a_q from LDS and
// one launch replaces three. All the block's work sits on one CU, so the ~160
// workgroups of a decode batch stream side by side with eight wavefronts each
// (enough loads in flight to keep HBM busy at that count).
//
// Weight loads go through buffer resources made per K step or column group
// (scalar registers): a prefetch past the end gets a resource of zero length and
// returns zeros without touching memory, so no load is predicated and the
// compiler's memory waits stay exact. Everything the epilogues need per row or
// column is fetched in the prologue: a load issued behind a prefetch can only be
// waited for together with it.
#include "common.hpp"

namespace srmoe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXMaxH = 5120;                    // largest H whose x rows fit the LDS budget
constexpr int kXMaxHB = kXMaxH / kGroup;
constexpr int kRunK = 1024;                     // K bytes of a phase-1 batch per row
constexpr int kHalfRS = kRunK / 2 + 16;         // LDS row stride of a staged half batch
constexpr int kOutRS = 128 + 16;                // LDS row stride of a staged group of output rows

// Raw buffer resource over [base, base + bytes) (GFX9 descriptor word 3); loads at
// offsets past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// Cache policy of the weight loads: non-temporal (every weight byte is read once per
// layer; streaming them past the caches keeps the small per-token data of the other
// launches cached, which was measured faster overall).
constexpr int kWeightPolicy = 2;
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kWeightPolicy);
}

template <int NT>
struct ExpertDecodeLds {
  static constexpr int I = NT * 64;
  static constexpr int kX = 16 * (kXMaxH + 16);                 // x rows (phase 1)
  static constexpr int kStage1 = 8 * 16 * kHalfRS;              // per-wavefront half batches (phase 1)
  static constexpr int kGU = 16 * (2 * I + 4) * 4;              // g|u float32 (phase 1 -> 2)
  static constexpr int kStage3 = 8 * 64 * (I + 16);             // per-wavefront w2 groups (phase 3)
  static constexpr int kOut = 8 * 8 * kOutRS;                    // per-wavefront output rows (phase 3)
  static constexpr int kP3 = kStage3 + kOut;
  static constexpr int kBig = (kX + kStage1) > kP3 ? ((kX + kStage1) > kGU ? kX + kStage1 : kGU)
                                                   : (kP3 > kGU ? kP3 : kGU);
};

// The in-kernel align (kAlign): every workgroup derives the expert-sorted layout of
// the T*K1 <= kAlignMaxN routed entries itself and writes its share of the align
// outputs (see the prologue).
constexpr int kAlignMaxN = 4096;
struct AlignOut {
  const int32_t* topk_ids;   // [T*K1] in
  int32_t* counts;           // [E1] out (workgroup 0)
  int32_t* offsets;          // [E1+1] out (workgroup 0)
  int32_t* num_padded;       // [1] out (workgroup 0)
  int E1;
};

template <bool kBlock, int NT, bool kAlign>   // NT = I / 64
__global__ void __launch_bounds__(512) expert_ffn_decode_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ sx, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const uint8_t* __restrict__ w2, const float* __restrict__ s2,
    int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert, AlignOut al,
    const float* __restrict__ topk_w, float* __restrict__ a_out, uint16_t* __restrict__ slot_out,
    int T, int H, int K1) {
  using Lds = ExpertDecodeLds<NT>;
  constexpr int I = Lds::I;
  constexpr int AS = I + 16;                // a_q row stride
  constexpr int GS = 2 * I + 4;             // g|u row stride (floats)
  constexpr int NI = I / 16;                // 1 KB runs per 64-row w2 group
  constexpr int C = I / 32;                 // phase-2 columns per thread
  __shared__ __align__(16) uint8_t big[Lds::kBig];
  __shared__ __align__(16) uint8_t aqs[16 * AS];
  __shared__ float rsc_s[16];
  __shared__ float sa_s[16][2];
  __shared__ int srow_s[16];
  __shared__ float wgt_s[16];
  __shared__ __align__(16) float sxs[kBlock ? kXMaxHB * 16 : 16];
  __shared__ float s13s[kBlock ? (2 * I / kGroup) * kXMaxHB : 1];   // w13[e]'s block scales

  const int b = blockIdx.x;
  int bb = b;   // the block of the sorted layout this workgroup computes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control
  const int r16 = lane & 15, kq = lane >> 4;
  const int sentinel = T * K1;
  const uint64_t magic = slot_div_magic(K1);
  const int HB = H / kGroup, nsteps = H / kGroup;
  const int XS = H + 16;
  uint8_t* xs = big;
  uint8_t* stg1 = big + Lds::kX + wv * (16 * kHalfRS);

  // ---- the block: its expert e (-1 past the used rows) and its 16 sorted rows -> srow_s
  int e;
  if (!kAlign) {
    // the used blocks in reverse, walked per XCD, as in the align branch below
    const int nu = min(al.num_padded[0] / 16, (int)gridDim.x);
    bb = b < nu ? nu - 1 - xcd_tile(b, nu) : b;
    e = block_expert[bb];
    if (e < 0) return;
    if (tid < 16) srow_s[tid] = sorted[bb * 16 + tid];
  } else {
    // The layout of the align call, derived here from topk_ids: per-expert counts
    // (LDS atomics; counts do not depend on their order), each expert's segment padded
    // to 16 rows in ascending expert order, then the block's rows = the entries of its
    // expert ranked 16 (b - first block) .. + 15 in flat-slot order (ballots), padding
    // rows = the sentinel. Entry s = 512 j + tid is held by thread tid.
    __shared__ int e_s, bb_s;
    int* cnt_l = reinterpret_cast<int*>(big);   // [256]
    int* pad_l = cnt_l + 256;                   // [256] first row of each expert
    int* wc_l = pad_l + 256;                    // [8][8] entries of e per (j, wavefront)
    constexpr int kJ = kAlignMaxN / 512;
    int idv[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) idv[j] = 512 * j + tid < sentinel ? al.topk_ids[512 * j + tid] : -1;
    if (tid < 256) cnt_l[tid] = 0;
    if (tid < 16) srow_s[tid] = sentinel;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      if (idv[j] >= 0) atomicAdd(&cnt_l[idv[j]], 1);
    __syncthreads();
    if (wv == 0) {   // exclusive scan of the padded counts, 4 experts per lane
      int pc[4], sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ex = lane * 4 + u;
        pc[u] = ex < al.E1 ? (cnt_l[ex] + 15) & ~15 : 0;
        sum += pc[u];
      }
      int inc = sum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += n;
      }
      const int total = __shfl(inc, kWave - 1, kWave);
      // the used blocks in reverse, walked per XCD: the shared expert's blocks (the last
      // ones) share one XCD's L2, the one that takes the extra block when 8 does not
      // divide their number
      const int nu = total / 16;
      const int bp = b < nu ? nu - 1 - xcd_tile(b, nu) : b;
      int run = inc - sum;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ex = lane * 4 + u;
        if (ex < al.E1) {
          pad_l[ex] = run;
          if (b == 0) {
            al.counts[ex] = cnt_l[ex];
            al.offsets[ex] = run;
          }
        }
        if (pc[u] > 0 && bp * 16 >= run && bp * 16 < run + pc[u]) e_s = ex;
        run += pc[u];
      }
      if (lane == 0) {
        bb_s = bp;
        if (bp * 16 >= total) e_s = -1;
        if (b == 0) {
          al.offsets[al.E1] = total;
          al.num_padded[0] = total;
        }
      }
    }
    __syncthreads();
    e = e_s;
    bb = bb_s;
    if (e >= 0) {
      const int first = bb * 16 - pad_l[e];   // rank of the block's first row within e
      const uint64_t lower = (1ull << lane) - 1ull;
      uint64_t m[kJ];
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        m[j] = __ballot(idv[j] == e);
        if (lane == 0) wc_l[j * 8 + wv] = __popcll(m[j]);
      }
      __syncthreads();
      int before = 0;   // entries of e in (j, wavefront) pairs ahead of this one
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        int mine = before;
        for (int w = 0; w < 8; ++w) {
          const int c = wc_l[j * 8 + w];
          mine += w < wv ? c : 0;
          before += c;
        }
        if (idv[j] == e) {
          const int r = mine + __popcll(m[j] & lower) - first;
          if (r >= 0 && r < 16) srow_s[r] = 512 * j + tid;
        }
      }
    }
    __syncthreads();
    if (tid < 16) sorted[bb * 16 + tid] = srow_s[tid];
    if (tid == 0) block_expert[bb] = e;
    if (e < 0) return;
  }
  __syncthreads();

  // ---- phase 1 prologue: per-row and per-column data, x rows into LDS, first weight batch
  const uint8_t* w13e = w13 + (size_t)e * 2 * I * H;
  const int tile0 = wv * NT;   // first of the wavefront's 16-row tiles of w13[e]
  // Batch q = (tile pass q / nchunks, K chunk q % nchunks): row r of the tile is load r, at
  // scalar offset r * H; lane l takes bytes 16 l .. 16 l + 15 of the chunk (an out-of-range
  // offset, read as zero, past the end of a row). Batches past the last get a zero-length
  // resource.
  const int nchunks = (H + kRunK - 1) / kRunK;
  const int nq = NT * nchunks;
  // (the blocks of one expert, the shared expert's at decode, run on one XCD and walk
  // the same K chunks in step, so that its L2 serves the lines they share)
  auto batch_load = [&](int q, u32x4 (&L)[16]) __attribute__((always_inline)) {
    const int n = q / nchunks, c = q - n * nchunks;
    const bool in = q < nq;
    const __amdgpu_buffer_rsrc_t r =
        slice_rsrc(w13e + (in ? (size_t)16 * (tile0 + n) * H : 0), in ? (uint32_t)(16 * H) : 0u);
    const int o = c * kRunK + lane * 16;
    const uint32_t vo = o < H ? (uint32_t)o : 0x80000000u;
#pragma unroll
    for (int i = 0; i < 16; ++i) L[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, i * H, kWeightPolicy);
  };
  float sc13[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) sc13[n] = kBlock ? 1.f : s13[(size_t)e * 2 * I + 16 * (tile0 + n) + r16];
  if (tid < 16) {
    const int s = srow_s[tid];
    wgt_s[tid] = s < sentinel ? topk_w[s] : 0.f;
  }
  if (kBlock) {
    for (int i = tid; i < (2 * I / kGroup) * HB; i += 512) s13s[i] = s13[(size_t)e * (2 * I / kGroup) * HB + i];
    for (int i = tid; i < 16 * HB; i += 512) {
      const int r = i & 15, kb = i >> 4;
      const int s = srow_s[r];
      sxs[i] = s < sentinel ? sx[(size_t)slot_token(s, magic) * HB + kb] : 0.f;
    }
  } else if (tid < 16) {
    const int s = srow_s[tid];
    sxs[tid] = s < sentinel ? sx[slot_token(s, magic)] : 0.f;
  }
  u32x4 LA[16], LB[16];
  {
    // thread -> (row tid / 32, 16-byte chunks part, part + 32, ...); padding rows read token 0
    const int xr = tid >> 5, part = tid & 31;
    const int s_x = srow_s[xr];
    const int tx = s_x < sentinel ? slot_token(s_x, magic) : 0;
    const uint8_t* src = xq + (size_t)tx * H;
    constexpr int kMaxChunks = kXMaxH / 16 / 32;
    u32x4 xv[kMaxChunks];
#pragma unroll
    for (int m = 0; m < kMaxChunks; ++m) {
      const int c = part + 32 * m;
      if (c < H / 16) xv[m] = *reinterpret_cast<const u32x4*>(src + c * 16);
    }
    // the first weight batch goes out behind the x rows, so that waiting for x leaves it in flight
    batch_load(0, LA);
#pragma unroll
    for (int m = 0; m < kMaxChunks; ++m) {
      const int c = part + 32 * m;
      // opaque: a plain load-then-store pair would be merged into one copy placed at the store
      asm volatile("" : "+v"(xv[m]));
      if (c < H / 16) *reinterpret_cast<u32x4*>(xs + xr * XS + c * 16) = xv[m];
    }
  }
  __syncthreads();

  // ---- phase 1: gate/up
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  // cur accumulates the tile being streamed; at the end of a tile pass it is pushed onto
  // acc[] (static register indices), which then holds the passes in order
  v4f acc[NT], cur = zero4;
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = zero4;
  auto process = [&](u32x4 (&L)[16], int q) __attribute__((always_inline)) {
    const int n = q / nchunks, c = q - n * nchunks;
    const int srow13 = (16 * (tile0 + n)) / kGroup;   // the tile's block row of w13[e]'s scales
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if ((lane >> 5) == h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) *reinterpret_cast<u32x4*>(stg1 + i * kHalfRS + (lane & 31) * 16) = L[i];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // past the end of K the weights read as zero; x stays on a real step (finite codes)
        const int kb = min(c * 8 + h * 4 + j, nsteps - 1);
        const v8i A = load32(xs + r16 * XS + kb * kGroup + kq * 32);
        const v8i B = load32(stg1 + r16 * kHalfRS + j * kGroup + kq * 32);
        if (!kBlock) {
          cur = mfma_16x16x128_fp8(A, B, cur);
        } else {
          const v4f t = mfma_16x16x128_fp8(A, B, zero4);
          const float sw = s13s[srow13 * HB + kb];
          const float4 sxr = *reinterpret_cast<const float4*>(&sxs[kb * 16 + 4 * kq]);
          cur[0] += t[0] * (sxr.x * sw);
          cur[1] += t[1] * (sxr.y * sw);
          cur[2] += t[2] * (sxr.z * sw);
          cur[3] += t[3] * (sxr.w * sw);
        }
      }
      // bounds how far the scheduler hoists fragment reads (registers: two batches are live)
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" : "+v"(cur));   // the batch's MFMAs stay in the batch (not sunk into the next)
    if (q < nq && c == nchunks - 1) {   // the pass's last batch
#pragma unroll
      for (int m = 0; m + 1 < NT; ++m) acc[m] = acc[m + 1];
      acc[NT - 1] = cur;
      cur = zero4;
    }
  };
#pragma unroll 1
  for (int q = 0; q < nq; q += 2) {
    batch_load(q + 1, LB);
    __builtin_amdgcn_sched_barrier(0);
    process(LA, q);
    batch_load(q + 2, LA);
    __builtin_amdgcn_sched_barrier(0);
    process(LB, q + 1);
  }

  // ---- phase 3 prologue: the wavefront's first w2 group starts loading now
  const int ng = H / 64;
  const int n_my = (ng - wv + 7) >> 3;   // groups wv, wv + 8, ... below ng
  // the wavefront's i-th group; i >= n_my maps past the end (an empty load, no stores)
  auto group_of = [&](int i) __attribute__((always_inline)) { return i < n_my ? wv + 8 * i : ng; };
  const uint8_t* w2e = w2 + (size_t)e * H * I;
  const float* s2e = s2 + (size_t)e * H;
  // the wavefront's i-th group: its 64 rows of w2[e] and their 64 channel scales
  auto load_group = [&](int i, u32x4 (&W)[NI], u32x4 (&S)[4]) __attribute__((always_inline)) {
    const int g = group_of(i);
    const bool in = g < ng;
    const __amdgpu_buffer_rsrc_t r = slice_rsrc(w2e + (in ? g * 64 * I : 0), in ? 64u * I : 0u);
#pragma unroll
    for (int j = 0; j < NI; ++j) W[j] = bload(r, (uint32_t)(j * 1024 + lane * 16));
    if (!kBlock) {
      const __amdgpu_buffer_rsrc_t rs = slice_rsrc(s2e + (in ? g * 64 : 0), in ? 256u : 0u);
#pragma unroll
      for (int c = 0; c < 4; ++c) S[c] = bload(rs, (uint32_t)(kq * 64 + c * 16));
    }
  };
  u32x4 WA[NI], WB[NI], SA[4], SB[4];
  load_group(0, WA, SA);

  // ---- phase 1 epilogue: scaled g|u tiles to LDS (x and the K-step buffers are free after the barrier)
  __syncthreads();
  float* gu = reinterpret_cast<float*>(big);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int col = 16 * (tile0 + n) + r16;   // w13 row: gate for col < I, up above
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 4 * kq + q;
      gu[row * GS + col] = kBlock ? acc[n][q] : acc[n][q] * sxs[row] * sc13[n];
    }
  }
  __syncthreads();

  // ---- phase 2: a = silu(g) * u, FP8 with absmax scales
  {
    const int r = tid >> 5, part = tid & 31;
    const bool valid = srow_s[r] < sentinel;
    float av[C];
    float amax = 0.f;
#pragma unroll
    for (int m = 0; m < C; ++m) {
      const int c = part * C + m;
      const float g = gu[r * GS + c], u = gu[r * GS + I + c];
      av[m] = valid ? silu(g) * u : 0.f;
      amax = fmaxf(amax, fabsf(av[m]));
    }
    // the float32 product also goes to the workspace (sorted-row order), where the split path
    // keeps it, unless a_out is null (the whole-layer call, which never reads it back)
    if (a_out) {
      float* arow = a_out + (size_t)(bb * 16 + r) * I + part * C;
#pragma unroll
      for (int m = 0; m < C; m += 2) *reinterpret_cast<float2*>(arow + m) = make_float2(av[m], av[m + 1]);
    }
    const float wgt = wgt_s[r];
    // per channel: the row's 32 threads; block: the 128 / C threads of a 128-column group
    const float scale = fp8_scale(group_max(amax, kBlock ? kGroup / C : 32));
    const ScaleDiv q = scale_div(scale);
#pragma unroll
    for (int m = 0; m < C; m += 2)   // C = I / 32 is even
      *reinterpret_cast<uint16_t*>(&aqs[r * AS + part * C + m]) = (uint16_t)quant2(q, av[m], av[m + 1]);
    if (!kBlock) {
      if (part == 0) rsc_s[r] = wgt * scale;
    } else {
      if (part == 0) rsc_s[r] = wgt;
      if ((part * C) % kGroup == 0) sa_s[r][(part * C) / kGroup] = scale;
    }
  }
  __syncthreads();

  // ---- phase 3: down
  uint8_t* stg3 = big + wv * 64 * AS;
  uint8_t* ost = big + Lds::kStage3 + wv * 8 * kOutRS;
  uint32_t kc[2];
  v8i avq[2];
  float sr[2] = {0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int koff = u * kGroup + kq * 32;
    const bool in = koff < I;
    kc[u] = in ? koff : I - 32;
    const v8i t = load32(aqs + r16 * AS + kc[u]);
    const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    avq[u] = in ? t : zero8;
    if (kBlock && u * kGroup < I) sr[u] = sa_s[r16][u];
  }
  const float rsc = rsc_s[r16];
  // lane's LDS slot for each 16-byte piece of a group: column c = o / I of the 64 goes to
  // row 16 ((c / 4) % 4) + 4 (c / 16) + c % 4 so that MFMA tile n reads rows 16 n .. 16 n + 15
  int soff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int o = i * 1024 + lane * 16;
    const int c = o / I, byte = o - c * I;
    soff[i] = (16 * ((c >> 2) & 3) + 4 * (c >> 4) + (c & 3)) * AS + byte;
  }
  auto down_group = [&](u32x4 (&W)[NI], u32x4 (&S)[4], int i) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NI; ++j) *reinterpret_cast<u32x4*>(stg3 + soff[j]) = W[j];
    v4f d[4] = {zero4, zero4, zero4, zero4};
#pragma unroll
    for (int u = 0; u < (I > kGroup ? 2 : 1); ++u) {
      v8i bw[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) bw[n] = load32(stg3 + (16 * n + r16) * AS + kc[u]);
      if (!kBlock) {
#pragma unroll
        for (int n = 0; n < 4; ++n) d[n] = mfma_16x16x128_fp8(bw[n], avq[u], d[n]);
      } else {
        // a group's 64 columns lie in one 128-column block of w2's scales
        const int g = min(group_of(i), ng - 1);
        const float swb = s2[((size_t)e * (H / kGroup) + (g * 64) / kGroup) * (I / kGroup) + u];
        const float f = sr[u] * swb;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const v4f t = mfma_16x16x128_fp8(bw[n], avq[u], zero4);
#pragma unroll
          for (int q = 0; q < 4; ++q) d[n][q] += t[q] * f;
        }
      }
    }
    // the MFMAs read operands across the whole wavefront: keep them ahead of the exits below
#pragma unroll
    for (int n = 0; n < 4; ++n) asm volatile("" : "+v"(d[n]));
    const int h0 = group_of(i) * 64;
    if (h0 >= H) return;   // uniform: past the wavefront's groups
    float sw[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sw[4 * c] = kBlock ? 1.f : __uint_as_float(S[c].x);
      sw[4 * c + 1] = kBlock ? 1.f : __uint_as_float(S[c].y);
      sw[4 * c + 2] = kBlock ? 1.f : __uint_as_float(S[c].z);
      sw[4 * c + 3] = kBlock ? 1.f : __uint_as_float(S[c].w);
    }
    uint32_t packed[8];
#pragma unroll
    for (int c = 0; c < 16; c += 2) {   // column c = 4 n + q of the lane's 16
      const float y0 = d[c >> 2][c & 3] * sw[c] * rsc;
      const float y1 = d[(c + 1) >> 2][(c + 1) & 3] * sw[c + 1] * rsc;
      packed[c >> 1] = pack_bf16x2(y0, y1);
    }
    // through the wavefront's 8 LDS rows, 8 output rows at a time, so that each store
    // writes 8 rows x 128 whole bytes (a wavefront's LDS operations complete in order);
    // padding rows are not stored
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      if ((r16 >> 3) == ps) {
        uint4* sp = reinterpret_cast<uint4*>(ost + (r16 & 7) * kOutRS + kq * 32);
        sp[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        sp[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      }
      const int sr = srow_s[8 * ps + (lane >> 3)];
      const uint4 v = *reinterpret_cast<const uint4*>(ost + (lane >> 3) * kOutRS + (lane & 7) * 16);
      if (sr < sentinel) *reinterpret_cast<uint4*>(slot_out + (size_t)sr * H + h0 + (lane & 7) * 8) = v;
    }
  };
#pragma unroll 1
  for (int i = 0; i < n_my; i += 2) {
    load_group(i + 1, WB, SB);
    __builtin_amdgcn_sched_barrier(0);
    down_group(WA, SA, i);
    load_group(i + 2, WA, SA);
    __builtin_amdgcn_sched_barrier(0);
    down_group(WB, SB, i + 1);
  }
}

bool expert_ffn_decode_supported(int H, int I) {
  return I % 64 == 0 && I >= 64 && I <= 256 && H % kGroup == 0 && H <= kXMaxH;
}
bool expert_ffn_decode_align_supported(int T, int K1) { return (size_t)T * K1 <= kAlignMaxN; }

// align == nullptr: sorted / block_expert are inputs (from the align call). Otherwise
// the kernel derives them from align->topk_ids and writes them with the other align
// outputs (T*K1 <= kAlignMaxN).
hipError_t launch_expert_ffn_decode(const uint8_t* xq, const float* sx, const uint8_t* w13,
                                    const float* s13, const uint8_t* w2, const float* s2, bool block,
                                    int32_t* sorted, int32_t* block_expert, const int32_t* num_padded,
                                    const AlignOut* align, const float* topk_w, float* a_out,
                                    uint16_t* slot_out, int T, int H, int I, int E1, int K1,
                                    hipStream_t stream) {
  const int P_max = (int)sorted_capacity(T, K1, E1, 16);
  const dim3 grid(P_max / 16), blk(512);
  const AlignOut al = align ? *align : AlignOut{nullptr, nullptr, nullptr, const_cast<int32_t*>(num_padded), E1};
#define SRMOE_EFD(B, N, A)                                                                          \
  hipLaunchKernelGGL((expert_ffn_decode_kernel<B, N, A>), grid, blk, 0, stream, xq, sx, w13, s13, w2, \
                     s2, sorted, block_expert, al, topk_w, a_out, slot_out, T, H, K1)
#define SRMOE_EFD2(N)                              \
  if (block) {                                     \
    if (align) SRMOE_EFD(true, N, true);           \
    else SRMOE_EFD(true, N, false);                \
  } else {                                         \
    if (align) SRMOE_EFD(false, N, true);          \
    else SRMOE_EFD(false, N, false);               \
  }                                                \
  break;
  switch (I / 64) {
    case 1: SRMOE_EFD2(1)
    case 2: SRMOE_EFD2(2)
    case 3: SRMOE_EFD2(3)
    default: SRMOE_EFD2(4)
  }
#undef SRMOE_EFD2
#undef SRMOE_EFD
  return hipGetLastError();
}

}  // namespace srmoe
