// Prefill-shaped expert GEMMs (block_m == 128) with LDS-staged tiles.
//
// With hundreds of rows per expert every weight fragment can feed many MFMAs,
// so the workgroup stages both operands through LDS: per 128-byte K step it
// loads the block's 128 gathered x_q rows (A) and 128 weight rows (64 gate rows
// and the matching 64 up rows of w13[e]) into a double-buffered LDS tile, and
// its 2x2 wavefronts each compute a 64-row x (32 gate + 32 up) sub-tile as
// 4 x 4 MFMAs of 16x16x128. The global loads of step k+1 are in flight while
// step k computes. LDS rows are padded from 128 to 144 bytes so that the 16
// rows a fragment read touches land on distinct banks.
//
// gate_up: grid (P_max / 128, ceil(I / 64)); epilogue as in the other gate_up
// kernels: a = silu(g) * u in float32 per sorted row (0 for padding rows). In block
// mode every K step's products are rescaled by (x scale x weight block scale) before
// they are accumulated; there the weights are the MFMA's A operand, so that a lane's 4
// results share one token and one weight block and the rescale takes one product per
// tile (per channel, the x rows are A and the scales are applied once, in the epilogue).
// down: grid (P_max / 128, H / 128); the same double-buffered K loop over
// K = I (a partial last step is zero-filled in LDS) with the weights as the
// MFMA A operand, so D holds [column][token]; inside a wavefront's 64 columns
// tile n row r holds column (r / 4) * 16 + 4 * n + r % 4, which leaves each
// lane with 16 consecutive output columns of one token to store as two
// 16-byte bf16 writes (slot_out = bf16(row_scale * s2 * y)).
#include "common.hpp"

namespace srmoe {

namespace {
constexpr int kTBM = 128;             // rows per block
constexpr int kTBN = 128;             // weight rows per workgroup: 64 gate + 64 up
constexpr int kTLD = kGroup + 16;     // padded LDS row stride (bytes)
constexpr int kTile = (kTBM + kTBN) * kTLD;

}  // namespace

template <bool kBlock>
__global__ void __launch_bounds__(256, 2) gate_up_tile_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ sx, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    const int32_t* __restrict__ expert_offsets, float* __restrict__ a_out, int T, int H, int I, int K1) {
  __shared__ __align__(16) uint8_t lds[2][kTile];
  // tiles (row block, 64-column group) walked per XCD: grouped by expert when the offsets
  // are given (grouped_tile), else in row-block-major order
  const int ny = (I + 63) / 64;
  const int tile = xcd_tile(blockIdx.x, num_padded[0] / kTBM * ny);
  if (tile < 0) return;
  int b = tile / ny, cy = tile - b * ny;
  if (expert_offsets) grouped_tile(tile, ny, kTBM, block_expert, expert_offsets, &b, &cy);
  const int e = block_expert[b];
  if (e < 0) return;
  const int c0 = cy * 64;  // first intermediate column of this workgroup
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int wm = wv >> 1, wn = wv & 1;
  const int sentinel = T * K1;
  const int HB = H / kGroup;

  // Global -> LDS assignment: 2048 16-byte chunks per K step (rows 0..127 A,
  // 128..255 B; 8 chunks per 128-byte row). Thread tid moves chunk part tid & 7 of
  // A rows tid/8 + 32 i and of B rows tid/8 + 32 i (i = 0..3). Padding rows read
  // token 0 and weight columns past I read row 0 (both discarded in the
  // epilogue), so no load is predicated.
  const int part = tid & 7, r0 = tid >> 3;
  // the sorted slot ids the staging needs, loaded together before any is used
  int sA[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sA[i] = sorted[b * kTBM + r0 + 32 * i];
  const int sS = kBlock ? sorted[b * kTBM + (tid & (kTBM - 1))] : 0;
  const uint64_t kmagic = slot_div_magic(K1);
  uint32_t aoff[4], boff[4];   // byte offsets of the rows (T*H and 2*I*H are < 2^31)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = slot_token(sA[i], kmagic);
    aoff[i] = (uint32_t)(sA[i] < sentinel ? t : 0) * (uint32_t)H;
    const int r = r0 + 32 * i;                      // 0..63 gate, 64..127 up
    const int col = c0 + (r & 63);
    boff[i] = (uint32_t)(col < I ? (r < 64 ? col : I + col) : 0) * (uint32_t)H;
  }
  const uint8_t* abase = xq + part * 16;
  const uint8_t* bbase = w13 + (size_t)e * 2 * I * H + part * 16;
  // Block mode: each K step's scales travel with its tiles through LDS (a global
  // load waited on inside the step would also wait for the prefetch). Entries
  // 0..127: x scale of block row i (0 for padding rows); 128 + 4 * wn + n: the
  // weight block scale of B tile n of column half wn. Thread tid fetches entry tid.
  __shared__ __align__(16) float scl[2][kBlock ? kTBM + 8 : 4];
  const float* sptr = sx;
  bool sval = false;
  if (kBlock) {
    if (tid < kTBM) {
      sval = sS < sentinel;
      sptr = sx + (size_t)(sval ? slot_token(sS, kmagic) : 0) * HB;
    } else if (tid < kTBM + 8) {
      const int c = tid - kTBM, n = c & 3;
      const int col = c0 + 32 * (c >> 2) + 16 * (n & 1);   // 16-column tiles never straddle a 128 block
      const int nb = (n >= 2 ? I + min(col, I - 16) : min(col, I - 16)) / kGroup;
      sptr = s13 + ((size_t)e * (2 * I / kGroup) + nb) * HB;
      sval = true;
    }
  }
  // Two register sets of staged chunks: while step k computes from LDS, set
  // (k + 1) & 1 holds step k + 1's chunks (loaded a step earlier) and set k & 1
  // receives step k + 2's, so every load has two steps to arrive.
  uint4 g0_0, g0_1, g0_2, g0_3, g0_4, g0_5, g0_6, g0_7;
  uint4 g1_0, g1_1, g1_2, g1_3, g1_4, g1_5, g1_6, g1_7;
  float sc0 = 0.f, sc1 = 0.f;
#define SRMOE_TILE_GLOAD(S, k)                                                \
  if (kBlock) sc##S = sptr[(k) / kGroup];                                     \
  g##S##_0 = *reinterpret_cast<const uint4*>(abase + aoff[0] + (k));          \
  g##S##_1 = *reinterpret_cast<const uint4*>(abase + aoff[1] + (k));          \
  g##S##_2 = *reinterpret_cast<const uint4*>(abase + aoff[2] + (k));          \
  g##S##_3 = *reinterpret_cast<const uint4*>(abase + aoff[3] + (k));          \
  g##S##_4 = *reinterpret_cast<const uint4*>(bbase + boff[0] + (k));          \
  g##S##_5 = *reinterpret_cast<const uint4*>(bbase + boff[1] + (k));          \
  g##S##_6 = *reinterpret_cast<const uint4*>(bbase + boff[2] + (k));          \
  g##S##_7 = *reinterpret_cast<const uint4*>(bbase + boff[3] + (k));
#define SRMOE_TILE_LSTORE(S, buf)                                                              \
  *reinterpret_cast<uint4*>(&lds[buf][(r0 + 0) * kTLD + part * 16]) = g##S##_0;               \
  *reinterpret_cast<uint4*>(&lds[buf][(r0 + 32) * kTLD + part * 16]) = g##S##_1;              \
  *reinterpret_cast<uint4*>(&lds[buf][(r0 + 64) * kTLD + part * 16]) = g##S##_2;              \
  *reinterpret_cast<uint4*>(&lds[buf][(r0 + 96) * kTLD + part * 16]) = g##S##_3;              \
  *reinterpret_cast<uint4*>(&lds[buf][(kTBM + r0 + 0) * kTLD + part * 16]) = g##S##_4;        \
  *reinterpret_cast<uint4*>(&lds[buf][(kTBM + r0 + 32) * kTLD + part * 16]) = g##S##_5;       \
  *reinterpret_cast<uint4*>(&lds[buf][(kTBM + r0 + 64) * kTLD + part * 16]) = g##S##_6;       \
  *reinterpret_cast<uint4*>(&lds[buf][(kTBM + r0 + 96) * kTLD + part * 16]) = g##S##_7;       \
  if (kBlock && tid < kTBM + 8) scl[buf][tid] = sval ? sc##S : 0.f;

  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = zero4;

  // LDS rows of this wavefront's fragments: A rows 64*wm + 16*m + r16; B rows
  // (gate tiles n = 0,1, up tiles n = 2,3) 128 + {32*wn, 32*wn+16, 64+32*wn, 64+32*wn+16} + r16.
  const int arow0 = (64 * wm + r16) * kTLD + kq * 32;
  int brow[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
    brow[n] = (kTBM + (n >= 2 ? 64 : 0) + 32 * wn + 16 * (n & 1) + r16) * kTLD + kq * 32;

#define SRMOE_TILE_COMPUTE(buf)                                                                \
  {                                                                                            \
    v8i af[4], bf[4];                                                                          \
    _Pragma("unroll") for (int m = 0; m < 4; ++m) af[m] = load32(&lds[buf][arow0 + 16 * m * kTLD]); \
    _Pragma("unroll") for (int n = 0; n < 4; ++n) bf[n] = load32(&lds[buf][brow[n]]);          \
    if (!kBlock) {                                                                             \
      _Pragma("unroll") for (int m = 0; m < 4; ++m)                                            \
      _Pragma("unroll") for (int n = 0; n < 4; ++n)                                            \
        acc[m][n] = mfma_16x16x128_fp8(af[m], bf[n], acc[m][n]);                               \
    } else {                                                                                   \
      /* weights as the A operand: the lane's 4 results are 4 weight rows of one token, so the \
         step's rescale is one product of the token's and the tile's scale per tile */         \
      const float4 sw = *reinterpret_cast<const float4*>(&scl[buf][kTBM + 4 * wn]);            \
      const float swn[4] = {sw.x, sw.y, sw.z, sw.w};                                           \
      _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                          \
        const float sxm = scl[buf][64 * wm + 16 * m + r16];                                    \
        _Pragma("unroll") for (int n = 0; n < 4; ++n) {                                        \
          const v4f t = mfma_16x16x128_fp8(bf[n], af[m], zero4);                               \
          const float sc = sxm * swn[n];                                                       \
          _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[m][n][j] += t[j] * sc;             \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
  }
  // one K step: prefetch step ks + 2 into set SL, compute step ks, stage step
  // ks + 1 from set SS into the other LDS buffer (past the end the last step is
  // re-read rather than branched around; it is never stored)
#define SRMOE_TILE_STEP(ks, SL, SS)                                           \
  {                                                                           \
    const int buf = (ks) & 1;                                                 \
    SRMOE_TILE_GLOAD(SL, min((ks) + 2, nk - 1) * kGroup)                      \
    SRMOE_TILE_COMPUTE(buf)                                                   \
    if ((ks) + 1 < nk) {                                                      \
      SRMOE_TILE_LSTORE(SS, buf ^ 1)                                          \
    }                                                                         \
    __syncthreads();                                                          \
  }

  const int nk = H / kGroup;
  SRMOE_TILE_GLOAD(0, 0)
  SRMOE_TILE_GLOAD(1, min(1, nk - 1) * kGroup)
  SRMOE_TILE_LSTORE(0, 0)
  __syncthreads();
  for (int ks = 0; ks < nk; ks += 2) {
    SRMOE_TILE_STEP(ks, 0, 1)
    if (ks + 1 < nk) SRMOE_TILE_STEP(ks + 1, 1, 0)
  }
#undef SRMOE_TILE_STEP
#undef SRMOE_TILE_COMPUTE
#undef SRMOE_TILE_GLOAD
#undef SRMOE_TILE_LSTORE

  // epilogue: gate tile n pairs with up tile n + 2 (same intermediate columns).
  if (kBlock) {
    // block mode (weights were the A operand): element j of tile (m, n) is intermediate
    // column c0 + 32 wn + 16 n + 4 kq + j of token row 64 wm + 16 m + r16, already scaled;
    // each lane stores 4 consecutive columns (I % 128 == 0: every column exists)
    bool valid[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) valid[m] = sorted[b * kTBM + 64 * wm + 16 * m + r16] < sentinel;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int col = c0 + 32 * wn + 16 * n + 4 * kq;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int p = b * kTBM + 64 * wm + 16 * m + r16;
        float4 av;
        av.x = valid[m] ? silu(acc[m][n][0]) * acc[m][n + 2][0] : 0.f;
        av.y = valid[m] ? silu(acc[m][n][1]) * acc[m][n + 2][1] : 0.f;
        av.z = valid[m] ? silu(acc[m][n][2]) * acc[m][n + 2][2] : 0.f;
        av.w = valid[m] ? silu(acc[m][n][3]) * acc[m][n + 2][3] : 0.f;
        *reinterpret_cast<float4*>(a_out + (size_t)p * I + col) = av;
      }
    }
    return;
  }
  // per channel: tokens of this lane's output rows (-1 for padding rows) are re-read here
  // rather than held through the K loop; all scales are fetched before any is used.
  int otok[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int4 sv = *reinterpret_cast<const int4*>(sorted + b * kTBM + 64 * wm + 16 * m + 4 * kq);
    const int sm[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) otok[m][j] = sm[j] < sentinel ? slot_token(sm[j], kmagic) : -1;
  }
  float sxo[4][4], sg[2], su[2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) sxo[m][j] = sx[max(otok[m][j], 0)];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int colc = min(c0 + 32 * wn + 16 * n + r16, I - 1);
    sg[n] = s13[(size_t)e * 2 * I + colc];
    su[n] = s13[(size_t)e * 2 * I + I + colc];
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int col = c0 + 32 * wn + 16 * n + r16;
    if (col >= I) continue;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = b * kTBM + 64 * wm + 16 * m + 4 * kq + j;
        const float g = acc[m][n][j] * (sxo[m][j] * sg[n]);
        const float u = acc[m][n + 2][j] * (sxo[m][j] * su[n]);
        a_out[(size_t)p * I + col] = otok[m][j] >= 0 ? silu(g) * u : 0.f;
      }
  }
}

template <bool kBlock>
__global__ void __launch_bounds__(256, 2) down_tile_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ sa, const uint8_t* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    const int32_t* __restrict__ expert_offsets, const float* __restrict__ row_scale,
    uint16_t* __restrict__ slot_out, int T, int H, int I, int K1) {
  __shared__ __align__(16) uint8_t lds[2][kTile];   // rows 0..127 weights (h), 128..255 a_q rows
  const int ny = H / 128;
  const int tile = xcd_tile(blockIdx.x, num_padded[0] / kTBM * ny);
  if (tile < 0) return;
  int b = tile / ny, cy = tile - b * ny;
  if (expert_offsets) grouped_tile(tile, ny, kTBM, block_expert, expert_offsets, &b, &cy);
  const int e = block_expert[b];
  if (e < 0) return;
  const int h0 = cy * 128;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int wh = wv >> 1, wt = wv & 1;   // 64-column half, 64-token half
  const int sentinel = T * K1;
  const int IB = I / kGroup;

  // Global -> LDS: thread tid moves chunk part tid & 7 (16 bytes of a 128-byte K step)
  // of weight rows h0 + tid/8 + 32 i and of a_q rows tid/8 + 32 i (i = 0..3).
  // Chunks past I are clamped to the row's last 16 bytes and replaced by zeros.
  const int part = tid & 7, r0 = tid >> 3;
  const uint8_t* wbase = w2 + ((size_t)e * H + h0 + r0) * I;
  const uint8_t* abase = aq + ((size_t)b * kTBM + r0) * I;
  const size_t rstep = (size_t)32 * I;
  const uint4 z4 = {0u, 0u, 0u, 0u};
  // Block mode: each K step's scales travel with its tiles through LDS: entries
  // 0..127 the a_q row scales, 128 the w2 block scale of this column block.
  __shared__ __align__(16) float scl[2][kBlock ? kTBM + 4 : 4];
  const float* sptr = kBlock ? (tid < kTBM ? sa + ((size_t)b * kTBM + tid) * IB
                                           : s2 + ((size_t)e * (H / kGroup) + h0 / kGroup) * IB)
                             : sa;
  // two register sets of staged chunks, as in gate_up_tile_kernel
  uint4 g0_0, g0_1, g0_2, g0_3, g0_4, g0_5, g0_6, g0_7;
  uint4 g1_0, g1_1, g1_2, g1_3, g1_4, g1_5, g1_6, g1_7;
  float sc0 = 0.f, sc1 = 0.f;
#define SRMOE_DTILE_GLOAD(S, k)                                                           \
  {                                                                                       \
    if (kBlock) sc##S = sptr[(k) / kGroup];                                               \
    const int ko = (k) + part * 16;                                                       \
    const bool in = ko < I;                                                               \
    const int kc = in ? ko : I - 16;                                                      \
    g##S##_0 = *reinterpret_cast<const uint4*>(wbase + kc);                               \
    g##S##_1 = *reinterpret_cast<const uint4*>(wbase + rstep + kc);                       \
    g##S##_2 = *reinterpret_cast<const uint4*>(wbase + 2 * rstep + kc);                   \
    g##S##_3 = *reinterpret_cast<const uint4*>(wbase + 3 * rstep + kc);                   \
    g##S##_4 = *reinterpret_cast<const uint4*>(abase + kc);                               \
    g##S##_5 = *reinterpret_cast<const uint4*>(abase + rstep + kc);                       \
    g##S##_6 = *reinterpret_cast<const uint4*>(abase + 2 * rstep + kc);                   \
    g##S##_7 = *reinterpret_cast<const uint4*>(abase + 3 * rstep + kc);                   \
    if (!in) {                                                                            \
      g##S##_0 = g##S##_1 = g##S##_2 = g##S##_3 = z4;                                     \
      g##S##_4 = g##S##_5 = g##S##_6 = g##S##_7 = z4;                                     \
    }                                                                                     \
  }
#define SRMOE_DTILE_LSTORE(S, buf)                                                             \
  *reinterpret_cast<uint4*>(&lds[buf][(r0 + 0) * kTLD + part * 16]) = g##S##_0;               \
  *reinterpret_cast<uint4*>(&lds[buf][(r0 + 32) * kTLD + part * 16]) = g##S##_1;              \
  *reinterpret_cast<uint4*>(&lds[buf][(r0 + 64) * kTLD + part * 16]) = g##S##_2;              \
  *reinterpret_cast<uint4*>(&lds[buf][(r0 + 96) * kTLD + part * 16]) = g##S##_3;              \
  *reinterpret_cast<uint4*>(&lds[buf][(kTBM + r0 + 0) * kTLD + part * 16]) = g##S##_4;        \
  *reinterpret_cast<uint4*>(&lds[buf][(kTBM + r0 + 32) * kTLD + part * 16]) = g##S##_5;       \
  *reinterpret_cast<uint4*>(&lds[buf][(kTBM + r0 + 64) * kTLD + part * 16]) = g##S##_6;       \
  *reinterpret_cast<uint4*>(&lds[buf][(kTBM + r0 + 96) * kTLD + part * 16]) = g##S##_7;       \
  if (kBlock && tid <= kTBM) scl[buf][tid] = sc##S;

  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f acc[4][4];   // [column tile n][token tile m]
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[n][m] = zero4;
  // fragment rows: weights (A) 64*wh + (r16/4)*16 + 4n + r16%4; tokens (B) 128 + 64*wt + 16m + r16
  const int wrow0 = (64 * wh + (r16 >> 2) * 16 + (r16 & 3)) * kTLD + kq * 32;
  const int trow0 = (kTBM + 64 * wt + r16) * kTLD + kq * 32;

#define SRMOE_DTILE_COMPUTE(buf)                                                               \
  {                                                                                            \
    v8i wf[4], tf[4];                                                                          \
    _Pragma("unroll") for (int n = 0; n < 4; ++n) wf[n] = load32(&lds[buf][wrow0 + 4 * n * kTLD]); \
    _Pragma("unroll") for (int m = 0; m < 4; ++m) tf[m] = load32(&lds[buf][trow0 + 16 * m * kTLD]); \
    if (!kBlock) {                                                                             \
      _Pragma("unroll") for (int n = 0; n < 4; ++n)                                            \
      _Pragma("unroll") for (int m = 0; m < 4; ++m)                                            \
        acc[n][m] = mfma_16x16x128_fp8(wf[n], tf[m], acc[n][m]);                               \
    } else {                                                                                   \
      /* the workgroup's 128 columns are one 128-column block of w2's scales */               \
      const float swb = scl[buf][kTBM];                                                        \
      _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                          \
        const float sr = scl[buf][64 * wt + 16 * m + r16] * swb;                               \
        _Pragma("unroll") for (int n = 0; n < 4; ++n) {                                        \
          const v4f t = mfma_16x16x128_fp8(wf[n], tf[m], zero4);                               \
          _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[n][m][j] += t[j] * sr;             \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
  }
#define SRMOE_DTILE_STEP(ks, SL, SS)                                          \
  {                                                                           \
    const int buf = (ks) & 1;                                                 \
    SRMOE_DTILE_GLOAD(SL, min((ks) + 2, nk - 1) * kGroup)                     \
    SRMOE_DTILE_COMPUTE(buf)                                                  \
    if ((ks) + 1 < nk) {                                                      \
      SRMOE_DTILE_LSTORE(SS, buf ^ 1)                                         \
    }                                                                         \
    __syncthreads();                                                          \
  }

  const int nk = (I + kGroup - 1) / kGroup;
  SRMOE_DTILE_GLOAD(0, 0)
  SRMOE_DTILE_GLOAD(1, min(1, nk - 1) * kGroup)
  SRMOE_DTILE_LSTORE(0, 0)
  __syncthreads();
  for (int ks = 0; ks < nk; ks += 2) {
    SRMOE_DTILE_STEP(ks, 0, 1)
    if (ks + 1 < nk) SRMOE_DTILE_STEP(ks + 1, 1, 0)
  }
#undef SRMOE_DTILE_STEP
#undef SRMOE_DTILE_COMPUTE
#undef SRMOE_DTILE_GLOAD
#undef SRMOE_DTILE_LSTORE

  // epilogue row data and this lane's 16 per-channel column scales
  int srow[4];
  float rsc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    srow[m] = sorted[b * kTBM + 64 * wt + 16 * m + r16];
    rsc[m] = row_scale[b * kTBM + 64 * wt + 16 * m + r16];
  }
  const int hl = h0 + 64 * wh + 16 * kq;   // this lane's first output column
  float swc[16];
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
    const float4 v = kBlock ? make_float4(1.f, 1.f, 1.f, 1.f)
                            : *reinterpret_cast<const float4*>(s2 + (size_t)e * H + hl + c);
    swc[c] = v.x; swc[c + 1] = v.y; swc[c + 2] = v.z; swc[c + 3] = v.w;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int s = srow[m];
    if (s >= sentinel) continue;
    uint32_t packed[8];
#pragma unroll
    for (int c = 0; c < 16; c += 2) {   // column c = 4 * n + j of this lane's 16
      const float y0 = acc[c >> 2][m][c & 3] * swc[c] * rsc[m];
      const float y1 = acc[(c + 1) >> 2][m][(c + 1) & 3] * swc[c + 1] * rsc[m];
      packed[c >> 1] = pack_bf16x2(y0, y1);
    }
    uint4* dst = reinterpret_cast<uint4*>(slot_out + (size_t)s * H + hl);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  }
}

// down for I <= 256 with 32x32x64 MFMAs: K = I in ceil(I / 64) steps of 64 bytes (three
// exact steps at I = 192; a partial last step is zero-filled). Workgroup = 2 row halves x
// 2 column streams; stream wc takes the 64-column tiles g * 2 NTL + wc + 2 j of w2[e]
// (j < NTL), in 128 * NTL columns per workgroup, tiles ordered row block major and walked
// per XCD.
//  - Each wavefront holds its 64 a_q rows as the MFMA B operand for the whole launch,
//    loaded once (lane l: row l % 32 of a 32-row tile, K bytes 32 (l / 32) of each step).
//  - A tile's 64 rows of w2[e] are 64 * I contiguous bytes: the stream's two wavefronts load
//    half each as 1 KB runs (16 bytes per lane: whole lines per instruction), a tile ahead,
//    and store them to the stream's LDS buffer (rows padded by 16 bytes); the weight
//    fragments (the A operand) are read from there. Weight row rho of a 32-row MFMA tile is
//    output column 16 ((rho / 4) % 2) + 4 (rho / 8) + rho % 4, so that lane l ends with the 16
//    consecutive columns 16 (l / 32) .. + 15 of token l % 32.
//  - The bf16 results go through a wavefront-private LDS buffer so that 8 lanes write each
//    row's 128 contiguous bytes with one non-temporal store: slot_out is written once and
//    read once by the combine, and whole-line streaming stores keep it from evicting the
//    w2 tiles that the block's neighbours re-read from L2.
constexpr int kDownTiles = 4;
constexpr int kDownTilesWide = 10;         // 1,280 columns per workgroup (down_wide_tiles_wide)
constexpr int kCombTiles = 1;              // 64-column tiles per wavefront in the combining launch
constexpr int kStageLD = 128 + 16;         // LDS row stride of an output staging buffer

typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// D(32x32,f32) += A(32x64,fp8 e4m3) * B(64x32,fp8 e4m3): lane l supplies row/column l % 32
// and the 32 K bytes at 32 (l / 32) of the 64-byte K step (A and B share the K mapping);
// element v of lane l is D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]. Format 0 = OCP E4M3 for
// both operands, E8M0 block scales fixed at 127 (= 1).
__device__ __forceinline__ v16f mfma_32x32x64_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// acc[c] += the c-th of the 8 bf16 values in v (low half of each word first)
__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[2 * j] += bf16_to_f32(w[j] & 0xFFFFu);
    acc[2 * j + 1] += bf16_to_f32(w[j] >> 16);
  }
}

// Where the rows' bf16 results go (kOut):
//  kRowsOut    the blocks of rows 0 .. rows[0] - 1; each row's result to its slot row of
//              slot_out, [T*K1 + 1, H] (moe_ffn_down's layout);
//  kBlockedOut the same rows, with slot_out in 128-column blocks: the piece of slot row
//              s at columns 128 cb .. 128 cb + 127 at element (cb * (T*K1 + 1) + s) * 128;
//  kCombineOut the comb_blocks blocks from row rows[0] on (the shared expert's segment,
//              one row per token in token order); each row's result is added to the
//              token's routed slot rows, left column-blocked in slot_out by a kBlockedOut
//              launch over the rows before, and the sum is stored to out.
// In the blocked layout the combining launch reads, per 128-token block and column block,
// one contiguous run of 128 * K1 pieces of 256 bytes (the row layout scatters them).
constexpr int kRowsOut = 0, kBlockedOut = 1, kCombineOut = 2;
template <bool kBlock, int KT, int NTL, int kOut>
__global__ void __launch_bounds__(256, 2) down_wide_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ sa, const uint8_t* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ expert_offsets, const float* __restrict__ row_scale,
    uint16_t* __restrict__ slot_out, int T, int H, int I, int K1, uint16_t* __restrict__ out, int comb_blocks) {
  constexpr int kSLD = 64 * KT + 16;   // LDS row stride of a staged weight tile (bytes)
  constexpr int kCols = 128 * NTL;     // columns per workgroup
  constexpr int KG = (KT + 1) / 2;     // 128-byte K groups (block-scale mode)
  constexpr int kRuns = 2 * KT;        // 1 KB runs per wavefront and tile at most (32 rows * I bytes)
  __shared__ __align__(16) uint8_t wst[2][64 * kSLD];
  __shared__ __align__(16) uint8_t ost[4][64 * kStageLD];
  __shared__ __align__(16) float scol[kBlock ? kCols / kGroup * KG : kCols];
  const int ng = (H + kCols - 1) / kCols;
  constexpr bool kComb = kOut == kCombineOut;
  const int tile = xcd_tile(blockIdx.x, (kComb ? comb_blocks : rows[0] / kTBM) * ng);
  if (tile < 0) return;
  // with the offsets: the routed rows grouped by expert (grouped_tile), the combining
  // launch's blocks (all the shared expert's) column group by column group
  int bt = tile / ng, g = tile - bt * ng;
  if (expert_offsets) {
    if (kComb) {
      g = tile / comb_blocks;
      bt = tile - g * comb_blocks;
    } else {
      grouped_tile(tile, ng, kTBM, block_expert, expert_offsets, &bt, &g);
    }
  }
  const int b = kComb ? rows[0] / kTBM + bt : bt;
  const int e = block_expert[b];
  if (e < 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wv & 1, wc = wv >> 1;   // row half, column stream
  const int l32 = lane & 31, h = lane >> 5;
  const int nct = H / 64;
  const int sentinel = T * K1;
  const uint64_t magic = slot_div_magic(K1);
  const size_t nrows = (size_t)sentinel + 1;   // slot rows, with the padding rows' spare
  const int c0 = g * kCols;   // first column of the workgroup

  // ---- the wavefront's a_q rows as B fragments, zero past I (K bytes ks * 64 + 32 h)
  v8i aqf[2][KT];
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const uint8_t* arow = aq + ((size_t)b * kTBM + 64 * wt + 32 * mt + l32) * I + 32 * h;
#pragma unroll
    for (int ks = 0; ks < KT; ++ks) aqf[mt][ks] = 64 * ks + 32 * h < I ? load32(arow + 64 * ks) : zero8;
  }
  // w2 scales of the workgroup's columns -> LDS (per channel: kCols floats; block mode:
  // per 128-column block and K group), clamped past H
  if (!kBlock) {
#pragma unroll
    for (int c = tid; c < kCols; c += 256) scol[c] = s2[(size_t)e * H + min(c0 + c, H - 1)];
  } else if (tid < kCols / kGroup * KG) {
    const int cb = min(c0 / kGroup + tid / KG, H / kGroup - 1);
    scol[tid] = s2[((size_t)e * (H / kGroup) + cb) * (I / kGroup) + tid % KG];
  }
  // this lane's rows: output scale (and block-mode activation scales) in the MFMA layout
  // (rows 64 wt + 32 mt + l32), slot ids in the store layout (rows 64 wt + 8 q + lane / 8)
  float rsc[2], sar[2][KG];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int p = b * kTBM + 64 * wt + 32 * mt + l32;
    rsc[mt] = row_scale[p];
#pragma unroll
    for (int gk = 0; gk < KG; ++gk) sar[mt][gk] = kBlock ? sa[(size_t)p * (I / kGroup) + gk] : 1.f;
  }
  int srow[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)   // padding rows go to the spare row after the T*K1 slot rows
    srow[q] = min(sorted[b * kTBM + 64 * wt + 8 * q + (lane >> 3)], sentinel);

  // ---- weight tiles: the wavefront's half (rows 32 wt .. 32 wt + 31 of the tile, 32 I bytes)
  // as 16-byte pieces at 1024 r + 16 lane; a tile past the last reads zeros
  const int t0 = g * 2 * NTL + wc;   // this stream's first 64-column tile
  const uint8_t* w2e = w2 + (size_t)e * H * I;
  const int nrun = I / 32;           // 1 KB runs in 32 I bytes
  u32x4_nt wr[kRuns];
  auto wload = [&](int tj) __attribute__((always_inline)) {
    const bool in = tj < nct;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w2e + (in ? (size_t)tj * 64 * I + (size_t)32 * wt * I : 0)), 0,
        in ? 32 * I : 0, 0x00020000);
#pragma unroll
    for (int q = 0; q < kRuns; ++q)
      if (q < nrun) wr[q] = __builtin_amdgcn_raw_buffer_load_b128(r, q * 1024 + lane * 16, 0, 2);
  };
  auto wstore = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kRuns; ++q)
      if (q < nrun) {
        const int o = 32 * wt * I + q * 1024 + lane * 16;   // byte of the tile's 64 * I
        const int r = o / I, k = o - r * I;
        *reinterpret_cast<u32x4_nt*>(&wst[wc][r * kSLD + k]) = wr[q];
      }
  };
  // A-fragment row of lane l in a 32-row MFMA tile: the tile's output column
  const int wcol = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);

  // combining launch (one 64-column tile per wavefront): the slot rows that the first two
  // rows add do not depend on the GEMM, so their loads go out now
  static_assert(!kComb || NTL == 1, "the combining launch takes one tile per wavefront");
  const int nr = K1 - 1;
  const int last = nr > 0 ? nr - 1 : 0;
  const int tc0 = t0 < nct ? t0 : 0;
  const int hs0 = tc0 * 64 + (lane & 7) * 8;
  const size_t cbase = (size_t)(hs0 >> 7) * nrows;   // the column block's first row
  const int hc = hs0 & 127;
  uint4 sv[2][2][8];
  auto slot_issue = [&](int q, uint4 (&v)[2][8]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int first = srow[q + u] < sentinel ? srow[q + u] - nr : 0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[u][k] = *reinterpret_cast<const uint4*>(slot_out + (cbase + first + min(k, last)) * 128 + hc);
    }
  };

  wload(t0);
  if (kComb) slot_issue(0, sv[0]);
  const v16f zero16 = {};
  uint8_t* stg = ost[wv];
#pragma unroll 1
  for (int j = 0; j < NTL; ++j) {
    const int tj = t0 + 2 * j;
    __syncthreads();   // the stream's buffer is free (the previous tile's fragments are read)
    wstore();
    if (j + 1 < NTL) wload(tj + 2);
    __syncthreads();   // the tile is in LDS (and the scales, at j == 0)
    // (H % 128 == 0 makes the tile count even, so both streams run out of tiles at the same j:
    // the break is uniform over the workgroup and no barrier is left waiting)
    if (tj >= nct) break;
    v16f acc[2][2];   // [column tile ct][row tile mt]
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[ct][mt] = zero16;
    const uint8_t* wrow0 = &wst[wc][wcol * kSLD + 32 * h];
    if (!kBlock) {
#pragma unroll
      for (int ks = 0; ks < KT; ++ks) {
        const bool kin = 64 * ks + 32 * h < I;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const v8i wf = kin ? load32(wrow0 + 32 * ct * kSLD + 64 * ks) : zero8;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) acc[ct][mt] = mfma_32x32x64_fp8(wf, aqf[mt][ks], acc[ct][mt]);
        }
      }
    } else {
      // a 64-column tile lies in one 128-column block of w2's scales; one factor per
      // lane, row tile and 128-byte K group
#pragma unroll
      for (int gk = 0; gk < KG; ++gk) {
        v16f t[2][2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) t[ct][mt] = zero16;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ks = 2 * gk + kk;
          if (ks >= KT) break;
          const bool kin = 64 * ks + 32 * h < I;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const v8i wf = kin ? load32(wrow0 + 32 * ct * kSLD + 64 * ks) : zero8;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) t[ct][mt] = mfma_32x32x64_fp8(wf, aqf[mt][ks], t[ct][mt]);
          }
        }
        const float sb = scol[((tj * 64 - c0) / kGroup) * KG + gk];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const float f = sar[mt][gk] * sb;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ct][mt][v] += t[ct][mt][v] * f;
        }
      }
    }
    // scale, round and stage: lane (l32, h) holds columns 32 ct + 16 h .. + 15 of row
    // 32 mt + l32 of the wavefront's 64
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float swc[16];
#pragma unroll
      for (int c = 0; c < 16; c += 4) {
        const float4 v = kBlock ? make_float4(1.f, 1.f, 1.f, 1.f)
                                : *reinterpret_cast<const float4*>(&scol[tj * 64 - c0 + 32 * ct + 16 * h + c]);
        swc[c] = v.x; swc[c + 1] = v.y; swc[c + 2] = v.z; swc[c + 3] = v.w;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        uint32_t packed[8];
#pragma unroll
        for (int c = 0; c < 16; c += 2)
          packed[c >> 1] = pack_bf16x2(acc[ct][mt][c] * swc[c] * rsc[mt], acc[ct][mt][c + 1] * swc[c + 1] * rsc[mt]);
        uint4* sp = reinterpret_cast<uint4*>(stg + (32 * mt + l32) * kStageLD + (32 * ct + 16 * h) * 2);
        sp[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        sp[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      }
    }
    // store: 8 lanes per row, 8 rows per instruction, each row's 128 bytes whole
    // (a wavefront's LDS operations complete in order, so no barrier is needed)
    const int hs = tj * 64 + (lane & 7) * 8;
    if (!kComb) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(stg + (8 * q + (lane >> 3)) * kStageLD + (lane & 7) * 16);
        const u32x4_nt nv = {v.x, v.y, v.z, v.w};
        const size_t o = kOut == kRowsOut ? (size_t)srow[q] * H + hs
                                          : ((size_t)(hs >> 7) * nrows + srow[q]) * 128 + (hs & 127);
        __builtin_nontemporal_store(nv, reinterpret_cast<u32x4_nt*>(slot_out + o));
      }
    } else {
      // the combine's sum for the row's token t: float32 from 0, routed slot rows t*K1 ..
      // t*K1 + K1 - 2 in order, then this row's bf16 value (slot K1 - 1). Two rows at a
      // time with the next two rows' slot loads in flight; slots 0..7 are always loaded
      // (a row past the token's last is masked to +0.0, which leaves a sum that started
      // at +0.0 unchanged), slots 8.. one at a time. Padding rows read token 0's rows and
      // store nothing.
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        if (q + 2 < 8) slot_issue(q + 2, sv[((q >> 1) + 1) & 1]);
        uint4 (&v)[2][8] = sv[(q >> 1) & 1];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int srw = srow[q + u];
          float acs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t m = k < nr ? 0xFFFFFFFFu : 0u;
            add_bf16x8(acs, make_uint4(v[u][k].x & m, v[u][k].y & m, v[u][k].z & m, v[u][k].w & m));
          }
          const int first = srw < sentinel ? srw - nr : 0;
          for (int k = 8; k < nr; ++k)
            add_bf16x8(acs, *reinterpret_cast<const uint4*>(slot_out + (cbase + first + k) * 128 + hc));
          add_bf16x8(acs, *reinterpret_cast<const uint4*>(stg + (8 * (q + u) + (lane >> 3)) * kStageLD + (lane & 7) * 16));
          if (srw < sentinel) {
            const u32x4_nt nv = {pack_bf16x2(acs[0], acs[1]), pack_bf16x2(acs[2], acs[3]),
                                 pack_bf16x2(acs[4], acs[5]), pack_bf16x2(acs[6], acs[7])};
            __builtin_nontemporal_store(nv, reinterpret_cast<u32x4_nt*>(out + (size_t)slot_token(srw, magic) * H + hs));
          }
        }
      }
    }
  }
}

// Column tiles per down_wide workgroup. 128 rows x 512 columns while the routed rows give
// few row blocks; 1,280 columns once that width still leaves four full rounds of resident
// workgroups (2 per CU). The wider workgroup spreads its prologue (a_q fragments, scales,
// slot ids) over 2.5x the columns; the narrower one keeps the last round short. Measured at
// H = 5120, I = 192: 4,096 tokens 120 us (4) against 127 us (10); 16k tokens 406 us
// against 364 us.
static bool down_wide_tiles_wide(int T, int H, int K1) {
  const size_t blocks = (size_t)T * K1 / kTBM;
  return blocks * ((H + 128 * kDownTilesWide - 1) / (128 * kDownTilesWide)) >= 2048;
}

hipError_t launch_down_tile(const uint8_t* aq, const float* sa, const uint8_t* w2, const float* s2,
                            bool block, const int32_t* sorted, const int32_t* block_expert,
                            const int32_t* num_padded, const int32_t* expert_offsets, const float* row_scale,
                            uint16_t* slot_out, int T, int H, int I, int E1, int K1, hipStream_t stream) {
  const int nb = (int)(sorted_capacity(T, K1, E1, kTBM) / kTBM);
  const dim3 blk(256);
  if (I <= 2 * kGroup) {
    const bool wide = down_wide_tiles_wide(T, H, K1);
    const int ntl = wide ? kDownTilesWide : kDownTiles;
    const dim3 grid(nb * ((H + 128 * ntl - 1) / (128 * ntl)));
#define SRMOE_DOWN_WIDE(B, KT, NTL)                                                                   \
  hipLaunchKernelGGL((down_wide_kernel<B, KT, NTL, kRowsOut>), grid, blk, 0, stream, aq, sa, w2, s2, \
                     sorted, block_expert, num_padded, expert_offsets, row_scale, slot_out, T, H, I, K1, nullptr, 0)
#define SRMOE_DOWN_WIDE2(KT)                                   \
  if (wide) {                                                  \
    if (block) SRMOE_DOWN_WIDE(true, KT, kDownTilesWide);      \
    else SRMOE_DOWN_WIDE(false, KT, kDownTilesWide);           \
  } else {                                                     \
    if (block) SRMOE_DOWN_WIDE(true, KT, kDownTiles);          \
    else SRMOE_DOWN_WIDE(false, KT, kDownTiles);               \
  }
    switch ((I + 63) / 64) {
      case 1: SRMOE_DOWN_WIDE2(1) break;
      case 2: SRMOE_DOWN_WIDE2(2) break;
      case 3: SRMOE_DOWN_WIDE2(3) break;
      default: SRMOE_DOWN_WIDE2(4) break;
    }
#undef SRMOE_DOWN_WIDE2
#undef SRMOE_DOWN_WIDE
    return hipGetLastError();
  }
  const dim3 grid(nb * (H / 128));
  if (block)
    hipLaunchKernelGGL(down_tile_kernel<true>, grid, blk, 0, stream, aq, sa, w2, s2, sorted,
                       block_expert, num_padded, expert_offsets, row_scale, slot_out, T, H, I, K1);
  else
    hipLaunchKernelGGL(down_tile_kernel<false>, grid, blk, 0, stream, aq, sa, w2, s2, sorted,
                       block_expert, num_padded, expert_offsets, row_scale, slot_out, T, H, I, K1);
  return hipGetLastError();
}

bool down_wide_supported(int I) { return I <= 2 * kGroup; }

// The down GEMM and the combine of the layer in two launches: the routed experts' rows
// (those before the shared expert's segment, which starts at row *shared_first) to
// slot_out in the column-blocked layout, then the shared expert's ceil(T / 128) blocks,
// whose rows add the token's routed slot rows and store out. The shared expert's slot
// rows are never written.
hipError_t launch_down_wide_combine(const uint8_t* aq, const float* sa, const uint8_t* w2, const float* s2,
                                    bool block, const int32_t* sorted, const int32_t* block_expert,
                                    const int32_t* expert_offsets, const float* row_scale,
                                    uint16_t* slot_out, uint16_t* out, int T, int H, int I, int E1, int K1,
                                    int parts, hipStream_t stream) {
  const int32_t* shared_first = expert_offsets + (E1 - 1);   // the shared expert's first row
  // parts: bit 0 the routed experts' launch, bit 1 the shared expert's launch with the combine
  if (!down_wide_supported(I)) return hipErrorInvalidValue;
  const int nb = (int)(sorted_capacity(T, K1, E1, kTBM) / kTBM);
  const int nbs = (T + kTBM - 1) / kTBM;
  const dim3 blk(256);
  const bool wide = down_wide_tiles_wide(T, H, K1);
  const int ntl = wide ? kDownTilesWide : kDownTiles;
  const dim3 grid(nb * ((H + 128 * ntl - 1) / (128 * ntl)));
  const dim3 grid_c(nbs * ((H + 128 * kCombTiles - 1) / (128 * kCombTiles)));
#define SRMOE_DOWN_COMB(B, KT)                                                                          \
  do {                                                                                                  \
    if ((parts & 1) && wide)                                                                            \
      hipLaunchKernelGGL((down_wide_kernel<B, KT, kDownTilesWide, kBlockedOut>), grid, blk, 0, stream, aq, \
                         sa, w2, s2, sorted, block_expert, shared_first, expert_offsets, row_scale, slot_out, \
                         T, H, I, K1, nullptr, 0);                                                      \
    else if (parts & 1)                                                                                 \
      hipLaunchKernelGGL((down_wide_kernel<B, KT, kDownTiles, kBlockedOut>), grid, blk, 0, stream, aq, sa, \
                         w2, s2, sorted, block_expert, shared_first, expert_offsets, row_scale, slot_out, T, \
                         H, I, K1, nullptr, 0);                                                         \
    if (parts & 2)                                                                                      \
      hipLaunchKernelGGL((down_wide_kernel<B, KT, kCombTiles, kCombineOut>), grid_c, blk, 0, stream, aq, sa, \
                         w2, s2, sorted, block_expert, shared_first, expert_offsets, row_scale, slot_out, T, \
                         H, I, K1, out, nbs);                                                           \
  } while (0)
#define SRMOE_DOWN_COMB2(KT) \
  if (block) SRMOE_DOWN_COMB(true, KT); else SRMOE_DOWN_COMB(false, KT);
  switch ((I + 63) / 64) {
    case 1: SRMOE_DOWN_COMB2(1) break;
    case 2: SRMOE_DOWN_COMB2(2) break;
    case 3: SRMOE_DOWN_COMB2(3) break;
    default: SRMOE_DOWN_COMB2(4) break;
  }
#undef SRMOE_DOWN_COMB2
#undef SRMOE_DOWN_COMB
  return hipGetLastError();
}

hipError_t launch_gate_up_tile(const uint8_t* xq, const float* sx, const uint8_t* w13,
                               const float* s13, bool block, const int32_t* sorted,
                               const int32_t* block_expert, const int32_t* num_padded,
                               const int32_t* expert_offsets, float* a, int T, int H, int I, int E1, int K1,
                               hipStream_t stream) {
  const int nb = (int)(sorted_capacity(T, K1, E1, kTBM) / kTBM);
  const dim3 grid(nb * ((I + 63) / 64));
  // Tile order. When an expert's gate/up weights exceed half an XCD's L2 (2 MB), its tiles
  // go column tile by column tile (grouped_tile), so that its row blocks read each weight
  // slice while it is in L2. Otherwise row block by row block: a block's x rows stay in L2
  // for its column tiles while the expert's whole weights stay there too. Measured at
  // H = 5120, I = 192: 150 -> 145 us at 4,096 tokens, 405 -> 390 us at 16k.
  if ((size_t)2 * I * H <= ((size_t)2 << 20)) expert_offsets = nullptr;
  if (block)
    hipLaunchKernelGGL(gate_up_tile_kernel<true>, grid, dim3(256), 0, stream, xq, sx, w13, s13,
                       sorted, block_expert, num_padded, expert_offsets, a, T, H, I, K1);
  else
    hipLaunchKernelGGL(gate_up_tile_kernel<false>, grid, dim3(256), 0, stream, xq, sx, w13, s13,
                       sorted, block_expert, num_padded, expert_offsets, a, T, H, I, K1);
  return hipGetLastError();
}

}  // namespace srmoe
