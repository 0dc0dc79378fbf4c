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
// kernels: a = silu(g) * u in float32 per sorted row (0 for padding rows).
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
    float* __restrict__ a_out, int T, int H, int I, int K1) {
  __shared__ __align__(16) uint8_t lds[2][kTile];
  // tiles (row block, 64-column group) in row-block-major order, walked per XCD
  const int ny = (I + 63) / 64;
  const int tile = xcd_tile(blockIdx.x, num_padded[0] / kTBM * ny);
  if (tile < 0) return;
  const int b = tile / ny;
  const int e = block_expert[b];
  if (e < 0) return;
  const int c0 = (tile - b * ny) * 64;  // first intermediate column of this workgroup
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
      const float4 sw = *reinterpret_cast<const float4*>(&scl[buf][kTBM + 4 * wn]);            \
      const float swn[4] = {sw.x, sw.y, sw.z, sw.w};                                           \
      _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                          \
        const float4 sv = *reinterpret_cast<const float4*>(&scl[buf][64 * wm + 16 * m + 4 * kq]); \
        const float sxv[4] = {sv.x, sv.y, sv.z, sv.w};                                         \
        _Pragma("unroll") for (int n = 0; n < 4; ++n) {                                        \
          const v4f t = mfma_16x16x128_fp8(af[m], bf[n], zero4);                               \
          _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[m][n][j] += t[j] * (sxv[j] * swn[n]); \
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
  // Tokens of this lane's output rows (-1 for padding rows) are re-read here
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
    for (int j = 0; j < 4; ++j) sxo[m][j] = kBlock ? 1.f : sx[max(otok[m][j], 0)];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int colc = min(c0 + 32 * wn + 16 * n + r16, I - 1);
    sg[n] = kBlock ? 1.f : s13[(size_t)e * 2 * I + colc];
    su[n] = kBlock ? 1.f : s13[(size_t)e * 2 * I + I + colc];
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
    const float* __restrict__ row_scale, uint16_t* __restrict__ slot_out, int T, int H, int I,
    int K1) {
  __shared__ __align__(16) uint8_t lds[2][kTile];   // rows 0..127 weights (h), 128..255 a_q rows
  const int ny = H / 128;
  const int tile = xcd_tile(blockIdx.x, num_padded[0] / kTBM * ny);
  if (tile < 0) return;
  const int b = tile / ny;
  const int e = block_expert[b];
  if (e < 0) return;
  const int h0 = (tile - b * ny) * 128;
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

// down for I <= 256 (at most two 128-byte K steps): no K loop. The workgroup
// stages its block's 128 a_q rows (zero-filled from I to the K-step boundary)
// and the w2 scales of its columns in LDS once; each wavefront then sweeps
// kDownTiles 64-column tiles of w2[e] for one 64-row half, with the weights as
// the MFMA A operand and two tiles' weight fragments in registers (a tile's set is
// refilled two tiles ahead as soon as its MFMAs have consumed it). Inside a tile, row r of MFMA
// tile n holds column (r / 4) * 16 + 4 * n + r % 4, so each lane ends with 16
// consecutive output columns of a row. The bf16 tile then goes through a
// wavefront-private LDS buffer so that 8 lanes write each row's 128 contiguous
// bytes with one non-temporal store: slot_out is written once and read once by
// the combine, and whole-line streaming stores keep it from evicting the w2
// slices that the block's neighbours re-read from L2 (mixed with partial-line
// stores the same reads and writes took about 1.7x as long). Workgroup = 2 row
// halves x 2 interleaved column streams over 128 * kDownTiles columns; tiles
// are ordered row block major and walked per XCD.
constexpr int kDownTiles = 4;
constexpr int kCombTiles = 1;              // 64-column tiles per wavefront in the combining launch
constexpr int kDownLD = 2 * kGroup + 16;   // LDS row stride of the a_q tile (bytes)
constexpr int kStageLD = 128 + 16;         // LDS row stride of an output staging buffer

typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

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
template <bool kBlock, int KS, int NTL, int kOut>
__global__ void __launch_bounds__(256, 2) down_wide_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ sa, const uint8_t* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ rows,
    const float* __restrict__ row_scale, uint16_t* __restrict__ slot_out, int T, int H, int I,
    int K1, uint16_t* __restrict__ out, int comb_blocks) {
  constexpr int kCols = 128 * NTL;   // columns per workgroup
  __shared__ __align__(16) uint8_t atile[kTBM * kDownLD];
  __shared__ __align__(16) uint8_t stage[4][64 * kStageLD];
  __shared__ __align__(16) float scol[kBlock ? kCols / kGroup * KS : kCols];
  const int ng = (H + kCols - 1) / kCols;
  constexpr bool kComb = kOut == kCombineOut;
  const int tile = xcd_tile(blockIdx.x, (kComb ? comb_blocks : rows[0] / kTBM) * ng);
  if (tile < 0) return;
  const int bt = tile / ng;
  const int b = kComb ? rows[0] / kTBM + bt : bt;
  const int e = block_expert[b];
  if (e < 0) return;
  const int g = tile - bt * ng;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int wt = wv & 1, wc = wv >> 1;
  const int nct = H / 64;
  const int sentinel = T * K1;
  const uint64_t magic = slot_div_magic(K1);
  const size_t nrows = (size_t)sentinel + 1;   // slot rows, with the padding rows' spare
  const int c0 = g * kCols;   // first column of the workgroup

  // a_q rows of the block -> LDS, bytes [I, KS * 128) of each row zeroed: 4 * KS
  // 16-byte chunks per thread, from unconditional (clamped) loads so that the
  // unrolled copy issues them all before the first store waits
  {
    constexpr int cpr = KS * kGroup / 16;   // chunks per LDS row
#pragma unroll
    for (int i = 0; i < 4 * KS; ++i) {
      const int c = tid + 256 * i, r = c / cpr, k = (c % cpr) * 16;
      const uint4 v = *reinterpret_cast<const uint4*>(aq + ((size_t)b * kTBM + r) * I + (k < I ? k : 0));
      const uint32_t msk = k < I ? 0xFFFFFFFFu : 0u;   // a per-word mask: a select of whole
                                                       // uint4 values would go through scratch
      *reinterpret_cast<uint4*>(&atile[r * kDownLD + k]) =
          make_uint4(v.x & msk, v.y & msk, v.z & msk, v.w & msk);
    }
  }
  // w2 scales of the workgroup's columns -> LDS (per channel: kCols floats;
  // block mode: per 128-column block and K step), clamped past H
  if (!kBlock) {
#pragma unroll
    for (int c = tid; c < kCols; c += 256) scol[c] = s2[(size_t)e * H + min(c0 + c, H - 1)];
  } else if (tid < kCols / kGroup * KS) {
    const int cb = min(c0 / kGroup + tid / KS, H / kGroup - 1);
    scol[tid] = s2[((size_t)e * (H / kGroup) + cb) * (I / kGroup) + tid % KS];
  }
  // this lane's rows: output scale in the MFMA layout (rows 64 wt + 16 m + r16)
  // and slot ids in the store layout (rows 64 wt + 8 q + lane / 8)
  float rsc[4], sar[4][KS];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int p = b * kTBM + 64 * wt + 16 * m + r16;
    rsc[m] = row_scale[p];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sar[m][ks] = kBlock ? sa[(size_t)p * (I / kGroup) + ks] : 1.f;
  }
  int srow[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)   // padding rows go to the spare row after the T*K1 slot rows
    srow[q] = min(sorted[b * kTBM + 64 * wt + 8 * q + (lane >> 3)], sentinel);
  // K slices of this lane: bytes ks * 128 + kq * 32 .. +32. Weight slices past I
  // are clamped to the row's first bytes (finite weights) and meet zeros in the
  // a_q tile, so each such product is exactly 0.
  uint32_t koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int k = ks * kGroup + kq * 32;
    koff[ks] = k < I ? k : 0;
  }
  int t = g * 2 * NTL + wc;   // this wavefront's first 64-column tile
  const bool active = t < nct;
  const int t0 = active ? t : 0;
  // weight fragment rows: row r16 of MFMA tile n is column (r16/4)*16 + 4n + r16%4
  const uint8_t* wb = w2 + (size_t)e * H * I + (size_t)((r16 >> 2) * 16 + (r16 & 3)) * I;
  // two register sets of weight fragments: tile j computes from set j & 1 while the set
  // of tile j + 1 is in flight, and set j & 1 is refilled with tile j + 2 as soon as its
  // MFMAs have consumed it
  v8i wf[2][4][KS];
  auto wload = [&](v8i (&w)[4][KS], int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) w[n][ks] = load32(wb + (size_t)(tile * 64 + 4 * n) * I + koff[ks]);
  };
  wload(wf[0], t0);
  if (NTL > 1) wload(wf[1], min(t0 + 2, nct - 1));
  // combining launch (one 64-column tile per wavefront): the slot rows that the first two
  // rows add do not depend on the GEMM, so their loads go out now
  static_assert(!kComb || NTL == 1, "the combining launch takes one tile per wavefront");
  const int nr = K1 - 1;
  const int last = nr > 0 ? nr - 1 : 0;
  const int hs0 = t0 * 64 + (lane & 7) * 8;
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
  // (not with block scales over two K steps: their extra live registers would spill)
  constexpr bool kEarly = kComb && !(kBlock && KS == 2);
  if (kEarly) slot_issue(0, sv[0]);
  __syncthreads();   // the a_q tile and the scales are in LDS
  if (!active) return;

  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* trow = &atile[(64 * wt + r16) * kDownLD + kq * 32];
  uint8_t* stg = stage[wv];
#pragma unroll
  for (int j = 0; j < NTL; ++j) {
    const int cur = j & 1;
    const int tj = t + 2 * j;
    if (tj >= nct) break;
    const int tl = min(tj + 4, nct - 1);   // the tile two steps ahead (re-read past the end)
    v4f acc[4][4];   // [column tile n][row tile m]
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[n][m] = zero4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      v8i tf[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) tf[m] = load32(trow + 16 * m * kDownLD + ks * kGroup);
      const float sb = kBlock ? scol[((tj * 64 - c0) / kGroup) * KS + ks] : 1.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          if (!kBlock) {
            acc[n][m] = mfma_16x16x128_fp8(wf[cur][n][ks], tf[m], acc[n][m]);
          } else {
            const v4f p4 = mfma_16x16x128_fp8(wf[cur][n][ks], tf[m], zero4);
            const float sc = sar[m][ks] * sb;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[n][m][q] += p4[q] * sc;
          }
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j + 2 < NTL) wload(wf[cur], tl);
    __builtin_amdgcn_sched_barrier(0);
    // scale, round and stage: lane (r16, kq) holds columns 16 kq .. 16 kq + 15 of
    // rows 16 m + r16 of the wavefront's 64
    float swc[16];
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
      const float4 v = kBlock ? make_float4(1.f, 1.f, 1.f, 1.f)
                              : *reinterpret_cast<const float4*>(&scol[tj * 64 - c0 + 16 * kq + c]);
      swc[c] = v.x; swc[c + 1] = v.y; swc[c + 2] = v.z; swc[c + 3] = v.w;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t packed[8];
#pragma unroll
      for (int c = 0; c < 16; c += 2) {   // column c = 4 * n + q of this lane's 16
        const float y0 = acc[c >> 2][m][c & 3] * swc[c] * rsc[m];
        const float y1 = acc[(c + 1) >> 2][m][(c + 1) & 3] * swc[c + 1] * rsc[m];
        packed[c >> 1] = pack_bf16x2(y0, y1);
      }
      uint4* sp = reinterpret_cast<uint4*>(stg + (16 * m + r16) * kStageLD + kq * 32);
      sp[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      sp[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
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
      if (!kEarly) slot_issue(0, sv[0]);
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        if (q + 2 < 8) slot_issue(q + 2, sv[((q >> 1) + 1) & 1]);
        uint4 (&v)[2][8] = sv[(q >> 1) & 1];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int srw = srow[q + u];
          float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t m = k < nr ? 0xFFFFFFFFu : 0u;
            add_bf16x8(acc, make_uint4(v[u][k].x & m, v[u][k].y & m, v[u][k].z & m, v[u][k].w & m));
          }
          const int first = srw < sentinel ? srw - nr : 0;
          for (int k = 8; k < nr; ++k)
            add_bf16x8(acc, *reinterpret_cast<const uint4*>(slot_out + (cbase + first + k) * 128 + hc));
          add_bf16x8(acc, *reinterpret_cast<const uint4*>(stg + (8 * (q + u) + (lane >> 3)) * kStageLD + (lane & 7) * 16));
          if (srw < sentinel) {
            const u32x4_nt nv = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                 pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
            __builtin_nontemporal_store(nv, reinterpret_cast<u32x4_nt*>(out + (size_t)slot_token(srw, magic) * H + hs));
          }
        }
      }
    }
  }
}

hipError_t launch_down_tile(const uint8_t* aq, const float* sa, const uint8_t* w2, const float* s2,
                            bool block, const int32_t* sorted, const int32_t* block_expert,
                            const int32_t* num_padded, const float* row_scale, uint16_t* slot_out,
                            int T, int H, int I, int E1, int K1, hipStream_t stream) {
  const int nb = (int)(sorted_capacity(T, K1, E1, kTBM) / kTBM);
  const dim3 blk(256);
  if (I <= 2 * kGroup) {
    const dim3 grid(nb * ((H + 128 * kDownTiles - 1) / (128 * kDownTiles)));
#define SRMOE_DOWN_WIDE(B, KS)                                                                        \
  hipLaunchKernelGGL((down_wide_kernel<B, KS, kDownTiles, kRowsOut>), grid, blk, 0, stream, aq, sa, w2, s2, \
                     sorted, block_expert, num_padded, row_scale, slot_out, T, H, I, K1, nullptr, 0)
    if (I <= kGroup) {
      if (block) SRMOE_DOWN_WIDE(true, 1); else SRMOE_DOWN_WIDE(false, 1);
    } else {
      if (block) SRMOE_DOWN_WIDE(true, 2); else SRMOE_DOWN_WIDE(false, 2);
    }
#undef SRMOE_DOWN_WIDE
    return hipGetLastError();
  }
  const dim3 grid(nb * (H / 128));
  if (block)
    hipLaunchKernelGGL(down_tile_kernel<true>, grid, blk, 0, stream, aq, sa, w2, s2, sorted,
                       block_expert, num_padded, row_scale, slot_out, T, H, I, K1);
  else
    hipLaunchKernelGGL(down_tile_kernel<false>, grid, blk, 0, stream, aq, sa, w2, s2, sorted,
                       block_expert, num_padded, row_scale, slot_out, T, H, I, K1);
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
                                    const int32_t* shared_first, const float* row_scale,
                                    uint16_t* slot_out, uint16_t* out, int T, int H, int I, int E1, int K1,
                                    int parts, hipStream_t stream) {
  // parts: bit 0 the routed experts' launch, bit 1 the shared expert's launch with the combine
  if (!down_wide_supported(I)) return hipErrorInvalidValue;
  const int nb = (int)(sorted_capacity(T, K1, E1, kTBM) / kTBM);
  const int nbs = (T + kTBM - 1) / kTBM;
  const dim3 blk(256);
  const dim3 grid(nb * ((H + 128 * kDownTiles - 1) / (128 * kDownTiles)));
  const dim3 grid_c(nbs * ((H + 128 * kCombTiles - 1) / (128 * kCombTiles)));
#define SRMOE_DOWN_COMB(B, KS)                                                                          \
  do {                                                                                                  \
    if (parts & 1)                                                                                      \
      hipLaunchKernelGGL((down_wide_kernel<B, KS, kDownTiles, kBlockedOut>), grid, blk, 0, stream, aq, sa, \
                         w2, s2, sorted, block_expert, shared_first, row_scale, slot_out, T, H, I, K1,   \
                         nullptr, 0);                                                                   \
    if (parts & 2)                                                                                      \
      hipLaunchKernelGGL((down_wide_kernel<B, KS, kCombTiles, kCombineOut>), grid_c, blk, 0, stream, aq, sa, \
                         w2, s2, sorted, block_expert, shared_first, row_scale, slot_out, T, H, I, K1, out, \
                         nbs);                                                                          \
  } while (0)
  if (I <= kGroup) {
    if (block) SRMOE_DOWN_COMB(true, 1); else SRMOE_DOWN_COMB(false, 1);
  } else {
    if (block) SRMOE_DOWN_COMB(true, 2); else SRMOE_DOWN_COMB(false, 2);
  }
#undef SRMOE_DOWN_COMB
  return hipGetLastError();
}

hipError_t launch_gate_up_tile(const uint8_t* xq, const float* sx, const uint8_t* w13,
                               const float* s13, bool block, const int32_t* sorted,
                               const int32_t* block_expert, const int32_t* num_padded, float* a,
                               int T, int H, int I, int E1, int K1, hipStream_t stream) {
  const int nb = (int)(sorted_capacity(T, K1, E1, kTBM) / kTBM);
  const dim3 grid(nb * ((I + 63) / 64));
  if (block)
    hipLaunchKernelGGL(gate_up_tile_kernel<true>, grid, dim3(256), 0, stream, xq, sx, w13, s13,
                       sorted, block_expert, num_padded, a, T, H, I, K1);
  else
    hipLaunchKernelGGL(gate_up_tile_kernel<false>, grid, dim3(256), 0, stream, xq, sx, w13, s13,
                       sorted, block_expert, num_padded, a, T, H, I, K1);
  return hipGetLastError();
}

}  // namespace srmoe
