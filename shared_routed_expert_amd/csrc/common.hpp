// Device helpers shared by the kernels of the fused shared + routed MoE layer (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace srmoe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 128;         // activation group / weight block edge in block-scale mode
constexpr float kFp8Max = 448.0f;   // largest finite OCP E4M3FN magnitude

// D(16x16,f32) += A(16x128,fp8 e4m3) * B(128x16,fp8 e4m3) on the gfx950 matrix cores.
// Format code 0 selects OCP E4M3 for both operands; the E8M0 block scales are
// fixed at 127 (= 2^0), so this is the plain unscaled product.
// Operand layout used by every kernel here: lane l supplies row/column (l & 15)
// and 32 consecutive K bytes starting at 32 * (l >> 4); A and B use the same
// K mapping, so the dot products do not depend on how the hardware orders K.
// Result: element j of lane l is D[4 * (l >> 4) + j][l & 15].
__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// OCP FP8 E4M3FN codes of two finite values with |v| <= 448 (1 + 2^-20) (the quotients
// v / scale of the quantisers never exceed that): gfx950's conversion instruction,
// which rounds to the nearest representable value with ties to the even code and
// keeps the sign (-0 and negative values that round to zero give 0x80). On that range
// it equals an encoder written from the format definition (3 mantissa bits with
// round-to-nearest-even, exponent bias 7, a uniform 2^-9 grid below 2^-6) on every
// float32. Bits 0..7: the code of a, bits 8..15: that of b.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// float -> bfloat16 bits, round to nearest even (finite inputs): gfx950 converts in
// hardware (v_cvt_pk_bf16_f32, two values per instruction, in the current rounding
// mode, which is to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two floats -> their bf16 bits packed in one word (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Cross-lane moves through the DPP network (GFX9 encodings), much cheaper than the
// LDS-routed ds_bpermute behind __shfl_xor. Lanes outside row_mask keep their value.
enum : int {
  kDppXor1 = 0xB1,          // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,          // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
  kDppRowBcast15 = 0x142,   // lane 15 of each row -> next row
  kDppRowBcast31 = 0x143,   // lane 31 -> rows 2 and 3
};

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), kCtrl,
                                                    kRowMask, 0xF, false));
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtrl, kRowMask, 0xF, false);
}

// Max over each row of 16 lanes; every lane of the row ends with the row's max.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}

// Reduce max within aligned groups of `width` lanes (16, 32 or 64).
__device__ __forceinline__ float group_max(float v, int width) {
  v = row16_max(v);
  if (width >= 32) v = fmaxf(v, __shfl_xor(v, 16, kWave));
  if (width >= 64) v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t max_dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<kCtrl, kRowMask>((uint32_t)v);
  const uint32_t hi = dpp_u32<kCtrl, kRowMask>((uint32_t)(v >> 32));
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Max of a 64-bit key over the wavefront, returned to every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_dpp_u64<kDppXor1, 0xF>(v);
  v = max_dpp_u64<kDppXor2, 0xF>(v);
  v = max_dpp_u64<kDppRowHalfMirror, 0xF>(v);
  v = max_dpp_u64<kDppRowMirror, 0xF>(v);
  v = max_dpp_u64<kDppRowBcast15, 0xA>(v);
  v = max_dpp_u64<kDppRowBcast31, 0xC>(v);   // lane 63 now holds the maximum
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Absmax scale for FP8 quantisation, taken in float32: amax / 448, or 1 when amax == 0.
__device__ __forceinline__ float fp8_scale(float amax) {
  return amax > 0.0f ? __fdiv_rn(amax, kFp8Max) : 1.0f;
}

// v / s for many v sharing one scale s, for FP8 codes. With y = 1/s correctly rounded,
// q0 = v y and the remainder r = v - q0 s (exact in one FMA), q0 + r y is the correctly
// rounded quotient whenever nothing underflows (Markstein's theorem on division with a
// fused multiply-add). Scales below 2^-90 take the division itself; above, r can only
// underflow for quotients below 2^-12, whose code is 0 whichever way they round. So the
// FP8 code always equals that of the correctly rounded v / s (also checked on every
// pair of bf16 values and on billions of random float32 pairs).
struct ScaleDiv {
  float s, y;
};
__device__ __forceinline__ ScaleDiv scale_div(float s) { return {s, __fdiv_rn(1.0f, s)}; }
__device__ __forceinline__ float div_by(const ScaleDiv& d, float v) {
  if (d.s < 0x1p-90f) return __fdiv_rn(v, d.s);
  const float q0 = v * d.y;
  return __builtin_fmaf(__builtin_fmaf(-q0, d.s, v), d.y, q0);
}
// E4M3 codes of a / s and b / s (bits 0..7 and 8..15)
__device__ __forceinline__ uint32_t quant2(const ScaleDiv& d, float a, float b) {
  return e4m3_pack2(div_by(d, a), div_by(d, b));
}

// SwiGLU gate activation silu(z) = z * sigmoid(z), in float32.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 32 bytes (one MFMA operand's K slice for a lane) from a 16-byte aligned address.
__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// The command processor hands workgroup i of a launch to XCD i % 8, and each
// XCD has its own L2. For a 1-D grid of at least n workgroups, map dispatch slot
// i to a logical tile so that every XCD walks a contiguous run of the n tiles in
// order (neighbouring tiles then share operands through one L2), every XCD gets
// within one tile of the same count, and the slots left over get -1.
__device__ __forceinline__ int xcd_tile(int i, int n) {
  const int x = i & 7, j = i >> 3;
  const int q = n >> 3, r = n & 7;
  if (j >= q + (x < r ? 1 : 0)) return -1;
  return x * q + (x < r ? x : r) + j;
}

// Tile t (0 <= t < used blocks * ny, in the order xcd_tile walks) -> (row block, column
// tile) with the tiles of one expert grouped column tile by column tile: the ny tiles of
// each of the expert's nb_e blocks occupy the same range of t as in row-block-major order,
// but inside it the expert's blocks take each column tile back to back. Those tiles read the
// same weight slice at the same time, so one XCD's L2 serves it to all of them (in row-block
// order the same slice comes back ny tiles later, after it has left the L2). block_expert and
// expert_offsets are the align outputs (offsets in rows, multiples of block_m).
__device__ __forceinline__ void grouped_tile(int t, int ny, int block_m, const int32_t* __restrict__ block_expert,
                                             const int32_t* __restrict__ expert_offsets, int* b, int* cy) {
  const int e = block_expert[t / ny];
  const int b0 = expert_offsets[e] / block_m;
  const int nbe = expert_offsets[e + 1] / block_m - b0;
  const int u = t - b0 * ny;
  *cy = u / nbe;
  *b = b0 + (u - *cy * nbe);
}

// Token of sorted slot id s = t * K1 + k, i.e. floor(s / K1), as a multiply by
// magic = ceil(2^32 / K1) (slot_div_magic). Exact for K1 <= 16 and s <= 2^24:
// the error term s * (magic * K1 - 2^32) / (K1 * 2^32) stays below 1 / (16 K1).
__device__ __forceinline__ uint64_t slot_div_magic(int K1) {
  return (uint64_t)(0xFFFFFFFFu / (uint32_t)K1) + 1u;
}
__device__ __forceinline__ int slot_token(int s, uint64_t magic) {
  return (int)(((uint64_t)(uint32_t)s * magic) >> 32);
}

__host__ __device__ __forceinline__ size_t sorted_capacity(int T, int K1, int E1, int block_m) {
  size_t n = (size_t)T * K1 + (size_t)E1 * (block_m - 1);
  return (n + block_m - 1) / block_m * block_m;
}

}  // namespace srmoe
