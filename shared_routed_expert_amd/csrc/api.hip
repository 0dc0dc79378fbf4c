// C ABI of the fused shared + routed MoE layer: argument checks, workspace
// layout and kernel launches on the caller's stream. See include/srmoe.h.
#include "srmoe.h"

#include <functional>
#include <mutex>

#include "front_dev.hpp"

namespace srmoe {
hipError_t launch_route(const LogitSrc&, int, int, int, float, int32_t*, float*, hipStream_t);
hipError_t launch_route_topk(const float*, int, int, int, int32_t*, float*, hipStream_t);
size_t router_workspace_bytes(int T, int H, int E);
int router_splits(int T, int H, int E);
hipError_t launch_router_gemm(const uint16_t*, const float*, const float*, int, int, int, float*, hipStream_t);
hipError_t launch_router(const uint16_t*, const float*, const float*, int, int, int, float*, float*,
                         hipStream_t);
size_t align_workspace_bytes(int T, int K1, int E1);
hipError_t launch_align(const int32_t*, int, int, int, int, int32_t*, int32_t*, int32_t*, int32_t*,
                        int32_t*, void*, hipStream_t);
hipError_t launch_quant_x(const uint16_t*, int, int, bool, uint8_t*, float*, hipStream_t);
hipError_t launch_quant_a(const float*, int, int, bool, const int32_t*, const float*, int, const int32_t*,
                          uint8_t*, float*, float*, hipStream_t);
hipError_t launch_gate_up(const uint8_t*, const float*, const uint8_t*, const float*, bool,
                          const int32_t*, const int32_t*, const int32_t*, const int32_t*, float*, int, int,
                          int, int, int, int, hipStream_t);
hipError_t launch_down(const uint8_t*, const float*, const uint8_t*, const float*, bool,
                       const int32_t*, const int32_t*, const int32_t*, const int32_t*, const float*,
                       uint16_t*, int, int, int, int, int, int, hipStream_t);
hipError_t launch_combine(const uint16_t*, const uint16_t*, int, int, int, uint16_t*, hipStream_t);
bool down_wide_supported(int I);
hipError_t launch_down_wide_combine(const uint8_t*, const float*, const uint8_t*, const float*, bool,
                                    const int32_t*, const int32_t*, const int32_t*, const float*, uint16_t*,
                                    uint16_t*, int, int, int, int, int, int, hipStream_t);
hipError_t launch_gate_up_decode(const uint8_t*, const float*, const uint8_t*, const float*, bool,
                                 const int32_t*, const int32_t*, float*, int, int, int, int, int,
                                 hipStream_t);
hipError_t launch_layer_front(const LogitSrc&, int, int, int, float, int32_t*, float*, const uint16_t*,
                              int, bool, uint8_t*, float*, hipStream_t);
bool expert_ffn_decode_supported(int H, int I);
bool expert_ffn_decode_align_supported(int T, int K1);
struct AlignOut {
  const int32_t* topk_ids;
  int32_t* counts;
  int32_t* offsets;
  int32_t* num_padded;
  int E1;
};
hipError_t launch_expert_ffn_decode(const uint8_t*, const float*, const uint8_t*, const float*,
                                    const uint8_t*, const float*, bool, int32_t*, int32_t*, const int32_t*,
                                    const AlignOut*, const float*, float*, uint16_t*, int, int, int,
                                    int, int, hipStream_t);
hipError_t launch_qk_norm_rope(uint16_t*, int, int, int, int, int, bool, const float*, const float*, float,
                               const int32_t*, const float*, int, bool, hipStream_t);
hipError_t launch_rope_table(float*, int, int, double, hipStream_t);
}  // namespace srmoe

using namespace srmoe;

// The array behind moe_layer_forward_noalloc (one copy per device; see there). In host code
// this name is only a handle for hipGetSymbolAddress, never a device address.
static __device__ __align__(256) uint8_t scratch[SRMOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxT = 1 << 20;
constexpr int kMaxNoAllocDevices = 64;

inline size_t al256(size_t n) { return (n + 255) / 256 * 256; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SRMOE_OK;
  g_last_hip_error = (int)e;
  return SRMOE_ERR_HIP;
}

// FFN workspace: slot_out first (moe_combine reads it at offset 0) plus one
// spare row that takes the down GEMM's stores for padding rows (so its stores
// need no branch), then the quantised activations, the SwiGLU product in
// float32, its quantised copy and the per-row output scale of the down GEMM.
struct FfnLayout {
  size_t slot_out, xq, sx, a, aq, sa, rs, total;
};

FfnLayout ffn_layout(int T, int H, int I, int E1, int K1, int block_m, int mode) {
  const size_t P = sorted_capacity(T, K1, E1, block_m);
  const size_t gh = mode == SRMOE_SCALE_BLOCK128 ? (size_t)H / kGroup : 1;
  const size_t gi = mode == SRMOE_SCALE_BLOCK128 ? (size_t)I / kGroup : 1;
  FfnLayout L{};
  size_t off = 0;
  L.slot_out = off; off += al256(((size_t)T * K1 + 1) * H * 2);
  L.xq = off;       off += al256((size_t)T * H);
  L.sx = off;       off += al256((size_t)T * gh * 4);
  L.a = off;        off += al256(P * I * 4);
  L.aq = off;       off += al256(P * I);
  L.sa = off;       off += al256(P * gi * 4);
  L.rs = off;       off += al256(P * 4);
  L.total = off;
  return L;
}

bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }

// Shape checks shared by the FFN entry points; 0 if fine.
int check_ffn_dims(int scale_mode, int T, int H, int I, int E1, int K1, int block_m) {
  if (T < 0 || T > kMaxT || H <= 0 || I <= 0 || E1 < 1 || K1 < 1) return SRMOE_ERR_INVALID_ARG;
  if (scale_mode != SRMOE_SCALE_PER_CHANNEL && scale_mode != SRMOE_SCALE_BLOCK128)
    return SRMOE_ERR_INVALID_ARG;
  if (E1 > 256 || K1 > 16 || K1 > E1) return SRMOE_ERR_UNSUPPORTED;
  if (!valid_block_m(block_m)) return SRMOE_ERR_UNSUPPORTED;
  if (H % 128 != 0 || I % 32 != 0) return SRMOE_ERR_UNSUPPORTED;
  if (scale_mode == SRMOE_SCALE_BLOCK128 && I % 128 != 0) return SRMOE_ERR_UNSUPPORTED;
  if (H > 65536 || I > 3072) return SRMOE_ERR_UNSUPPORTED;
  if ((size_t)T * K1 * H >= ((size_t)1 << 31)) return SRMOE_ERR_UNSUPPORTED;
  return SRMOE_OK;
}

}  // namespace

extern "C" {

size_t moe_sorted_capacity(int T, int K1, int E1, int block_m) {
  if (T < 0 || K1 < 1 || E1 < 1 || !valid_block_m(block_m)) return 0;
  return sorted_capacity(T, K1, E1, block_m);
}

size_t moe_align_workspace_bytes(int T, int K1, int E1) {
  if (T < 0 || K1 < 1 || E1 < 1) return 0;
  const size_t n = align_workspace_bytes(T, K1, E1);
  return n > 256 ? n : 256;
}

size_t moe_ffn_workspace_bytes(int T, int H, int I, int E1, int K1, int block_m, int scale_mode) {
  if (check_ffn_dims(scale_mode, T, H, I, E1, K1, block_m) != SRMOE_OK) return 0;
  return ffn_layout(T, H, I, E1, K1, block_m, scale_mode).total;
}

int moe_ffn_workspace_offsets(int T, int H, int I, int E1, int K1, int block_m, int scale_mode,
                              size_t* out) {
  const int st = check_ffn_dims(scale_mode, T, H, I, E1, K1, block_m);
  if (st != SRMOE_OK) return st;
  if (!out) return SRMOE_ERR_INVALID_ARG;
  const FfnLayout L = ffn_layout(T, H, I, E1, K1, block_m, scale_mode);
  out[0] = L.slot_out; out[1] = L.xq; out[2] = L.sx; out[3] = L.a; out[4] = L.aq; out[5] = L.sa;
  out[6] = L.rs; out[7] = L.total;
  return SRMOE_OK;
}

const char* srmoe_status_string(int status) {
  switch (status) {
    case SRMOE_OK: return "ok";
    case SRMOE_ERR_INVALID_ARG: return "invalid argument";
    case SRMOE_ERR_UNSUPPORTED: return "unsupported shape";
    case SRMOE_ERR_WORKSPACE: return "workspace too small";
    case SRMOE_ERR_HIP: return "HIP launch failed (see srmoe_last_hip_error)";
    default: return "unknown status";
  }
}

const char* moe_status_string(int status) { return srmoe_status_string(status); }

int srmoe_last_hip_error(void) { return g_last_hip_error; }

#ifndef SRMOE_SOURCE_HASH
#define SRMOE_SOURCE_HASH "unstamped"
#endif
const char* srmoe_source_hash(void) { return SRMOE_SOURCE_HASH; }

size_t moe_workspace_bytes(int T, int H, int I, int E1, int K1, int block_m, int scale_mode) {
  const size_t f = moe_ffn_workspace_bytes(T, H, I, E1, K1, block_m, scale_mode);
  if (f == 0) return 0;
  const size_t a = moe_align_workspace_bytes(T, K1, E1);
  return f > a ? f : a;
}

int moe_route_topk_plus_shared(const float* logits, int T, int E, int K, float shared_weight,
                               int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || T > kMaxT || E < 1 || K < 0) return SRMOE_ERR_INVALID_ARG;
  if (E > 255 || K > E || K > 15) return SRMOE_ERR_UNSUPPORTED;
  if (T == 0) return SRMOE_OK;
  if (!logits || !topk_ids || !topk_w) return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return SRMOE_ERR_INVALID_ARG;
  return hip_status(launch_route(LogitSrc{logits, nullptr, 0, 0}, T, E, K, shared_weight, topk_ids, topk_w,
                                  as_stream(stream)));
}

size_t moe_router_workspace_bytes(int T, int H, int E) {
  if (T < 0 || H <= 0 || E < 1) return 0;
  const size_t n = router_workspace_bytes(T, H, E);
  return n > 256 ? n : 256;
}

int moe_router_logits(const uint16_t* x, const float* w_router, const float* bias, int T, int H, int E,
                      float* logits, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || T > kMaxT || H <= 0 || E < 1) return SRMOE_ERR_INVALID_ARG;
  if (H % 128 != 0 || E > 256) return SRMOE_ERR_UNSUPPORTED;
  if (T == 0) return SRMOE_OK;
  if (!x || !w_router || !logits || !workspace) return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits) || !aligned16(workspace) ||
      (bias && !aligned16(bias)))
    return SRMOE_ERR_INVALID_ARG;
  if (ws_bytes < moe_router_workspace_bytes(T, H, E)) return SRMOE_ERR_WORKSPACE;
  return hip_status(launch_router(x, w_router, bias, T, H, E, logits, static_cast<float*>(workspace),
                                  as_stream(stream)));
}

int moe_route_topk(const float* logits, int T, int E, int K, int32_t* topk_ids, float* topk_w,
                   void* stream) {
  if (T < 0 || T > kMaxT || E < 1 || K < 1) return SRMOE_ERR_INVALID_ARG;
  if (E > 256 || K > E || K > 15) return SRMOE_ERR_UNSUPPORTED;
  if (T == 0) return SRMOE_OK;
  if (!logits || !topk_ids || !topk_w) return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return SRMOE_ERR_INVALID_ARG;
  return hip_status(launch_route_topk(logits, T, E, K, topk_ids, topk_w, as_stream(stream)));
}

int moe_align_by_expert(const int32_t* topk_ids, int T, int K1, int E1, int block_m,
                        int32_t* sorted_slot_ids, int32_t* block_expert, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* num_padded, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (T < 0 || T > kMaxT || K1 < 1 || E1 < 1) return SRMOE_ERR_INVALID_ARG;
  if (K1 > 16 || E1 > 256 || !valid_block_m(block_m)) return SRMOE_ERR_UNSUPPORTED;
  if ((T > 0 && !topk_ids) || !sorted_slot_ids || !block_expert || !expert_counts ||
      !expert_offsets || !num_padded || !workspace)
    return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(topk_ids) || !aligned16(sorted_slot_ids) || !aligned16(block_expert) ||
      !aligned16(expert_counts) || !aligned16(expert_offsets) || !aligned16(num_padded) ||
      !aligned16(workspace))
    return SRMOE_ERR_INVALID_ARG;
  if (ws_bytes < moe_align_workspace_bytes(T, K1, E1)) return SRMOE_ERR_WORKSPACE;
  // T == 0 still defines the (empty) layout: counts and offsets 0, all rows sentinel.
  return hip_status(launch_align(topk_ids, T, K1, E1, block_m, sorted_slot_ids, block_expert,
                                 expert_counts, expert_offsets, num_padded, workspace,
                                 as_stream(stream)));
}

int moe_ffn_quant_x(const uint16_t* x, int scale_mode, int T, int H, int I, int E1, int K1,
                    int block_m, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_ffn_dims(scale_mode, T, H, I, E1, K1, block_m);
  if (st != SRMOE_OK) return st;
  if (T == 0) return SRMOE_OK;
  if (!x || !workspace || !aligned16(x) || !aligned16(workspace)) return SRMOE_ERR_INVALID_ARG;
  const FfnLayout L = ffn_layout(T, H, I, E1, K1, block_m, scale_mode);
  if (ws_bytes < L.total) return SRMOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return hip_status(launch_quant_x(x, T, H, scale_mode == SRMOE_SCALE_BLOCK128,
                                   reinterpret_cast<uint8_t*>(ws + L.xq),
                                   reinterpret_cast<float*>(ws + L.sx), as_stream(stream)));
}

int moe_ffn_gate_up(const uint8_t* w13, const float* s13, int scale_mode, int T, int H, int I,
                    int E1, int K1, int block_m, const int32_t* sorted_slot_ids,
                    const int32_t* block_expert, const int32_t* num_padded, void* workspace,
                    size_t ws_bytes, void* stream) {
  int st = check_ffn_dims(scale_mode, T, H, I, E1, K1, block_m);
  if (st != SRMOE_OK) return st;
  if (T == 0) return SRMOE_OK;
  if (!w13 || !s13 || !sorted_slot_ids || !block_expert || !num_padded || !workspace)
    return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(w13) || !aligned16(s13) || !aligned16(sorted_slot_ids) || !aligned16(block_expert) ||
      !aligned16(num_padded) || !aligned16(workspace))
    return SRMOE_ERR_INVALID_ARG;
  const FfnLayout L = ffn_layout(T, H, I, E1, K1, block_m, scale_mode);
  if (ws_bytes < L.total) return SRMOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const bool blk = scale_mode == SRMOE_SCALE_BLOCK128;
  if (block_m == 16)
    return hip_status(launch_gate_up_decode(reinterpret_cast<const uint8_t*>(ws + L.xq),
                                            reinterpret_cast<const float*>(ws + L.sx), w13, s13, blk,
                                            sorted_slot_ids, block_expert,
                                            reinterpret_cast<float*>(ws + L.a), T, H, I, E1, K1,
                                            as_stream(stream)));
  return hip_status(launch_gate_up(reinterpret_cast<const uint8_t*>(ws + L.xq),
                                   reinterpret_cast<const float*>(ws + L.sx), w13, s13, blk,
                                   sorted_slot_ids, block_expert, num_padded, nullptr,
                                   reinterpret_cast<float*>(ws + L.a), T, H, I, E1, K1, block_m,
                                   as_stream(stream)));
}

int moe_ffn_down(const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E1,
                 int K1, int block_m, const int32_t* sorted_slot_ids, const int32_t* block_expert,
                 const int32_t* num_padded, const float* topk_w, void* workspace, size_t ws_bytes,
                 void* stream) {
  int st = check_ffn_dims(scale_mode, T, H, I, E1, K1, block_m);
  if (st != SRMOE_OK) return st;
  if (T == 0) return SRMOE_OK;
  if (!w2 || !s2 || !sorted_slot_ids || !block_expert || !num_padded || !topk_w || !workspace)
    return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(w2) || !aligned16(s2) || !aligned16(sorted_slot_ids) || !aligned16(block_expert) ||
      !aligned16(num_padded) || !aligned16(topk_w) || !aligned16(workspace))
    return SRMOE_ERR_INVALID_ARG;
  const FfnLayout L = ffn_layout(T, H, I, E1, K1, block_m, scale_mode);
  if (ws_bytes < L.total) return SRMOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const bool blk = scale_mode == SRMOE_SCALE_BLOCK128;
  const int P_max = (int)sorted_capacity(T, K1, E1, block_m);
  hipError_t e = launch_quant_a(reinterpret_cast<const float*>(ws + L.a), P_max, I, blk,
                                sorted_slot_ids, topk_w, T * K1, num_padded,
                                reinterpret_cast<uint8_t*>(ws + L.aq),
                                reinterpret_cast<float*>(ws + L.sa),
                                reinterpret_cast<float*>(ws + L.rs), as_stream(stream));
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_down(reinterpret_cast<const uint8_t*>(ws + L.aq),
                                reinterpret_cast<const float*>(ws + L.sa), w2, s2, blk,
                                sorted_slot_ids, block_expert, num_padded, nullptr,
                                reinterpret_cast<const float*>(ws + L.rs),
                                reinterpret_cast<uint16_t*>(ws + L.slot_out), T, H, I, E1, K1,
                                block_m, as_stream(stream)));
}

int moe_ffn_experts_one_kernel(int H, int I, int block_m) {
  return block_m == 16 && expert_ffn_decode_supported(H, I) ? 1 : 0;
}

int moe_ffn_experts(const uint8_t* w13, const float* s13, const uint8_t* w2, const float* s2,
                    int scale_mode, int T, int H, int I, int E1, int K1, int block_m,
                    const int32_t* sorted_slot_ids, const int32_t* block_expert,
                    const int32_t* num_padded, const float* topk_w, void* workspace, size_t ws_bytes,
                    void* stream) {
  int st = check_ffn_dims(scale_mode, T, H, I, E1, K1, block_m);
  if (st != SRMOE_OK) return st;
  if (T == 0) return SRMOE_OK;
  if (!w13 || !s13 || !w2 || !s2 || !sorted_slot_ids || !block_expert || !num_padded || !topk_w ||
      !workspace)
    return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(w13) || !aligned16(s13) || !aligned16(w2) || !aligned16(s2) ||
      !aligned16(sorted_slot_ids) || !aligned16(block_expert) || !aligned16(num_padded) ||
      !aligned16(topk_w) || !aligned16(workspace))
    return SRMOE_ERR_INVALID_ARG;
  const FfnLayout L = ffn_layout(T, H, I, E1, K1, block_m, scale_mode);
  if (ws_bytes < L.total) return SRMOE_ERR_WORKSPACE;
  if (!moe_ffn_experts_one_kernel(H, I, block_m)) {
    st = moe_ffn_gate_up(w13, s13, scale_mode, T, H, I, E1, K1, block_m, sorted_slot_ids,
                         block_expert, num_padded, workspace, ws_bytes, stream);
    if (st != SRMOE_OK) return st;
    return moe_ffn_down(w2, s2, scale_mode, T, H, I, E1, K1, block_m, sorted_slot_ids, block_expert,
                        num_padded, topk_w, workspace, ws_bytes, stream);
  }
  char* ws = static_cast<char*>(workspace);
  // sorted_slot_ids / block_expert are only read when no align output is requested
  return hip_status(launch_expert_ffn_decode(
      reinterpret_cast<const uint8_t*>(ws + L.xq), reinterpret_cast<const float*>(ws + L.sx), w13, s13,
      w2, s2, scale_mode == SRMOE_SCALE_BLOCK128, const_cast<int32_t*>(sorted_slot_ids),
      const_cast<int32_t*>(block_expert), num_padded, nullptr, topk_w, reinterpret_cast<float*>(ws + L.a),
      reinterpret_cast<uint16_t*>(ws + L.slot_out), T, H, I, E1, K1, as_stream(stream)));
}

int moe_fused_ffn(const uint16_t* x, const uint8_t* w13, const float* s13, const uint8_t* w2,
                  const float* s2, int scale_mode, int T, int H, int I, int E1, int K1,
                  int block_m, const int32_t* sorted_slot_ids, const int32_t* block_expert,
                  const int32_t* num_padded, const float* topk_w, void* workspace,
                  size_t ws_bytes, void* stream) {
  int st = check_ffn_dims(scale_mode, T, H, I, E1, K1, block_m);
  if (st != SRMOE_OK) return st;
  if (T == 0) return SRMOE_OK;
  // all pointer checks up front so that a bad call launches nothing
  if (!x || !w13 || !s13 || !w2 || !s2 || !sorted_slot_ids || !block_expert || !num_padded ||
      !topk_w || !workspace)
    return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(s13) || !aligned16(w2) || !aligned16(s2) ||
      !aligned16(sorted_slot_ids) || !aligned16(block_expert) || !aligned16(num_padded) ||
      !aligned16(topk_w) || !aligned16(workspace))
    return SRMOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_layout(T, H, I, E1, K1, block_m, scale_mode).total) return SRMOE_ERR_WORKSPACE;
  st = moe_ffn_quant_x(x, scale_mode, T, H, I, E1, K1, block_m, workspace, ws_bytes, stream);
  if (st != SRMOE_OK) return st;
  return moe_ffn_experts(w13, s13, w2, s2, scale_mode, T, H, I, E1, K1, block_m, sorted_slot_ids,
                         block_expert, num_padded, topk_w, workspace, ws_bytes, stream);
}

// Events recorded between the stages of one layer call (for measurement): events[0] before
// the first launch, events[i] after stage i, and the stage's name in names[i - 1].
struct StageMarks {
  void* const* events;
  int n_events;
  const char** names;
  int recorded;
};

static int layer_forward(const uint16_t* x, const LogitSrc& src, const void* logits, const uint8_t* w13, const float* s13,
                      const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E,
                      int K, float shared_weight, int block_m, int32_t* topk_ids, float* topk_w,
                      int32_t* sorted_slot_ids, int32_t* block_expert, int32_t* expert_counts,
                      int32_t* expert_offsets, int32_t* num_padded, void* align_ws,
                      size_t align_ws_bytes, void* ffn_ws, size_t ffn_ws_bytes, uint16_t* out,
                      void* stream, const std::function<int(LogitSrc*, hipStream_t)>& gate,
                      StageMarks* marks = nullptr) {
  // every check of the four calls, before anything is launched
  if (T < 0 || T > kMaxT || E < 1 || K < 0) return SRMOE_ERR_INVALID_ARG;
  if (E > 255 || K > E || K > 15) return SRMOE_ERR_UNSUPPORTED;
  const int E1 = E + 1, K1 = K + 1;
  int st = check_ffn_dims(scale_mode, T, H, I, E1, K1, block_m);
  if (st != SRMOE_OK) return st;
  if (T == 0) return SRMOE_OK;
  const void* ptrs[] = {x, logits, w13, s13, w2, s2, topk_ids, topk_w, sorted_slot_ids, block_expert,
                        expert_counts, expert_offsets, num_padded, align_ws, ffn_ws, out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return SRMOE_ERR_INVALID_ARG;
  if (align_ws_bytes < moe_align_workspace_bytes(T, K1, E1)) return SRMOE_ERR_WORKSPACE;
  const FfnLayout L = ffn_layout(T, H, I, E1, K1, block_m, scale_mode);
  if (ffn_ws_bytes < L.total) return SRMOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(ffn_ws);
  {
    // x_q is written before the align runs: an align workspace that overlaps the FFN workspace
    // must keep its scratch inside the slot-row region in front of x_q (it always does when the
    // two start at the same address: the align scratch is a few bytes per entry, a slot row H*2)
    const char* a0 = static_cast<const char*>(align_ws);
    const size_t need = moe_align_workspace_bytes(T, K1, E1);
    if (a0 < ws + L.total && ws < a0 + need && (a0 < ws || a0 + need > ws + L.xq)) return SRMOE_ERR_WORKSPACE;
  }
  const bool blk = scale_mode == SRMOE_SCALE_BLOCK128;
  hipStream_t sm = as_stream(stream);
  // after a stage: record the next event (when asked to) and pass the status on
  auto mark = [&](int status, const char* name) -> int {
    if (status != SRMOE_OK || !marks || marks->recorded >= marks->n_events) return status;
    if (marks->names && marks->recorded > 0) marks->names[marks->recorded - 1] = name;
    const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(marks->events[marks->recorded]), sm);
    if (e != hipSuccess) return hip_status(e);
    marks->recorded++;
    return SRMOE_OK;
  };
  st = mark(SRMOE_OK, "");
  if (st != SRMOE_OK) return st;
  LogitSrc lsrc = src;
  if (gate) {
    st = mark(gate(&lsrc, sm), "router_gate");
    if (st != SRMOE_OK) return st;
  }
  st = mark(hip_status(launch_layer_front(lsrc, T, E, K, shared_weight, topk_ids, topk_w, x, H, blk,
                                          reinterpret_cast<uint8_t*>(ws + L.xq),
                                          reinterpret_cast<float*>(ws + L.sx), sm)),
            "front");
  if (st != SRMOE_OK) return st;
  if (moe_ffn_experts_one_kernel(H, I, block_m) && expert_ffn_decode_align_supported(T, K1)) {
    // decode shapes: the expert kernel derives the align layout itself (every workgroup
    // from topk_ids) and writes the align outputs, so the layer is three launches
    const AlignOut al{topk_ids, expert_counts, expert_offsets, num_padded, E1};
    st = mark(hip_status(launch_expert_ffn_decode(
                  reinterpret_cast<const uint8_t*>(ws + L.xq), reinterpret_cast<const float*>(ws + L.sx), w13,
                  s13, w2, s2, blk, sorted_slot_ids, block_expert, num_padded, &al, topk_w, nullptr,
                  reinterpret_cast<uint16_t*>(ws + L.slot_out), T, H, I, E1, K1, sm)),
              "experts");
    if (st != SRMOE_OK) return st;
    return mark(moe_combine(topk_w, T, K1, H, ffn_ws, ffn_ws_bytes, out, stream), "combine");
  }
  st = mark(moe_align_by_expert(topk_ids, T, K1, E1, block_m, sorted_slot_ids, block_expert, expert_counts,
                                expert_offsets, num_padded, align_ws, align_ws_bytes, stream),
            "align");
  if (st != SRMOE_OK) return st;
  if (block_m == 128) {
    // prefill shapes: gate/up, the FP8 quantisation of a, then the down GEMM
    const int P_max = (int)sorted_capacity(T, K1, E1, block_m);
    // (the tiles of one expert grouped by the align's offsets, so that its blocks share the
    // weight slices through L2)
    st = mark(hip_status(launch_gate_up(reinterpret_cast<const uint8_t*>(ws + L.xq),
                                        reinterpret_cast<const float*>(ws + L.sx), w13, s13, blk, sorted_slot_ids,
                                        block_expert, num_padded, expert_offsets,
                                        reinterpret_cast<float*>(ws + L.a), T, H, I, E1, K1, block_m, sm)),
              "gate_up");
    if (st != SRMOE_OK) return st;
    st = mark(hip_status(launch_quant_a(reinterpret_cast<const float*>(ws + L.a), P_max, I, blk, sorted_slot_ids,
                                        topk_w, T * K1, num_padded, reinterpret_cast<uint8_t*>(ws + L.aq),
                                        reinterpret_cast<float*>(ws + L.sa), reinterpret_cast<float*>(ws + L.rs),
                                        sm)),
              "quant_a");
    if (st != SRMOE_OK) return st;
    if (!down_wide_supported(I)) {
      // I > 256: the K-looped down GEMM, then the combine
      st = mark(hip_status(launch_down(reinterpret_cast<const uint8_t*>(ws + L.aq),
                                       reinterpret_cast<const float*>(ws + L.sa), w2, s2, blk, sorted_slot_ids,
                                       block_expert, num_padded, expert_offsets,
                                       reinterpret_cast<const float*>(ws + L.rs),
                                       reinterpret_cast<uint16_t*>(ws + L.slot_out), T, H, I, E1, K1, block_m,
                                       sm)),
                "down");
      if (st != SRMOE_OK) return st;
      return mark(moe_combine(topk_w, T, K1, H, ffn_ws, ffn_ws_bytes, out, stream), "combine");
    }
    // the shared expert's down GEMM and the combine are one launch (the shared expert's
    // segment is the last one; its rows add the token's routed slot rows, left by the
    // routed experts' down launch before it, and store out)
    for (int part = 1; part <= 2; ++part) {
      st = mark(hip_status(launch_down_wide_combine(
                    reinterpret_cast<const uint8_t*>(ws + L.aq), reinterpret_cast<const float*>(ws + L.sa), w2,
                    s2, blk, sorted_slot_ids, block_expert, expert_offsets,
                    reinterpret_cast<const float*>(ws + L.rs), reinterpret_cast<uint16_t*>(ws + L.slot_out), out,
                    T, H, I, E1, K1, part, sm)),
                part == 1 ? "down_routed" : "down_shared_combine");
      if (st != SRMOE_OK) return st;
    }
    return SRMOE_OK;
  }
  st = mark(moe_ffn_experts(w13, s13, w2, s2, scale_mode, T, H, I, E1, K1, block_m, sorted_slot_ids,
                            block_expert, num_padded, topk_w, ffn_ws, ffn_ws_bytes, stream),
            moe_ffn_experts_one_kernel(H, I, block_m) ? "experts" : "gate_up+quant_a+down");
  if (st != SRMOE_OK) return st;
  return mark(moe_combine(topk_w, T, K1, H, ffn_ws, ffn_ws_bytes, out, stream), "combine");
}

int moe_layer_forward(const uint16_t* x, const float* logits, const uint8_t* w13, const float* s13,
                      const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E,
                      int K, float shared_weight, int block_m, int32_t* topk_ids, float* topk_w,
                      int32_t* sorted_slot_ids, int32_t* block_expert, int32_t* expert_counts,
                      int32_t* expert_offsets, int32_t* num_padded, void* align_ws,
                      size_t align_ws_bytes, void* ffn_ws, size_t ffn_ws_bytes, uint16_t* out,
                      void* stream) {
  return layer_forward(x, LogitSrc{logits, nullptr, 0, 0}, logits, w13, s13, w2, s2, scale_mode, T, H, I, E, K,
                       shared_weight, block_m, topk_ids, topk_w, sorted_slot_ids, block_expert,
                       expert_counts, expert_offsets, num_padded, align_ws, align_ws_bytes, ffn_ws,
                       ffn_ws_bytes, out, stream, nullptr);
}

int moe_layer_forward_staged(const uint16_t* x, const float* logits, const uint8_t* w13, const float* s13,
                             const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E,
                             int K, float shared_weight, int block_m, int32_t* topk_ids, float* topk_w,
                             int32_t* sorted_slot_ids, int32_t* block_expert, int32_t* expert_counts,
                             int32_t* expert_offsets, int32_t* num_padded, void* align_ws,
                             size_t align_ws_bytes, void* ffn_ws, size_t ffn_ws_bytes, uint16_t* out,
                             void* stream, void* const* events, int n_events, const char** stage_names,
                             int* n_recorded) {
  if (n_events < 0 || (n_events > 0 && !events)) return SRMOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return SRMOE_ERR_INVALID_ARG;
  StageMarks marks{events, n_events, stage_names, 0};
  const int st = layer_forward(x, LogitSrc{logits, nullptr, 0, 0}, logits, w13, s13, w2, s2, scale_mode, T, H, I,
                               E, K, shared_weight, block_m, topk_ids, topk_w, sorted_slot_ids, block_expert,
                               expert_counts, expert_offsets, num_padded, align_ws, align_ws_bytes, ffn_ws,
                               ffn_ws_bytes, out, stream, nullptr, &marks);
  if (n_recorded) *n_recorded = marks.recorded;
  return st;
}

// ---------------------------------------------------------------------------------------
// moe_layer_forward_noalloc: the layer with every intermediate (routing tables, sort arrays,
// align and FFN workspaces) in the library's own device array, for callers that cannot
// allocate. Each device that runs it holds its own copy of the array until the process ends;
// its device address is looked up once per device (hipGetSymbolAddress) and only that
// address is handed to the kernels. Calls on one device share the array: calls that overlap
// in time on one device race.
static std::mutex g_noalloc_mu;
static void* g_noalloc_ptr[kMaxNoAllocDevices];

static int noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxNoAllocDevices) return SRMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return SRMOE_ERR_HIP;
    g_noalloc_ptr[dev] = p;
  }
  *ptr = g_noalloc_ptr[dev];
  return SRMOE_OK;
}

// Carve of the array for one call (each piece 256-byte aligned); 0 when the shape is invalid.
struct NoAllocLayout {
  size_t ids, w, sorted, bexp, counts, offsets, npad, align_ws, ffn_ws, align_bytes, ffn_bytes, total;
};
static NoAllocLayout noalloc_layout(int T, int H, int I, int E, int K, int block_m, int scale_mode) {
  NoAllocLayout L{};
  const int E1 = E + 1, K1 = K + 1;
  const size_t P = sorted_capacity(T, K1, E1, block_m);
  size_t off = 0;
  L.ids = off;      off += al256((size_t)T * K1 * 4);
  L.w = off;        off += al256((size_t)T * K1 * 4);
  L.sorted = off;   off += al256(P * 4);
  L.bexp = off;     off += al256(P / block_m * 4);
  L.counts = off;   off += al256((size_t)E1 * 4);
  L.offsets = off;  off += al256((size_t)(E1 + 1) * 4);
  L.npad = off;     off += 256;
  L.align_bytes = moe_align_workspace_bytes(T, K1, E1);
  L.align_ws = off; off += al256(L.align_bytes);
  L.ffn_bytes = moe_ffn_workspace_bytes(T, H, I, E1, K1, block_m, scale_mode);
  L.ffn_ws = off;   off += al256(L.ffn_bytes);
  L.total = off;
  return L;
}

int moe_layer_forward_noalloc(const uint16_t* x, const float* logits, const uint8_t* w13, const float* s13,
                              const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E,
                              int K, float shared_weight, int block_m, uint16_t* out, void* stream) {
  // the shape checks of moe_layer_forward first (nothing of the array is touched before them)
  if (T < 0 || T > kMaxT || E < 1 || K < 0) return SRMOE_ERR_INVALID_ARG;
  if (E > 255 || K > E || K > 15) return SRMOE_ERR_UNSUPPORTED;
  int st = check_ffn_dims(scale_mode, T, H, I, E + 1, K + 1, block_m);
  if (st != SRMOE_OK) return st;
  if (T == 0) return SRMOE_OK;
  const NoAllocLayout L = noalloc_layout(T, H, I, E, K, block_m, scale_mode);
  if (L.ffn_bytes == 0 || L.total > (size_t)SRMOE_NOALLOC_SCRATCH_BYTES) return SRMOE_ERR_WORKSPACE;
  const void* ptrs[] = {x, logits, w13, s13, w2, s2, out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return SRMOE_ERR_INVALID_ARG;
  void* base = nullptr;
  st = noalloc_scratch(&base);
  if (st != SRMOE_OK) return st;
  char* sb = static_cast<char*>(base);
  return layer_forward(x, LogitSrc{logits, nullptr, 0, 0}, logits, w13, s13, w2, s2, scale_mode, T, H, I, E, K,
                       shared_weight, block_m, reinterpret_cast<int32_t*>(sb + L.ids),
                       reinterpret_cast<float*>(sb + L.w), reinterpret_cast<int32_t*>(sb + L.sorted),
                       reinterpret_cast<int32_t*>(sb + L.bexp), reinterpret_cast<int32_t*>(sb + L.counts),
                       reinterpret_cast<int32_t*>(sb + L.offsets), reinterpret_cast<int32_t*>(sb + L.npad),
                       sb + L.align_ws, L.align_bytes, sb + L.ffn_ws, L.ffn_bytes, out, stream, nullptr);
}

size_t moe_route_from_x_workspace_bytes(int T, int H, int E) {
  if (T <= 0 || H <= 0 || E < 1) return 0;
  const int ks = router_splits(T, H, E);
  return (size_t)(ks > 1 ? ks : 1) * T * E * sizeof(float);
}

// Router gate into the workspace (partial tiles, or the logits themselves when the gate
// runs in one K chunk); the routing kernels then read it through a LogitSrc.
static int router_into(const uint16_t* x, const float* w_router, const float* bias, int T, int H, int E,
                       void* ws, LogitSrc* src, hipStream_t sm) {
  float* dst = static_cast<float*>(ws);
  const int ks = router_splits(T, H, E);
  const int st = hip_status(launch_router_gemm(x, w_router, bias, T, H, E, dst, sm));
  *src = ks > 1 ? LogitSrc{dst, bias, ks, (size_t)T * E} : LogitSrc{dst, nullptr, 0, 0};
  return st;
}

static int check_router_args(const uint16_t* x, const float* w_router, const float* bias, int T, int H,
                             int E, const void* ws, size_t ws_bytes) {
  if (H <= 0) return SRMOE_ERR_INVALID_ARG;
  if (H % 128 != 0) return SRMOE_ERR_UNSUPPORTED;
  if (T == 0) return SRMOE_OK;
  if (!x || !w_router || !ws || !aligned16(x) || !aligned16(w_router) || !aligned16(ws) ||
      (bias && !aligned16(bias)))
    return SRMOE_ERR_INVALID_ARG;
  if (ws_bytes < moe_route_from_x_workspace_bytes(T, H, E)) return SRMOE_ERR_WORKSPACE;
  return SRMOE_OK;
}

int moe_route_from_x(const uint16_t* x, const float* w_router, const float* bias, int T, int H, int E, int K,
                     float shared_weight, int32_t* topk_ids, float* topk_w, void* workspace, size_t ws_bytes,
                     void* stream) {
  if (T < 0 || T > kMaxT || E < 1 || K < 0) return SRMOE_ERR_INVALID_ARG;
  if (E > 255 || K > E || K > 15) return SRMOE_ERR_UNSUPPORTED;
  int st = check_router_args(x, w_router, bias, T, H, E, workspace, ws_bytes);
  if (st != SRMOE_OK || T == 0) return st;
  if (!topk_ids || !topk_w || !aligned16(topk_ids) || !aligned16(topk_w)) return SRMOE_ERR_INVALID_ARG;
  hipStream_t sm = as_stream(stream);
  LogitSrc src;
  st = router_into(x, w_router, bias, T, H, E, workspace, &src, sm);
  if (st != SRMOE_OK) return st;
  return hip_status(launch_route(src, T, E, K, shared_weight, topk_ids, topk_w, sm));
}

int moe_layer_forward_from_x(const uint16_t* x, const float* w_router, const float* bias,
                             const uint8_t* w13, const float* s13, const uint8_t* w2, const float* s2,
                             int scale_mode, int T, int H, int I, int E, int K, float shared_weight,
                             int block_m, int32_t* topk_ids, float* topk_w, int32_t* sorted_slot_ids,
                             int32_t* block_expert, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* num_padded, void* router_ws, size_t router_ws_bytes, void* align_ws,
                             size_t align_ws_bytes, void* ffn_ws, size_t ffn_ws_bytes, uint16_t* out,
                             void* stream) {
  // the shape checks of the layer first, then the gate's
  if (T < 0 || T > kMaxT || E < 1 || K < 0) return SRMOE_ERR_INVALID_ARG;
  if (E > 255 || K > E || K > 15) return SRMOE_ERR_UNSUPPORTED;
  int st = check_ffn_dims(scale_mode, T, H, I, E + 1, K + 1, block_m);
  if (st != SRMOE_OK) return st;
  st = check_router_args(x, w_router, bias, T, H, E, router_ws, router_ws_bytes);
  if (st != SRMOE_OK) return st;
  // a stand-in for the logits pointer, so that the layer's own checks pass before the gate runs
  return layer_forward(x, LogitSrc{nullptr, nullptr, 0, 0}, router_ws, w13, s13, w2, s2, scale_mode, T, H, I,
                       E, K, shared_weight, block_m, topk_ids, topk_w, sorted_slot_ids, block_expert,
                       expert_counts, expert_offsets, num_padded, align_ws, align_ws_bytes, ffn_ws,
                       ffn_ws_bytes, out, stream, [&](LogitSrc* src, hipStream_t sm) {
                         return router_into(x, w_router, bias, T, H, E, router_ws, src, sm);
                       });
}

int moe_combine(const float* topk_w, int T, int K1, int H, const void* workspace, size_t ws_bytes,
                uint16_t* out, void* stream) {
  if (T < 0 || T > kMaxT || K1 < 1 || H <= 0) return SRMOE_ERR_INVALID_ARG;
  if (K1 > 16 || H % 128 != 0 || (size_t)T * K1 * H >= ((size_t)1 << 31)) return SRMOE_ERR_UNSUPPORTED;
  if (T == 0) return SRMOE_OK;
  if (!workspace || !out || !aligned16(workspace) || !aligned16(out)) return SRMOE_ERR_INVALID_ARG;
  // the slot rows already carry their routing weight (the down GEMM's epilogue applies it), so
  // topk_w is not read here; it may be NULL
  if (topk_w && !aligned16(topk_w)) return SRMOE_ERR_INVALID_ARG;
  if (ws_bytes < (size_t)T * K1 * H * 2) return SRMOE_ERR_WORKSPACE;
  return hip_status(launch_combine(static_cast<const uint16_t*>(workspace), nullptr, T, K1, H, out,
                                   as_stream(stream)));
}

int moe_combine_unfused(int T, int K, int H, const void* routed_ws, size_t routed_ws_bytes,
                        const void* shared_ws, size_t shared_ws_bytes, uint16_t* out, void* stream) {
  if (T < 0 || T > kMaxT || K < 1 || H <= 0) return SRMOE_ERR_INVALID_ARG;
  if (K > 16 || H % 128 != 0 || (size_t)T * K * H >= ((size_t)1 << 31)) return SRMOE_ERR_UNSUPPORTED;
  if (T == 0) return SRMOE_OK;
  if (!routed_ws || !shared_ws || !out || !aligned16(routed_ws) || !aligned16(shared_ws) ||
      !aligned16(out))
    return SRMOE_ERR_INVALID_ARG;
  if (routed_ws_bytes < (size_t)T * K * H * 2 || shared_ws_bytes < (size_t)T * H * 2)
    return SRMOE_ERR_WORKSPACE;
  return hip_status(launch_combine(static_cast<const uint16_t*>(routed_ws),
                                   static_cast<const uint16_t*>(shared_ws), T, K, H, out,
                                   as_stream(stream)));
}

// head_dim in {64, 128, 256}; rotary_dim a power of two in [16, head_dim]
static bool qk_dims_supported(int head_dim, int rotary_dim) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return false;
  return rotary_dim >= 16 && rotary_dim <= head_dim && (rotary_dim & (rotary_dim - 1)) == 0;
}

int moe_rope_cos_sin_table(float* cos_sin, int max_pos, int rotary_dim, double theta, void* stream) {
  if (max_pos < 1 || rotary_dim < 2 || rotary_dim % 2 != 0 || !(theta > 1.0)) return SRMOE_ERR_INVALID_ARG;
  if ((size_t)max_pos * rotary_dim >= ((size_t)1 << 31)) return SRMOE_ERR_UNSUPPORTED;
  if (!cos_sin || !aligned16(cos_sin)) return SRMOE_ERR_INVALID_ARG;
  return hip_status(launch_rope_table(cos_sin, max_pos, rotary_dim, theta, as_stream(stream)));
}

int moe_qk_norm_rope(uint16_t* qkv, int T, int num_q_heads, int num_kv_heads, int head_dim, int rotary_dim,
                     int neox, const float* q_norm_w, const float* k_norm_w, float eps,
                     const int32_t* positions, const float* cos_sin, int max_pos, int fused, void* stream) {
  if (T < 0 || T > kMaxT || num_q_heads < 0 || num_kv_heads < 0 || num_q_heads + num_kv_heads < 1 ||
      max_pos < 1 || !(eps >= 0.f) || !(eps < 1e30f))
    return SRMOE_ERR_INVALID_ARG;
  if (!qk_dims_supported(head_dim, rotary_dim) || num_q_heads + 2 * num_kv_heads > 1024)
    return SRMOE_ERR_UNSUPPORTED;
  if ((size_t)max_pos * rotary_dim >= ((size_t)1 << 31)) return SRMOE_ERR_UNSUPPORTED;
  if (T == 0) return SRMOE_OK;
  if (!qkv || !positions || !cos_sin || (num_q_heads > 0 && !q_norm_w) || (num_kv_heads > 0 && !k_norm_w))
    return SRMOE_ERR_INVALID_ARG;
  if (!aligned16(qkv) || !aligned16(positions) || !aligned16(cos_sin) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w))
    return SRMOE_ERR_INVALID_ARG;
  return hip_status(launch_qk_norm_rope(qkv, T, num_q_heads, num_kv_heads, head_dim, rotary_dim, neox != 0,
                                        q_norm_w, k_norm_w, eps, positions, cos_sin, max_pos, fused != 0,
                                        as_stream(stream)));
}

}  // extern "C"
