/*
 * srmoe.h -- C ABI of the fused shared + routed MoE layer for AMD MI355X (gfx950).
 *
 * The layer (Optimizing GLM4-MoE for production, Novita AI, section 1 "Shared
 * Experts Fusion"; intelliparadigm, GLM4-MoE production optimisation, section
 * 2.1): every token goes through one shared expert and through the top-K of E
 * routed experts chosen by its router, and the outputs are summed with the
 * routing weights. The fusion treats the shared expert as one more routed
 * expert (id E, the (E+1)-th), appends it to every token's routing table in
 * the last slot (slot K, the 9th of 9 for K = 8) with coefficient 1.0, and runs
 * all K+1 slots as one grouped expert-FFN pass:
 *
 *     out_t = sum_{k=0..K} w[t,k] * FFN_{ids[t,k]}(x_t),  ids[t,K] = E, w[t,K] = 1
 *     FFN_e(v) = W2_e ( silu(Wgate_e v) * (Wup_e v) )      (SwiGLU)
 *
 * with FP8 E4M3 expert weights (the pages serve the model in FP8 at TP8, where
 * the per-GPU expert intermediate size is 192).
 *
 * Conventions for every entry point below
 *   - Pointers are DEVICE pointers unless marked "host". Arrays are row-major
 *     and contiguous. bf16 values are passed as their uint16 bit patterns; FP8
 *     values are OCP E4M3FN bytes (bias 7, max 448, no infinities).
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the default stream). Buffers must stay alive until that work completes.
 *     Nothing is synchronised and no device-to-host copy is made.
 *   - The caller owns and allocates every buffer (including workspaces). The
 *     library allocates no device memory, keeps no state between calls except
 *     a thread-local copy of the last HIP error, and is reentrant.
 *   - Argument checks run on the host before any launch. On failure a
 *     negative srmoe_status is returned and no output is touched. A failed
 *     launch returns SRMOE_ERR_HIP; srmoe_last_hip_error() gives the hipError_t.
 *     Nothing throws, prints or aborts.
 *   - T == 0 is valid everywhere. Route, FFN and combine then launch nothing;
 *     align still writes its empty layout (all rows sentinel, counts 0).
 *   - Inputs outside the contract (non-finite logits or activations, ids or
 *     sort arrays not produced by this library) give undefined results.
 *   - Pointers must be 16-byte aligned.
 */
#ifndef SRMOE_H_
#define SRMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SRMOE_OK = 0,
  SRMOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer    */
  SRMOE_ERR_UNSUPPORTED = -2, /* a shape outside the supported set             */
  SRMOE_ERR_WORKSPACE = -3,   /* workspace smaller than the *_workspace_bytes   */
  SRMOE_ERR_HIP = -4          /* a HIP launch failed; see srmoe_last_hip_error() */
} srmoe_status;

typedef enum {
  SRMOE_SCALE_PER_CHANNEL = 0, /* s13 [E1,2I], s2 [E1,H]; activations: one scale per row  */
  SRMOE_SCALE_BLOCK128 = 1     /* s13 [E1,2I/128,H/128], s2 [E1,H/128,I/128]; activations:
                                  one scale per row and 128-wide column group             */
} srmoe_scale_mode;

/* ---------------------------------------------------------------------------
 * Step 1: router top-K plus the shared slot.
 * Per token t: the K routed experts with the largest logits, ordered by
 * (logit descending, expert id ascending) -- equal logits go to the lower id;
 * weights w[t,k] = p_k / sum_{j in top-K} p_j with p = softmax(logits[t,0:E]);
 * then slot K gets the shared expert: ids[t,K] = E, w[t,K] = shared_weight.
 * (Shared expert as routed expert number E+1 in the last of K+1 positions:
 * intelliparadigm section 2.1; Novita AI section 1. Softmax with renormalised
 * top-K is the plainest router reading; the pages do not name it.)
 *   logits   [T,E] float32 (router output for the E routed experts)
 *   topk_ids [T,K+1] int32 out;  topk_w [T,K+1] float32 out
 *   limits: 1 <= E <= 255, 0 <= K <= min(E,15).
 * ------------------------------------------------------------------------- */
int moe_route_topk_plus_shared(const float* logits, int T, int E, int K, float shared_weight,
                               int32_t* topk_ids, float* topk_w, void* stream);

/* ---------------------------------------------------------------------------
 * The router gate, upstream of step 1 (each token scores the E routed experts;
 * Novita AI section 1): logits[t,e] = sum_h x[t,h] * w_router[e,h] + bias[e].
 *   x [T,H] bf16; w_router [E,H] float32; bias [E] float32 or NULL; logits [T,E]
 *   float32 out (the input of moe_route_topk_plus_shared).
 *   Float32-accurate on the bf16 matrix cores: each weight is split into three bf16
 *   parts that carry its 24 significand bits, so every product with the bf16 x is
 *   exact and the sums are float32. Deterministic (K-split partials are summed in a
 *   fixed order).
 *   workspace >= moe_router_workspace_bytes(T,H,E) bytes (those partials), device.
 *   limits: H % 128 == 0, 1 <= E <= 256.
 * ------------------------------------------------------------------------- */
int moe_router_logits(const uint16_t* x, const float* w_router, const float* bias, int T, int H, int E,
                      float* logits, void* workspace, size_t ws_bytes, void* stream);
size_t moe_router_workspace_bytes(int T, int H, int E); /* host */

/* ---------------------------------------------------------------------------
 * The router gate folded into the route call: routing straight from x (the router
 * scores every token over the routed experts ahead of the top-K: Optimizing GLM4-MoE
 * for production, section 1; the fused routing table: intelliparadigm section 2.1).
 * moe_route_from_x = the gate of moe_router_logits followed by the routing of
 * moe_route_topk_plus_shared, with the gate's K-split partial tiles summed inside the
 * routing kernel (in chunk order, then + bias: the same float32 operations as the gate's
 * own reduction), so ids and weights equal those of the two calls bit for bit, one
 * launch and one [T,E] round trip fewer. Arguments as in those two calls;
 * workspace >= moe_route_from_x_workspace_bytes(T,H,E) bytes (device): the partial
 * tiles, or the logits when the gate runs in one K chunk.
 * limits: H % 128 == 0, 1 <= E <= 255, 0 <= K <= min(E, 15).
 * ------------------------------------------------------------------------- */
int moe_route_from_x(const uint16_t* x, const float* w_router, const float* bias, int T, int H, int E, int K,
                     float shared_weight, int32_t* topk_ids, float* topk_w, void* workspace, size_t ws_bytes,
                     void* stream);
size_t moe_route_from_x_workspace_bytes(int T, int H, int E); /* host; 0 for empty shapes */

/* The whole layer from x: moe_layer_forward with the router gate in front of it and the
 * gate's partial tiles summed by the routing part of its first launch (so the outputs
 * equal moe_router_logits + moe_layer_forward bit for bit). router_ws as for
 * moe_route_from_x; every other argument as for moe_layer_forward. */
int moe_layer_forward_from_x(const uint16_t* x, const float* w_router, const float* bias,
                             const uint8_t* w13, const float* s13, const uint8_t* w2, const float* s2,
                             int scale_mode, int T, int H, int I, int E, int K, float shared_weight,
                             int block_m, int32_t* topk_ids, float* topk_w, int32_t* sorted_slot_ids,
                             int32_t* block_expert, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* num_padded, void* router_ws, size_t router_ws_bytes, void* align_ws,
                             size_t align_ws_bytes, void* ffn_ws, size_t ffn_ws_bytes, uint16_t* out,
                             void* stream);

/* ---------------------------------------------------------------------------
 * The unfused layer, for the fused-vs-unfused comparison: the routed experts and
 * the shared expert computed as two passes and added (the pages' formulation
 * before the fusion: intelliparadigm section 2.1, shared output plus the weighted
 * routed outputs).
 *
 * moe_route_topk: step 1 without the shared slot -- the same top-K, order and
 * weights, rows of K entries.   topk_ids / topk_w [T,K] out; limits 1 <= K <=
 * min(E,15), E <= 256.
 *
 * The routed pass is then moe_align_by_expert + moe_fused_ffn with K1 = K, E1 = E
 * (the first E experts of w13/s13/w2/s2); the shared pass is moe_fused_ffn with
 * K1 = 1, E1 = 1 (the shared expert's weights; every token routed to it with
 * weight shared_weight, a layout that does not depend on the routing).
 *
 * moe_combine_unfused: out[t,:] = bf16( sum_{k<K} routed[t,k,:] + shared[t,:] ),
 * accumulated in float32 in that order -- the order of moe_combine over the fused
 * K+1 slots, so the two layers agree bit for bit. routed_ws / shared_ws are the
 * workspaces of the two passes (>= T*K*H*2 and T*H*2 bytes of slot rows).
 * ------------------------------------------------------------------------- */
int moe_route_topk(const float* logits, int T, int E, int K, int32_t* topk_ids, float* topk_w,
                   void* stream);
int moe_combine_unfused(int T, int K, int H, const void* routed_ws, size_t routed_ws_bytes,
                        const void* shared_ws, size_t shared_ws_bytes, uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Step 2: align / sort / pad the T*(K+1) (token, slot) entries by expert.
 * Entry s = t*K1 + k has expert topk_ids[s]. Output, for experts in ascending
 * id, the entries of each expert in ascending s (a stable counting sort),
 * each expert's segment padded to a multiple of block_m with the sentinel
 * T*K1 (an expert with no entries takes no rows), and the sentinel again up
 * to P_max = moe_sorted_capacity(T,K1,E1,block_m).
 *   topk_ids        [T*K1] int32 in, values in 0..E1-1
 *   sorted_slot_ids [P_max] int32 out
 *   block_expert    [P_max/block_m] int32 out: owning expert of rows
 *                   b*block_m..(b+1)*block_m-1, or -1 past the used rows
 *   expert_counts   [E1] int32 out: entries per expert
 *   expert_offsets  [E1+1] int32 out: exclusive scan of the padded counts
 *   num_padded      [1] int32 out: expert_offsets[E1]
 *   workspace       >= moe_align_workspace_bytes(T,K1,E1) bytes, device
 *   limits: 1 <= K1 <= 16, 1 <= E1 <= 256, block_m in {16,32,64,128}.
 * Integer-only; results are deterministic and independent of scheduling.
 * ------------------------------------------------------------------------- */
int moe_align_by_expert(const int32_t* topk_ids, int T, int K1, int E1, int block_m,
                        int32_t* sorted_slot_ids, int32_t* block_expert, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* num_padded, void* workspace,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Step 3: the grouped SwiGLU expert FFN over all K+1 slots (one pass for the
 * shared and the routed experts). For each sorted row with slot s = t*K1+k:
 *   x_q      = FP8 absmax fake-quant of x[t] (scale amax/448, RNE, saturating;
 *              per row, or per 128 group in block mode) -- activation step a3
 *   g, u     = dequantised x_q against gate rows 0..I-1 / up rows I..2I-1 of
 *              w13[e] (fp8 MFMA, fp32 accumulate, per-channel or per-block
 *              scales)                                       -- step a4
 *   a        = silu(g) * u (float32), FP8 absmax-quantised per row over I
 *              (per 128 group in block mode)
 *   y        = dequantised a against w2[e]                   -- step a5
 *   slot_out[s,:] = bf16( topk_w[s] * y )   (kept in the workspace)
 * Inputs:
 *   x        [T,H] bf16;   w13 [E1,2I,H] e4m3;  w2 [E1,H,I] e4m3
 *   s13, s2  float32 scales, shapes per scale_mode (see srmoe_scale_mode)
 *   sorted_slot_ids, block_expert, num_padded: outputs of step 2 (same block_m)
 *   topk_w   [T,K1] float32 routing weights (step 1)
 *   workspace >= moe_ffn_workspace_bytes(...) bytes; also read by moe_combine
 *   limits: H % 128 == 0, H <= 65536; I % 32 == 0 (block mode: I % 128 == 0),
 *           I <= 3072; E1 <= 256; 1 <= K1 <= 16; block_m in {16,32,64,128}.
 * ------------------------------------------------------------------------- */
int moe_fused_ffn(const uint16_t* x, const uint8_t* w13, const float* s13, const uint8_t* w2,
                  const float* s2, int scale_mode, int T, int H, int I, int E1, int K1,
                  int block_m, const int32_t* sorted_slot_ids, const int32_t* block_expert,
                  const int32_t* num_padded, const float* topk_w, void* workspace,
                  size_t ws_bytes, void* stream);

/* The stages of moe_fused_ffn, callable one at a time (same arguments, same
 * workspace). moe_fused_ffn == moe_ffn_quant_x then moe_ffn_experts.
 *
 * moe_ffn_experts: gate/up, a = silu(g)*u, a's FP8 quantisation and down, from the
 * x_q that moe_ffn_quant_x left in the workspace; leaves slot_out (and the float32
 * a) in the workspace. For 16-row blocks (block_m == 16) with I a multiple of 64 in
 * 64..256 and H <= 5120 this is one kernel per layer (moe_ffn_experts_one_kernel
 * says whether it is, returning 1 or 0); otherwise it is moe_ffn_gate_up followed by
 * moe_ffn_down, which can also be called on their own (in that order). Both routes
 * compute the same quantities; their float32 sums may round differently.
 * Errors as moe_fused_ffn; nothing is launched when a check fails. */
int moe_ffn_quant_x(const uint16_t* x, int scale_mode, int T, int H, int I, int E1, int K1,
                    int block_m, void* workspace, size_t ws_bytes, void* stream);
int moe_ffn_experts(const uint8_t* w13, const float* s13, const uint8_t* w2, const float* s2,
                    int scale_mode, int T, int H, int I, int E1, int K1, int block_m,
                    const int32_t* sorted_slot_ids, const int32_t* block_expert,
                    const int32_t* num_padded, const float* topk_w, void* workspace, size_t ws_bytes,
                    void* stream);
int moe_ffn_experts_one_kernel(int H, int I, int block_m);
int moe_ffn_gate_up(const uint8_t* w13, const float* s13, int scale_mode, int T, int H, int I,
                    int E1, int K1, int block_m, const int32_t* sorted_slot_ids,
                    const int32_t* block_expert, const int32_t* num_padded, void* workspace,
                    size_t ws_bytes, void* stream);
int moe_ffn_down(const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E1,
                 int K1, int block_m, const int32_t* sorted_slot_ids,
                 const int32_t* block_expert, const int32_t* num_padded, const float* topk_w,
                 void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Step 4: weighted combine (Novita AI section 1: the experts' outputs are
 * weighted and aggregated). out[t,:] = bf16( sum_{k=0..K1-1} slot_out[t*K1+k,:] )
 * accumulated in float32 in slot order 0..K1-1, where slot_out is the one
 * moe_fused_ffn left in `workspace`.
 *   topk_w [T,K1] float32, the routing weights of step 1 (may be NULL). The
 *          weighting itself happens in moe_fused_ffn's down GEMM, which stores
 *          each slot row as bf16(topk_w[s] * y): the weight is one factor of the
 *          row's dequantisation scale there, so the combine is a plain sum and the
 *          weighted rows are rounded once. The argument is part of the call so
 *          that the weighting can move between the two kernels without an ABI
 *          change; the current kernels do not read it.
 *   out [T,H] bf16 out.
 * ------------------------------------------------------------------------- */
int moe_combine(const float* topk_w, int T, int K1, int H, const void* workspace, size_t ws_bytes,
                uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * The whole layer in one call: steps 1-4 with the arguments of the four calls
 * above (K routed slots, E routed experts; K1 = K+1, E1 = E+1) and the same
 * outputs, bit for bit. The routing and the FP8 quantisation of x do not depend
 * on each other and share one launch, so the layer takes one launch fewer than
 * the four calls. With block_m == 128 and I <= 256 the shared expert's down GEMM
 * and step 4 are one launch as well: the shared expert's rows (the last segment of
 * the sorted layout, one per token) add the token's routed slot rows and store out,
 * with the same float32 sum in the same order as moe_combine. align_ws/ffn_ws as for
 * moe_align_by_expert/moe_fused_ffn; what ffn_ws holds afterwards is not part of the
 * result (in that case the routed slot rows are kept in 128-column blocks and the
 * shared expert's are not written).
 * ------------------------------------------------------------------------- */
int moe_layer_forward(const uint16_t* x, const float* logits, const uint8_t* w13, const float* s13,
                      const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E,
                      int K, float shared_weight, int block_m, int32_t* topk_ids, float* topk_w,
                      int32_t* sorted_slot_ids, int32_t* block_expert, int32_t* expert_counts,
                      int32_t* expert_offsets, int32_t* num_padded, void* align_ws,
                      size_t align_ws_bytes, void* ffn_ws, size_t ffn_ws_bytes, uint16_t* out,
                      void* stream);

/* Measurement form of moe_layer_forward: the same launches and outputs, with caller-created
 * hipEvent_t events (host array `events` of n_events handles) recorded on `stream` between
 * the layer's stages: events[0] before the first launch, events[i] after stage i, for as
 * many stages as there are events. stage_names (host, may be NULL) receives in entry i - 1
 * a static name for stage i ("front", "align", "experts", "gate_up", "quant_a",
 * "down_routed", "down_shared_combine", "combine", ...); *n_recorded (host, may be NULL) the number of events
 * recorded. The elapsed time between events i - 1 and i is stage i's share of the layer. */
int moe_layer_forward_staged(const uint16_t* x, const float* logits, const uint8_t* w13, const float* s13,
                             const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E,
                             int K, float shared_weight, int block_m, int32_t* topk_ids, float* topk_w,
                             int32_t* sorted_slot_ids, int32_t* block_expert, int32_t* expert_counts,
                             int32_t* expert_offsets, int32_t* num_padded, void* align_ws,
                             size_t align_ws_bytes, void* ffn_ws, size_t ffn_ws_bytes, uint16_t* out,
                             void* stream, void* const* events, int n_events, const char** stage_names,
                             int* n_recorded);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_layer_forward with every
 * intermediate -- routing tables, sort arrays, align and FFN workspaces -- in a device
 * array inside the library instead of caller buffers. The caller passes the inputs and
 * `out` only; arguments and result are those of moe_layer_forward (same kernels, same
 * bits). The call allocates nothing: no hipMalloc, hipFree or allocating library routine.
 *   - The array holds SRMOE_NOALLOC_SCRATCH_BYTES (64 MiB) on each device it runs on, from
 *     the first call on that device until the process ends.
 *   - Sizes whose intermediates need more than that return SRMOE_ERR_WORKSPACE before
 *     anything is launched: the carve is the routing tables, the sort arrays, the align
 *     workspace and moe_ffn_workspace_bytes(...), each rounded up to 256 bytes (at H =
 *     5120, I = 192, 161 experts and 9 slots: up to 609 tokens with 16-row blocks, 444
 *     with 128-row blocks).
 *   - Every call on a device shares that device's array and leaves the last call's
 *     contents there: calls that overlap in time on one device (other streams, other host
 *     threads) race. Nothing in the array needs to start at zero.
 * ------------------------------------------------------------------------- */
#define SRMOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_forward_noalloc(const uint16_t* x, const float* logits, const uint8_t* w13, const float* s13,
                              const uint8_t* w2, const float* s2, int scale_mode, int T, int H, int I, int E,
                              int K, float shared_weight, int block_m, uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Attention side of the same model: the per-head QK norm fused with the rotary
 * position embedding (intelliparadigm section 2.2; Optimizing GLM4-MoE for
 * production section 2: both are per-head steps, so one kernel does both; GLM4-MoE
 * rotates only part of each head).
 *
 * moe_qk_norm_rope works IN PLACE on qkv [T, (num_q_heads + 2*num_kv_heads) *
 * head_dim] bf16, the qkv projection output (per token: the q heads, the k heads,
 * the v heads). For every q and k head of token t (v heads are left untouched):
 *     y = x / sqrt(mean(x^2) + eps) * w            (w = q_norm_w or k_norm_w, [head_dim] float32)
 *     the first rotary_dim dims of y are rotated by angle(p, i) = p * theta^(-2i/rotary_dim),
 *     i < rotary_dim/2, p = positions[t]; neox != 0 pairs dim i with i + rotary_dim/2
 *     (rotate-half), neox == 0 pairs 2i with 2i+1 (interleaved); dims >= rotary_dim
 *     keep y.
 *   Float32 arithmetic, one bf16 rounding (round to nearest even) per value.
 *   fused == 0 runs the two steps as two passes with y stored as bf16 in between (the
 *   unfused form, for comparison).
 *   positions [T] int32; a position outside [0, max_pos) is clamped into it.
 *   cos_sin [max_pos, rotary_dim] float32: for each position rotary_dim/2 cosines
 *   then rotary_dim/2 sines, as written by moe_rope_cos_sin_table.
 *   limits: head_dim in {64, 128, 256}; rotary_dim a power of two, 16 <= rotary_dim
 *   <= head_dim; num_q_heads + 2*num_kv_heads <= 1024; eps >= 0.
 *   q_norm_w may be NULL when num_q_heads == 0, k_norm_w when num_kv_heads == 0.
 * ------------------------------------------------------------------------- */
int moe_qk_norm_rope(uint16_t* qkv, int T, int num_q_heads, int num_kv_heads, int head_dim, int rotary_dim,
                     int neox, const float* q_norm_w, const float* k_norm_w, float eps,
                     const int32_t* positions, const float* cos_sin, int max_pos, int fused, void* stream);
/* cos_sin [max_pos, rotary_dim] float32 (device, written): cos_sin[p][i] = cos(a),
 * cos_sin[p][rotary_dim/2 + i] = sin(a), a = p * theta^(-2i/rotary_dim), i < rotary_dim/2;
 * computed in float64 and rounded to float32. rotary_dim even, theta > 1. */
int moe_rope_cos_sin_table(float* cos_sin, int max_pos, int rotary_dim, double theta, void* stream);

/* Host helpers. */
size_t moe_sorted_capacity(int T, int K1, int E1, int block_m); /* P_max, rows */
size_t moe_align_workspace_bytes(int T, int K1, int E1);
size_t moe_ffn_workspace_bytes(int T, int H, int I, int E1, int K1, int block_m, int scale_mode);
/* Byte offsets inside the FFN workspace (host): out[0] slot_out [T*K1,H] bf16 (always 0;
 * followed by one scratch row of H that padding rows are written to),
 * out[1] x_q [T,H] e4m3, out[2] x scales, out[3] a [P_max,I] float32 (sorted-row order),
 * out[4] a_q [P_max,I] e4m3, out[5] a scales, out[6] per-row output scales [P_max] float32,
 * out[7] total. For inspecting the stages; returns SRMOE_OK or SRMOE_ERR_INVALID_ARG /
 * SRMOE_ERR_UNSUPPORTED for bad shapes. */
int moe_ffn_workspace_offsets(int T, int H, int I, int E1, int K1, int block_m, int scale_mode,
                              size_t* out /* host, 8 entries */);
/* Bytes of ONE device workspace that serves moe_align_by_expert, moe_fused_ffn (and its
 * stages) and moe_combine for these sizes: the larger of moe_align_workspace_bytes and
 * moe_ffn_workspace_bytes (0 for an unsupported shape). The same buffer may be passed to all
 * of them, and as both align_ws and ffn_ws of moe_layer_forward: align's scratch is dead
 * once it returns, before the FFN writes there (calls on one stream run in order). */
size_t moe_workspace_bytes(int T, int H, int I, int E1, int K1, int block_m, int scale_mode);
/* Text of a status code (static storage). srmoe_status_string is the same function. */
const char* moe_status_string(int status);
const char* srmoe_status_string(int status);
int srmoe_last_hip_error(void); /* hipError_t of this thread's last failed launch, 0 if none */
/* Build stamp: 16 hex digits of the sha256 over the csrc and include sources the library was
 * compiled from (shared_routed_expert_amd/build.py, source_hash), or "unstamped" for a build
 * that did not set it. Static storage, never null. The Python binding refuses to load a
 * library whose stamp differs from the sources beside it. */
const char* srmoe_source_hash(void);

#ifdef __cplusplus
}
#endif
#endif /* SRMOE_H_ */
