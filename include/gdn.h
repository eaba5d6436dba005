/*
 * gdn.h - C ABI of libgdn.so, the MI355X (gfx950) Gated DeltaNet decode path.
 *
 * The operations are the GDN (linear-attention) layer steps of the page
 * "linear_attention.rs" (spark_model/forward/qwen3_5, forward_linear_attention):
 *   step 3    fused causal_conv1d_update + SiLU + per-head L2 norm of Q and K
 *   steps 4-5 gate alpha = exp(softplus(dt + dt_bias) * -exp(A_log)), beta = sigmoid(b)
 *   step 6    qkv split into Q | K | V
 *   step 7    gated_delta_rule_decode: per v-head state update and readout
 *   step 8    per-head RMSNorm of the readout with one norm_weight vector of d_v
 *   steps 9-11  silu(z) (.) y_norm, the gated input of out_proj (out_proj itself is
 *             not part of this library)
 * The delta rule of step 7 is the published gated delta rule (Gated DeltaNet):
 *   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t / sqrt(d_k).
 * The conv state is rolled in place, the convention the page "ple.rs" documents for
 * ple_conv, so one call serves decode (T = 1) and multi-token input (T > 1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every buffer pointer is a DEVICE pointer (HIP device memory of the current
 *   device), owned by the caller; the library allocates no memory and keeps no state
 *   between calls. The shape struct is a HOST pointer, read during the call only.
 * Stream: `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *   work and return; results are ready when the stream is synchronised.
 * Layouts (row-major, C order; B = batch, C = 2*H_k*d_k + H_v*d_v channels):
 *   conv1d_state  [B][K-1][C]   act dtype; row 0 = oldest token; read and rolled in place
 *   state         [B][H_v][d_k][d_v] fp32, d_v contiguous: H[i][j] with S = H^T, so the
 *                 readout is o_j = sum_i H[i][j] q_i / sqrt(d_k); updated in place
 *   qkv           [B][C] act dtype: Q of k-head g at g*d_k, K at H_k*d_k + g*d_k, V of
 *                 v-head h at 2*H_k*d_k + h*d_v (step 6)
 *   conv1d_weight [C][K] act dtype: tap K-1 multiplies the current token; no bias
 *   dt_raw, b_raw [B][H_v] act dtype (one per v-head, steps 4-5)
 *   z             [B][H_v*d_v] act dtype
 *   A_log, dt_bias [H_v] fp32; norm_weight [d_v] fp32
 *   v-head h reads the Q/K of k-head h / G, G = H_v / H_k (consecutive v-heads share).
 * Validation: every argument is checked on the host before anything is enqueued; on any
 *   error the call returns a negative gdn_status_t and writes nothing.
 *   - NULL buffer pointers -> GDN_ERR_NULL (allowed only when batch, or T, is 0)
 *   - batch < 0, heads < 1, H_v % H_k != 0, K outside [2, 8], eps < 0 or not finite,
 *     T < 0, grid too large, or (gdn_sequence, since ABI 1.4) B x T times the largest
 *     token row of qkv, z or out above 2^62 bytes -> GDN_ERR_SHAPE
 *   - act_dtype / out_dtype not a gdn_dtype_t -> GDN_ERR_DTYPE
 *   - qkv, conv1d_state, state, conv1d_weight, z, qkv_act, y, out not 16-byte aligned,
 *     or another buffer not aligned to its element size -> GDN_ERR_ALIGN
 *   - a buffer the call writes overlaps any other buffer of the call -> GDN_ERR_ALIAS
 *   - head dims without a compiled kernel (supported: d_k == d_v in {32, 64, 128})
 *     -> GDN_ERR_UNSUPPORTED
 *   - the HIP runtime rejects the launch -> GDN_ERR_HIP (kernels may already be queued
 *     for an earlier part of the call only in gdn_sequence's multi-launch path).
 *   Faults inside a kernel surface asynchronously at the caller's next synchronisation.
 * Concurrency: calls on one stream are ordered; two calls that touch the same state
 *   buffers on different streams race. Within one call every conv-state channel and
 *   every state element is read and written by exactly one workgroup.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype_t;

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,
  GDN_ERR_SHAPE = -2,
  GDN_ERR_DTYPE = -3,
  GDN_ERR_ALIGN = -4,
  GDN_ERR_ALIAS = -5,
  GDN_ERR_WORKSPACE = -6,
  GDN_ERR_UNSUPPORTED = -7,
  GDN_ERR_HIP = -8
} gdn_status_t;

/* Layer shape and precision, named after the config fields of the page
 * "linear_attention.rs" (k_head_dim_lin, v_head_dim_lin, num_k_heads_lin,
 * num_v_heads_lin, conv_kernel_size, rms_eps) plus the step-3 l2_eps. */
typedef struct {
  int32_t batch;       /* B: independent sequences (>= 0; 0 is a no-op) */
  int32_t num_k_heads; /* H_k */
  int32_t num_v_heads; /* H_v, a multiple of H_k */
  int32_t head_k_dim;  /* d_k */
  int32_t head_v_dim;  /* d_v */
  int32_t conv_kernel; /* K taps, 2..8 */
  float l2_eps;        /* epsilon of the Q/K L2 norm: q / sqrt(sum q^2 + l2_eps); 1e-6 on the page */
  float rms_eps;       /* epsilon of the per-head RMSNorm: o / sqrt(mean o^2 + rms_eps) */
  int32_t act_dtype;   /* gdn_dtype_t of qkv, z, dt_raw, b_raw, conv1d_weight, conv1d_state */
  int32_t out_dtype;   /* gdn_dtype_t of y / out (GDN_F32 keeps full precision) */
} gdn_shape_t;

/* Step 3 alone ("linear_attention.rs", step 3: fused causal_conv1d_update_l2norm).
 * For every sequence and channel c: u = sum_j conv1d_weight[c][j] * w_j over the window
 * w = (conv1d_state rows 0..K-2, qkv[c]), a = silu(u); Q and K segments of each k-head
 * are then divided by sqrt(sum a^2 + l2_eps); V keeps silu(u). The conv state is rolled
 * in place (rows shift up one, row K-2 <- qkv, bit-exact copy).
 * Writes qkv_act [B][C] fp32 (device). */
gdn_status_t gdn_conv_update(const gdn_shape_t* shape, void* conv1d_state, const void* qkv,
                             const void* conv1d_weight, float* qkv_act, void* stream);

/* Steps 4, 5 and 7 ("linear_attention.rs", steps 4-7: gdn_gate, sigmoid,
 * gated_delta_rule_decode). Reads qkv_act [B][C] fp32 as written by gdn_conv_update
 * (Q and K already unit-normalised). Per (b, v-head h): alpha, beta from dt_raw, b_raw,
 * A_log, dt_bias; m = H^T k; H <- alpha H + k (beta (v - alpha m))^T (in place);
 * y = H^T q / sqrt(d_k) with the updated H, written as y [B][H_v][d_v] in out_dtype. */
gdn_status_t gdn_recurrent_step(const gdn_shape_t* shape, float* state, const float* qkv_act,
                                const void* dt_raw, const void* b_raw, const float* A_log,
                                const float* dt_bias, void* y, void* stream);

/* One fused decode step, steps 3-11 of "linear_attention.rs" up to (excluding) the
 * out_proj GEMV: conv update, gates, delta-rule update and readout, then
 * out = y / sqrt(mean_j y_j^2 + rms_eps) * norm_weight * silu(z) per v-head.
 * conv1d_state and state are updated in place; out is [B][H_v*d_v] in out_dtype.
 * Each state element is read once and written once. */
gdn_status_t gdn_decode_layer(const gdn_shape_t* shape, void* conv1d_state, float* state,
                              const void* qkv, const void* conv1d_weight, const void* dt_raw,
                              const void* b_raw, const void* z, const float* A_log,
                              const float* dt_bias, const float* norm_weight, void* out,
                              void* stream);

/* gdn_decode_layer with intermediate taps, for staged debugging: the same step (states
 * updated in place, out written), plus the intermediates that the page
 * "linear_attention.rs" can dump after its optional stream synchronisation (the
 * intra-layer dump at the end of forward_linear_attention: the smoothed qkv, the gates,
 * y and y_norm). Every tap is optional (NULL: not written), fp32, device, and must not
 * overlap another buffer:
 *   qkv_act_tap [B][C]          q and k after the L2 norms, v after SiLU (step 3)
 *   alpha_tap, beta_tap [B][H_v] the gates of steps 4-5
 *   y_tap      [B][H_v][d_v]    the readout y = S q / sqrt(d_k) (step 7)
 *   y_norm_tap [B][H_v][d_v]    y / sqrt(mean y^2 + rms_eps) * norm_weight (step 8,
 *                               before the silu(z) gate of steps 9-11)
 * y_tap and y_norm_tap must be 16-byte aligned, the others 4-byte. The step runs on the
 * shape-generic kernel (slower than gdn_decode_layer; for tests and debugging), with
 * the same validation and errors as gdn_decode_layer. */
gdn_status_t gdn_decode_layer_debug(const gdn_shape_t* shape, void* conv1d_state, float* state,
                                    const void* qkv, const void* conv1d_weight, const void* dt_raw,
                                    const void* b_raw, const void* z, const float* A_log,
                                    const float* dt_bias, const float* norm_weight, void* out,
                                    float* qkv_act_tap, float* alpha_tap, float* beta_tap,
                                    float* y_tap, float* y_norm_tap, void* stream);

/* gdn_decode_layer for a batch whose states live in a pool (continuous batching).
 * For callers that keep one state slot per live sequence and run a changing subset
 * of them each step. Sequence b of the batch (its qkv, dt_raw, b_raw and z rows, and
 * its out row) uses the conv state and recurrent state of pool slot slots[b]:
 *   slots           [B] int32 (device): slot per sequence; a value outside
 *                   [0, pool_size) marks an inactive sequence. Its slot is not touched
 *                   and its out row is not written.
 *   conv1d_state_pool [pool_size][K-1][C] act dtype, state_pool
 *                   [pool_size][H_v][d_k][d_v] fp32; active slots are updated in place.
 * The arithmetic is the same as gdn_decode_layer's. Two active sequences of one call
 * must not share a slot: their updates would race (slot values are device data and
 * are not checked on the host). Validation and errors are as for gdn_decode_layer,
 * plus pool_size < 0 -> GDN_ERR_SHAPE. */
gdn_status_t gdn_decode_layer_pooled(const gdn_shape_t* shape, int32_t pool_size, const int32_t* slots,
                                     void* conv1d_state_pool, float* state_pool, const void* qkv,
                                     const void* conv1d_weight, const void* dt_raw, const void* b_raw,
                                     const void* z, const float* A_log, const float* dt_bias,
                                     const float* norm_weight, void* out, void* stream);

/* T consecutive tokens of gdn_decode_layer per sequence, with both states carried
 * from token to token (the rolled conv state of "ple.rs" serves prefill and decode
 * alike). Inputs are [B][T][...]: qkv [B][T][C], dt_raw and b_raw [B][T][H_v],
 * z [B][T][H_v*d_v]; out is [B][T][H_v*d_v]. Equal, up to rounding, to T calls of
 * gdn_decode_layer. `workspace` (device, may be NULL when the query returns 0) must
 * hold gdn_sequence_workspace_bytes(shape, T) bytes -> else GDN_ERR_WORKSPACE.
 * With d_k = d_v = 128 and K = 4 the tokens go in chunks of 32 through the chunked form
 * of the rule on the matrix cores once T reaches 6, 10 or 14 tokens (B x H_v fitting one,
 * two or more passes over the device's compute units), with every operand split into
 * two fp16 halves (22 significant bits): the recurrent state and the per-token deltas
 * must stay below the fp16 range (6.5e4 in magnitude; the layer's values are orders of
 * magnitude smaller). The state and the deltas are split unscaled, so their low halves
 * can fall in fp16's subnormal range: with fp32 activations this form agrees with the
 * fp64 recurrence to about 2e-5 relative, where the token-by-token path reaches about
 * 1e-6. Shorter sequences and other shapes run token by token in fp32. Since the choice
 * depends on T and on B x H_v, the same sequence may be evaluated at either precision
 * (and to different bits) at a different batch size. */
gdn_status_t gdn_sequence(const gdn_shape_t* shape, int32_t T, void* conv1d_state, float* state,
                          const void* qkv, const void* conv1d_weight, const void* dt_raw,
                          const void* b_raw, const void* z, const float* A_log,
                          const float* dt_bias, const float* norm_weight, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes gdn_sequence needs for this shape and T (0 if none; SIZE_MAX if the
 * shape or T is invalid, the 2^62-byte bound included). Host-only, no HIP call. */
size_t gdn_sequence_workspace_bytes(const gdn_shape_t* shape, int32_t T);

/* Speculative decoding: verify T draft tokens, then commit the accepted prefix.
 * The page "glm5next_dsa/layer.rs" (decode_k, and its lockstep check of the indexer
 * cache) decodes k tokens per call and rewinds its caches past a rejected draft. A recurrent state cannot be
 * rewound, so verification leaves both states untouched and records, per token, the
 * rank-one update of the delta rule (step 7 of "linear_attention.rs"):
 *   H_t = alpha_t H_{t-1} + k_t delta_t^T,  delta_t = beta_t (v_t - alpha_t H_{t-1}^T k_t),
 * from which the commit rebuilds the state after any accepted prefix with one read
 * and one write of the state.
 *
 * Trail (device, caller-owned, fp32; gdn_verify_trail_bytes(shape, T) bytes): delta
 * [B][T][H_v][d_v], then unit-norm k [B][T][H_k][d_k], then alpha [B][T][H_v]. */
#define GDN_MAX_VERIFY_TOKENS 8

/* Trail bytes for this shape and T (SIZE_MAX if the shape is invalid or T is outside
 * [0, GDN_MAX_VERIFY_TOKENS]). Host-only, no HIP call. */
size_t gdn_verify_trail_bytes(const gdn_shape_t* shape, int32_t T);

/* T draft tokens per sequence (0 <= T <= GDN_MAX_VERIFY_TOKENS, else GDN_ERR_SHAPE),
 * inputs [B][T][...] as for gdn_sequence. out [B][T][H_v*d_v] receives, for every draft
 * token, what gdn_sequence would give (up to rounding) from the current states; the
 * states conv1d_state and state are only read. trail_bytes < the query's value ->
 * GDN_ERR_WORKSPACE. Any H_v / H_k and K. */
gdn_status_t gdn_decode_verify(const gdn_shape_t* shape, int32_t T, const void* conv1d_state,
                               const float* state, const void* qkv, const void* conv1d_weight,
                               const void* dt_raw, const void* b_raw, const void* z,
                               const float* A_log, const float* dt_bias, const float* norm_weight,
                               void* out, void* trail, size_t trail_bytes, void* stream);

/* Advance each sequence b by its first n = accepted[b] draft tokens of the preceding
 * gdn_decode_verify call (same shape, T, qkv and trail): the state becomes the state
 * after those n tokens (the recorded updates H <- alpha_t H + k_t delta_t^T replayed in
 * order, with the deltas verify formed its outputs from) and the conv state is rolled
 * by n tokens (bit-exact copies of the draft's qkv rows).
 * accepted: [B] int32 (device). n = 0 leaves the sequence untouched, and so does a
 * value outside [0, T] (device data, not checked on the host). qkv and trail are read,
 * conv1d_state and state updated in place. */
gdn_status_t gdn_decode_commit(const gdn_shape_t* shape, int32_t T, const int32_t* accepted,
                               void* conv1d_state, float* state, const void* qkv, const void* trail,
                               size_t trail_bytes, void* stream);

/* The projections on either side of the layer, with caller-provided (for example
 * synthetic) weights: step 2 of "linear_attention.rs" (in_proj_qkv, in_proj_z and the
 * fused in_proj_a / in_proj_b GEMVs of x_norm) and steps 9-11 (out_proj applied to
 * silu(z) (.) y_norm, which gdn_decode_layer already writes as `out`). Each output is
 * Y[b][n] = sum_k X[b][k] W[n][k] with bf16 X and W, fp32 accumulation and one final
 * rounding to the output dtype (round to nearest even for bf16). One launch each.
 * Requirements: act_dtype == GDN_BF16 and the contraction length (hidden for
 * gdn_in_proj, H_v*d_v for gdn_out_proj) a multiple of 64, else GDN_ERR_UNSUPPORTED
 * (gdn_out_proj's hidden, its number of outputs, may be any value >= 1 since ABI 1.3);
 * hidden < 1 -> GDN_ERR_SHAPE. Alignment: 16 bytes for every buffer except dt_raw and
 * b_raw (2). Weights are row-major [outputs][inputs] (K contiguous). */

/* x_norm [B][hidden] bf16 -> qkv [B][C], z [B][H_v*d_v], dt_raw [B][H_v], b_raw
 * [B][H_v], all bf16 (the act-dtype inputs of gdn_decode_layer), with w_qkv [C][hidden],
 * w_z [H_v*d_v][hidden], w_a and w_b [H_v][hidden] (bf16). */
gdn_status_t gdn_in_proj(const gdn_shape_t* shape, int32_t hidden, const void* x_norm, const void* w_qkv,
                         const void* w_z, const void* w_a, const void* w_b, void* qkv, void* z,
                         void* dt_raw, void* b_raw, void* stream);

/* gated [B][H_v*d_v] bf16 (gdn_decode_layer's out in bf16) -> y [B][hidden] in
 * out_dtype, with w_out [hidden][H_v*d_v] bf16. */
gdn_status_t gdn_out_proj(const gdn_shape_t* shape, int32_t hidden, const void* gated, const void* w_out,
                          void* y, void* stream);

/* Static, NUL-terminated description of a status code. Host-only. */
const char* gdn_status_string(int32_t status);

/* ABI version of this header: (major << 16) | minor. Host-only. */
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
