/*
 * fp64 CPU oracle of the Gated DeltaNet (GDN) single-token decode step.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may call this file. It shares no code, header, table or helper with
 * the HIP library; the library never loads it.
 *
 * What it computes, per sequence and decode step, in the order of the page
 * "linear_attention.rs" (spark_model/forward/qwen3_5), forward_linear_attention:
 *   step 3  fused causal conv1d update over the rolled per-channel state, SiLU, then
 *           a per-head L2 norm on Q and K (V gets SiLU only); l2_eps is 1e-6 there.
 *           The state layout [K-1][C], rolled in place, is the one the page "ple.rs"
 *           documents for ple_conv.
 *   step 4  gate  alpha = exp(softplus(dt + dt_bias) * -exp(A_log)), one per v-head.
 *   step 5  beta  = sigmoid(b_raw), one per v-head.
 *   step 6  qkv split: Q | K | V, consecutive in the channel axis.
 *   step 7  gated_delta_rule_decode (state, q, k, v, gate, beta -> y). The page shows
 *           only the call; the rule is the published gated delta rule of Gated
 *           DeltaNet (Yang, Kautz, Hatamizadeh, ICLR 2025):
 *               S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *               o_t = S_t q_t,
 *           with the 1/sqrt(d) factor applied at the kernel output (the comment after
 *           step 3 on the same page).
 *   step 8  per-head RMSNorm of y over d_v with the one norm_weight vector.
 *   steps 9-11  the gate silu(z) (.) y_norm that feeds out_proj (out_proj itself is
 *           a trained-weight GEMV and not part of this oracle).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - state H is stored [d_k][d_v] per head, d_v contiguous; S = H^T, so
 *     m_j = sum_i H[i][j] k_i and o_j = sum_i H[i][j] q_i / sqrt(d_k);
 *   - conv tap K-1 multiplies the current token, row 0 of the conv state is the
 *     oldest token, no conv bias (the page passes none);
 *   - L2 norm is x / sqrt(sum x^2 + eps);
 *   - RMSNorm is x * w / sqrt(mean x^2 + eps), eps = rms_eps argument;
 *   - v-head h reads k-head floor(h / G), G = H_v / H_k;
 *   - the readout uses the updated state.
 *
 * Arithmetic is double throughout; every float input is widened exactly. Loops run
 * in ascending index order. OpenMP only distributes independent (sequence, k-head)
 * units; each unit's arithmetic is the same with any thread count.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdn_oracle_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

static double silu(double u) { return u / (1.0 + exp(-u)); }

/* softplus(x) = log(1 + e^x), written in a form that does not overflow. */
static double softplus(double x) { return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x))); }

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Channel index of element i of the Q / K segment of k-head g, and of the V segment
 * of v-head h (page "linear_attention.rs", step 6: Q | K | V). */
static long q_chan(const gdn_oracle_shape* s, int g, int i) { return (long)g * s->head_k_dim + i; }
static long k_chan(const gdn_oracle_shape* s, int g, int i) {
  return (long)s->num_k_heads * s->head_k_dim + (long)g * s->head_k_dim + i;
}
static long v_chan(const gdn_oracle_shape* s, int h, int j) {
  return 2L * s->num_k_heads * s->head_k_dim + (long)h * s->head_v_dim + j;
}

static long n_channels(const gdn_oracle_shape* s) {
  return 2L * s->num_k_heads * s->head_k_dim + (long)s->num_v_heads * s->head_v_dim;
}

/* Step 3 for one channel of one sequence: conv over (state rows, current input),
 * SiLU, then roll the state by one token. Returns silu(u). */
static double conv_channel(const gdn_oracle_shape* s, double* conv_state, const float* qkv,
                           const float* conv_w, long c) {
  const int K = s->conv_kernel;
  const long C = n_channels(s);
  double u = 0.0;
  for (int j = 0; j < K; ++j) {
    double x = (j < K - 1) ? conv_state[(long)j * C + c] : (double)qkv[c];
    u += (double)conv_w[c * K + j] * x;
  }
  for (int j = 0; j + 1 < K - 1; ++j) conv_state[(long)j * C + c] = conv_state[(long)(j + 1) * C + c];
  conv_state[(long)(K - 2) * C + c] = (double)qkv[c];
  return silu(u);
}

/* Step 3 for the channels of k-head g of one sequence: q, k of head g and v of the
 * G v-heads that read it; q and k are then L2-normalised. Writes act[C]. */
static void conv_unit(const gdn_oracle_shape* s, int g, double* conv_state, const float* qkv,
                      const float* conv_w, double* act) {
  const int dk = s->head_k_dim, dv = s->head_v_dim;
  const int G = s->num_v_heads / s->num_k_heads;
  for (int i = 0; i < dk; ++i) act[q_chan(s, g, i)] = conv_channel(s, conv_state, qkv, conv_w, q_chan(s, g, i));
  for (int i = 0; i < dk; ++i) act[k_chan(s, g, i)] = conv_channel(s, conv_state, qkv, conv_w, k_chan(s, g, i));
  for (int h = g * G; h < (g + 1) * G; ++h)
    for (int j = 0; j < dv; ++j) act[v_chan(s, h, j)] = conv_channel(s, conv_state, qkv, conv_w, v_chan(s, h, j));
  double sq = 0.0, sk = 0.0;
  for (int i = 0; i < dk; ++i) {
    sq += act[q_chan(s, g, i)] * act[q_chan(s, g, i)];
    sk += act[k_chan(s, g, i)] * act[k_chan(s, g, i)];
  }
  const double rq = 1.0 / sqrt(sq + s->l2_eps), rk = 1.0 / sqrt(sk + s->l2_eps);
  for (int i = 0; i < dk; ++i) {
    act[q_chan(s, g, i)] *= rq;
    act[k_chan(s, g, i)] *= rk;
  }
}

/* Steps 4, 5 and 7 for v-head h of one sequence. act holds the normalised q, k and
 * the v of this sequence; H is the head's [d_k][d_v] state, updated in place. */
static void recurrence_head(const gdn_oracle_shape* s, int h, double* H, const double* act,
                            const float* dt_raw, const float* b_raw, const float* A_log,
                            const float* dt_bias, double* o, double* alpha_out, double* beta_out) {
  const int dk = s->head_k_dim, dv = s->head_v_dim;
  const int g = h / (s->num_v_heads / s->num_k_heads);
  const double alpha = exp(-exp((double)A_log[h]) * softplus((double)dt_raw[h] + (double)dt_bias[h]));
  const double beta = sigmoid((double)b_raw[h]);
  if (alpha_out) alpha_out[h] = alpha;
  if (beta_out) beta_out[h] = beta;
  double* m = (double*)calloc((size_t)dv, sizeof(double));
  /* m = H^T k: what the state currently returns for key k */
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) m[j] += H[(long)i * dv + j] * act[k_chan(s, g, i)];
  /* delta rule: H <- alpha H + k (beta (v - alpha m))^T */
  for (int j = 0; j < dv; ++j) m[j] = beta * (act[v_chan(s, h, j)] - alpha * m[j]);
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j)
      H[(long)i * dv + j] = alpha * H[(long)i * dv + j] + act[k_chan(s, g, i)] * m[j];
  /* readout of the updated state, scaled by 1/sqrt(d_k) */
  for (int j = 0; j < dv; ++j) o[(long)h * dv + j] = 0.0;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) o[(long)h * dv + j] += H[(long)i * dv + j] * act[q_chan(s, g, i)];
  const double scale = 1.0 / sqrt((double)dk);
  for (int j = 0; j < dv; ++j) o[(long)h * dv + j] *= scale;
  free(m);
}

/* Step 8 and the silu(z) gate of steps 9-11 for v-head h of one sequence. */
static void gated_norm_head(const gdn_oracle_shape* s, int h, const double* o, const float* z,
                            const float* norm_w, double* y_norm, double* out) {
  const int dv = s->head_v_dim;
  double ms = 0.0;
  for (int j = 0; j < dv; ++j) ms += o[(long)h * dv + j] * o[(long)h * dv + j];
  ms /= (double)dv;
  const double r = 1.0 / sqrt(ms + s->rms_eps);
  for (int j = 0; j < dv; ++j) {
    const long e = (long)h * dv + j;
    const double yn = o[e] * r * (double)norm_w[j];
    if (y_norm) y_norm[e] = yn;
    out[e] = yn * silu((double)z[e]);
  }
}

int gdn_oracle_check_shape(const gdn_oracle_shape* s) {
  if (!s) return -1;
  if (s->batch < 0 || s->num_k_heads <= 0 || s->num_v_heads <= 0 || s->head_k_dim <= 0 ||
      s->head_v_dim <= 0 || s->conv_kernel < 2)
    return -2;
  if (s->num_v_heads % s->num_k_heads != 0) return -2;
  return 0;
}

void gdn_oracle_conv_update(const gdn_oracle_shape* s, double* conv_state, const float* qkv,
                            const float* conv_w, double* qkv_act) {
  const long C = n_channels(s);
  const long cs_stride = (long)(s->conv_kernel - 1) * C;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < s->batch; ++b)
    for (int g = 0; g < s->num_k_heads; ++g)
      conv_unit(s, g, conv_state + b * cs_stride, qkv + b * C, conv_w, qkv_act + b * C);
}

void gdn_oracle_recurrent_step(const gdn_oracle_shape* s, double* state, const double* qkv_act,
                               const float* dt_raw, const float* b_raw, const float* A_log,
                               const float* dt_bias, double* o, double* alpha, double* beta) {
  const long C = n_channels(s);
  const int Hv = s->num_v_heads;
  const long hs = (long)s->head_k_dim * s->head_v_dim;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < s->batch; ++b)
    for (int h = 0; h < Hv; ++h)
      recurrence_head(s, h, state + ((long)b * Hv + h) * hs, qkv_act + b * C, dt_raw + (long)b * Hv,
                      b_raw + (long)b * Hv, A_log, dt_bias, o + (long)b * Hv * s->head_v_dim,
                      alpha ? alpha + (long)b * Hv : NULL, beta ? beta + (long)b * Hv : NULL);
}

void gdn_oracle_gated_rmsnorm(const gdn_oracle_shape* s, const double* o, const float* z,
                              const float* norm_w, double* y_norm, double* out) {
  const int Hv = s->num_v_heads;
  const long zd = (long)Hv * s->head_v_dim;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < s->batch; ++b)
    for (int h = 0; h < Hv; ++h)
      gated_norm_head(s, h, o + b * zd, z + b * zd, norm_w, y_norm ? y_norm + b * zd : NULL, out + b * zd);
}

/* One token of one (sequence, k-head) unit: step 3 for the unit's channels, then
 * steps 4-11 for each v-head that reads k-head g. */
static void decode_unit(const gdn_oracle_shape* s, int g, double* conv_state, double* state_b,
                        const float* qkv, const float* conv_w, const float* dt_raw,
                        const float* b_raw, const float* z, const float* A_log,
                        const float* dt_bias, const float* norm_w, double* act, double* o,
                        double* out) {
  const int G = s->num_v_heads / s->num_k_heads;
  const long hs = (long)s->head_k_dim * s->head_v_dim;
  conv_unit(s, g, conv_state, qkv, conv_w, act);
  for (int h = g * G; h < (g + 1) * G; ++h) {
    recurrence_head(s, h, state_b + h * hs, act, dt_raw, b_raw, A_log, dt_bias, o, NULL, NULL);
    gated_norm_head(s, h, o, z, norm_w, NULL, out);
  }
}

void gdn_oracle_decode_step(const gdn_oracle_shape* s, double* conv_state, double* state,
                            const float* qkv, const float* conv_w, const float* dt_raw,
                            const float* b_raw, const float* z, const float* A_log,
                            const float* dt_bias, const float* norm_w, double* out) {
  gdn_oracle_sequence(s, 1, conv_state, state, qkv, conv_w, dt_raw, b_raw, z, A_log, dt_bias,
                      norm_w, out);
}

void gdn_oracle_sequence(const gdn_oracle_shape* s, int T, double* conv_state, double* state,
                         const float* qkv, const float* conv_w, const float* dt_raw,
                         const float* b_raw, const float* z, const float* A_log,
                         const float* dt_bias, const float* norm_w, double* out) {
  const long C = n_channels(s);
  const int Hv = s->num_v_heads;
  const long zd = (long)Hv * s->head_v_dim;
  const long cs_stride = (long)(s->conv_kernel - 1) * C;
  const long st_stride = (long)Hv * s->head_k_dim * s->head_v_dim;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < s->batch; ++b)
    for (int g = 0; g < s->num_k_heads; ++g) {
      double* act = (double*)calloc((size_t)C, sizeof(double));
      double* o = (double*)calloc((size_t)zd, sizeof(double));
      for (int t = 0; t < T; ++t) {
        const long bt = (long)b * T + t;
        decode_unit(s, g, conv_state + b * cs_stride, state + b * st_stride, qkv + bt * C, conv_w,
                    dt_raw + bt * Hv, b_raw + bt * Hv, z + bt * zd, A_log, dt_bias, norm_w, act, o,
                    out + bt * zd);
      }
      free(act);
      free(o);
    }
}

/* Page "linear_attention.rs", step 2 (in_proj_qkv, in_proj_z, in_proj_a, in_proj_b:
 * x_norm -> qkv, z, dt_raw, b_raw) and steps 9-11 (out_proj applied to the gated
 * output): each is a matrix-vector product per row. Sum in ascending k. */
void gdn_oracle_linear(int M, int N, int K, const float* x, const float* w, double* y) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += (double)x[(long)m * K + k] * (double)w[(long)n * K + k];
      y[(long)m * N + n] = acc;
    }
}
