/*
 * fp64 CPU oracle of the GDN decode step: declarations. TEST INFRASTRUCTURE, not part
 * of the library; see gdn_oracle.c for what each function follows.
 *
 * Layouts (row-major, per sequence b):
 *   conv_state [B][K-1][C]   row 0 = oldest token; updated in place (double)
 *   state      [B][H_v][d_k][d_v]  updated in place (double)
 *   qkv        [B][C]        C = 2*H_k*d_k + H_v*d_v, Q | K | V  (float, exact values)
 *   conv_w     [C][K]        tap K-1 multiplies the current token
 *   dt_raw, b_raw [B][H_v]; A_log, dt_bias [H_v]; norm_w [d_v]; z [B][H_v*d_v]
 *   qkv_act    [B][C]        silu(conv), Q and K L2-normalised
 *   o          [B][H_v][d_v] S q / sqrt(d_k) with the updated S
 *   out        [B][H_v*d_v]  rmsnorm(o) * norm_w * silu(z)
 * A sequence call takes qkv [B][T][C], dt_raw/b_raw [B][T][H_v], z and out
 * [B][T][H_v*d_v].
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int batch, num_k_heads, num_v_heads, head_k_dim, head_v_dim, conv_kernel;
  double l2_eps, rms_eps;
} gdn_oracle_shape;

int gdn_oracle_check_shape(const gdn_oracle_shape* s);

/* Sets the OpenMP thread count when n > 0; returns the count in use. */
int gdn_oracle_threads(int n);

void gdn_oracle_conv_update(const gdn_oracle_shape* s, double* conv_state, const float* qkv,
                            const float* conv_w, double* qkv_act);

void gdn_oracle_recurrent_step(const gdn_oracle_shape* s, double* state, const double* qkv_act,
                               const float* dt_raw, const float* b_raw, const float* A_log,
                               const float* dt_bias, double* o, double* alpha, double* beta);

void gdn_oracle_gated_rmsnorm(const gdn_oracle_shape* s, const double* o, const float* z,
                              const float* norm_w, double* y_norm, double* out);

void gdn_oracle_decode_step(const gdn_oracle_shape* s, double* conv_state, double* state,
                            const float* qkv, const float* conv_w, const float* dt_raw,
                            const float* b_raw, const float* z, const float* A_log,
                            const float* dt_bias, const float* norm_w, double* out);

void gdn_oracle_sequence(const gdn_oracle_shape* s, int T, double* conv_state, double* state,
                         const float* qkv, const float* conv_w, const float* dt_raw,
                         const float* b_raw, const float* z, const float* A_log,
                         const float* dt_bias, const float* norm_w, double* out);

/* Dense projection y[m][n] = sum_k x[m][k] w[n][k] in fp64 (x [M][K], w [N][K], exact
 * float values; y [M][N]): the in_proj_* GEMVs of step 2 and the out_proj GEMV of steps
 * 9-11 of "linear_attention.rs", one GEMV per row m. */
void gdn_oracle_linear(int M, int N, int K, const float* x, const float* w, double* y);

#ifdef __cplusplus
}
#endif
#endif
