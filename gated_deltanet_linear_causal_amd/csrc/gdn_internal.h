// Internal interface between the host side (validation, dispatch) and the HIP
// kernels of libgdn.so. Not installed; the public ABI is include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kMaxConvTaps = 8;

// Everything a kernel launch needs. Element strides are in elements of the buffer's
// own dtype. "bs" = stride between sequences, "ts" = stride between tokens.
struct KernelArgs {
  int B, Hk, Hv, G, K, C, T;
  float l2_eps, rms_eps;
  int act_bf16, out_bf16;
  int stream_state;        // 1: state accesses marked non-temporal (state larger than the cache)
  const int* slots;        // [B] state-pool slot of each sequence, or null (slot = b)
  int pool;                // number of state slots; slots outside [0, pool) are skipped
  void* conv_state;        // [B][K-1][C] act dtype, in place
  float* state;            // [B][Hv][D][D] fp32, in place
  const void* qkv;         // act dtype
  const void* conv_w;      // [C][K] act dtype
  const float* qkv_act_in; // [B][C] fp32 (recurrence-only mode)
  float* qkv_act_out;      // [B][C] fp32 (conv-only mode)
  const void* dt_raw;      // act dtype
  const void* b_raw;       // act dtype
  const void* z;           // act dtype
  const float* A_log;      // [Hv]
  const float* dt_bias;    // [Hv]
  const float* norm_w;     // [D]
  void* out;               // y (recurrence-only) or gated output, out dtype
  long qkv_bs, qkv_ts;
  long ab_bs, ab_ts;
  long z_bs, z_ts;
  long out_bs, out_ts;
  // speculative verification: per-token updates of the draft, and the accepted counts
  float* trail_delta;      // [B][T][Hv][D]  delta_t of each v-head
  float* trail_k;          // [B][T][Hk][D]  unit-norm k_t of each k-head
  float* trail_alpha;      // [B][T][Hv]     alpha_t of each v-head
  const int* accepted;     // [B] tokens to commit per sequence
  // intermediate taps of a fused decode step (generic kernel only; each may be null)
  float* tap_act;          // [B][C]       q, k after the L2 norms, v after SiLU
  float* tap_alpha;        // [B][Hv]
  float* tap_beta;         // [B][Hv]
  float* tap_y;            // [B][Hv][D]   readout o = H'^T q / sqrt(d_k)
  float* tap_y_norm;       // [B][Hv][D]   o r norm_weight (before the silu(z) gate)
  int taps;                // 1: some tap is set (the launcher then takes the generic kernel)
};

enum Mode : int { kModeConv = 0, kModeRec = 1, kModeFused = 2 };

// Launchers (gdn_kernels.hip). Return the hipError_t of the launch.
// d: head dim (d_k == d_v); p: v-heads per pass (1 or 2). Grid = B * Hk workgroups.
bool step_supported(int d, int p);
hipError_t launch_step(int mode, int d, int p, const KernelArgs& a, hipStream_t stream);
// Multi-token kernel that keeps the state on chip for all T tokens, every v-head of a
// k-head resident (p == G); sequence_supported(G, K): 1 <= G <= 4 and 2 <= K <= 5.
bool sequence_supported(int G, int K);
hipError_t launch_sequence(int d, int p, const KernelArgs& a, hipStream_t stream);
// Chunked multi-token form on MFMA (gdn_chunked.hip): d == 128, K == 4, any G. One
// workgroup per (sequence, v-head); enqueues the chunk kernel and the conv-state tail.
bool chunked_supported(int d, int K);
hipError_t launch_chunked_sequence(const KernelArgs& a, hipStream_t stream);
// Speculative verification (gdn_kernels.hip): up to kMaxVerifyTokens draft tokens per
// sequence with both states read only, writing the outputs and the trail; and the
// commit of the accepted prefix (state and conv state). Grid B * Hv (any G and K).
constexpr int kMaxVerifyTokens = 8;
hipError_t launch_verify(int d, const KernelArgs& a, hipStream_t stream);
hipError_t launch_commit(int d, const KernelArgs& a, hipStream_t stream);

// Projections (gdn_proj.hip): Y_s[m][n] = sum_k X[m][k] W_s[n][k] for up to
// kMaxProjSegs weight segments sharing X; bf16 operands, fp32 accumulation.
constexpr int kMaxProjSegs = 4;
struct ProjSeg {
  const uint16_t* w;  // [n][K] bf16
  void* y;            // [M][n] fp32, or bf16 when y_bf16
  long n;             // rows of W = columns of Y
  int y_bf16;
  long row0;          // first row in the concatenation of all segments (set by launch_proj)
  int tile0;          // first column tile (set by launch_proj)
};
struct ProjArgs {
  int M, K;           // rows of X, contraction length (a multiple of 64)
  const uint16_t* x;  // [M][K] bf16
  int nseg;
  long rows;          // sum of the segments' n (set by launch_proj)
  int ntiles, mblocks;  // column tiles and row blocks of a tiled launch (set by its launcher)
  int krot;            // 1: the DMA-ring workgroups start their contraction at staggered stages
  ProjSeg seg[kMaxProjSegs];
};
hipError_t launch_proj(ProjArgs p, hipStream_t stream);

}  // namespace gdn
