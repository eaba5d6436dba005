// HIP kernels of the GDN decode path for CDNA4 (gfx950).
//
// Work unit: one workgroup per (sequence b, k-head g). It owns
//   * the conv channels of Q_g, K_g and of V for the G v-heads that read k-head g
//     (page "linear_attention.rs", step 6: v-head h reads k-head h / G), so it is the
//     only reader and the only writer of those conv-state columns and the in-place
//     roll is race-free inside one launch;
//   * the [d x d] fp32 state of each of those G v-heads, processed P heads at a time.
// The state of a pass lives in VGPRs: lane (ph, rg, cg) holds rows rg*R .. rg*R+R-1
// and columns 4cg .. 4cg+3 of head ph as R float4. Each element is read once and
// written once per step; the step is HBM-bound (~0.74 flop per byte).
// Load order matters on gfx9: vmcnt counts loads AND stores and retires in order, so
// every small input (conv window, taps, gates, z, norm weight) is loaded before the R
// 128-bit state loads. The conv / L2 prelude then only waits for its own loads while
// the state is still in flight, and nothing waits for the store drain.
// Lanes that share a column group differ only in the lane bits above log2(64/RG),
// inside one wave, so m = H^T k and p = H^T q are finished with xor shuffles.

#include <type_traits>

#include "gdn_device.h"

namespace gdn {
namespace {


// Channel of conv-unit index c for k-head g: [0, D) -> Q_g, [D, 2D) -> K_g,
// [2D, 2D + G*D) -> V of v-heads g*G .. g*G+G-1 (page "linear_attention.rs", step 6).
template <int D>
__device__ __forceinline__ long unit_channel(int c, int g, int Hk, int G) {
  if (c < D) return static_cast<long>(g) * D + c;
  if (c < 2 * D) return static_cast<long>(Hk) * D + static_cast<long>(g) * D + (c - D);
  return 2L * Hk * D + static_cast<long>(g) * G * D + (c - 2 * D);
}

// Conv taps of channel gc: K consecutive elements of conv_w[gc][*].
template <bool BF, int KT>
__device__ __forceinline__ void load_taps(const void* w, long gc, float (&wt)[KT]) {
  if constexpr (KT == 4) {
    const float4 v = Act<BF>::load4(w, gc * 4);
    wt[0] = v.x;
    wt[1] = v.y;
    wt[2] = v.z;
    wt[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < KT; ++j) wt[j] = Act<BF>::load(w, gc * KT + j);
  }
}

// ----------------------------------------------------------------------------------
// Conv prelude for a fixed tap count KT and a single pass (G == P): every lane owns
// NCPL channels at fixed positions. Split into "issue loads" and "compute" so the
// loads can be placed ahead of the state loads.
// ----------------------------------------------------------------------------------
template <bool BF, int KT, int NCH, int NT, int D>
struct ConvRegs {
  static constexpr int NCPL = (NCH + NT - 1) / NT;
  using raw_t = typename Act<BF>::raw_t;
  raw_t win[NCPL][KT - 1];
  raw_t x[NCPL];
  float wt[NCPL][KT];
  long gch[NCPL];

  __device__ __forceinline__ bool owns(int m) const {
    return (NCH % NT == 0) || (static_cast<int>(threadIdx.x) + m * NT < NCH);
  }
  __device__ __forceinline__ void channels(int g, int Hk, int G) {
#pragma unroll
    for (int m = 0; m < NCPL; ++m) gch[m] = owns(m) ? unit_channel<D>(threadIdx.x + m * NT, g, Hk, G) : 0;
  }
  __device__ __forceinline__ void load_window(const void* cs, long cs_base, long C) {
#pragma unroll
    for (int m = 0; m < NCPL; ++m)
      if (owns(m)) {
#pragma unroll
        for (int j = 0; j < KT - 1; ++j) win[m][j] = Act<BF>::raw(cs, cs_base + j * C + gch[m]);
      }
  }
  __device__ __forceinline__ void load_taps_all(const void* w) {
#pragma unroll
    for (int m = 0; m < NCPL; ++m)
      if (owns(m)) load_taps<BF, KT>(w, gch[m], wt[m]);
  }
  __device__ __forceinline__ void load_x(const void* qkv, long base) {
#pragma unroll
    for (int m = 0; m < NCPL; ++m)
      if (owns(m)) x[m] = Act<BF>::raw(qkv, base + gch[m]);
  }
  // u = sum_j w_j * window_j (tap KT-1 on the current token), silu(u) into LDS.
  __device__ __forceinline__ void compute(float* s_q, float* s_k, float* s_v) {
#pragma unroll
    for (int m = 0; m < NCPL; ++m)
      if (owns(m)) {
        float u = 0.0f;
#pragma unroll
        for (int j = 0; j < KT - 1; ++j) u = fmaf(wt[m][j], Act<BF>::f(win[m][j]), u);
        u = fmaf(wt[m][KT - 1], Act<BF>::f(x[m]), u);
        const float v = silu(u);
        const int c = threadIdx.x + m * NT;
        if (c < D) s_q[c] = v;
        else if (c < 2 * D) s_k[c - D] = v;
        else s_v[c - 2 * D] = v;
      }
  }
  // shift the window by one token (registers only)
  __device__ __forceinline__ void roll() {
#pragma unroll
    for (int m = 0; m < NCPL; ++m) {
#pragma unroll
      for (int j = 0; j < KT - 2; ++j) win[m][j] = win[m][j + 1];
      win[m][KT - 2] = x[m];
    }
  }
  __device__ __forceinline__ void store_window(void* cs, long cs_base, long C) const {
#pragma unroll
    for (int m = 0; m < NCPL; ++m)
      if (owns(m)) {
#pragma unroll
        for (int j = 0; j < KT - 1; ++j) Act<BF>::put(cs, cs_base + j * C + gch[m], win[m][j]);
      }
  }
};

// Generic conv of one channel (runtime K): window loads, conv, SiLU, in-place roll.
template <bool BF>
__device__ __forceinline__ float conv_channel_generic(const KernelArgs& a, long b, long sb, long gc) {
  using raw_t = typename Act<BF>::raw_t;
  const long cs0 = sb * (a.K - 1) * static_cast<long>(a.C) + gc;
  raw_t win[kMaxConvTaps];
  for (int j = 0; j < a.K - 1; ++j) win[j] = Act<BF>::raw(a.conv_state, cs0 + static_cast<long>(j) * a.C);
  win[a.K - 1] = Act<BF>::raw(a.qkv, b * a.qkv_bs + gc);
  float u = 0.0f;
  for (int j = 0; j < a.K; ++j) u = fmaf(Act<BF>::load(a.conv_w, gc * a.K + j), Act<BF>::f(win[j]), u);
  for (int j = 0; j < a.K - 1; ++j) Act<BF>::put(a.conv_state, cs0 + static_cast<long>(j) * a.C, win[j + 1]);
  return silu(u);
}


// ----------------------------------------------------------------------------------
// One decode step, single pass (G == P) with KT conv taps. MODE: kModeConv (step 3),
// kModeRec (steps 4-7 from qkv_act), kModeFused (steps 3-11).
// Grid: B*Hk workgroups of Layout::NT lanes. LDS: q[D], k[D], v[P*D], red, hred.
// ----------------------------------------------------------------------------------
template <int D, int P, int MODE, bool BF, int KT, bool STREAM>
__global__ __launch_bounds__((Layout<D, P>::NT)) void gdn_step_fast(const KernelArgs a) {
  using L = Layout<D, P>;
  using CR = ConvRegs<BF, KT, (2 + P) * D, L::NT, D>;
  constexpr int NT = L::NT, R = L::R, CGL = L::CGL, NW = L::NW, NCPL = CR::NCPL;
  constexpr uint32_t kHeadBytes = D * D * 4, kRowBytes = D * 4;
  __shared__ __attribute__((aligned(16))) float s_q[D];
  __shared__ __attribute__((aligned(16))) float s_k[D];
  __shared__ __attribute__((aligned(16))) float s_v[P * D];
  __shared__ float red[NW * 4];
  __shared__ float hred[NW];

  const int t = threadIdx.x;
  const int b = blockIdx.x / a.Hk;
  const int g = blockIdx.x - b * a.Hk;
  const int ph = t / L::LPH;
  const int u = t - ph * L::LPH;
  const int cg = (u >> 6) * CGL + (u & (CGL - 1));
  const int rg = (u & 63) / CGL;
  const int h = g * P + ph;
  // state slot of sequence b: b itself, or a pool entry; a slot outside the pool marks
  // an inactive sequence whose workgroups do nothing (uniform per workgroup)
  const int sb = a.slots ? a.slots[b] : b;
  if (sb < 0 || sb >= a.pool) return;
  const long cs_base = static_cast<long>(sb) * (KT - 1) * a.C;

  // ---- 1. small loads first
  CR cr;
  float act_in[NCPL];
  cr.channels(g, a.Hk, P);
  if constexpr (MODE == kModeRec) {
#pragma unroll
    for (int m = 0; m < NCPL; ++m)
      if (cr.owns(m)) act_in[m] = a.qkv_act_in[static_cast<long>(b) * a.C + cr.gch[m]];
  } else {
    cr.load_window(a.conv_state, cs_base, a.C);
    cr.load_x(a.qkv, b * a.qkv_bs);
    cr.load_taps_all(a.conv_w);
  }
  float dt = 0.0f, braw = 0.0f, A_log = 0.0f, dt_bias = 0.0f;
  typename Act<BF>::raw4_t z_raw{};
  float4 w4 = f4(0.0f);
  if constexpr (MODE != kModeConv) {
    dt = Act<BF>::load(a.dt_raw, b * a.ab_bs + h);
    braw = Act<BF>::load(a.b_raw, b * a.ab_bs + h);
    A_log = a.A_log[h];
    dt_bias = a.dt_bias[h];
  }
  if constexpr (MODE == kModeFused) {
    // every lane loads (the output lanes are row group 0; the others repeat their
    // addresses): a load inside a branch is waited for at the join, which would hold
    // the state loads below until all small loads had returned
    z_raw = Act<BF>::raw4(a.z, b * a.z_bs + static_cast<long>(h) * D + 4 * cg);
    w4 = *reinterpret_cast<const float4*>(a.norm_w + 4 * cg);
  }

  // ---- 2. the state (the step's whole cost), P heads of k-head g
  const uint32_t voff = static_cast<uint32_t>(ph) * kHeadBytes + static_cast<uint32_t>(rg * R) * kRowBytes +
                        static_cast<uint32_t>(cg) * 16u;
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(a.state + (static_cast<long>(sb) * a.Hv + static_cast<long>(g) * P) * (D * D), P * kHeadBytes);
  float4 hreg[R];
  if constexpr (MODE != kModeConv) {
#pragma unroll
    for (int k = 0; k < R; ++k) hreg[k] = buf_load4<STREAM>(srs, voff, k * kRowBytes);
  }

  // ---- 3. prelude: conv + SiLU (+ roll), L2 norms of q and k
  float kq;
  if constexpr (MODE == kModeRec) {
#pragma unroll
    for (int m = 0; m < NCPL; ++m)
      if (cr.owns(m)) {
        const int c = t + m * NT;
        if (c < D) s_q[c] = act_in[m];
        else if (c < 2 * D) s_k[c - D] = act_in[m];
        else s_v[c - 2 * D] = act_in[m];
      }
    __syncthreads();
    float s1[1] = {0.0f};
    for (int i = t; i < D; i += NT) s1[0] = fmaf(s_q[i], s_k[i], s1[0]);
    block_sum<NW, 1>(s1, red);
    kq = s1[0];
  } else {
    cr.compute(s_q, s_k, s_v);
    cr.roll();
    cr.store_window(a.conv_state, cs_base, a.C);
    if constexpr (MODE == kModeConv) {
#pragma unroll
      for (int m = 0; m < NCPL; ++m)
        if (cr.owns(m) && t + m * NT >= 2 * D)
          a.qkv_act_out[static_cast<long>(b) * a.C + cr.gch[m]] = s_v[t + m * NT - 2 * D];
    }
    __syncthreads();
    float s3[3] = {0.0f, 0.0f, 0.0f};
    for (int i = t; i < D; i += NT) {
      const float q = s_q[i], k = s_k[i];
      s3[0] = fmaf(q, q, s3[0]);
      s3[1] = fmaf(k, k, s3[1]);
      s3[2] = fmaf(q, k, s3[2]);
    }
    block_sum<NW, 3>(s3, red);
    const float rq = 1.0f / sqrtf(s3[0] + a.l2_eps);
    const float rk = 1.0f / sqrtf(s3[1] + a.l2_eps);
    kq = s3[2] * rq * rk;
    for (int i = t; i < D; i += NT) {
      const float qn = s_q[i] * rq, kn = s_k[i] * rk;
      if constexpr (MODE == kModeConv) {
        float* act = a.qkv_act_out + static_cast<long>(b) * a.C;
        act[static_cast<long>(g) * D + i] = qn;
        act[static_cast<long>(a.Hk) * D + static_cast<long>(g) * D + i] = kn;
      } else {
        s_q[i] = qn;
        s_k[i] = kn;
      }
    }
    if constexpr (MODE == kModeConv) return;
    __syncthreads();
  }

  // ---- 4. gates, delta rule, readout
  if constexpr (MODE != kModeConv) {
    const float alpha = gate_alpha(dt, dt_bias, A_log);
    const float beta = gate_beta(braw);
    const float4 v4 = *reinterpret_cast<const float4*>(s_v + ph * D + 4 * cg);
    const float4 o = delta_rule<D, P, true, STREAM>(hreg, s_k + rg * R, s_q + rg * R, v4, alpha, beta, kq, srs, voff, 0);
    if constexpr (MODE == kModeRec) {
      if (rg == 0) store_out4(a.out, b * a.out_bs + static_cast<long>(h) * D + 4 * cg, o, a.out_bf16 != 0);
    } else {
      const float r = head_rms_scale<D, P>(o, rg == 0, ph, hred, a.rms_eps);
      if (rg == 0)
        store_out4(a.out, b * a.out_bs + static_cast<long>(h) * D + 4 * cg, gated(o, r, w4, Act<BF>::cvt4(z_raw)),
                   a.out_bf16 != 0);
    }
  }
}

// ----------------------------------------------------------------------------------
// Generic decode step: runtime K and G (G/P passes of P heads). Correct for every
// supported shape; the fast kernel covers K = 4 with G <= 2.
// Dynamic LDS: q[D], k[D], v[G*D], red[NW*4], hred[NW] floats.
// ----------------------------------------------------------------------------------
template <int D, int P, int MODE, bool BF, bool STREAM>
__global__ __launch_bounds__((Layout<D, P>::NT)) void gdn_step_generic(const KernelArgs a) {
  using L = Layout<D, P>;
  constexpr int NT = L::NT, R = L::R, CGL = L::CGL, NW = L::NW;
  constexpr uint32_t kHeadBytes = D * D * 4, kRowBytes = D * 4;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int G = a.G;
  float* s_q = smem;
  float* s_k = s_q + D;
  float* s_v = s_k + D;
  float* red = s_v + G * D;
  float* hred = red + NW * 4;

  const int t = threadIdx.x;
  const int b = blockIdx.x / a.Hk;
  const int g = blockIdx.x - b * a.Hk;
  const int ph = t / L::LPH;
  const int u = t - ph * L::LPH;
  const int cg = (u >> 6) * CGL + (u & (CGL - 1));
  const int rg = (u & 63) / CGL;
  const int nch = (2 + G) * D;
  const int sb = a.slots ? a.slots[b] : b;  // state slot (see gdn_step_fast)
  if (sb < 0 || sb >= a.pool) return;

  float kq;
  if constexpr (MODE == kModeRec) {
    const float* act = a.qkv_act_in + static_cast<long>(b) * a.C;
    for (int c = t; c < nch; c += NT) {
      const float v = act[unit_channel<D>(c, g, a.Hk, G)];
      if (c < D) s_q[c] = v;
      else if (c < 2 * D) s_k[c - D] = v;
      else s_v[c - 2 * D] = v;
    }
    __syncthreads();
    float s1[1] = {0.0f};
    for (int i = t; i < D; i += NT) s1[0] = fmaf(s_q[i], s_k[i], s1[0]);
    block_sum<NW, 1>(s1, red);
    kq = s1[0];
  } else {
    for (int c = t; c < nch; c += NT) {
      const long gc = unit_channel<D>(c, g, a.Hk, G);
      const float v = conv_channel_generic<BF>(a, b, sb, gc);
      if (c < D) s_q[c] = v;
      else if (c < 2 * D) s_k[c - D] = v;
      else {
        s_v[c - 2 * D] = v;
        if constexpr (MODE == kModeConv) a.qkv_act_out[static_cast<long>(b) * a.C + gc] = v;
        if constexpr (MODE == kModeFused) {
          if (a.tap_act) a.tap_act[static_cast<long>(b) * a.C + gc] = v;
        }
      }
    }
    __syncthreads();
    float s3[3] = {0.0f, 0.0f, 0.0f};
    for (int i = t; i < D; i += NT) {
      const float q = s_q[i], k = s_k[i];
      s3[0] = fmaf(q, q, s3[0]);
      s3[1] = fmaf(k, k, s3[1]);
      s3[2] = fmaf(q, k, s3[2]);
    }
    block_sum<NW, 3>(s3, red);
    const float rq = 1.0f / sqrtf(s3[0] + a.l2_eps);
    const float rk = 1.0f / sqrtf(s3[1] + a.l2_eps);
    kq = s3[2] * rq * rk;
    for (int i = t; i < D; i += NT) {
      const float qn = s_q[i] * rq, kn = s_k[i] * rk;
      if constexpr (MODE == kModeConv) {
        float* act = a.qkv_act_out + static_cast<long>(b) * a.C;
        act[static_cast<long>(g) * D + i] = qn;
        act[static_cast<long>(a.Hk) * D + static_cast<long>(g) * D + i] = kn;
      } else {
        s_q[i] = qn;
        s_k[i] = kn;
        if (MODE == kModeFused && a.tap_act) {
          float* act = a.tap_act + static_cast<long>(b) * a.C;
          act[static_cast<long>(g) * D + i] = qn;
          act[static_cast<long>(a.Hk) * D + static_cast<long>(g) * D + i] = kn;
        }
      }
    }
    if constexpr (MODE == kModeConv) return;
    __syncthreads();
  }

  if constexpr (MODE != kModeConv) {
    const uint32_t voff = static_cast<uint32_t>(ph) * kHeadBytes + static_cast<uint32_t>(rg * R) * kRowBytes +
                          static_cast<uint32_t>(cg) * 16u;
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(a.state + (static_cast<long>(sb) * a.Hv + static_cast<long>(g) * G) * (D * D),
                  static_cast<uint32_t>(G) * kHeadBytes);
    const int passes = G / P;
    for (int pass = 0; pass < passes; ++pass) {
      const int hl = pass * P + ph;
      const int h = g * G + hl;
      const uint32_t soff = static_cast<uint32_t>(pass * P) * kHeadBytes;
      typename Act<BF>::raw4_t z_raw{};  // loaded by every lane, widened where used
      float4 w4 = f4(0.0f);
      if constexpr (MODE == kModeFused) {
        z_raw = Act<BF>::raw4(a.z, b * a.z_bs + static_cast<long>(h) * D + 4 * cg);
        w4 = *reinterpret_cast<const float4*>(a.norm_w + 4 * cg);
      }
      const float alpha = gate_alpha(Act<BF>::load(a.dt_raw, b * a.ab_bs + h), a.dt_bias[h], a.A_log[h]);
      const float beta = gate_beta(Act<BF>::load(a.b_raw, b * a.ab_bs + h));
      float4 hreg[R];
#pragma unroll
      for (int k = 0; k < R; ++k) hreg[k] = buf_load4<STREAM>(srs, voff, soff + k * kRowBytes);
      const float4 v4 = *reinterpret_cast<const float4*>(s_v + hl * D + 4 * cg);
      const float4 o =
          delta_rule<D, P, true, STREAM>(hreg, s_k + rg * R, s_q + rg * R, v4, alpha, beta, kq, srs, voff, soff);
      if constexpr (MODE == kModeRec) {
        if (rg == 0) store_out4(a.out, b * a.out_bs + static_cast<long>(h) * D + 4 * cg, o, a.out_bf16 != 0);
      } else {
        const float r = head_rms_scale<D, P>(o, rg == 0, ph, hred, a.rms_eps);
        if (rg == 0)
          store_out4(a.out, b * a.out_bs + static_cast<long>(h) * D + 4 * cg, gated(o, r, w4, Act<BF>::cvt4(z_raw)),
                     a.out_bf16 != 0);
        if (MODE == kModeFused && a.taps) {
          const long hb = static_cast<long>(b) * a.Hv + h;
          if (rg == 0 && a.tap_y) *reinterpret_cast<float4*>(a.tap_y + hb * D + 4 * cg) = o;
          if (rg == 0 && a.tap_y_norm)
            *reinterpret_cast<float4*>(a.tap_y_norm + hb * D + 4 * cg) =
                make_float4(o.x * r * w4.x, o.y * r * w4.y, o.z * r * w4.z, o.w * r * w4.w);
          if (u == 0 && a.tap_alpha) a.tap_alpha[hb] = alpha;
          if (u == 0 && a.tap_beta) a.tap_beta[hb] = beta;
        }
        if (pass + 1 < passes) __syncthreads();  // hred is rewritten by the next pass
      }
    }
  }
}

// ----------------------------------------------------------------------------------
// T tokens with the state held in VGPRs for the whole sequence (G == P: every v-head of
// the group is resident) and KT conv taps. Conv windows live in registers of the lane
// that owns the channel; the final conv state is the window's last KT-1 raw values.
// The next token's inputs are loaded while the current token is computed.
// ----------------------------------------------------------------------------------
template <int D, int P, bool BF, int KT>
__global__ __launch_bounds__((Layout<D, P>::NT)) void gdn_seq_kernel(const KernelArgs a) {
  using L = Layout<D, P>;
  using CR = ConvRegs<BF, KT, (2 + P) * D, L::NT, D>;
  constexpr int NT = L::NT, R = L::R, CGL = L::CGL, NW = L::NW;
  constexpr uint32_t kHeadBytes = D * D * 4, kRowBytes = D * 4;
  __shared__ __attribute__((aligned(16))) float s_q[D];
  __shared__ __attribute__((aligned(16))) float s_k[D];
  __shared__ __attribute__((aligned(16))) float s_v[P * D];
  __shared__ float red[NW * 4];
  __shared__ float hred[NW];

  const int t = threadIdx.x;
  const int b = blockIdx.x / a.Hk;
  const int g = blockIdx.x - b * a.Hk;
  const int ph = t / L::LPH;
  const int u = t - ph * L::LPH;
  const int cg = (u >> 6) * CGL + (u & (CGL - 1));
  const int rg = (u & 63) / CGL;
  const int h = g * P + ph;
  const long cs_base = static_cast<long>(b) * (KT - 1) * a.C;
  const bool obf = a.out_bf16 != 0;

  CR cr;
  cr.channels(g, a.Hk, P);
  cr.load_window(a.conv_state, cs_base, a.C);
  cr.load_taps_all(a.conv_w);
  cr.load_x(a.qkv, b * a.qkv_bs);
  const long ab0 = b * a.ab_bs + h;
  float dt = Act<BF>::load(a.dt_raw, ab0), braw = Act<BF>::load(a.b_raw, ab0);
  const long z0 = b * a.z_bs + static_cast<long>(h) * D + 4 * cg;
  typename Act<BF>::raw4_t z_raw = Act<BF>::raw4(a.z, z0);  // every lane: no wait at a branch join
  const float4 w4 = *reinterpret_cast<const float4*>(a.norm_w + 4 * cg);
  const float A_log = a.A_log[h], dt_bias = a.dt_bias[h];

  const uint32_t voff = static_cast<uint32_t>(ph) * kHeadBytes + static_cast<uint32_t>(rg * R) * kRowBytes +
                        static_cast<uint32_t>(cg) * 16u;
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(a.state + (static_cast<long>(b) * a.Hv + static_cast<long>(g) * P) * (D * D), P * kHeadBytes);
  float4 hreg[R];
#pragma unroll
  for (int k = 0; k < R; ++k) hreg[k] = buf_load4<false>(srs, voff, k * kRowBytes);

  for (int tok = 0; tok < a.T; ++tok) {
    cr.compute(s_q, s_k, s_v);
    cr.roll();
    const float alpha = gate_alpha(dt, dt_bias, A_log);
    const float beta = gate_beta(braw);
    const float4 zc = Act<BF>::cvt4(z_raw);
    // prefetch the next token's inputs
    if (tok + 1 < a.T) {
      cr.load_x(a.qkv, b * a.qkv_bs + (tok + 1) * a.qkv_ts);
      dt = Act<BF>::load(a.dt_raw, ab0 + (tok + 1) * a.ab_ts);
      braw = Act<BF>::load(a.b_raw, ab0 + (tok + 1) * a.ab_ts);
      z_raw = Act<BF>::raw4(a.z, z0 + (tok + 1) * a.z_ts);
    }
    __syncthreads();
    float s3[3] = {0.0f, 0.0f, 0.0f};
    for (int i = t; i < D; i += NT) {
      const float q = s_q[i], k = s_k[i];
      s3[0] = fmaf(q, q, s3[0]);
      s3[1] = fmaf(k, k, s3[1]);
      s3[2] = fmaf(q, k, s3[2]);
    }
    block_sum<NW, 3>(s3, red);
    const float rq = 1.0f / sqrtf(s3[0] + a.l2_eps);
    const float rk = 1.0f / sqrtf(s3[1] + a.l2_eps);
    const float kq = s3[2] * rq * rk;
    for (int i = t; i < D; i += NT) {
      s_q[i] *= rq;
      s_k[i] *= rk;
    }
    __syncthreads();
    const float4 v4 = *reinterpret_cast<const float4*>(s_v + ph * D + 4 * cg);
    const float4 o = delta_rule<D, P, false, false>(hreg, s_k + rg * R, s_q + rg * R, v4, alpha, beta, kq, srs, voff, 0);
    const float r = head_rms_scale<D, P>(o, rg == 0, ph, hred, a.rms_eps);
    if (rg == 0)
      store_out4(a.out, b * a.out_bs + tok * a.out_ts + static_cast<long>(h) * D + 4 * cg, gated(o, r, w4, zc), obf);
    __syncthreads();  // LDS is rewritten by the next token
  }

#pragma unroll
  for (int k = 0; k < R; ++k) buf_store4<false>(srs, voff, k * kRowBytes, hreg[k]);
  cr.store_window(a.conv_state, cs_base, a.C);
}

// ----------------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------------

template <int D, int P, bool BF, bool ST>
void launch_step_s(int mode, bool fast, const KernelArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hk));
  const dim3 block(Layout<D, P>::NT);
  if (fast) {
    switch (mode) {
      case kModeConv: gdn_step_fast<D, P, kModeConv, BF, 4, false><<<grid, block, 0, s>>>(a); break;
      case kModeRec: gdn_step_fast<D, P, kModeRec, BF, 4, ST><<<grid, block, 0, s>>>(a); break;
      default: gdn_step_fast<D, P, kModeFused, BF, 4, ST><<<grid, block, 0, s>>>(a); break;
    }
  } else {
    const size_t lds =
        sizeof(float) * (2 * D + static_cast<size_t>(a.G) * D + Layout<D, P>::NW * 4 + Layout<D, P>::NW);
    switch (mode) {
      case kModeConv: gdn_step_generic<D, P, kModeConv, BF, false><<<grid, block, lds, s>>>(a); break;
      case kModeRec: gdn_step_generic<D, P, kModeRec, BF, ST><<<grid, block, lds, s>>>(a); break;
      default: gdn_step_generic<D, P, kModeFused, BF, ST><<<grid, block, lds, s>>>(a); break;
    }
  }
}

template <int D, int P, bool BF>
hipError_t launch_step_d(int mode, bool fast, const KernelArgs& a, hipStream_t s) {
  if (a.stream_state)
    launch_step_s<D, P, BF, true>(mode, fast, a, s);
  else
    launch_step_s<D, P, BF, false>(mode, fast, a, s);
  return hipGetLastError();
}

template <int D, int P>
hipError_t launch_step_p(int mode, bool fast, const KernelArgs& a, hipStream_t s) {
  return a.act_bf16 ? launch_step_d<D, P, true>(mode, fast, a, s) : launch_step_d<D, P, false>(mode, fast, a, s);
}

template <int D, int P, int KT>
void launch_seq_k(const KernelArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hk));
  const dim3 block(Layout<D, P>::NT);
  if (a.act_bf16)
    gdn_seq_kernel<D, P, true, KT><<<grid, block, 0, s>>>(a);
  else
    gdn_seq_kernel<D, P, false, KT><<<grid, block, 0, s>>>(a);
}

template <int D, int P>
hipError_t launch_seq_t(const KernelArgs& a, hipStream_t s) {
  switch (a.K) {
    case 2: launch_seq_k<D, P, 2>(a, s); break;
    case 3: launch_seq_k<D, P, 3>(a, s); break;
    case 5: launch_seq_k<D, P, 5>(a, s); break;
    default: launch_seq_k<D, P, 4>(a, s); break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_seq_g(int p, const KernelArgs& a, hipStream_t s) {
  switch (p) {
    case 1: return launch_seq_t<D, 1>(a, s);
    case 2: return launch_seq_t<D, 2>(a, s);
    case 3: return launch_seq_t<D, 3>(a, s);
    default: return launch_seq_t<D, 4>(a, s);
  }
}

}  // namespace

bool step_supported(int d, int p) { return (d == 32 || d == 64 || d == 128) && (p == 1 || p == 2); }

hipError_t launch_step(int mode, int d, int p, const KernelArgs& a, hipStream_t s) {
  // fast path: K = 4 and a single pass (G == P); every other shape, and a step with
  // taps, takes the generic one
  const bool fast = (a.K == 4) && (a.G == p) && !a.taps;
  if (d == 128) return p == 2 ? launch_step_p<128, 2>(mode, fast, a, s) : launch_step_p<128, 1>(mode, fast, a, s);
  if (d == 64) return p == 2 ? launch_step_p<64, 2>(mode, fast, a, s) : launch_step_p<64, 1>(mode, fast, a, s);
  return p == 2 ? launch_step_p<32, 2>(mode, fast, a, s) : launch_step_p<32, 1>(mode, fast, a, s);
}

bool sequence_supported(int G, int K) { return G >= 1 && G <= 4 && K >= 2 && K <= 5; }

hipError_t launch_sequence(int d, int p, const KernelArgs& a, hipStream_t s) {
  if (d == 128) return launch_seq_g<128>(p, a, s);
  if (d == 64) return launch_seq_g<64>(p, a, s);
  return launch_seq_g<32>(p, a, s);
}

}  // namespace gdn
