// HIP kernels of speculative decoding for CDNA4 (gfx950): gdn_decode_verify runs the
// draft tokens of each sequence with both states read only and records each token's
// update; gdn_decode_commit applies the accepted prefix (see include/gdn.h).

#include "gdn_device.h"

namespace gdn {
namespace {

// ----------------------------------------------------------------------------------
// Speculative verification of T <= kMaxVerifyTokens draft tokens. One workgroup per
// (sequence b, v-head h), any G and K: both states are only read, so the G workgroups
// of a k-head may all read its Q/K conv columns. Per token: the output gdn_decode_layer
// would give after the previous draft tokens, and the trail of the token's update
// H <- alpha H + k delta^T (delta, unit k, alpha), from which gdn_commit_kernel
// rebuilds the state after any accepted prefix.
// Only the delta rule depends on the previous token, so the kernel runs in three
// phases: (A) conv, gates and L2 norms of all T tokens at once (one block reduction),
// (B) the T delta-rule steps on the VGPR-resident state with no barrier between them,
// (C) the per-head RMSNorm and the outputs of all T tokens (one block reduction).
// ----------------------------------------------------------------------------------
// d = 128 uses 16 state rows per lane (4 waves per head, 64 state VGPRs): the per-token
// work per lane halves and more workgroups stay resident.
template <int D>
using VerifyLayout = Layout<D, 1, D == 128 ? 16 : 0>;

template <int D, bool BF>
__global__ __launch_bounds__((VerifyLayout<D>::NT)) void gdn_verify_kernel(const KernelArgs a) {
  using L = VerifyLayout<D>;
  constexpr int NT = L::NT, R = L::R, CGL = L::CGL, NW = L::NW;
  constexpr int NCH = 3 * D;
  constexpr int kTM = kMaxVerifyTokens;
  constexpr int kRows = kMaxConvTaps - 1 + kTM;
  constexpr uint32_t kRowBytes = D * 4;
  using raw_t = typename Act<BF>::raw_t;  // stored values, widened on use
  __shared__ __attribute__((aligned(16))) raw_t s_x[kRows][NCH];  // K-1 conv-state rows, then T token rows
  __shared__ __attribute__((aligned(16))) raw_t s_w[NCH * kMaxConvTaps];  // taps [NCH][K]
  __shared__ __attribute__((aligned(16))) float s_q[kTM][D];
  __shared__ __attribute__((aligned(16))) float s_k[kTM][D];
  __shared__ __attribute__((aligned(16))) float s_v[kTM][D];
  __shared__ __attribute__((aligned(16))) float s_o[kTM][D];  // readouts, for the RMSNorm of phase C
  __shared__ __attribute__((aligned(16))) raw_t s_z[kTM][D];  // z rows of the tokens, staged in phase A
  __shared__ float s_gate[3][kTM];      // alpha, beta, k.q per token
  __shared__ float red[NW][3 * kTM];    // per-wave partial sums

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int bh = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x));  // (b, h), uniform
  const int b = bh / a.Hv;
  const int h = bh - b * a.Hv;
  const int g = h / a.G;
  const int cg = (t >> 6) * CGL + (t & (CGL - 1));
  const int rg = (t & 63) / CGL;
  const int K = a.K, T = a.T;
  const long C = a.C;
  // unit channel c: [0, D) Q of k-head g, [D, 2D) K of k-head g, [2D, 3D) V of v-head h
  auto chan = [&](int c) -> long {
    return c < D ? static_cast<long>(g) * D + c
                 : (c < 2 * D ? static_cast<long>(a.Hk + g) * D + (c - D) : static_cast<long>(2 * a.Hk + h) * D + (c - 2 * D));
  };

  const uint32_t voff = static_cast<uint32_t>(rg * R) * kRowBytes + static_cast<uint32_t>(cg) * 16u;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.state + static_cast<long>(bh) * (D * D), D * D * 4);
  float4 hreg[R];
  raw_t gdt = 0, gbr = 0;  // raw gate inputs of token t (t < T), converted where used

  // ---- A. conv inputs and taps into LDS, then conv + SiLU of every (token, channel), gates
  {
    // 16-byte pieces of 8 consecutive unit channels (a segment's D channels are
    // consecutive in a qkv row and in conv1d_weight). The pieces are assigned segment by
    // segment, so the segment's channel offset is uniform and each lane's address is a
    // row base plus a fixed piece offset. Every load is issued before the first LDS store.
    constexpr int kE = BF ? 1 : 2;             // 16-byte words per 8 elements
    constexpr int kEs = BF ? 2 : 4;            // bytes per element
    constexpr int kPR = D / 8;                 // pieces per row and segment
    constexpr int kXPer = (kRows * kPR + NT - 1) / NT;
    constexpr int kWPer = (D * kMaxConvTaps / 8 + NT - 1) / NT;
    constexpr int kZPer = (kTM * kPR + NT - 1) / NT;
    const int nrow = K - 1 + T;
    const int npw = D * K / 8;                 // tap pieces per segment
    u32x4 xr[3][kXPer][kE], wr[3][kWPer][kE], zr[kZPer][kE];
    auto ld8 = [&](const char* p, u32x4(&dst)[kE]) {
#pragma unroll
      for (int e = 0; e < kE; ++e) dst[e] = *reinterpret_cast<const u32x4*>(p + 16 * e);
    };
    // first channel of each segment: Q and K of k-head g, V of v-head h
    const long ch[3] = {static_cast<long>(g) * D, static_cast<long>(a.Hk + g) * D, static_cast<long>(2 * a.Hk + h) * D};
    const char* cs_row0 = static_cast<const char*>(a.conv_state) + static_cast<long>(b) * (K - 1) * C * kEs;
    const char* x_row0 = static_cast<const char*>(a.qkv) + b * a.qkv_bs * kEs;
    // Loads are unconditional, with indices clamped to valid rows (only the LDS stores
    // below are conditional): a load inside a branch is waited for where the branch
    // joins, which would put each load's latency in series.
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int it = min(t + i * NT, nrow * kPR - 1), j = it / kPR, pc = it - j * kPR;
      // rows 0..K-2 come from the conv state, the rest are the draft tokens
      const char* row = j < K - 1 ? cs_row0 + static_cast<long>(j) * C * kEs : x_row0 + (j - (K - 1)) * a.qkv_ts * kEs;
#pragma unroll
      for (int sg = 0; sg < 3; ++sg) ld8(row + (ch[sg] + 8 * pc) * kEs, xr[sg][i]);
    }
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int it = min(t + i * NT, npw - 1);
#pragma unroll
      for (int sg = 0; sg < 3; ++sg)
        ld8(static_cast<const char*>(a.conv_w) + (ch[sg] * K + 8 * it) * kEs, wr[sg][i]);
    }
#pragma unroll
    for (int i = 0; i < kZPer; ++i) {
      const int it = min(t + i * NT, T * kPR - 1), tok = it / kPR, pc = it - tok * kPR;
      ld8(static_cast<const char*>(a.z) + (b * a.z_bs + tok * a.z_ts + static_cast<long>(h) * D + 8 * pc) * kEs,
          zr[i]);
    }
    // the gate inputs and then the state of head h (read only) go out before the first
    // LDS store waits for the loads above, so all three latencies overlap; the state is
    // issued last (vmcnt retires in order) and stays in flight during the conv and norms
    {
      const long ab = b * a.ab_bs + min(t, T - 1) * a.ab_ts + h;  // T >= 1
      gdt = Act<BF>::raw(a.dt_raw, ab);
      gbr = Act<BF>::raw(a.b_raw, ab);
    }
#pragma unroll
    for (int k = 0; k < R; ++k) hreg[k] = buf_load4<false>(srs, voff, k * kRowBytes);
    auto put8 = [&](raw_t* dst, const u32x4(&src)[kE]) {  // 8 stored values, as they are
#pragma unroll
      for (int e = 0; e < kE; ++e) *reinterpret_cast<u32x4*>(dst + e * (16 / sizeof(raw_t))) = src[e];
    };
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int it = t + i * NT, j = it / kPR, pc = it - j * kPR;
      if (j < nrow)
#pragma unroll
        for (int sg = 0; sg < 3; ++sg) put8(&s_x[j][sg * D + 8 * pc], xr[sg][i]);
    }
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int it = t + i * NT;
      if (it < npw)
#pragma unroll
        for (int sg = 0; sg < 3; ++sg) put8(&s_w[sg * D * K + 8 * it], wr[sg][i]);
    }
#pragma unroll
    for (int i = 0; i < kZPer; ++i) {
      const int it = t + i * NT, tok = it / kPR, pc = it - tok * kPR;
      if (tok < T) put8(&s_z[tok][8 * pc], zr[i]);
    }
  }
  if (t < T) {
    s_gate[0][t] = gate_alpha(Act<BF>::f(gdt), a.dt_bias[h], a.A_log[h]);
    s_gate[1][t] = gate_beta(Act<BF>::f(gbr));
  }
  __syncthreads();
  for (int c = t; c < NCH; c += NT) {
    float(*dst)[D] = c < D ? s_q : (c < 2 * D ? s_k : s_v);
    const int e = c < D ? c : (c < 2 * D ? c - D : c - 2 * D);
    if (K == 4) {
      // the common width: taps in registers and a sliding window of the last three
      // inputs, so each input is read from LDS once
      const float w0 = Act<BF>::f(s_w[4 * c]), w1 = Act<BF>::f(s_w[4 * c + 1]), w2 = Act<BF>::f(s_w[4 * c + 2]),
                  w3 = Act<BF>::f(s_w[4 * c + 3]);
      float x0 = Act<BF>::f(s_x[0][c]), x1 = Act<BF>::f(s_x[1][c]), x2 = Act<BF>::f(s_x[2][c]);
      for (int tok = 0; tok < T; ++tok) {
        const float x3 = Act<BF>::f(s_x[tok + 3][c]);  // tap 3 on the token itself
        dst[tok][e] = silu_rcp(fmaf(w3, x3, fmaf(w2, x2, fmaf(w1, x1, w0 * x0))));
        x0 = x1;
        x1 = x2;
        x2 = x3;
      }
    } else {
      for (int tok = 0; tok < T; ++tok) {
        float u = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxConvTaps; ++j)
          if (j < K) u = fmaf(Act<BF>::f(s_w[c * K + j]), Act<BF>::f(s_x[tok + j][c]), u);  // tap K-1 on the token itself
        dst[tok][e] = silu_rcp(u);
      }
    }
  }
  __syncthreads();
  // L2 norms of q and k and their dot product, all tokens in one reduction
  float s3[3 * kTM];
#pragma unroll
  for (int i = 0; i < 3 * kTM; ++i) s3[i] = 0.0f;
  for (int i = t; i < D; i += NT)
#pragma unroll
    for (int tok = 0; tok < kTM; ++tok)
      if (tok < T) {
        const float q = s_q[tok][i], k = s_k[tok][i];
        s3[3 * tok] = fmaf(q, q, s3[3 * tok]);
        s3[3 * tok + 1] = fmaf(k, k, s3[3 * tok + 1]);
        s3[3 * tok + 2] = fmaf(q, k, s3[3 * tok + 2]);
      }
  {
    float s6[3 * kTM / 4];  // row r holds sum j + 6 (r & 1) + 12 (r >> 1) in register j
    wave_sums_t<3 * kTM>(s3, s6);
    if ((lane & 15) == 0) {
      const int r = lane >> 4;
#pragma unroll
      for (int j = 0; j < 3 * kTM / 4; ++j) red[wv][j + (3 * kTM / 4) * (r & 1) + (3 * kTM / 2) * (r >> 1)] = s6[j];
    }
  }
  __syncthreads();
  const long bt0 = static_cast<long>(b) * T;
  for (int tok = 0; tok < T; ++tok) {
    float sq = 0.0f, sk = 0.0f, sqk = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sq += red[w][3 * tok];
      sk += red[w][3 * tok + 1];
      sqk += red[w][3 * tok + 2];
    }
    const float rq = __builtin_amdgcn_rsqf(sq + a.l2_eps), rk = __builtin_amdgcn_rsqf(sk + a.l2_eps);
    if (t == 0) s_gate[2][tok] = sqk * rq * rk;
    // elements 0..D-1 scale q, D..2D-1 scale k (and record it in the trail)
    for (int i = t; i < 2 * D; i += NT) {
      if (i < D) {
        s_q[tok][i] *= rq;
      } else {
        const float kn = s_k[tok][i - D] * rk;
        s_k[tok][i - D] = kn;
        if (h % a.G == 0) a.trail_k[((bt0 + tok) * a.Hk + g) * D + (i - D)] = kn;
      }
    }
  }
  __syncthreads();

  // ---- B. the T delta-rule steps (no barrier: each lane reads LDS written above). The
  // state after the last token is not needed here (commit rebuilds it from the trail),
  // so the last step only forms delta and the readout.
  auto step = [&](int tok, auto form) {
    const float alpha = s_gate[0][tok], beta = s_gate[1][tok];
    const float4 v4 = *reinterpret_cast<const float4*>(&s_v[tok][4 * cg]);
    float4 delta;
    const float4 ot = delta_rule<D, 1, false, false, R, decltype(form)::value>(
        hreg, &s_k[tok][rg * R], &s_q[tok][rg * R], v4, alpha, beta, s_gate[2][tok], srs, voff, 0, &delta);
    if (rg == 0) {
      *reinterpret_cast<float4*>(&s_o[tok][4 * cg]) = ot;
      *reinterpret_cast<float4*>(a.trail_delta + ((bt0 + tok) * a.Hv + h) * D + 4 * cg) = delta;
    }
    if (t == 0) a.trail_alpha[(bt0 + tok) * a.Hv + h] = alpha;
  };
  for (int tok = 0; tok + 1 < T; ++tok) step(tok, std::integral_constant<int, 1>{});
  step(T - 1, std::integral_constant<int, 2>{});  // T >= 1

  // ---- C. per-head RMSNorm and gated outputs of all tokens
  float ss[kTM];
#pragma unroll
  for (int tok = 0; tok < kTM; ++tok) {
    float v = 0.0f;
    if (rg == 0 && tok < T) {
      const float4 o = *reinterpret_cast<const float4*>(&s_o[tok][4 * cg]);
      v = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
    }
    ss[tok] = v;
  }
  {
    float s2[kTM / 4];  // row r holds token j + 2 (r & 1) + 4 (r >> 1) in register j
    wave_sums_t<kTM>(ss, s2);
    if ((lane & 15) == 0) {
      const int r = lane >> 4;
#pragma unroll
      for (int j = 0; j < kTM / 4; ++j) red[wv][j + (kTM / 4) * (r & 1) + (kTM / 2) * (r >> 1)] = s2[j];
    }
  }
  __syncthreads();
  if (rg == 0) {
    const float4 w4 = *reinterpret_cast<const float4*>(a.norm_w + 4 * cg);
    const bool obf = a.out_bf16 != 0;
    for (int tok = 0; tok < T; ++tok) {
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += red[w][tok];
      const float r = __builtin_amdgcn_rsqf(tot / static_cast<float>(D) + a.rms_eps);
      const float4 z4 = Act<BF>::load4(&s_z[tok][0], 4 * cg);
      const float4 o = *reinterpret_cast<const float4*>(&s_o[tok][4 * cg]);
      store_out4(a.out, b * a.out_bs + tok * a.out_ts + static_cast<long>(h) * D + 4 * cg, gated<true>(o, r, w4, z4),
                 obf);
    }
  }
}

// Commit of the accepted prefix: H <- alpha_t H + k_t delta_t^T for t < n = accepted[b]
// (the expression delta_rule evaluates, so the result is bit-identical to the verify
// kernel's state after n tokens). n outside [1, T] leaves the sequence untouched.
template <int D>
__global__ __launch_bounds__((Layout<D, 1>::NT)) void gdn_commit_kernel(const KernelArgs a) {
  using L = Layout<D, 1>;
  constexpr int R = L::R, CGL = L::CGL;
  constexpr uint32_t kRowBytes = D * 4;
  const int t = threadIdx.x;
  const int bh = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x));  // (b, h), uniform
  const int b = bh / a.Hv;
  const int h = bh - b * a.Hv;
  const int g = h / a.G;
  const int n = a.accepted[b];
  if (n < 1 || n > a.T) return;
  const int cg = (t >> 6) * CGL + (t & (CGL - 1));
  const int rg = (t & 63) / CGL;
  const uint32_t voff = static_cast<uint32_t>(rg * R) * kRowBytes + static_cast<uint32_t>(cg) * 16u;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.state + static_cast<long>(bh) * (D * D), D * D * 4);
  float4 hreg[R];
#pragma unroll
  for (int k = 0; k < R; ++k) hreg[k] = buf_load4<false>(srs, voff, k * kRowBytes);
  for (int tok = 0; tok < n; ++tok) {
    const long bt = static_cast<long>(b) * a.T + tok;
    const float alpha = a.trail_alpha[bt * a.Hv + h];
    const float4 delta = *reinterpret_cast<const float4*>(a.trail_delta + (bt * a.Hv + h) * D + 4 * cg);
    const float* kr = a.trail_k + (bt * a.Hk + g) * D + rg * R;
#pragma unroll
    for (int k4 = 0; k4 < R / 4; ++k4) {
      const float4 kk = *reinterpret_cast<const float4*>(kr + 4 * k4);
      const float kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float4& hh = hreg[4 * k4 + e];
        hh.x = fmaf(kv[e], delta.x, alpha * hh.x);
        hh.y = fmaf(kv[e], delta.y, alpha * hh.y);
        hh.z = fmaf(kv[e], delta.z, alpha * hh.z);
        hh.w = fmaf(kv[e], delta.w, alpha * hh.w);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < R; ++k) buf_store4<false>(srs, voff, k * kRowBytes, hreg[k]);
}

// Conv state after the accepted prefix: row j <- element n + j of (old rows 0..K-2,
// x_0 .. x_{T-1}), a bit-exact copy; rows in increasing order, so an old row is read
// before it is overwritten. One thread per (sequence, channel).
template <bool BF>
__global__ __launch_bounds__(256) void gdn_conv_commit(const KernelArgs a) {
  const long C = a.C;
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(a.B) * C) return;
  const long b = idx / C, c = idx - b * C;
  const int n = a.accepted[b];
  if (n < 1 || n > a.T) return;
  const int Km1 = a.K - 1;
  for (int j = 0; j < Km1; ++j) {
    const int e = n + j;
    const auto v = e < Km1 ? Act<BF>::raw(a.conv_state, (b * Km1 + e) * C + c)
                           : Act<BF>::raw(a.qkv, b * a.qkv_bs + (e - Km1) * a.qkv_ts + c);
    Act<BF>::put(a.conv_state, (b * Km1 + j) * C + c, v);
  }
}

template <int D>
hipError_t launch_verify_d(const KernelArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv));
  if (a.act_bf16)
    gdn_verify_kernel<D, true><<<grid, VerifyLayout<D>::NT, 0, s>>>(a);
  else
    gdn_verify_kernel<D, false><<<grid, VerifyLayout<D>::NT, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_commit_d(const KernelArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv));
  gdn_commit_kernel<D><<<grid, Layout<D, 1>::NT, 0, s>>>(a);
  const dim3 cgrid(static_cast<unsigned>((static_cast<long>(a.B) * a.C + 255) / 256));
  if (a.act_bf16)
    gdn_conv_commit<true><<<cgrid, 256, 0, s>>>(a);
  else
    gdn_conv_commit<false><<<cgrid, 256, 0, s>>>(a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_verify(int d, const KernelArgs& a, hipStream_t s) {
  if (d == 128) return launch_verify_d<128>(a, s);
  if (d == 64) return launch_verify_d<64>(a, s);
  return launch_verify_d<32>(a, s);
}

hipError_t launch_commit(int d, const KernelArgs& a, hipStream_t s) {
  if (d == 128) return launch_commit_d<128>(a, s);
  if (d == 64) return launch_commit_d<64>(a, s);
  return launch_commit_d<32>(a, s);
}

}  // namespace gdn
