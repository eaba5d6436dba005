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
// The states are not written, so the state after each draft token is never formed:
// with H0 the state before the draft and G(i, j) = alpha_i ... alpha_j (1 when i > j),
// the rule H_t = alpha_t H_{t-1} + k_t delta_t^T unrolls to
//   m_t = H_{t-1}^T k_t = G(0, t-1) H0^T k_t + sum_{s<t} G(s+1, t-1) (k_s . k_t) delta_s,
//   delta_t = beta_t (v_t - alpha_t m_t),
//   o_t = H_t^T q_t / sqrt(d) = (G(0, t) H0^T q_t + sum_{s<=t} G(s+1, t) (k_s . q_t) delta_s) / sqrt(d),
// so one pass over H0 gives every token's H0^T k_t and H0^T q_t (two matrix-vector
// products per token instead of two plus the rank-one update), and the rest is the
// T x T products k_s . k_t, k_s . q_t and the decay products. Phases: (A) conv, gates
// and the L2 norms of all T tokens (one block reduction), then the T^2 token products;
// (B) per token, H0^T k_t and H0^T q_t on the VGPR-resident state, reduced over the
// row groups, then delta_t and o_t, one thread per column (the L2 norms enter as
// factors of those products, q and k are never rescaled in place); (C) the per-head
// RMSNorm and the outputs of all T tokens on the same threads (one block reduction).
// ----------------------------------------------------------------------------------
// d = 128 uses 16 state rows per lane (4 waves per head, 64 state VGPRs): the per-token
// work per lane halves and more workgroups stay resident.
template <int D>
using VerifyLayout = Layout<D, 1, D == 128 ? 16 : 0>;

template <int D, bool BF, int TM>
__global__ __launch_bounds__((VerifyLayout<D>::NT)) void gdn_verify_kernel(const KernelArgs a) {
  using L = VerifyLayout<D>;
  constexpr int NT = L::NT, R = L::R, CGL = L::CGL, NW = L::NW;
  constexpr int NCH = 3 * D;
  constexpr int kTM = TM;  // draft tokens the LDS and register arrays hold (T <= TM)
  constexpr int kRows = kMaxConvTaps - 1 + kTM;
  constexpr uint32_t kRowBytes = D * 4;
  using raw_t = typename Act<BF>::raw_t;  // stored values, widened on use
  // The conv inputs and taps are dead once the conv has run; the reduced state products
  // of phase B reuse their storage.
  union Reused {
    struct {
      raw_t x[kRows][NCH];            // K-1 conv-state rows, then T token rows
      raw_t w[NCH * kMaxConvTaps];    // taps [NCH][K]
    } conv;
    struct {
      float hk[kTM][D];               // H0^T k_t, reduced (k before its L2 norm)
      float hq[kTM][D];               // H0^T q_t, reduced (q before its L2 norm)
    } prod;
  };
  __shared__ __attribute__((aligned(16))) Reused reused;
  auto& s_x = reused.conv.x;
  auto& s_w = reused.conv.w;
  auto& s_hk = reused.prod.hk;
  auto& s_hq = reused.prod.hq;
  __shared__ __attribute__((aligned(16))) float s_q[kTM][D];
  __shared__ __attribute__((aligned(16))) float s_k[kTM][D];
  __shared__ __attribute__((aligned(16))) float s_v[kTM][D];
  __shared__ __attribute__((aligned(16))) raw_t s_z[kTM][D];  // z rows of the tokens, staged in phase A
  __shared__ float s_gate[2][kTM];      // alpha, beta per token
  __shared__ float s_kk[kTM][kTM];      // [t][s]: k_s . k_t for s < t (before the L2 norms)
  __shared__ float s_kq[kTM][kTM];      // [t][s]: k_s . q_t for s <= t (before the L2 norms)
  __shared__ float red[NW][2 * kTM];    // per-wave partial sums

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
  // L2 norms of q and k, all tokens in one reduction
  float s2n[2 * kTM];
#pragma unroll
  for (int i = 0; i < 2 * kTM; ++i) s2n[i] = 0.0f;
  for (int i = t; i < D; i += NT)
#pragma unroll
    for (int tok = 0; tok < kTM; ++tok)
      if (tok < T) {
        const float q = s_q[tok][i], k = s_k[tok][i];
        s2n[2 * tok] = fmaf(q, q, s2n[2 * tok]);
        s2n[2 * tok + 1] = fmaf(k, k, s2n[2 * tok + 1]);
      }
  {
    float s4[2 * kTM / 4];  // row r holds sum j + 4 (r & 1) + 8 (r >> 1) in register j
    wave_sums_t<2 * kTM>(s2n, s4);
    if ((lane & 15) == 0) {
      const int r = lane >> 4;
#pragma unroll
      for (int j = 0; j < 2 * kTM / 4; ++j) red[wv][j + (2 * kTM / 4) * (r & 1) + (2 * kTM / 2) * (r >> 1)] = s4[j];
    }
  }
  __syncthreads();
  const long bt0 = static_cast<long>(b) * T;
  // 1 / |q_t| and 1 / |k_t| of every token, in every thread: q and k stay as the conv
  // left them, and the factors are applied where their products are used (B2)
  float rq[kTM], rk[kTM];
#pragma unroll
  for (int tok = 0; tok < kTM; ++tok) {
    float sq = 0.0f, sk = 0.0f;
    if (tok < T) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sq += red[w][2 * tok];
        sk += red[w][2 * tok + 1];
      }
    }
    rq[tok] = __builtin_amdgcn_rsqf(sq + a.l2_eps);
    rk[tok] = __builtin_amdgcn_rsqf(sk + a.l2_eps);
  }
  // the trail's unit k
  if (h % a.G == 0) {
#pragma unroll
    for (int tok = 0; tok < kTM; ++tok) {
      if (tok >= T) break;
      for (int i = t; i < D; i += NT) a.trail_k[((bt0 + tok) * a.Hk + g) * D + i] = s_k[tok][i] * rk[tok];
    }
  }

  // The T^2 products of q and k (as the conv left them; B2 scales them to unit vectors):
  // pair p = i T + j is k_j . k_i for j < i and k_i . q_j for j >= i. 16 pairs per wave
  // and pass, 4 lanes per pair, each lane D / 4 consecutive elements, then a sum over
  // the 4 lanes.
  {
    constexpr int EPL = D / 4;
    const int sub = lane >> 2, part = lane & 3;
    for (int p0 = 0; p0 < T * T; p0 += 16 * NW) {
      const int p = p0 + 16 * wv + sub;
      const bool live = p < T * T;
      const int pi = live ? p / T : 0, pj = live ? p - pi * T : 0;
      const bool kk = pj < pi;
      const float* x = &s_k[kk ? pj : pi][part * EPL];
      const float* y = kk ? &s_k[pi][part * EPL] : &s_q[pj][part * EPL];
      float acc = 0.0f;
      // two pieces of each vector in flight: the state is live in registers here
#pragma unroll 2
      for (int e = 0; e < EPL; e += 4) {
        const float4 xv = *reinterpret_cast<const float4*>(x + e), yv = *reinterpret_cast<const float4*>(y + e);
        acc = fmaf(xv.x, yv.x, acc);
        acc = fmaf(xv.y, yv.y, acc);
        acc = fmaf(xv.z, yv.z, acc);
        acc = fmaf(xv.w, yv.w, acc);
      }
      acc = xor_add<1>(acc);
      acc = xor_add<2>(acc);
      if (live && part == 0) {
        if (kk)
          s_kk[pi][pj] = acc;
        else
          s_kq[pj][pi] = acc;
      }
    }
  }
  // (read in B2, after the barrier that ends B1)

  // ---- B1. H0^T k_t and H0^T q_t of every token (k and q not yet scaled to unit length)
  // on the VGPR-resident state, summed
  // over the lane's rows (no barrier: each lane reads LDS written above), then over the
  // row groups and stored to LDS
  auto partial = [&](int tok, float4& m, float4& pq) {
    const float* kr = &s_k[tok][rg * R];
    const float* qr = &s_q[tok][rg * R];
    m = f4(0.0f);
    pq = f4(0.0f);
#pragma unroll
    for (int k4 = 0; k4 < R / 4; ++k4) {
      const float4 kk = *reinterpret_cast<const float4*>(kr + 4 * k4);
      const float4 qq = *reinterpret_cast<const float4*>(qr + 4 * k4);
      m = fma4(hreg[4 * k4 + 0], kk.x, m);
      m = fma4(hreg[4 * k4 + 1], kk.y, m);
      m = fma4(hreg[4 * k4 + 2], kk.z, m);
      m = fma4(hreg[4 * k4 + 3], kk.w, m);
      pq = fma4(hreg[4 * k4 + 0], qq.x, pq);
      pq = fma4(hreg[4 * k4 + 1], qq.y, pq);
      pq = fma4(hreg[4 * k4 + 2], qq.z, pq);
      pq = fma4(hreg[4 * k4 + 3], qq.w, pq);
    }
  };
  // one token: each value summed over lanes l ^ CGL, l ^ 2 CGL, ... up to l ^ 32
  auto single = [&](int tok) {
    float4 m, pq;
    partial(tok, m, pq);
    if constexpr (CGL <= 1) xor_round<1>(m, pq);
    if constexpr (CGL <= 2) xor_round<2>(m, pq);
    if constexpr (CGL <= 4) xor_round<4>(m, pq);
    if constexpr (CGL <= 8) xor_round<8>(m, pq);
    if constexpr (CGL <= 16) xor_round<16>(m, pq);
    xor_round<32>(m, pq);
    if (rg == 0) {
      *reinterpret_cast<float4*>(&s_hk[tok][4 * cg]) = m;
      *reinterpret_cast<float4*>(&s_hq[tok][4 * cg]) = pq;
    }
  };
  if constexpr (CGL == 8) {
    // Row groups are lane bits 3-5. Two tokens at a time, transposed: the 16 values
    // (m, pq of token t0, then of t0 + 1) go through the 32-lane swaps (register i of
    // the lower half-wave keeps value i, of the upper value i + 8), the 16-lane swaps
    // (register j of row r holds value j + 4 (r & 1) + 8 (r >> 1)) and a DPP row_ror:8
    // sum; lanes with bit 3 clear store their 4 values. An odd last token goes alone.
    int t0 = 0;
    for (; t0 + 1 < T; t0 += 2) {
      float4 m0, p0, m1, p1;
      partial(t0, m0, p0);
      partial(t0 + 1, m1, p1);
      float v[16] = {m0.x, m0.y, m0.z, m0.w, p0.x, p0.y, p0.z, p0.w, m1.x, m1.y, m1.z, m1.w, p1.x, p1.y, p1.z, p1.w};
      float hh[8], qq[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float x0 = v[i], x1 = v[i + 8];
        asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x0), "+v"(x1));
        hh[i] = x0 + x1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x0 = hh[j], x1 = hh[j + 4];
        asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x0), "+v"(x1));
        qq[j] = x0 + x1;
        qq[j] += dpp_mov<0x128>(qq[j]);
      }
      const int r = lane >> 4, vb = 4 * (r & 1) + 8 * (r >> 1);  // value index of qq[0]
      const int tok = vb < 8 ? t0 : t0 + 1;
      if ((lane & 8) == 0) {
        float* dst = (vb & 4) ? &s_hq[tok][4 * cg] : &s_hk[tok][4 * cg];
        *reinterpret_cast<float4*>(dst) = make_float4(qq[0], qq[1], qq[2], qq[3]);
      }
    }
    if (t0 < T) single(t0);
  } else {
    for (int tok = 0; tok < T; ++tok) single(tok);
  }
  __syncthreads();

  // ---- B2. delta_t and o_t, one thread per column c: dl holds the deltas so far,
  // gs[s] = G(s+1, t-1) and g0 = G(0, t-1) before token t's gate is applied; the
  // readouts stay in registers for phase C
  float ov[kTM];
#pragma unroll
  for (int tok = 0; tok < kTM; ++tok) ov[tok] = 0.0f;
  if (t < D) {
    const int c = t;
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    float dl[kTM], gs[kTM];
    float g0 = 1.0f;
#pragma unroll
    for (int tok = 0; tok < kTM; ++tok) {
      if (tok >= T) break;
      const float alpha = s_gate[0][tok], beta = s_gate[1][tok];
      float mt = g0 * (s_hk[tok][c] * rk[tok]);
#pragma unroll
      for (int s = 0; s < tok; ++s) mt = fmaf(gs[s] * (s_kk[tok][s] * (rk[s] * rk[tok])), dl[s], mt);
      const float delta = beta * (s_v[tok][c] - alpha * mt);
      dl[tok] = delta;
      g0 *= alpha;
#pragma unroll
      for (int s = 0; s < tok; ++s) gs[s] *= alpha;
      gs[tok] = 1.0f;
      float ot = g0 * (s_hq[tok][c] * rq[tok]);
#pragma unroll
      for (int s = 0; s <= tok; ++s) ot = fmaf(gs[s] * (s_kq[tok][s] * (rk[s] * rq[tok])), dl[s], ot);
      ov[tok] = scale * ot;
      a.trail_delta[((bt0 + tok) * a.Hv + h) * D + c] = delta;
    }
  }
  if (t < T) a.trail_alpha[(bt0 + t) * a.Hv + h] = s_gate[0][t];

  // ---- C. per-head RMSNorm: each token's squares summed over the D column threads (one
  // transposed reduction for all tokens), then the gated outputs, one column per thread
  float ss[kTM];
#pragma unroll
  for (int tok = 0; tok < kTM; ++tok) ss[tok] = (t < D && tok < T) ? ov[tok] * ov[tok] : 0.0f;
  {
    float s2[kTM / 4];  // row r holds token j + (kTM / 4) (r & 1) + (kTM / 2) (r >> 1) in register j
    wave_sums_t<kTM>(ss, s2);
    if ((lane & 15) == 0) {
      const int r = lane >> 4;
#pragma unroll
      for (int j = 0; j < kTM / 4; ++j) red[wv][j + (kTM / 4) * (r & 1) + (kTM / 2) * (r >> 1)] = s2[j];
    }
  }
  __syncthreads();
  if (t < D) {
    const int c = t;
    const float w = a.norm_w[c];
    const bool obf = a.out_bf16 != 0;
#pragma unroll
    for (int tok = 0; tok < kTM; ++tok) {
      if (tok >= T) break;
      float tot = 0.0f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) tot += red[ww][tok];
      const float r = __builtin_amdgcn_rsqf(tot / static_cast<float>(D) + a.rms_eps);
      const float y = ov[tok] * r * w * silu_rcp(Act<BF>::f(s_z[tok][c]));
      const long at = b * a.out_bs + tok * a.out_ts + static_cast<long>(h) * D + c;
      if (obf)
        static_cast<uint16_t*>(a.out)[at] = static_cast<uint16_t>(f32_to_bf16(y));
      else
        static_cast<float*>(a.out)[at] = y;
    }
  }
}


// Commit of the accepted prefix: H <- alpha_t H + k_t delta_t^T for t < n = accepted[b]
// with the recorded deltas (those the verify kernel formed its outputs from). n
// outside [1, T] leaves the sequence untouched.
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
  // up to 4 draft tokens: arrays for 4, half the LDS of the instance for 8
  if (a.T <= 4) {
    if (a.act_bf16)
      gdn_verify_kernel<D, true, 4><<<grid, VerifyLayout<D>::NT, 0, s>>>(a);
    else
      gdn_verify_kernel<D, false, 4><<<grid, VerifyLayout<D>::NT, 0, s>>>(a);
  } else {
    if (a.act_bf16)
      gdn_verify_kernel<D, true, kMaxVerifyTokens><<<grid, VerifyLayout<D>::NT, 0, s>>>(a);
    else
      gdn_verify_kernel<D, false, kMaxVerifyTokens><<<grid, VerifyLayout<D>::NT, 0, s>>>(a);
  }
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
