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

#include "gdn_internal.h"

namespace gdn {
namespace {

// ----------------------------------------------------------------------------------
// element access
// ----------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t u) { return __uint_as_float(u << 16); }

// Round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Activation storage: bf16 (BF = true) or fp32. Raw values are the stored bits.
template <bool BF>
struct Act {
  using raw_t = typename std::conditional<BF, uint16_t, uint32_t>::type;
  __device__ static __forceinline__ raw_t raw(const void* p, long i) { return static_cast<const raw_t*>(p)[i]; }
  __device__ static __forceinline__ void put(void* p, long i, raw_t v) { static_cast<raw_t*>(p)[i] = v; }
  __device__ static __forceinline__ float f(raw_t v) { return BF ? bf16_to_f32(v) : __uint_as_float(v); }
  __device__ static __forceinline__ float load(const void* p, long i) { return f(raw(p, i)); }
  // 4 consecutive elements (8-byte aligned for bf16, 16-byte for fp32)
  __device__ static __forceinline__ float4 load4(const void* p, long i) {
    if constexpr (BF) {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
      return make_float4(bf16_to_f32(w.x & 0xffffu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xffffu),
                         bf16_to_f32(w.y >> 16));
    } else {
      return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    }
  }
};

__device__ __forceinline__ void store_out4(void* p, long i, float4 v, bool bf16) {
  if (bf16) {
    uint2 w;
    w.x = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
    w.y = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = v;
  }
}

// Raw buffer access to a workgroup's state slice: the slice base and size live in
// SGPRs (buffer resource), each lane keeps one 32-bit byte offset, and the per-row
// offset is a uniform SGPR, so R in-flight 128-bit loads cost no address VGPRs.
// Word 3 = 0x00020000 is the raw-dword resource format of the gfx9 family.
// Accesses outside [0, bytes) read 0 and are not written (hardware range check).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// Cache policy of the state's buffer accesses (gfx940-family bits: 0 sc0, 1 nt, 4 sc1).
// STREAM = true marks loads and stores non-temporal (nt): for a state larger than the
// 256 MB Infinity Cache every step streams it from HBM anyway, and on MI355X the nt
// pair lifts the B = 512 step from ~5.45 to ~6.3 TB/s. A state that fits the cache is
// accessed with the default policy so the next step finds it there.
template <bool STREAM>
struct StatePolicy {
  static constexpr int kLoad = STREAM ? 2 : 0;
  static constexpr int kStore = STREAM ? 2 : 0;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
template <bool STREAM>
__device__ __forceinline__ float4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, StatePolicy<STREAM>::kLoad);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
template <bool STREAM>
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float4 f) {
  u32x4 v;
  v.x = __float_as_uint(f.x);
  v.y = __float_as_uint(f.y);
  v.z = __float_as_uint(f.z);
  v.w = __float_as_uint(f.w);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, StatePolicy<STREAM>::kStore);
}

// ----------------------------------------------------------------------------------
// arithmetic helpers
// ----------------------------------------------------------------------------------

__device__ __forceinline__ float silu(float u) { return u / (1.0f + __expf(-u)); }

__device__ __forceinline__ float softplus(float x) { return fmaxf(x, 0.0f) + log1pf(__expf(-fabsf(x))); }

// alpha = exp(-exp(A_log) softplus(dt + dt_bias)), beta = sigmoid(b)
// (page "linear_attention.rs", steps 4 and 5)
__device__ __forceinline__ float gate_alpha(float dt, float dt_bias, float A_log) {
  return __expf(-__expf(A_log) * softplus(dt + dt_bias));
}
__device__ __forceinline__ float gate_beta(float b) { return 1.0f / (1.0f + __expf(-b)); }

__device__ __forceinline__ float4 f4(float s) { return make_float4(s, s, s, s); }
__device__ __forceinline__ float4 operator+(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
__device__ __forceinline__ float4 operator-(float4 a, float4 b) { return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w); }
__device__ __forceinline__ float4 operator*(float s, float4 a) { return make_float4(s * a.x, s * a.y, s * a.z, s * a.w); }
__device__ __forceinline__ float4 fma4(float4 a, float s, float4 c) {
  return make_float4(fmaf(a.x, s, c.x), fmaf(a.y, s, c.y), fmaf(a.z, s, c.z), fmaf(a.w, s, c.w));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sum of NV values over the whole workgroup; every lane gets the same totals (same
// order everywhere). `red` is LDS scratch of NW*NV floats; a barrier is needed before
// `red` is written again.
template <int NW, int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float* red) {
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum(v[i]);
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) red[(threadIdx.x >> 6) * NV + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w * NV + i];
    v[i] = s;
  }
}

// Lane layout of the state pass for head dim D and P heads per pass.
template <int D, int P>
struct Layout {
  static constexpr int R = (D == 128) ? 32 : (D == 64 ? 16 : 4);  // rows per lane
  static constexpr int CG = D / 4;                                 // float4 column groups
  static constexpr int RG = D / R;                                 // row groups
  static constexpr int LPH = CG * RG;                              // lanes per head
  static constexpr int NT = P * LPH;                               // workgroup size
  static constexpr int NW = NT / 64;                               // waves
  static constexpr int WPH = LPH / 64;                             // waves per head
  static constexpr int CGL = 64 / RG;                              // column groups per wave band
  static_assert(LPH % 64 == 0, "a head must fill whole waves");
  static_assert(CG % CGL == 0, "column groups must tile the wave bands");
};

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
// State pass of one v-head for a lane: m = H^T k, p = H^T q (reduced over the row
// groups), delta = beta (v - alpha m), H <- alpha H + k delta^T (stored when STORE),
// and returns o = H'^T q / sqrt(D) = (alpha p + (k.q) delta) / sqrt(D) for the lane's
// 4 columns.
// ----------------------------------------------------------------------------------
template <int D, int P, bool STORE, bool STREAM, int R>
__device__ __forceinline__ float4 delta_rule(float4 (&hreg)[R], const float* kr, const float* qr, float4 v4,
                                             float alpha, float beta, float kq, __amdgpu_buffer_rsrc_t srs,
                                             uint32_t voff, uint32_t soff, float4* delta_out = nullptr) {
  using L = Layout<D, P>;
  static_assert(R == L::R, "rows per lane");
  constexpr int CGL = L::CGL;
  constexpr uint32_t kRowBytes = D * 4;
  float4 m = f4(0.0f), pq = f4(0.0f);
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
#pragma unroll
  for (int msk = CGL; msk < 64; msk <<= 1) {
    m.x += __shfl_xor(m.x, msk, 64);
    m.y += __shfl_xor(m.y, msk, 64);
    m.z += __shfl_xor(m.z, msk, 64);
    m.w += __shfl_xor(m.w, msk, 64);
    pq.x += __shfl_xor(pq.x, msk, 64);
    pq.y += __shfl_xor(pq.y, msk, 64);
    pq.z += __shfl_xor(pq.z, msk, 64);
    pq.w += __shfl_xor(pq.w, msk, 64);
  }
  const float4 delta = beta * (v4 - alpha * m);
  if (delta_out) *delta_out = delta;
  // keep k out of registers across the shuffles: re-read it from LDS
  __asm__ volatile("" ::: "memory");
#pragma unroll
  for (int k4 = 0; k4 < R / 4; ++k4) {
    const float4 kk = *reinterpret_cast<const float4*>(kr + 4 * k4);
    const float kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float4& h = hreg[4 * k4 + e];
      h.x = fmaf(kv[e], delta.x, alpha * h.x);
      h.y = fmaf(kv[e], delta.y, alpha * h.y);
      h.z = fmaf(kv[e], delta.z, alpha * h.z);
      h.w = fmaf(kv[e], delta.w, alpha * h.w);
      if constexpr (STORE) buf_store4<STREAM>(srs, voff, soff + (4 * k4 + e) * kRowBytes, h);
    }
  }
  return (1.0f / sqrtf(static_cast<float>(D))) * (alpha * pq + kq * delta);
}

// Step 8 for one head: 1/sqrt(mean o^2 + eps) over the head's D columns (lanes with
// holder == true carry them). hred: LDS of NW floats; callers fence before reusing it.
template <int D, int P>
__device__ __forceinline__ float head_rms_scale(float4 o, bool holder, int ph, float* hred, float rms_eps) {
  using L = Layout<D, P>;
  float ss = holder ? (o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w) : 0.0f;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) hred[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < L::WPH; ++w) tot += hred[ph * L::WPH + w];
  return 1.0f / sqrtf(tot / static_cast<float>(D) + rms_eps);
}

// norm_weight and the silu(z) gate of steps 8-11
__device__ __forceinline__ float4 gated(float4 o, float r, float4 w4, float4 z4) {
  return make_float4(o.x * r * w4.x * silu(z4.x), o.y * r * w4.y * silu(z4.y), o.z * r * w4.z * silu(z4.z),
                     o.w * r * w4.w * silu(z4.w));
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
  float4 z4 = f4(0.0f), w4 = f4(0.0f);
  if constexpr (MODE != kModeConv) {
    dt = Act<BF>::load(a.dt_raw, b * a.ab_bs + h);
    braw = Act<BF>::load(a.b_raw, b * a.ab_bs + h);
    A_log = a.A_log[h];
    dt_bias = a.dt_bias[h];
  }
  if constexpr (MODE == kModeFused) {
    if (rg == 0) {
      z4 = Act<BF>::load4(a.z, b * a.z_bs + static_cast<long>(h) * D + 4 * cg);
      w4 = *reinterpret_cast<const float4*>(a.norm_w + 4 * cg);
    }
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
        store_out4(a.out, b * a.out_bs + static_cast<long>(h) * D + 4 * cg, gated(o, r, w4, z4), a.out_bf16 != 0);
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
      float4 z4 = f4(0.0f), w4 = f4(0.0f);
      if constexpr (MODE == kModeFused)
        if (rg == 0) {
          z4 = Act<BF>::load4(a.z, b * a.z_bs + static_cast<long>(h) * D + 4 * cg);
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
          store_out4(a.out, b * a.out_bs + static_cast<long>(h) * D + 4 * cg, gated(o, r, w4, z4), a.out_bf16 != 0);
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
  float4 z4 = f4(0.0f), w4 = f4(0.0f);
  if (rg == 0) {
    z4 = Act<BF>::load4(a.z, z0);
    w4 = *reinterpret_cast<const float4*>(a.norm_w + 4 * cg);
  }
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
    const float4 zc = z4;
    // prefetch the next token's inputs
    if (tok + 1 < a.T) {
      cr.load_x(a.qkv, b * a.qkv_bs + (tok + 1) * a.qkv_ts);
      dt = Act<BF>::load(a.dt_raw, ab0 + (tok + 1) * a.ab_ts);
      braw = Act<BF>::load(a.b_raw, ab0 + (tok + 1) * a.ab_ts);
      if (rg == 0) z4 = Act<BF>::load4(a.z, z0 + (tok + 1) * a.z_ts);
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
// Speculative verification of T <= kMaxVerifyTokens draft tokens. One workgroup per
// (sequence b, v-head h), any G and K: both states are only read, so the G workgroups
// of a k-head may all read its Q/K conv columns. The K-1 conv-state rows and the T
// token rows of the workgroup's 3D conv channels are staged in LDS, the state stays in
// VGPRs. Per token: outputs as gdn_decode_layer would give after the previous draft
// tokens, and the trail of the token's update H <- alpha H + k delta^T (delta, unit k,
// alpha), from which gdn_commit_kernel rebuilds the state after any accepted prefix.
// ----------------------------------------------------------------------------------
template <int D, bool BF>
__global__ __launch_bounds__((Layout<D, 1>::NT)) void gdn_verify_kernel(const KernelArgs a) {
  using L = Layout<D, 1>;
  constexpr int NT = L::NT, R = L::R, CGL = L::CGL, NW = L::NW;
  constexpr int NCH = 3 * D, NCPL = (NCH + NT - 1) / NT;
  constexpr int kRows = kMaxConvTaps - 1 + kMaxVerifyTokens;
  constexpr uint32_t kRowBytes = D * 4;
  __shared__ __attribute__((aligned(16))) float s_x[kRows][NCH];  // K-1 conv-state rows, then T token rows
  __shared__ __attribute__((aligned(16))) float s_q[D];
  __shared__ __attribute__((aligned(16))) float s_k[D];
  __shared__ __attribute__((aligned(16))) float s_v[D];
  __shared__ float red[NW * 4];
  __shared__ float hred[NW];

  const int t = threadIdx.x;
  const int b = blockIdx.x / a.Hv;
  const int h = blockIdx.x - b * a.Hv;
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

  // ---- small loads: conv inputs into LDS, taps, norm weight
  float wt[NCPL][kMaxConvTaps];
#pragma unroll
  for (int m = 0; m < NCPL; ++m) {
    const int c = t + m * NT;
    if (c < NCH) {
      const long gc = chan(c);
      for (int j = 0; j < K - 1; ++j) s_x[j][c] = Act<BF>::load(a.conv_state, (static_cast<long>(b) * (K - 1) + j) * C + gc);
      for (int tok = 0; tok < T; ++tok) s_x[K - 1 + tok][c] = Act<BF>::load(a.qkv, b * a.qkv_bs + tok * a.qkv_ts + gc);
#pragma unroll
      for (int j = 0; j < kMaxConvTaps; ++j) wt[m][j] = j < K ? Act<BF>::load(a.conv_w, gc * K + j) : 0.0f;
    }
  }
  float4 w4 = f4(0.0f);
  if (rg == 0) w4 = *reinterpret_cast<const float4*>(a.norm_w + 4 * cg);
  const float A_log = a.A_log[h], dt_bias = a.dt_bias[h];

  // ---- the state of head h, read only
  const uint32_t voff = static_cast<uint32_t>(rg * R) * kRowBytes + static_cast<uint32_t>(cg) * 16u;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.state + (static_cast<long>(b) * a.Hv + h) * (D * D), D * D * 4);
  float4 hreg[R];
#pragma unroll
  for (int k = 0; k < R; ++k) hreg[k] = buf_load4<false>(srs, voff, k * kRowBytes);
  __syncthreads();

  const bool obf = a.out_bf16 != 0;
  for (int tok = 0; tok < T; ++tok) {
    // conv + SiLU of the token (tap K-1 on the token itself)
#pragma unroll
    for (int m = 0; m < NCPL; ++m) {
      const int c = t + m * NT;
      if (c < NCH) {
        float u = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxConvTaps; ++j)
          if (j < K) u = fmaf(wt[m][j], s_x[tok + j][c], u);
        const float v = silu(u);
        if (c < D) s_q[c] = v;
        else if (c < 2 * D) s_k[c - D] = v;
        else s_v[c - 2 * D] = v;
      }
    }
    const long ab = b * a.ab_bs + tok * a.ab_ts + h;
    const float alpha = gate_alpha(Act<BF>::load(a.dt_raw, ab), dt_bias, A_log);
    const float beta = gate_beta(Act<BF>::load(a.b_raw, ab));
    float4 z4 = f4(0.0f);
    if (rg == 0) z4 = Act<BF>::load4(a.z, b * a.z_bs + tok * a.z_ts + static_cast<long>(h) * D + 4 * cg);
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
    const long bt = static_cast<long>(b) * T + tok;
    for (int i = t; i < D; i += NT) {
      const float kn = s_k[i] * rk;
      s_q[i] *= rq;
      s_k[i] = kn;
      if (h % a.G == 0) a.trail_k[(bt * a.Hk + g) * D + i] = kn;
    }
    __syncthreads();
    const float4 v4 = *reinterpret_cast<const float4*>(s_v + 4 * cg);
    float4 delta;
    const float4 o =
        delta_rule<D, 1, false, false>(hreg, s_k + rg * R, s_q + rg * R, v4, alpha, beta, kq, srs, voff, 0, &delta);
    if (rg == 0) *reinterpret_cast<float4*>(a.trail_delta + (bt * a.Hv + h) * D + 4 * cg) = delta;
    if (t == 0) a.trail_alpha[bt * a.Hv + h] = alpha;
    const float r = head_rms_scale<D, 1>(o, rg == 0, 0, hred, a.rms_eps);
    if (rg == 0) store_out4(a.out, b * a.out_bs + tok * a.out_ts + static_cast<long>(h) * D + 4 * cg, gated(o, r, w4, z4), obf);
    __syncthreads();  // s_q, s_k, s_v, red and hred are rewritten by the next token
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
  const int b = blockIdx.x / a.Hv;
  const int h = blockIdx.x - b * a.Hv;
  const int g = h / a.G;
  const int n = a.accepted[b];
  if (n < 1 || n > a.T) return;
  const int cg = (t >> 6) * CGL + (t & (CGL - 1));
  const int rg = (t & 63) / CGL;
  const uint32_t voff = static_cast<uint32_t>(rg * R) * kRowBytes + static_cast<uint32_t>(cg) * 16u;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.state + (static_cast<long>(b) * a.Hv + h) * (D * D), D * D * 4);
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

template <int D, int P>
hipError_t launch_seq_t(const KernelArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hk));
  const dim3 block(Layout<D, P>::NT);
  if (a.act_bf16)
    gdn_seq_kernel<D, P, true, 4><<<grid, block, 0, s>>>(a);
  else
    gdn_seq_kernel<D, P, false, 4><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_verify_d(const KernelArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv));
  if (a.act_bf16)
    gdn_verify_kernel<D, true><<<grid, Layout<D, 1>::NT, 0, s>>>(a);
  else
    gdn_verify_kernel<D, false><<<grid, Layout<D, 1>::NT, 0, s>>>(a);
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

bool step_supported(int d, int p) { return (d == 32 || d == 64 || d == 128) && (p == 1 || p == 2); }

hipError_t launch_step(int mode, int d, int p, const KernelArgs& a, hipStream_t s) {
  // fast path: K = 4 and a single pass (G == P); every other shape takes the generic one
  const bool fast = (a.K == 4) && (a.G == p);
  if (d == 128) return p == 2 ? launch_step_p<128, 2>(mode, fast, a, s) : launch_step_p<128, 1>(mode, fast, a, s);
  if (d == 64) return p == 2 ? launch_step_p<64, 2>(mode, fast, a, s) : launch_step_p<64, 1>(mode, fast, a, s);
  return p == 2 ? launch_step_p<32, 2>(mode, fast, a, s) : launch_step_p<32, 1>(mode, fast, a, s);
}

hipError_t launch_sequence(int d, int p, const KernelArgs& a, hipStream_t s) {
  if (d == 128) return p == 2 ? launch_seq_t<128, 2>(a, s) : launch_seq_t<128, 1>(a, s);
  if (d == 64) return p == 2 ? launch_seq_t<64, 2>(a, s) : launch_seq_t<64, 1>(a, s);
  return p == 2 ? launch_seq_t<32, 2>(a, s) : launch_seq_t<32, 1>(a, s);
}

}  // namespace gdn
