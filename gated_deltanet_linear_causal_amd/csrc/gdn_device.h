// Device helpers shared by the decode kernels (gdn_kernels.hip) and the speculative
// verification kernels (gdn_verify.hip): element access, buffer-resource access to the
// state, gate and norm arithmetic, the lane layout of a state pass and the delta rule.
#pragma once

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
  // 4 consecutive elements (8-byte aligned for bf16, 16-byte for fp32): raw4 loads the
  // stored words, cvt4 widens them where they are used (a conversion right after a load
  // makes the wave wait for the load there)
  using raw4_t = typename std::conditional<BF, uint2, float4>::type;
  __device__ static __forceinline__ raw4_t raw4(const void* p, long i) {
    return *reinterpret_cast<const raw4_t*>(static_cast<const raw_t*>(p) + i);
  }
  __device__ static __forceinline__ float4 cvt4(raw4_t w) {
    if constexpr (BF)
      return make_float4(bf16_to_f32(w.x & 0xffffu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xffffu),
                         bf16_to_f32(w.y >> 16));
    else
      return w;
  }
  __device__ static __forceinline__ float4 load4(const void* p, long i) { return cvt4(raw4(p, i)); }
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
// the same with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an IEEE divide
__device__ __forceinline__ float silu_rcp(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

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

// v + (v of lane ^ M), computed on the VALU instead of through the LDS crossbar
// (ds_bpermute): every lane gets exactly the value of v + __shfl_xor(v, M) (the same
// two operands; fp addition is commutative). M = 1, 2: DPP quad permutations; 4: quad
// mirror then half-row mirror; 8: row rotate by 8; 16, 32: v_permlane16_swap /
// v_permlane32_swap of two copies of v, after which the two registers hold v and its
// partner in some order. The swaps are inline asm with both registers read and written
// (the compiler's builtins return one register for both results), after two wait states.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
template <int M>
__device__ __forceinline__ float xor_add(float v) {
  if constexpr (M == 1) {
    return v + dpp_mov<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return v + dpp_mov<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    return v + dpp_mov<0x141>(dpp_mov<0x1B>(v));  // quad_perm [3,2,1,0], then row_half_mirror
  } else if constexpr (M == 8) {
    return v + dpp_mov<0x128>(v);  // row_ror:8
  } else if constexpr (M == 16) {
    float a = v, b = v;
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return a + b;
  } else {
    static_assert(M == 32, "lane mask");
    float a = v, b = v;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return a + b;
  }
}

template <int M>
__device__ __forceinline__ void xor_round(float4& m, float4& pq) {
  m.x = xor_add<M>(m.x);
  m.y = xor_add<M>(m.y);
  m.z = xor_add<M>(m.z);
  m.w = xor_add<M>(m.w);
  pq.x = xor_add<M>(pq.x);
  pq.y = xor_add<M>(pq.y);
  pq.z = xor_add<M>(pq.z);
  pq.w = xor_add<M>(pq.w);
}

__device__ __forceinline__ float wave_sum(float v) {
  v = xor_add<32>(v);
  v = xor_add<16>(v);
  v = xor_add<8>(v);
  v = xor_add<4>(v);
  v = xor_add<2>(v);
  return xor_add<1>(v);
}

// Wave sums of N values at once (N a multiple of 4), transposed: each exchange step
// halves the registers a lane carries while doubling the lanes each covers. After the
// 32-lane swaps register i < N/2 holds value i (lanes 0-31) or value i + N/2 (lanes
// 32-63), summed over lanes l and l ^ 32; after the 16-lane swaps register j < N/4 of
// row r (16 lanes) holds value j + (N/4)(r & 1) + (N/2)(r >> 1), summed over l, l ^ 16,
// l ^ 32, l ^ 48; a DPP row sum completes it. out[j] is that total on every lane of row
// r. N/2 + N/4 swaps and N adds replace N wave sums (6N exchanges and adds).
template <int N>
__device__ __forceinline__ void wave_sums_t(const float (&v)[N], float (&out)[N / 4]) {
  static_assert(N % 4 == 0, "N");
  float h[N / 2];
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    float x0 = v[i], x1 = v[i + N / 2];
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x0), "+v"(x1));
    h[i] = x0 + x1;
  }
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    float x0 = h[j], x1 = h[j + N / 4];
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x0), "+v"(x1));
    float r = x0 + x1;
    r = xor_add<1>(r);
    r = xor_add<2>(r);
    r += dpp_mov<0x141>(r);  // row_half_mirror: the other quad of the half-row
    r += dpp_mov<0x140>(r);  // row_mirror: the other half of the row
    out[j] = r;
  }
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
// RR > 0 overrides the rows per lane (fewer rows: more lanes per head, fewer VGPRs).
template <int D, int P, int RR = 0>
struct Layout {
  static constexpr int R = RR > 0 ? RR : ((D == 128) ? 32 : (D == 64 ? 16 : 4));  // rows per lane
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
  using L = Layout<D, P, R>;
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
  // reduce over the row groups: lanes l ^ CGL, l ^ 2 CGL, ... up to l ^ 32
  if constexpr (CGL <= 1) xor_round<1>(m, pq);
  if constexpr (CGL <= 2) xor_round<2>(m, pq);
  if constexpr (CGL <= 4) xor_round<4>(m, pq);
  if constexpr (CGL <= 8) xor_round<8>(m, pq);
  if constexpr (CGL <= 16) xor_round<16>(m, pq);
  xor_round<32>(m, pq);
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
template <bool RCP = false>
__device__ __forceinline__ float4 gated(float4 o, float r, float4 w4, float4 z4) {
  auto sl = [](float x) { return RCP ? silu_rcp(x) : silu(x); };
  return make_float4(o.x * r * w4.x * sl(z4.x), o.y * r * w4.y * sl(z4.y), o.z * r * w4.z * sl(z4.z),
                     o.w * r * w4.w * sl(z4.w));
}
}  // namespace
}  // namespace gdn
