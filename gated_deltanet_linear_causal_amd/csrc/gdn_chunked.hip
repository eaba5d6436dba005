// Chunked multi-token GDN on MFMA (CDNA4, gfx950), head dim 128, conv taps 4.
//
// Reformulation of the per-token gated delta rule over a chunk of C tokens (derived
// from the rule of the page "linear_attention.rs", step 7, as in the published chunked
// form of Gated DeltaNet). With H0 the state before the chunk, g_t the running sum of
// log(alpha) inside the chunk and gamma_t = exp(g_t):
//   A[t][s] = beta_t exp(g_t - g_s) (k_t . k_s)   for s < t, else 0
//   (I + A) Delta = diag(beta) (V - diag(gamma) K H0)         (Delta rows = delta_t)
//   O = diag(gamma) Q H0 + P Delta,  P[t][s] = exp(g_t - g_s) (q_t . k_s) for s <= t
//   H_C = gamma_C H0 + K^T diag(exp(g_C - g)) Delta
// and o_t = O_t / sqrt(d), then the per-head gated RMSNorm as in the decode step.
// Tokens are processed in order; the result equals the token-by-token recurrence up
// to rounding.
//
// Work unit: one workgroup (4 waves) per (sequence, v-head), looping over chunks.
// The 128x128 state lives in MFMA accumulators for the whole sequence: wave w owns
// columns 32w .. 32w+31 (8 x 2 tiles of 16x16). An accumulator tile, lane l holding
// rows 4(l/16)+r, column l%16, is exactly the B-operand layout of the 16x16x32 f16
// MFMA when the contraction index of each 32-block is ordered (4q..4q+3, 16+4q..
// 16+4q+3) for lane group q: two stacked accumulator tiles feed B directly, and the
// A operand reads the same permuted columns from LDS (two 8-byte reads).
// Precision: every operand is split into two fp16 halves (x = hi + lo, 22 significant
// bits) and each product is evaluated as hi*hi + hi*lo + lo*hi with fp32 accumulation,
// ~2^-21 relative per product; the three MFMAs of an accumulator are issued apart,
// interleaved with independent ones. A bf16 split (8 + 8 bits) measured ~1e-4 relative
// error on the outputs, too coarse for the fp32 recurrence. Operands must stay below
// the fp16 range (6.5e4); the normalised q, k, the state and delta of this layer are
// orders of magnitude smaller.
// The running sums g_t are kept in fp64: in a strongly decaying head g reaches -1e3
// and beyond within a chunk, where an fp32 sum would carry ~1e-4 absolute error into
// every exp(g_t - g_s); each difference is formed in fp64 and only then rounded.
// The (I + A) solve is an fp32 forward substitution on VALU, two lanes per column.
// With bf16 activations, the next chunk's conv inputs, z rows and gate inputs are
// loaded while it runs and stored to LDS after it.
//
// The conv state is only read here; a separate epilogue launch writes the rolled
// state afterwards (two workgroups of a k-head read the same Q/K conv columns).

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kD = 128;   // head dim (d_k = d_v)
constexpr int kC = 32;    // tokens per chunk
constexpr int kNT = 256;  // 4 waves
constexpr int kQKLd = kD + 8;  // bf16 row stride of the [t][i] planes
constexpr int kKTLd = kC + 8;  // bf16 row stride of the [i][t] planes
constexpr int kPLd = kC + 8;   // bf16 row stride of the [t][s] planes
constexpr int kALd = kC + 4;   // fp32 row stride of A
constexpr int kXLd = kD + 4;   // fp32 row stride of the [t][j] buffers
constexpr int kRawLd = 2 * kD + 4;
// Operands bounded by 1 in magnitude (normalised q, k and the decayed scores P) are
// split after scaling by 2^15: fp16 keeps 11 significant bits only above 6.1e-5, so
// unscaled the strongly decayed entries of P would carry an absolute error of ~3e-8
// each (measured: ~1e-4 relative error on late tokens of a chunk). Products with
// these operands go to fresh accumulators and are scaled back by 2^-15 in fp32.
constexpr float kUp = 32768.0f, kDown = 1.0f / 32768.0f;

constexpr int kUnits = 3 * kD;  // conv channels of a workgroup: q, k of its k-head, v of its v-head
constexpr int kPairs = kUnits / 2;  // bf16 channel pairs (one dword each)
constexpr int kTaps = 4;             // conv taps (K)

// Inputs of the next chunk, prefetched into LDS while the current chunk is solved
// (bf16 activations only; with fp32 activations the inputs are read directly). Row
// j of x holds the conv inputs of token j - 3 of the chunk: rows 0..2 are the three
// inputs before it (the conv state for the first chunk), so every conv output of the
// chunk can be formed from LDS alone.
template <bool BF>
struct Staging {
  alignas(16) uint32_t x[kC + kTaps - 1][kPairs + 4];  // two bf16 channels per word
  alignas(16) uint32_t z[2][kC][kD / 2 + 4];           // z rows of this v-head, double-buffered by chunk parity
};
template <>
struct Staging<false> {};

template <bool BF>
struct alignas(16) ChunkSmem {
  alignas(16) uint16_t q_hi[kC][kQKLd], q_lo[kC][kQKLd];
  alignas(16) uint16_t k_hi[kC][kQKLd], k_lo[kC][kQKLd];
  alignas(16) uint16_t kt_hi[kD][kKTLd], kt_lo[kD][kKTLd];
  union {
    float raw[kC][kRawLd];  // silu(conv) of q (0..127) and k (128..255) before the L2 norm (steps 1-2)
    struct {
      alignas(16) float at[kC][kALd];  // -A transposed, at[s][16 (t & 1) + t / 2] = -A[t][s], zero for s >= t (steps 3-4)
      float x[kC][kXLd];    // right-hand side, then Delta (steps 3-5)
      uint16_t p_hi[kC][kPLd], p_lo[kC][kPLd];  // 2^15 P (steps 3-5)
    } s;
  } u;
  float v[kC][kXLd];        // silu(conv) of v
  alignas(16) double g[2][kC];  // running sum of log(alpha) inside the chunk (fp64), by chunk parity
  alignas(16) float beta[2][kC];
  alignas(16) float ss[kC][4];  // per-wave partial sums of o^2
  Staging<BF> st;
};

// Gates of the tokens of a chunk, computed by one wave (lanes 0..31, one token each):
// beta_t = sigmoid(b_t) and the inclusive running sum over the chunk of
// log(alpha_t) = -exp(A_log) softplus(dt_t + dt_bias). Tokens past T get 0 and 0.
// `left` = tokens of the sequence from the chunk's first on.
template <bool BF>
__device__ __forceinline__ void chunk_gate_inputs(const KernelArgs& a, int b, int h, int ch, int lane, float& dt,
                                                  float& br);
__device__ __forceinline__ void chunk_gates(int left, int lane, float dt, float br, float A_exp, float dt_bias,
                                            double* g_out, float* beta_out);

// Prefetch of chunk `ch` (bf16 activations) by the four waves, wave `wv` (wave-uniform)
// taking tokens 8 wv .. 8 wv + 7: conv inputs and z rows, and (wave 0) the gates. The
// global loads go to registers first (stage_load) and the LDS stores follow later
// (stage_store), so that the loads are in flight during the work in between. A row
// segment is 64 dwords (256 bytes); one 16-byte load per lane covers four rows, lanes
// 16 r .. 16 r + 15 taking row r, so a wave's 32 rows take 8 loads. Rows of tokens past
// T (last chunk) repeat the last token: the conv outputs and the outputs of such tokens
// are masked, so their values are never used.
struct StageRegs {
  u32x4 xv[6];   // conv inputs: segment k / 2 (q, k, v) of token 8 wv + 4 (k % 2) + lane / 16
  u32x4 zv[2];   // z row of token 8 wv + 4 k + lane / 16
  float dt, br;  // gate inputs of token `lane` (used by wave 0)
};

__device__ __forceinline__ int seg_offset(int sg, int g, int h, int hk) {  // dword offset of a conv segment
  return sg == 0 ? g * (kD / 2) : (sg == 1 ? (hk + g) * (kD / 2) : (2 * hk + h) * (kD / 2));
}

// Buffer resource over `bytes` bytes from `base` (raw dwords; word 3 = 0x00020000 is the
// raw-dword format of the gfx9 family): the base lives in SGPRs and each lane supplies a
// 32-bit byte offset, so a load needs no 64-bit address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

__device__ __forceinline__ void stage_load(const KernelArgs& a, int b, int g, int h, int ch, int lane, int wv,
                                           StageRegs& r) {
  const int T = a.T, t0 = ch * kC, nt = min(kC, T - t0);
  // Row strides and segment offsets in dwords, opaque to the optimiser so that they are
  // recomputed here (a few scalar ops) instead of being held across the chunk loop.
  int cw = a.C / 2, zw = a.Hv * (kD / 2), hk = a.Hk;
  asm volatile("" : "+s"(cw), "+s"(zw), "+s"(hk));
  chunk_gate_inputs<true>(a, b, h, ch, lane, r.dt, r.br);
  const uint32_t* xb = reinterpret_cast<const uint32_t*>(a.qkv) + (static_cast<long>(b) * T + t0) * cw;
  const uint32_t* zb = reinterpret_cast<const uint32_t*>(a.z) + (static_cast<long>(b) * T + t0) * zw + h * (kD / 2);
  const __amdgpu_buffer_rsrc_t xr = rows_rsrc(xb, static_cast<uint32_t>(nt * cw) * 4u);
  const __amdgpu_buffer_rsrc_t zr = rows_rsrc(zb, static_cast<uint32_t>(nt * zw) * 4u);
  const int col = 16 * (lane & 15);  // byte offset of the lane's 4 dwords in a segment
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int t = min(8 * wv + 4 * half + (lane >> 4), nt - 1);
#pragma unroll
    for (int sg = 0; sg < 3; ++sg)
      r.xv[2 * sg + half] = __builtin_amdgcn_raw_buffer_load_b128(xr, 4 * (t * cw + seg_offset(sg, g, h, hk)) + col, 0, 0);
    r.zv[half] = __builtin_amdgcn_raw_buffer_load_b128(zr, 4 * t * zw + col, 0, 0);
  }
}

// With `first`, rows 0..2 of the staged conv inputs come from the conv state; otherwise
// wave 3 first moves the previous chunk's last three rows there (it is the wave that
// overwrites them, and a wave's LDS accesses complete in order).
__device__ __forceinline__ void stage_store(ChunkSmem<true>& sm, const KernelArgs& a, int b, int g, int h, int ch,
                                            int lane, int wv, bool first, float A_exp, float dt_bias,
                                            const StageRegs& r) {
  Staging<true>& st = sm.st;
  constexpr int kHist = (kTaps - 1) * 3;  // history rows x segments
  if (first) {
    // conv state rows 0..2 ([B][K-1][C], same channel layout as a qkv row)
    int cw = a.C / 2, hk = a.Hk;
    asm volatile("" : "+s"(cw), "+s"(hk));
    const uint32_t* cb = reinterpret_cast<const uint32_t*>(a.conv_state) + static_cast<long>(b) * (kTaps - 1) * cw;
#pragma unroll
    for (int k = 0; k < (kHist + 3) / 4; ++k) {
      const int rr = wv + 4 * k;
      if (rr < kHist) {
        const int j = rr / 3, sg = rr - 3 * j;
        st.x[j][sg * (kD / 2) + lane] = cb[j * cw + seg_offset(sg, g, h, hk) + lane];
      }
    }
  } else if (wv == 3) {
    uint32_t hist[kHist];
#pragma unroll
    for (int rr = 0; rr < kHist; ++rr) hist[rr] = st.x[kC + rr / 3][(rr % 3) * (kD / 2) + lane];
#pragma unroll
    for (int rr = 0; rr < kHist; ++rr) st.x[rr / 3][(rr % 3) * (kD / 2) + lane] = hist[rr];
  }
  if (wv == 0) chunk_gates(a.T - ch * kC, lane, r.dt, r.br, A_exp, dt_bias, sm.g[ch & 1], sm.beta[ch & 1]);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int t = 8 * wv + 4 * half + (lane >> 4);
#pragma unroll
    for (int sg = 0; sg < 3; ++sg)
      *reinterpret_cast<u32x4*>(&st.x[kTaps - 1 + t][sg * (kD / 2) + 4 * (lane & 15)]) = r.xv[2 * sg + half];
    *reinterpret_cast<u32x4*>(&st.z[ch & 1][t][4 * (lane & 15)]) = r.zv[half];
  }
}

__device__ __forceinline__ float bf16_to_f32(uint32_t u) { return __uint_as_float(u << 16); }

template <bool BF>
__device__ __forceinline__ uint32_t load_raw(const void* p, long i) {
  if constexpr (BF)
    return static_cast<const uint16_t*>(p)[i];
  else
    return static_cast<const uint32_t*>(p)[i];
}
template <bool BF>
__device__ __forceinline__ float raw_f32(uint32_t v) {
  if constexpr (BF)
    return bf16_to_f32(v);
  else
    return __uint_as_float(v);
}

// silu with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an IEEE divide
__device__ __forceinline__ float silu(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }
// log2(e) silu(u) from u2 = log2(e) u: u2 / (1 + 2^-u2). The conv weights are scaled by
// log2(e) once, so the exponent needs no multiply; the factor log2(e) then cancels in
// the L2 norms of q and k (whose epsilon is scaled by log2(e)^2) and is taken out of v
// where v enters the right-hand side of the solve.
__device__ __forceinline__ float silu_l2e(float u2) {
  return u2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u2));
}
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;

// Cross-lane adds inside a row of 16 lanes via DPP (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
// the same move for an fp64 value, one DPP per half (a lane shifted in from outside
// the row reads +0.0 in both halves)
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
  const u32x2 w = __builtin_bit_cast(u32x2, v);
  u32x2 r;
  r[0] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(w[0]), CTRL, 0xf, 0xf, true));
  r[1] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(w[1]), CTRL, 0xf, 0xf, true));
  return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ double readlane64(double v, int lane) {
  const u32x2 w = __builtin_bit_cast(u32x2, v);
  u32x2 r;
  r[0] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(w[0]), lane));
  r[1] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(w[1]), lane));
  return __builtin_bit_cast(double, r);
}
// v_permlane32_swap: lanes 32-63 of a trade places with lanes 0-31 of b (afterwards a
// holds a[0..31], b[0..31] and b holds a[32..63], b[32..63]). v_permlane16_swap: the
// odd rows of 16 lanes of a trade places with the even rows of b. Written as inline
// asm with both registers read and written: the compiler's builtins for these return
// one register for both results. Two wait states before the swap cover a VALU write
// of either operand just before it.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_rows(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// sum over the 16 lanes of each row (every lane of the row gets it)
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}
template <bool BF>
__device__ __forceinline__ void chunk_gate_inputs(const KernelArgs& a, int b, int h, int ch, int lane, float& dt,
                                                  float& br) {
  // lanes past the end read the last token (the gates mask them)
  const int t0 = ch * kC;
  const long ai = (static_cast<long>(b) * a.T + t0 + min(lane, min(kC, a.T - t0) - 1)) * a.Hv + h;
  dt = raw_f32<BF>(load_raw<BF>(a.dt_raw, ai));
  br = raw_f32<BF>(load_raw<BF>(a.b_raw, ai));
}

__device__ __forceinline__ void chunk_gates(int left, int lane, float dt, float br, float A_exp, float dt_bias,
                                            double* g_out, float* beta_out) {
  float la = 0.0f, bt = 0.0f;
  if (lane < min(kC, left)) {
    // softplus(x) = max(x, 0) + log(1 + exp(-|x|)); the log's argument lies in (1, 2]
    const float x = dt + dt_bias;
    la = -A_exp * (fmaxf(x, 0.0f) + __logf(1.0f + __expf(-fabsf(x))));
    bt = __builtin_amdgcn_rcpf(1.0f + __expf(-br));
  }
  // inclusive scan in fp64 over lanes 0..31: within each row of 16 lanes by DPP row
  // shifts (lanes shifted in from outside the row read 0), then row 1 adds row 0's total
  double g = la;
  g += dpp64<0x111>(g);  // row_shr:1
  g += dpp64<0x112>(g);  // row_shr:2
  g += dpp64<0x114>(g);  // row_shr:4
  g += dpp64<0x118>(g);  // row_shr:8
  const double row0 = readlane64(g, 15);
  if (lane >= 16) g += row0;
  if (lane < kC) {
    g_out[lane] = g;
    beta_out[lane] = bt;
  }
}

// x = hi + lo in fp16, both rounded to nearest: hi = fp16(x), lo = fp16(x - hi)
// (x - hi is exact in fp32). 11 + 11 significant bits: |x - hi - lo| <= 2^-22 |x|
// for normal values, and <= 2^-25 absolute in the fp16 subnormal range.
// `one` is 1.0f held opaque to the optimiser: x * one - hi is then a single
// v_fma_mix_f32 reading the fp16 hi directly (exact, like the subtraction it replaces)
// instead of a conversion back to fp32 followed by a subtraction.
__device__ __forceinline__ void split1(float x, uint32_t& hi, uint32_t& lo, float one) {
  const _Float16 h = static_cast<_Float16>(x);
  const _Float16 r = static_cast<_Float16>(fmaf(x, one, -static_cast<float>(h)));
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, r);
}
// two fp32 -> packed fp16 pairs (hi0 | hi1 << 16), (lo0 | lo1 << 16), same rounding as
// split1 (v_cvt_pk_f16_f32 rounds to nearest even)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo, float one) {
  const f32x2 x = {x0, x1};
  const f16x2 h = __builtin_convertvector(x, f16x2);
  const f32x2 res = {fmaf(x0, one, -static_cast<float>(h[0])), fmaf(x1, one, -static_cast<float>(h[1]))};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(res, f16x2));
}
// four fp32 -> (hi pair, hi pair), (lo pair, lo pair)
__device__ __forceinline__ void split4(f32x4 x, u32x2& hi, u32x2& lo, float one) {
  uint32_t h0, h1, l0, l1;
  split2(x[0], x[1], h0, l0, one);
  split2(x[2], x[3], h1, l1, one);
  hi[0] = h0;
  hi[1] = h1;
  lo[0] = l0;
  lo[1] = l1;
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}
// A-operand fragment of a row-major bf16 plane: row `row`, 32-column block at `k0`,
// permuted order (k0+4q .. +3, k0+16+4q .. +3) for lane group q.
__device__ __forceinline__ u32x4 frag(const uint16_t* plane, int ld, int row, int k0, int q) {
  const uint16_t* p = plane + row * ld + k0 + 4 * q;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
  u32x4 r;
  r[0] = lo[0];
  r[1] = lo[1];
  r[2] = hi[0];
  r[3] = hi[1];
  return r;
}

// B-operand fragment from two stacked accumulator-layout tiles (rows 0..15, 16..31 of
// a 32-row block), split into hi and lo.
__device__ __forceinline__ void bfrag(f32x4 top, f32x4 bottom, u32x4& hi, u32x4& lo, float one) {
  u32x2 h0, l0, h1, l1;
  split4(top, h0, l0, one);
  split4(bottom, h1, l1, one);
  hi[0] = h0[0];
  hi[1] = h0[1];
  hi[2] = h1[0];
  hi[3] = h1[1];
  lo[0] = l0[0];
  lo[1] = l0[1];
  lo[2] = l1[0];
  lo[3] = l1[1];
}

__device__ __forceinline__ void put_split(uint16_t* hi_plane, uint16_t* lo_plane, int idx, float x, float one) {
  uint32_t h, l;
  split1(x, h, l, one);
  hi_plane[idx] = static_cast<uint16_t>(h);
  lo_plane[idx] = static_cast<uint16_t>(l);
}

// The 16 outputs of a lane (rows 16 (tt ^ hw) + 4q + r, columns 32w + 16jt + c16) as
// buffer stores at byte offset vo (the lane's row 4q and column) plus the row offset;
// bf16 outputs are rounded to nearest even.
template <bool OUT_BF16>
__device__ __forceinline__ void store_rows(const float (&y)[2][4][2], __amdgpu_buffer_rsrc_t ors, int vo, int hw,
                                           int zr) {
  constexpr int esz = OUT_BF16 ? 2 : 4;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ro = vo + (16 * (tt ^ hw) + r) * zr * esz;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const float x = y[tt][r][jt];
        if constexpr (OUT_BF16) {
          // round to nearest even; a NaN stays a (quiet) NaN
          uint32_t u = __float_as_uint(x);
          u = ((u & 0x7fffffffu) > 0x7f800000u) ? (u | 0x00400000u) : u + 0x7fffu + ((u >> 16) & 1u);
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(u >> 16), ors, ro + 16 * esz * jt, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), ors, ro + 16 * esz * jt, 0, 0);
        }
      }
    }
}

template <bool BF>
__global__ __launch_bounds__(kNT) void gdn_chunk_kernel(const KernelArgs a) {
  __shared__ ChunkSmem<BF> sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, q = l >> 4, c16 = l & 15;
  const int b = blockIdx.x / a.Hv;
  const int h = blockIdx.x - b * a.Hv;
  const int g = h / a.G;
  const int T = a.T;
  const long C = a.C;

  // ---- state: wave w holds H[16 it + 4q + r][32 w + 16 jt + c16]
  float* hst = a.state + (static_cast<long>(b) * a.Hv + h) * (kD * kD);
  f32x4 hacc[8][2];
#pragma unroll
  for (int it = 0; it < 8; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) hacc[it][jt][r] = hst[(16 * it + 4 * q + r) * kD + 32 * w + 16 * jt + c16];

  const float A_exp = __expf(a.A_log[h]);
  const float dt_bias = a.dt_bias[h];
  const float rsd = 1.0f / sqrtf(static_cast<float>(kD));
  const float nw[2] = {a.norm_w[32 * w + c16], a.norm_w[32 * w + 16 + c16]};  // norm weights of the output columns

  // ---- conv weights of this lane's channels. Unit channel c of the workgroup:
  // [0,128) q of k-head g, [128,256) k of k-head g, [256,384) v of v-head h.
  // bf16: lane takes 3 work units u = tid + 256 i, each the channel pair p = u % 192
  // (unit channels 2p, 2p+1) over the 8 tokens 8 (u / 192) .. +7 of a chunk.
  // fp32: lane takes unit channel tid, and tid + 256 when below 384, over all tokens.
  constexpr int kCU = BF ? 3 : 2;  // work units (bf16) or channels (fp32) of a lane
  constexpr int kCW = BF ? 2 : 1;  // channels per unit
  float wt[kCU][kCW][kTaps];
  auto unit_channel = [&](int c) -> long {  // unit channel -> channel of the qkv row
    return c < kD ? static_cast<long>(g) * kD + c
                  : (c < 2 * kD ? static_cast<long>(a.Hk + g) * kD + (c - kD)
                                : static_cast<long>(2 * a.Hk + h) * kD + (c - 2 * kD));
  };
#pragma unroll
  for (int i = 0; i < kCU; ++i) {
    const int c0 = BF ? 2 * ((tid + kNT * i) % kPairs) : min(tid + kNT * i, kUnits - 1);
#pragma unroll
    for (int e = 0; e < kCW; ++e) {
      const long gc = unit_channel(c0 + e);
#pragma unroll
      for (int j = 0; j < kTaps; ++j) wt[i][e][j] = kLog2e * raw_f32<BF>(load_raw<BF>(a.conv_w, gc * kTaps + j));
    }
  }
  float win[2][kTaps - 1];  // fp32: the channel's last three inputs
  if constexpr (!BF) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const long gc = unit_channel(min(tid + kNT * m, kUnits - 1));
#pragma unroll
      for (int j = 0; j < kTaps - 1; ++j)
        win[m][j] = raw_f32<BF>(load_raw<BF>(a.conv_state, (static_cast<long>(b) * (kTaps - 1) + j) * C + gc));
    }
  }

  const int nchunks = (T + kC - 1) / kC;
  if constexpr (BF) {
    if (nchunks > 0) {
      const int wv = __builtin_amdgcn_readfirstlane(w);
      StageRegs sr;
      stage_load(a, b, g, h, 0, l, wv, sr);
      stage_store(sm, a, b, g, h, 0, l, wv, true, A_exp, dt_bias, sr);
    }
    __syncthreads();
  }
  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * kC;
    const int nt = min(kC, T - t0);
    const int par = ch & 1;
    // lane indices re-derived per chunk (opaque to the optimiser), so that the many
    // lane-dependent LDS addresses are recomputed instead of held across the loop
    int tid_ = tid;
    asm volatile("" : "+v"(tid_));
    float one = 1.0f;
    asm volatile("" : "+s"(one));
    const int tid = tid_;
    const int w = tid >> 6, l = tid & 63, q = l >> 4, c16 = l & 15;
    const int hw = __builtin_amdgcn_readfirstlane(w) >> 1;  // row block of the wave's K K^T / Q K^T tile

    // ---- 1. conv + SiLU of this chunk's tokens (and, fp32, the gates)
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < kCU; ++i) {
        const int u = tid + kNT * i, p = u % kPairs, t8 = 8 * (u / kPairs);
        float xl[8 + kTaps - 1], xh[8 + kTaps - 1];  // inputs of channels 2p, 2p+1
#pragma unroll
        for (int j = 0; j < 8 + kTaps - 1; ++j) {
          const uint32_t wv = sm.st.x[t8 + j][p];
          xl[j] = bf16_to_f32(wv & 0xffffu);
          xh[j] = __uint_as_float(wv & 0xffff0000u);
        }
        float* dst = p < kD ? &sm.u.raw[0][2 * p] : &sm.v[0][2 * p - 2 * kD];
        const int ld = p < kD ? kRawLd : kXLd;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float u0 = wt[i][0][0] * xl[e], u1 = wt[i][1][0] * xh[e];
#pragma unroll
          for (int j = 1; j < kTaps; ++j) {
            u0 = fmaf(wt[i][0][j], xl[e + j], u0);
            u1 = fmaf(wt[i][1][j], xh[e + j], u1);
          }
          // tokens past the end (last chunk) repeat the last input row: finite values
          // whose beta is 0, so their delta rows are exactly 0 and they change nothing
          *reinterpret_cast<f32x2*>(dst + (t8 + e) * ld) = f32x2{silu_l2e(u0), silu_l2e(u1)};
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m == 1 && tid >= kUnits - kNT) break;
        const long gc = unit_channel(tid + kNT * m);
        constexpr int kTB = 8;  // tokens loaded per batch of loads
#pragma unroll 1
        for (int tb = 0; tb < kC; tb += kTB) {
          // tokens past the end (last chunk) repeat the last input: finite values whose
          // beta is 0, so their delta rows are exactly 0 and they change nothing (a zero
          // row would give 0 * rsq(0) = NaN in the L2 norm when l2_eps is 0)
          uint32_t xv[kTB];
#pragma unroll
          for (int e = 0; e < kTB; ++e)
            xv[e] = load_raw<BF>(a.qkv, (static_cast<long>(b) * T + t0 + min(tb + e, nt - 1)) * C + gc);
#pragma unroll
          for (int e = 0; e < kTB; ++e) {
            const int t = tb + e;
            const float xf = raw_f32<BF>(xv[e]);
            float uu = wt[m][0][0] * win[m][0];
            uu = fmaf(wt[m][0][1], win[m][1], uu);
            uu = fmaf(wt[m][0][2], win[m][2], uu);
            uu = fmaf(wt[m][0][3], xf, uu);
            const float val = silu_l2e(uu);
            if (m == 0)
              sm.u.raw[t][tid] = val;
            else
              sm.v[t][tid] = val;
            if (t < nt) {
              win[m][0] = win[m][1];
              win[m][1] = win[m][2];
              win[m][2] = xf;
            }
          }
        }
      }
      if (w == 0) {
        float dt = 0.0f, br = 0.0f;
        chunk_gate_inputs<BF>(a, b, h, ch, l, dt, br);
        chunk_gates(T - t0, l, dt, br, A_exp, dt_bias, sm.g[par], sm.beta[par]);
      }
    }
    __syncthreads();

    // The next chunk's inputs (bf16 activations) are loaded here and stored to LDS after
    // the solve: phases 2 and 3 cover the loads' latency.
    const int wv = __builtin_amdgcn_readfirstlane(w);
    [[maybe_unused]] StageRegs sr;
    const int chn = min(ch + 1, nchunks - 1);
    if constexpr (BF) stage_load(a, b, g, h, chn, l, wv, sr);

    // ---- 2. L2 norms of q and k; split planes [t][i] and [i][t]. Wave w takes tokens
    // 8w .. 8w+7, lane l channels 2l and 2l+1; the 16 reductions run side by side.
    {
      constexpr int kTW = kC / 4;
      const int tb = w * kTW;
      const float l2_eps = a.l2_eps * (kLog2e * kLog2e);  // q, k carry the factor log2(e)
      float2 qv[kTW], kv[kTW];
      float ss[2 * kTW];
#pragma unroll
      for (int tt = 0; tt < kTW; ++tt) {
        qv[tt] = *reinterpret_cast<const float2*>(&sm.u.raw[tb + tt][2 * l]);
        kv[tt] = *reinterpret_cast<const float2*>(&sm.u.raw[tb + tt][kD + 2 * l]);
      }
#pragma unroll
      for (int tt = 0; tt < kTW; ++tt) {
        ss[2 * tt] = qv[tt].x * qv[tt].x + qv[tt].y * qv[tt].y;
        ss[2 * tt + 1] = kv[tt].x * kv[tt].x + kv[tt].y * kv[tt].y;
      }
      // The 16 sums over the wave, transposed: each exchange step halves the values a
      // lane carries while doubling the lanes each covers. After the 32-lane swaps value
      // i (i < 8) lives in lanes 0-31 and value i + 8 in lanes 32-63, each summed over
      // lanes l and l ^ 32; after the 16-lane swaps register j of row r holds value
      // j + 4 r summed over l, l ^ 16, l ^ 32, l ^ 48; a row sum completes it.
      float h8[kTW];
#pragma unroll
      for (int i = 0; i < kTW; ++i) {
        float x0 = ss[i], x1 = ss[i + kTW];
        swap_halves(x0, x1);
        h8[i] = x0 + x1;
      }
      float h4[kTW / 2];
#pragma unroll
      for (int j = 0; j < kTW / 2; ++j) {
        float x0 = h8[j], x1 = h8[j + kTW / 2];
        swap_rows(x0, x1);
        h4[j] = __builtin_amdgcn_rsqf(row16_sum(x0 + x1) + l2_eps);
      }
#pragma unroll
      for (int i = 0; i < 2 * kTW; ++i)
        ss[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, h4[i % 4]), 16 * (i / 4)));
      float kn[2][kTW];  // normalised k of channels 2l, 2l+1
#pragma unroll
      for (int tt = 0; tt < kTW; ++tt) {
        const int t = tb + tt;
        const float rq = ss[2 * tt], rk = ss[2 * tt + 1];
        uint32_t h, lo;
        split2(qv[tt].x * rq * kUp, qv[tt].y * rq * kUp, h, lo, one);
        *reinterpret_cast<uint32_t*>(&sm.q_hi[t][2 * l]) = h;
        *reinterpret_cast<uint32_t*>(&sm.q_lo[t][2 * l]) = lo;
        kn[0][tt] = kv[tt].x * rk;
        kn[1][tt] = kv[tt].y * rk;
        split2(kn[0][tt] * kUp, kn[1][tt] * kUp, h, lo, one);
        *reinterpret_cast<uint32_t*>(&sm.k_hi[t][2 * l]) = h;
        *reinterpret_cast<uint32_t*>(&sm.k_lo[t][2 * l]) = lo;
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 hv, lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t h, lo;
          split2(kn[c][2 * e], kn[c][2 * e + 1], h, lo, one);
          hv[e] = h;
          lv[e] = lo;
        }
        *reinterpret_cast<u32x4*>(&sm.kt_hi[2 * l + c][tb]) = hv;
        *reinterpret_cast<u32x4*>(&sm.kt_lo[2 * l + c][tb]) = lv;
      }
    }
    __syncthreads();

    // ---- 3. K K^T and Q K^T (32 x 32), K H0 and Q H0 (this wave's columns) on MFMA, in
    // one pass over the K and Q fragments. Wave w computes tile (w/2, w%2) of K K^T and
    // Q K^T (tile (0, 1) lies above the diagonal: all its entries are masked). The wave
    // holds its fragments with its own row block first, slot lt holding row block
    // lt ^ hw (hw = w / 2), so the A operand of its K K^T / Q K^T tile is always slot 0;
    // the accumulators of K H0, Q H0 and O follow the same slots.
    f32x4 kh[2][2], qh[2][2];
#pragma unroll
    for (int lt = 0; lt < 2; ++lt)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        kh[lt][jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        qh[lt][jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    // two accumulators each for K K^T and Q K^T (even and odd blocks), so that the three
    // MFMAs of one are issued apart
    f32x4 kk2[2] = {}, qk2[2] = {};
    // Factors of the epilogues, formed before the products so that their LDS reads and
    // exponentials overlap the MFMAs. Tile (w/2, w%2), rows t = 16 hw + 4q + r, column
    // s = 16 (w % 2) + c16: ea = -beta_t exp(g_t - g_s) 2^-30 for s < t, else 0 (A from
    // 2^30 k_t.k_s), eb = exp(g_t - g_s) 2^-15 for s <= t, else 0 (2^15 P from 2^30 q_t.k_s).
    // Rows of slot lt (t = 16 (lt ^ hw) + 4q + r), column j: rhs = c1v + c3 (2^15 K H0) with
    // c1v = beta_t ln2 v_t[j] (v is stored as log2(e) v), c3 = -beta_t ln2 gamma_t 2^-15
    // log2(e); O starts as c4 (2^15 Q H0), c4 = gamma_t 2^-15.
    float ea[4], eb[4];
    {
      const int t4 = 16 * hw + 4 * q, s = 16 * (w & 1) + c16;
      const double* gt = &sm.g[par][t4];
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[par][t4]);
      const double gs = sm.g[par][s];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t4 + r;
        // exp(g_t - g_s) <= 1 for s <= t; the other entries are masked (argument clamped)
        const float e = (s <= t) ? __expf(fminf(static_cast<float>(gt[r] - gs), 0.0f)) : 0.0f;
        ea[r] = (s < t) ? -(bt[r] * e * (kDown * kDown)) : 0.0f;
        eb[r] = e * kDown;
      }
    }
    float c1v[2][4][2], c3[2][4], c4[2][4];
#pragma unroll
    for (int lt = 0; lt < 2; ++lt) {
      const int t4 = 16 * (lt ^ hw) + 4 * q;
      const double* gt = &sm.g[par][t4];
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[par][t4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gam = __expf(static_cast<float>(gt[r])), c1 = bt[r] * kLn2;
        c3[lt][r] = -c1 * (gam * (kDown * kLog2e));
        c4[lt][r] = gam * kDown;
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) c1v[lt][r][jt] = c1 * sm.v[t4 + r][32 * w + 16 * jt + c16];
      }
    }
    {
      const bool same = (w & 1) == hw;  // B operand (K rows of block w % 2) in slot 0, else slot 1
      // Operands of block kb: K and Q fragments fq[kb & 1] (8: slot lt, plane k_hi, k_lo,
      // q_hi, q_lo) and the split state hb*[kb & 1] (8 pairs: column tile jt, rows
      // 32 kb + 4q + {0,1 | 2,3} and 16 + ...). Those of block kb + 1 are produced one
      // slice at a time between the MFMAs of block kb, each slice with two MFMAs behind
      // a scheduling barrier, so that the loads and splits issue while the matrix core
      // works instead of before it.
      u32x4 fq[2][2][4];
      u32x4 hbh[2][2], hbl[2][2];
      auto frag_slice = [&](int kb, int k, u32x4(&dst)[2][4]) {
        const int lt = k >> 2, pl = k & 3;
        const uint16_t* plane = pl == 0 ? &sm.k_hi[0][0] : (pl == 1 ? &sm.k_lo[0][0] : (pl == 2 ? &sm.q_hi[0][0] : &sm.q_lo[0][0]));
        dst[lt][pl] = frag(plane, kQKLd, 16 * (lt ^ hw) + c16, 32 * kb, q);
      };
      auto split_slice = [&](int kb, int k, u32x4(&hh)[2], u32x4(&hl)[2]) {
        const int jt = k >> 2, e = k & 3;
        const f32x4 src = e < 2 ? hacc[2 * kb][jt] : hacc[2 * kb + 1][jt];
        uint32_t h_, l_;
        split2(src[2 * (e & 1)], src[2 * (e & 1) + 1], h_, l_, one);
        hh[jt][e] = h_;
        hl[jt][e] = l_;
      };
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        frag_slice(0, k, fq[0]);
        split_slice(0, k, hbh[0], hbl[0]);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int cb = kb & 1, nb = cb ^ 1;
        const u32x4(&f0)[4] = fq[cb][0];
        const u32x4 bkh = same ? fq[cb][0][0] : fq[cb][1][0];
        const u32x4 bkl = same ? fq[cb][0][1] : fq[cb][1][1];
        // hi*hi, hi*lo, lo*hi of all ten accumulators in turn (independent neighbours)
#pragma unroll
        for (int part = 0; part < 3; ++part) {
          kk2[kb & 1] = mfma(part == 2 ? f0[1] : f0[0], part == 1 ? bkl : bkh, kk2[kb & 1]);
          qk2[kb & 1] = mfma(part == 2 ? f0[3] : f0[2], part == 1 ? bkl : bkh, qk2[kb & 1]);
#pragma unroll
          for (int lt = 0; lt < 2; ++lt)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              const u32x4(&f)[4] = fq[cb][lt];
              const u32x4 bb = part == 1 ? hbl[cb][jt] : hbh[cb][jt];
              kh[lt][jt] = mfma(part == 2 ? f[1] : f[0], bb, kh[lt][jt]);
              qh[lt][jt] = mfma(part == 2 ? f[3] : f[2], bb, qh[lt][jt]);
              const int k = 4 * part + 2 * lt + jt;
              if (kb + 1 < 4 && k < 8) {
                frag_slice(kb + 1, k, fq[nb]);
                split_slice(kb + 1, k, hbh[nb], hbl[nb]);
              }
              // (the last block has no fences: the epilogues below may start among its
              // MFMAs once the products they read are final)
              if (kb + 1 < 4) __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
    }
    // A and P of tile (w / 2, w % 2)
    {
      const f32x4 kk = kk2[0] + kk2[1], qk = qk2[0] + qk2[1];
      const int t4 = 16 * hw + 4 * q, s = 16 * (w & 1) + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t4 + r;
        sm.u.s.at[s][16 * (t & 1) + (t >> 1)] = ea[r] * kk[r];
        put_split(&sm.u.s.p_hi[0][0], &sm.u.s.p_lo[0][0], t * kPLd + s, eb[r] * qk[r], one);  // = 2^15 P
      }
    }

    // rhs[t][j] = beta_t (v_t[j] - gamma_t (K H0)[t][j]);  O starts as gamma_t (Q H0)[t][j]
    f32x4 oacc[2][2];  // slot lt: rows of block lt ^ hw
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t4 = 16 * (tt ^ hw) + 4 * q;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          sm.u.s.x[t4 + r][32 * w + 16 * jt + c16] = fmaf(c3[tt][r], kh[tt][jt][r], c1v[tt][r][jt]);
          oacc[tt][jt][r] = c4[tt][r] * qh[tt][jt][r];
        }
    }
    __syncthreads();

    // ---- 4. forward substitution (I + A) Delta = rhs in right-looking order: once
    // delta_s is final it is eliminated from every later row, so the updates of different
    // rows are independent. Two lanes per column j (all four waves): lane parity p holds
    // the rows t = 2i + p; at step s the lane holding row s passes delta_s to its partner
    // by DPP. With bf16 activations the next chunk's inputs are stored to LDS afterwards.
    {
      const int j = 32 * w + (l >> 1), p = l & 1;
      float d[kC / 2];
#pragma unroll
      for (int i = 0; i < kC / 2; ++i) d[i] = sm.u.s.x[2 * i + p][j];
      // rows of -A^T (this lane's parity) are read two rows ahead of their use; at step s
      // the rows i >= lo(s) are updated (for s even and p = 0 that includes row s itself,
      // whose coefficient is 0)
      auto lo = [](int s_) { return (s_ & 1) ? (s_ >> 1) + 1 : (s_ >> 1); };
      constexpr int kAhead = 2;
      f32x4 ring[kAhead + 1][kC / 8];
      auto fetch = [&](int s_, f32x4(&dst)[kC / 8]) {
#pragma unroll
        for (int i4 = lo(s_) / 4; i4 < kC / 8; ++i4) dst[i4] = *reinterpret_cast<const f32x4*>(&sm.u.s.at[s_][16 * p + 4 * i4]);
      };
#pragma unroll
      for (int s = 0; s < kAhead; ++s) fetch(s, ring[s]);
      // delta_s from the lane holding row s: quad_perm [0,0,2,2] (even lane of the pair)
      // or [1,1,3,3] (odd lane)
      float ds = dpp<0xA0>(d[0]);
#pragma unroll
      for (int s = 0; s < kC - 1; ++s) {
        if (s + kAhead < kC - 1) fetch(s + kAhead, ring[(s + kAhead) % (kAhead + 1)]);
        const f32x4(&m)[kC / 8] = ring[s % (kAhead + 1)];
        // the next pivot row (s + 1, slot (s + 1) / 2, always updated at step s) first, so
        // that its hand-off overlaps the other updates of this step
        // (two more updates separate it from the DPP read of its result); scheduling
        // barriers keep the next step's updates, which wait for the hand-off, behind this
        // step's
        const int in = (s + 1) >> 1;
        d[in] = fmaf(m[in >> 2][in & 3], ds, d[in]);
#pragma unroll
        for (int i = in + 1; i < min(in + 3, kC / 2); ++i) d[i] = fmaf(m[i >> 2][i & 3], ds, d[i]);
        float dn = 0.0f;
        if (s + 1 < kC - 1) dn = ((s + 1) & 1) ? dpp<0xF5>(d[in]) : dpp<0xA0>(d[in]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = lo(s); i < kC / 2; ++i)
          if (i < in || i >= in + 3) d[i] = fmaf(m[i >> 2][i & 3], ds, d[i]);
        __builtin_amdgcn_sched_barrier(0);
        ds = dn;
      }
#pragma unroll
      for (int i = 0; i < kC / 2; ++i) sm.u.s.x[2 * i + p][j] = d[i];
      if constexpr (BF) {
        if (ch + 1 < nchunks) stage_store(sm, a, b, g, h, ch + 1, l, wv, false, A_exp, dt_bias, sr);
      }
    }
    __syncthreads();

    // ---- 5. O += P Delta;  H = gamma_C H + K^T diag(exp(g_C - g)) Delta
    {
      // operand fragments first: P rows of this wave's two row tiles, K^T rows of all 8
      u32x4 ph[2], pl[2], kth[8], ktl[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        ph[tt] = frag(&sm.u.s.p_hi[0][0], kPLd, 16 * (tt ^ hw) + c16, 0, q);  // slot order, as oacc
        pl[tt] = frag(&sm.u.s.p_lo[0][0], kPLd, 16 * (tt ^ hw) + c16, 0, q);
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        kth[it] = frag(&sm.kt_hi[0][0], kKTLd, 16 * it + c16, 0, q);
        ktl[it] = frag(&sm.kt_lo[0][0], kKTLd, 16 * it + c16, 0, q);
      }
      const double gC = sm.g[par][kC - 1];
      const float gamC = __expf(static_cast<float>(gC));
      const double* g0 = &sm.g[par][4 * q];
      const double* g1 = &sm.g[par][16 + 4 * q];
      u32x4 dh[2], dl[2], eh[2], el[2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const int j = 32 * w + 16 * jt + c16;
        f32x4 top, bot, top2, bot2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          top[r] = sm.u.s.x[4 * q + r][j];
          bot[r] = sm.u.s.x[16 + 4 * q + r][j];
          top2[r] = __expf(static_cast<float>(gC - g0[r])) * top[r];
          bot2[r] = __expf(static_cast<float>(gC - g1[r])) * bot[r];
        }
        bfrag(top, bot, dh[jt], dl[jt], one);
        bfrag(top2, bot2, eh[jt], el[jt], one);
      }
      f32x4 pd[2][2] = {};  // 2^15 P Delta
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
            pd[tt][jt] = mfma(part == 2 ? pl[tt] : ph[tt], part == 1 ? dl[jt] : dh[jt], pd[tt][jt]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[tt][jt][r] = fmaf(pd[tt][jt][r], kDown, oacc[tt][jt][r]);
#pragma unroll
      for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int r = 0; r < 4; ++r) hacc[it][jt][r] *= gamC;
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
            hacc[it][jt] = mfma(part == 2 ? ktl[it] : kth[it], part == 1 ? el[jt] : eh[jt], hacc[it][jt]);
    }

    // ---- 6. gated RMSNorm of o = O / sqrt(d) and the output rows
    {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float s4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = 0.0f;
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) v += oacc[tt][jt][r] * oacc[tt][jt][r];
          v = row16_sum(v);
          s4[r] = v;
        }
        if (c16 == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.ss[16 * (tt ^ hw) + 4 * q + r][w] = s4[r];
        }
      }
      __syncthreads();
      // all inputs first (row sums, z), then the 16 outputs of this lane, then the stores
      const long zrow = static_cast<long>(a.Hv) * kD;
      const long row0 = (static_cast<long>(b) * T + t0) * zrow + static_cast<long>(h) * kD;
      f32x4 sv[2][4];
      float zz[2][4][2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * (tt ^ hw) + 4 * q + r;
          sv[tt][r] = *reinterpret_cast<const f32x4*>(&sm.ss[t][0]);
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const int j = 32 * w + 16 * jt + c16;
            if constexpr (BF)
              zz[tt][r][jt] = bf16_to_f32((sm.st.z[par][t][j >> 1] >> (16 * (j & 1))) & 0xffffu);
            else
              zz[tt][r][jt] = raw_f32<BF>(load_raw<BF>(a.z, row0 + min(t, nt - 1) * zrow + j));
          }
        }
      float y[2][4][2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 v4 = sv[tt][r];
          const float tot = (v4[0] + v4[1] + v4[2] + v4[3]) * (rsd * rsd);
          const float rr = __builtin_amdgcn_rsqf(tot * (1.0f / kD) + a.rms_eps);
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) y[tt][r][jt] = oacc[tt][jt][r] * rsd * rr * nw[jt] * silu(zz[tt][r][jt]);
        }
      // The chunk's nt output rows form one buffer resource: rows past the end of the
      // sequence (last chunk) fall outside it and are not written (hardware range check).
      // The lane's part of the byte offset (row 4q, column 32w + c16) is fixed; the row
      // block and r are wave-uniform.
      const int esz = a.out_bf16 ? 2 : 4;
      const int zr = a.Hv * kD;  // elements per token row
      const __amdgpu_buffer_rsrc_t ors = rows_rsrc(
          static_cast<char*>(a.out) + ((static_cast<long>(b) * T + t0) * zr + static_cast<long>(h) * kD) * esz,
          static_cast<uint32_t>(nt * zr * esz));
      const int vo = (4 * q * zr + 32 * w + c16) * esz;
      if (a.out_bf16)
        store_rows<true>(y, ors, vo, hw, zr);
      else
        store_rows<false>(y, ors, vo, hw, zr);
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }

#pragma unroll
  for (int it = 0; it < 8; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) hst[(16 * it + 4 * q + r) * kD + 32 * w + 16 * jt + c16] = hacc[it][jt][r];
}

// Final conv state after T tokens: row j of the K-1 rows is element T + j of the
// sequence (old rows 0..K-2, x_0 .. x_{T-1}); a bit-exact copy. One thread per
// (sequence, channel); rows are visited in increasing order, so an old row is read
// before it is overwritten.
template <bool BF>
__global__ __launch_bounds__(256) void gdn_conv_state_tail(const KernelArgs a) {
  const long C = a.C;
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(a.B) * C) return;
  const long b = idx / C, c = idx - b * C;
  const int Km1 = a.K - 1;
  const long T = a.T;
  for (int j = 0; j < Km1; ++j) {
    const long e = T + j;  // element of the combined sequence
    uint32_t v;
    if (e < Km1)
      v = load_raw<BF>(a.conv_state, (b * Km1 + e) * C + c);
    else
      v = load_raw<BF>(a.qkv, (b * T + (e - Km1)) * C + c);
    if constexpr (BF)
      static_cast<uint16_t*>(a.conv_state)[(b * Km1 + j) * C + c] = static_cast<uint16_t>(v);
    else
      static_cast<uint32_t*>(a.conv_state)[(b * Km1 + j) * C + c] = v;
  }
}

}  // namespace

bool chunked_supported(int d, int K) { return d == kD && K == 4; }

hipError_t launch_chunked_sequence(const KernelArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv));
  const dim3 tail_grid(static_cast<unsigned>((static_cast<long>(a.B) * a.C + 255) / 256));
  if (a.act_bf16) {
    gdn_chunk_kernel<true><<<grid, kNT, 0, s>>>(a);
    gdn_conv_state_tail<true><<<tail_grid, 256, 0, s>>>(a);
  } else {
    gdn_chunk_kernel<false><<<grid, kNT, 0, s>>>(a);
    gdn_conv_state_tail<false><<<tail_grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace gdn
