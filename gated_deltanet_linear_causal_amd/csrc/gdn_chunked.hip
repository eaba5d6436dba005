// Chunked multi-token GDN on MFMA (CDNA4, gfx950), head dim 128, conv taps 4.
//
// Reformulation of the per-token gated delta rule over a chunk of C tokens (derived
// from the rule of the page "linear_attention.rs", step 7, as in the published chunked
// form of Gated DeltaNet). With H0 the state before the chunk, g_t the running sum of
// log(alpha) inside the chunk and gamma_t = exp(g_t):
//   A[t][s] = beta_t exp(g_t - g_s) (k_t . k_s)   for s < t, else 0
//   R = diag(beta) (V - diag(gamma) K H0),   Delta = (I + A)^-1 R      (rows delta_t)
//   O = diag(gamma) Q H0 + P Delta,  P[t][s] = exp(g_t - g_s) (q_t . k_s) for s <= t
//   H_C = gamma_C H0 + K^T diag(exp(g_C - g)) Delta
// and o_t = O_t / sqrt(d), then the per-head gated RMSNorm as in the decode step.
// (I + A)^-1 is taken in 2 x 2 blocks of 16 tokens: T11 = (I + A11)^-1, T22 =
// (I + A22)^-1, and Delta1 = T11 R1, Delta2 = T22 (R2 - A21 Delta1). Everything but
// the products with H0 and Delta is independent of the state.
//
// Work unit: one workgroup of 8 waves per (sequence, v-head), looping over the chunks.
// Waves 0-3 (consumers) hold the 128 x 128 state in MFMA accumulators for the whole
// sequence and do the state-dependent products of chunk c; waves 4-7 (producers)
// meanwhile build chunk c + 1's operands: its conv + SiLU, L2 norms and gates, and then
// K K^T, Q K^T, the two 16 x 16 block inverses, A21 and P. Waves w and w + 4 share a
// SIMD, so each SIMD runs one matrix-heavy and one vector-heavy wave. Two barriers per
// chunk:
//   phase 1  consumers: K H0, Q H0, R, Delta, O = gamma Q H0 + P Delta, row sums of O^2,
//                       then H = gamma_C H + K^T diag(exp(g_C - g)) Delta
//            producers: conv / norms of chunk c+1 into the other operand buffer, z rows
//                       of chunk c; then the loads of chunk c+2
//   phase 2  consumers: outputs of chunk c; Q K^T (1, 0), (1, 1) of chunk c+1 -> P
//                       (waves 0, 1); conv + SiLU of chunk c+1's v rows (waves 2, 3)
//            producers: K K^T (0, 0) -> T11, (1, 1) -> T22, (1, 0) -> A21, and
//                       Q K^T (0, 0) -> P of chunk c+1, one tile per wave; the last of
//                       them then the gates of chunk c+2 (bf16 inputs; with fp32 inputs
//                       the gates of chunk c+1 come in phase 1)
// The per-chunk buffers written in phase 1 (q, k planes, v) and the gates are
// double-buffered; those written in phase 2 (T, A21, P) are read by the consumers only
// in phase 1. The gates of chunk c+2 go into the buffer of chunk c, whose gates the
// consumers last read in phase 1.
// The A operand of the state update (K^T) is read from the [t][i] plane of k with the
// LDS transpose load (ds_read_b64_tr_b16): in each group of 16 lanes, lane i receives
// element i % 4 of the 8-byte slots addressed by lanes 4k + i / 4, k = 0..3.
//
// Precision: every operand is split into two fp16 halves (x = hi + lo, 22 significant
// bits for normal values) and each product is evaluated as hi*hi + hi*lo + lo*hi with
// fp32 accumulation. q and the scores P (bounded by 1) are scaled by 2^15 before the
// split, the products by 2^-15 after; k stays unscaled because the same plane feeds
// the state update. The 16 x 16 inverses are scaled by a power of two from their
// largest entry (T has a unit diagonal, so it may exceed 1). The running sums g_t are
// kept in fp64 and each difference is formed in fp64 before the exponential (in a
// strongly decaying head g passes -1e3 within a chunk). Operands must stay below the
// fp16 range (6.5e4); the normalised q, k, the state and delta of this layer are
// orders of magnitude smaller.
//
// The conv state is only read here; a separate launch writes the rolled state
// afterwards (two workgroups of a k-head read the same Q/K conv columns).

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;       // head dim (d_k = d_v)
constexpr int kC = 32;        // tokens per chunk
constexpr int kNT = 512;      // 8 waves: 4 consumers, 4 producers
constexpr int kTaps = 4;      // conv taps (K)
constexpr int kGateWave = 3;  // the producer wave that loads the gate inputs and scans the gates
                              // (bf16: in phase 2, after the lightest of the four tiles)
constexpr int kRows = 8 + kTaps - 1;  // conv input rows of a producer wave (8 tokens + history)
constexpr int kQKLd = kD + 4;  // halves per row of the [t][i] planes (66 dwords: the 16 rows of a
                               // fragment read start in 16 different even banks)
constexpr int kPLd = kC + 8;   // halves per row of the P planes
constexpr float kUp = 32768.0f, kDown = 1.0f / 32768.0f;
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;

// One chunk's operands, written by the producers in phase 1 (double-buffered). v row t
// keeps column j at j ^ vswz(t), so that the consumers' reads of rows t, t + 4, t + 8,
// t + 12 fall in different banks without padding.
struct Operands {
  alignas(16) uint16_t k_hi[kC][kQKLd], k_lo[kC][kQKLd];  // unit k rows
  alignas(16) uint16_t q_hi[kC][kQKLd], q_lo[kC][kQKLd];  // 2^15 unit q rows
  alignas(16) float v[kC][kD];                             // log2(e) v (see silu_l2e), swizzled
  alignas(16) double g[kC];                                // running log-gate sums
  alignas(16) float beta[kC];
  alignas(16) float gam[kC];                               // exp(g_t)
  alignas(16) float dec[kC];                               // exp(g_C - g_t), g_C = g[kC - 1]
};
__device__ __forceinline__ int vswz(int t) { return 16 * ((t >> 2) & 3); }

// z rows of this v-head for one chunk. bf16: 16 pieces of 16 bytes per row, piece pc of
// row t at position pc ^ zswz(t) (the consumers' reads of rows t, t + 4, t + 8, t + 12
// then fall in different banks); filled by DMA. fp32: padded rows, filled by stores.
template <bool BF>
struct ZRows {
  alignas(16) uint32_t z[kC][kD / 2];
};
template <>
struct ZRows<false> {
  alignas(16) float z[kC][kD + 4];
};
__device__ __forceinline__ int zswz(int t) { return 2 * ((t >> 2) & 3); }

// Conv inputs staged by DMA (bf16): per producer wave, the q, k and v segments of its 11
// rows (8 tokens and the 3 before them), 64 dwords each (two channels per dword).
template <bool BF>
struct Staging {
  alignas(16) uint32_t x[4][3][kRows][kD / 2];
};
template <>
struct Staging<false> {};

template <bool BF>
struct ChunkSmem {
  Operands op[2];
  alignas(16) uint16_t p_hi[kC][kPLd], p_lo[kC][kPLd];  // 2^15 P (tile (0,1) stays 0)
  alignas(16) uint16_t t_hi[2][16][16], t_lo[2][16][16];  // scaled T11, T22
  alignas(16) uint16_t a_hi[16][16], a_lo[16][16];        // 2^15 A21
  alignas(16) float lsc[2][16][4][4];  // L of A11, A22 for the inverses: [s][rho][kappa] = L[rho + 4 kappa][s]
  alignas(16) float wt[3 * kD][kTaps];  // log2(e) conv taps of the workgroup's q, k, v channels
  alignas(16) float rsum[kC][4];        // per consumer wave: sums of O^2 over its 32 columns
  float tscale[2];                      // 2^(E-15) of the scaled T11, T22
  ZRows<BF> zr;
  Staging<BF> stg;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t u) { return __uint_as_float(u << 16); }

// silu with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an IEEE divide
__device__ __forceinline__ float silu(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }
// log2(e) silu(u) from u2 = log2(e) u: u2 / (1 + 2^-u2). The conv taps are scaled by
// log2(e) once, so the exponent needs no multiply; the factor log2(e) then cancels in
// the L2 norms of q and k (whose epsilon is scaled by log2(e)^2) and is taken out of v
// where v enters R.
__device__ __forceinline__ float silu_l2e(float u2) {
  return u2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u2));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
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
// v_permlane32_swap: lanes 32-63 of a trade places with lanes 0-31 of b. v_permlane16_swap:
// the odd rows of 16 lanes of a trade places with the even rows of b. Inline asm with
// both registers read and written (the builtins return one register for both results);
// two wait states cover a VALU write of either operand just before the swap.
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
// maximum over the 64 lanes (every lane gets it)
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  float a = v, b = v;
  swap_rows(a, b);  // a: rows (0, 0, 2, 2), b: rows (1, 1, 3, 3)
  v = fmaxf(a, b);
  a = v;
  b = v;
  swap_halves(a, b);  // a: lanes 0-31 twice, b: lanes 32-63 twice
  return fmaxf(a, b);
}

// x = hi + lo in fp16, both rounded to nearest: hi = fp16(x), lo = fp16(x - hi)
// (x - hi is exact in fp32). `one` is 1.0f held opaque to the optimiser: x * one - hi is
// then a single v_fma_mix_f32 reading the fp16 hi directly.
__device__ __forceinline__ void split1(float x, uint32_t& hi, uint32_t& lo, float one) {
  const _Float16 hh = static_cast<_Float16>(x);
  const _Float16 rr = static_cast<_Float16>(fmaf(x, one, -static_cast<float>(hh)));
  hi = __builtin_bit_cast(uint16_t, hh);
  lo = __builtin_bit_cast(uint16_t, rr);
}
// two fp32 -> packed fp16 pairs (hi0 | hi1 << 16), (lo0 | lo1 << 16)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo, float one) {
  const f32x2 x = {x0, x1};
  const f16x2 hh = __builtin_convertvector(x, f16x2);
  const f32x2 res = {fmaf(x0, one, -static_cast<float>(hh[0])), fmaf(x1, one, -static_cast<float>(hh[1]))};
  hi = __builtin_bit_cast(uint32_t, hh);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(res, f16x2));
}
// four fp32 (an accumulator column of 4 rows) -> operand pieces of 4 halves
__device__ __forceinline__ void split4(f32x4 x, u32x2& hi, u32x2& lo, float one) {
  uint32_t h0, h1, l0, l1;
  split2(x[0], x[1], h0, l0, one);
  split2(x[2], x[3], h1, l1, one);
  hi = u32x2{h0, h1};
  lo = u32x2{l0, l1};
}
// B-operand fragment of the 16x16x32 product from two stacked accumulator tiles (rows
// 0..15 and 16..31 of a 32-row block): k-slots 0..3 of lane group q are rows 4q..4q+3
// of the top tile, slots 4..7 rows 16+4q..16+4q+3 of the bottom one. The A operands
// read their columns in the same order.
__device__ __forceinline__ void bfrag(f32x4 top, f32x4 bottom, u32x4& hi, u32x4& lo, float one) {
  typedef __attribute__((ext_vector_type(8))) float f32x8;
  const f32x8 x = {top[0], top[1], top[2], top[3], bottom[0], bottom[1], bottom[2], bottom[3]};
  const f16x8 h = __builtin_convertvector(x, f16x8);
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = fmaf(x[i], one, -static_cast<float>(h[i]));
  hi = __builtin_bit_cast(u32x4, h);
  lo = __builtin_bit_cast(u32x4, __builtin_convertvector(r, f16x8));
}

__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}
__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                               0);
}
// hi*hi + hi*lo + lo*hi
__device__ __forceinline__ f32x4 mfma32x3(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
  return mfma32(al, bh, mfma32(ah, bl, mfma32(ah, bh, c)));
}
__device__ __forceinline__ f32x4 mfma16x3(u32x2 ah, u32x2 al, u32x2 bh, u32x2 bl, f32x4 c) {
  return mfma16(al, bh, mfma16(ah, bl, mfma16(ah, bh, c)));
}

// A-operand fragment of a row-major fp16 plane for the 16x16x32 product: row `row`,
// 32-column block at k0, columns k0+4q..+3 and k0+16+4q..+3 for lane group q.
__device__ __forceinline__ u32x4 frag(const uint16_t* plane, int ld, int row, int k0, int q) {
  const uint16_t* p = plane + row * ld + k0 + 4 * q;
  const u32x2 a = *reinterpret_cast<const u32x2*>(p);
  const u32x2 b = *reinterpret_cast<const u32x2*>(p + 16);
  return u32x4{a[0], a[1], b[0], b[1]};
}
// A-operand fragment of the transposed [t][i] plane: rows i0 + c16 of plane^T, the 32
// columns t in the fragment order above (t = 4q + m, then 16 + 4q + m), by two transpose
// loads: lane (q, c16) addresses row 4q + c16/4 (then 16 + ...) at column i0 + 4 (c16 % 4).
__device__ __forceinline__ u32x4 frag_t(const uint16_t* plane, int i0, int q, int c16) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  uint16_t* p0 = const_cast<uint16_t*>(plane) + (4 * q + (c16 >> 2)) * kQKLd + i0 + 4 * (c16 & 3);
  uint16_t* p1 = p0 + 16 * kQKLd;
  const i16x4 ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 tb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  const u32x2 ua = __builtin_bit_cast(u32x2, ta), ub = __builtin_bit_cast(u32x2, tb);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// Buffer resource over `bytes` bytes from `base` (raw dwords; word 3 = 0x00020000 is the
// raw-dword format of the gfx9 family): base in SGPRs, a 32-bit byte offset per lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// ---------------------------------------------------------------------------------
// producer waves
// ---------------------------------------------------------------------------------

// LDS-only barrier: this wave's LDS accesses complete, then the workgroup barrier.
// (__syncthreads would also wait for every global load in flight, the DMA included.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Row of the conv inputs at token `tok` of sequence b, in dwords: the conv state before
// the sequence, the last token past its end (whose outputs are not stored and whose
// beta is 0).
__device__ __forceinline__ const uint32_t* input_row(const KernelArgs& a, int b, int tok, int cw) {
  return tok < 0 ? static_cast<const uint32_t*>(a.conv_state) + (static_cast<long>(b) * (kTaps - 1) + (kTaps - 1 + tok)) * cw
                 : static_cast<const uint32_t*>(a.qkv) + (static_cast<long>(b) * a.T + min(tok, a.T - 1)) * cw;
}

// bf16: producer wave p's conv inputs of chunk n (rows 8p-3 .. 8p+7 of the chunk) into
// its staging rows. Inside the sequence by DMA: per segment 3 instructions of 64 lanes x
// 16 bytes, each filling 4 rows (lane i: row e0 + i / 16, 16-byte piece i % 16; the last
// one 3 rows) from a wave-uniform row base. For the wave whose rows start before the
// sequence (conv state) or reach past its end (the last token repeated), by plain loads
// and LDS stores, which the barrier that follows makes visible.
// (one segment sg at a time, so that the instructions of a chunk can be spread over the
// conv of the chunk before)
__device__ __forceinline__ void stage_inputs(ChunkSmem<true>& sm, const KernelArgs& a, int b, int g, int h, int n,
                                             int p, int l, int sg) {
  int cw = a.C / 2, hk = a.Hk;  // dwords per token row; k-head count
  asm volatile("" : "+s"(cw), "+s"(hk));
  const int tok0 = n * kC + 8 * p - (kTaps - 1);  // token of row 0
  const int seg = (sg == 0 ? g : (sg == 1 ? hk + g : 2 * hk + h)) * (kD / 2);
  if (tok0 >= 0 && tok0 + kRows <= a.T) {
    const int lr = l >> 4, pc = l & 15;
    const uint32_t* base = static_cast<const uint32_t*>(a.qkv) + (static_cast<long>(b) * a.T + tok0) * cw + seg;
#pragma unroll
    for (int e0 = 0; e0 < kRows; e0 += 4)
      if (e0 + 4 <= kRows || lr < kRows - e0)
        __builtin_amdgcn_global_load_lds(base + (e0 + lr) * cw + 4 * pc, &sm.stg.x[p][sg][e0][0], 16, 0, 0);
  } else {
    const uint32_t* qkv = static_cast<const uint32_t*>(a.qkv) + static_cast<long>(b) * a.T * cw;
    const uint32_t* cst = static_cast<const uint32_t*>(a.conv_state) + static_cast<long>(b) * (kTaps - 1) * cw;
#pragma unroll
    for (int e = 0; e < kRows; ++e) {
      const int tok = tok0 + e;  // wave-uniform
      const uint32_t* row = tok < 0 ? cst + (kTaps - 1 + tok) * cw : qkv + static_cast<long>(min(tok, a.T - 1)) * cw;
      sm.stg.x[p][sg][e][l] = row[seg + l];
    }
  }
}

// bf16: DMA of the z rows 8p .. 8p+7 of chunk c of this v-head into the swizzled z
// buffer (rows past the end repeat the last token): 2 instructions.
__device__ __forceinline__ void stage_z(ChunkSmem<true>& sm, const KernelArgs& a, int b, int h, int c, int p,
                                        int l) {
  int zw = a.Hv * kD / 2;  // dwords per token row
  asm volatile("" : "+s"(zw));
  const uint32_t* zb = static_cast<const uint32_t*>(a.z) + static_cast<long>(b) * a.T * zw + h * (kD / 2);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int t = 8 * p + 4 * k + (l >> 4);  // LDS row of this lane's piece
    const int pc = (l & 15) ^ zswz(t);       // the piece that belongs at position l & 15
    const int tok = min(c * kC + t, a.T - 1);
    __builtin_amdgcn_global_load_lds(zb + static_cast<long>(tok) * zw + 4 * pc, &sm.zr.z[8 * p + 4 * k][0], 16, 0, 0);
  }
}

// fp32: a producer lane's conv inputs of one chunk (channel pair l of the q, k and v
// segments, rows 8p-3 .. 8p+7) and z pieces, loaded where they are used.
struct F32Inputs {
  uint32_t x[kRows][3][2];
  u32x4 zv[4];
};
__device__ __forceinline__ void load_inputs_f32(const KernelArgs& a, int b, int g, int h, int n, int p, int l,
                                                F32Inputs& r) {
  int cw = a.C, hk = a.Hk;
  asm volatile("" : "+s"(cw), "+s"(hk));
  const int seg[3] = {g * kD, (hk + g) * kD, (2 * hk + h) * kD};
#pragma unroll
  for (int e = 0; e < kRows; ++e) {
    const uint32_t* row = input_row(a, b, n * kC + 8 * p - (kTaps - 1) + e, cw);
#pragma unroll
    for (int sg = 0; sg < 3; ++sg) {
      const u32x2 v2 = *reinterpret_cast<const u32x2*>(row + seg[sg] + 2 * l);
      r.x[e][sg][0] = v2[0];
      r.x[e][sg][1] = v2[1];
    }
  }
}
__device__ __forceinline__ void copy_z_f32(ChunkSmem<false>& sm, const KernelArgs& a, int b, int h, int c, int p,
                                           int l) {
  int zw = a.Hv * kD;
  asm volatile("" : "+s"(zw));
  const float* zb = static_cast<const float*>(a.z) + static_cast<long>(b) * a.T * zw + h * kD;
  u32x4 zv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int f = 64 * k + l, t = 8 * p + (f >> 5);
    zv[k] = *reinterpret_cast<const u32x4*>(zb + static_cast<long>(min(c * kC + t, a.T - 1)) * zw + 4 * (f & 31));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int f = 64 * k + l;
    *reinterpret_cast<u32x4*>(&sm.zr.z[8 * p + (f >> 5)][4 * (f & 31)]) = zv[k];
  }
}

// raw gate inputs of token `lane` of chunk n (lanes past the end read the last token),
// widened only where they are used: a conversion right after a load waits for it
template <bool BF>
__device__ __forceinline__ void load_gate_inputs(const KernelArgs& a, int b, int h, int n, int lane, uint32_t& dt,
                                                 uint32_t& br) {
  const int t = min(n * kC + min(lane, kC - 1), a.T - 1);
  const long ai = (static_cast<long>(b) * a.T + t) * a.Hv + h;
  if constexpr (BF) {
    dt = static_cast<const uint16_t*>(a.dt_raw)[ai];
    br = static_cast<const uint16_t*>(a.b_raw)[ai];
  } else {
    dt = static_cast<const uint32_t*>(a.dt_raw)[ai];
    br = static_cast<const uint32_t*>(a.b_raw)[ai];
  }
}
template <bool BF>
__device__ __forceinline__ float gate_input(uint32_t raw) {
  return BF ? bf16_to_f32(raw) : __uint_as_float(raw);
}

// Gates of the chunk's tokens (lanes 0..31, one token each): beta_t = sigmoid(b_t) and
// the inclusive running sum of log(alpha_t) = -exp(A_log) softplus(dt_t + dt_bias), in
// fp64. Tokens past the end get beta 0 and log alpha 0.
__device__ __forceinline__ void chunk_gates(int left, int lane, float dt, float br, float A_exp, float dt_bias,
                                            Operands& op) {
  float la = 0.0f, bt = 0.0f;
  if (lane < min(kC, left)) {
    // softplus(x) = max(x, 0) + log(1 + exp(-|x|)); the log's argument lies in (1, 2]
    const float x = dt + dt_bias;
    la = -A_exp * (fmaxf(x, 0.0f) + __logf(1.0f + __expf(-fabsf(x))));
    bt = __builtin_amdgcn_rcpf(1.0f + __expf(-br));
  }
  // inclusive scan over lanes 0..31: within each row of 16 lanes by DPP row shifts
  // (lanes shifted in from outside the row read 0), then row 1 adds row 0's total
  double gg = la;
  gg += dpp64<0x111>(gg);  // row_shr:1
  gg += dpp64<0x112>(gg);  // row_shr:2
  gg += dpp64<0x114>(gg);  // row_shr:4
  gg += dpp64<0x118>(gg);  // row_shr:8
  const double row0 = readlane64(gg, 15);
  if (lane >= 16) gg += row0;
  // the decay factors the consumers apply to every row: gamma_t = exp(g_t) and
  // exp(g_C - g_t), each difference formed in fp64 before the exponential
  const double gC = readlane64(gg, kC - 1);
  if (lane < kC) {
    op.g[lane] = gg;
    op.beta[lane] = bt;
    op.gam[lane] = __expf(static_cast<float>(gg));
    op.dec[lane] = __expf(static_cast<float>(gC - gg));
  }
}

// Phase 1 of producer wave p (tokens 8p .. 8p+7) for chunk n: conv + SiLU of its q, k, v
// channel pairs, the L2 norms of q and k, and the split planes. fetch(sg, x0, x1) gives
// channels 2l, 2l+1 of the rows of segment sg; fetched(sg) runs once they are in
// registers.
template <bool BF, int NSEG, typename Fetch, typename Fetched>
__device__ __forceinline__ void produce_conv(ChunkSmem<BF>& sm, const KernelArgs& a, int n, int p, int l,
                                             Fetch fetch, Fetched fetched, float one) {
  Operands& op = sm.op[n & 1];
  float y[3][8][2];  // conv outputs of channels 2l, 2l+1 of segment sg (q, k, v) for token e
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sm.wt[sg * kD + 2 * l][0]);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sm.wt[sg * kD + 2 * l + 1][0]);
    float x0[kRows], x1[kRows];
    fetch(sg, x0, x1);
    fetched(sg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float u0 = w0[0] * x0[e], u1 = w1[0] * x1[e];
#pragma unroll
      for (int j = 1; j < kTaps; ++j) {
        u0 = fmaf(w0[j], x0[e + j], u0);
        u1 = fmaf(w1[j], x1[e + j], u1);
      }
      y[sg][e][0] = silu_l2e(u0);
      y[sg][e][1] = silu_l2e(u1);
    }
  }
  // The 16 sums of squares (8 tokens x q, k) over the wave, transposed: each exchange
  // step halves the values a lane carries while doubling the lanes each covers. After
  // the 32-lane swaps value i (i < 8) lives in lanes 0-31 and value i + 8 in lanes 32-63;
  // after the 16-lane swaps register j of row r holds value j + 4 r; a row sum ends it.
  float ss[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ss[2 * e] = y[0][e][0] * y[0][e][0] + y[0][e][1] * y[0][e][1];
    ss[2 * e + 1] = y[1][e][0] * y[1][e][0] + y[1][e][1] * y[1][e][1];
  }
  const float l2_eps = a.l2_eps * (kLog2e * kLog2e);  // q, k carry the factor log2(e)
  float h8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x0 = ss[i], x1 = ss[i + 8];
    swap_halves(x0, x1);
    h8[i] = x0 + x1;
  }
  float h4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float x0 = h8[j], x1 = h8[j + 4];
    swap_rows(x0, x1);
    h4[j] = __builtin_amdgcn_rsqf(row16_sum(x0 + x1) + l2_eps);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
    ss[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, h4[i % 4]), 16 * (i / 4)));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = 8 * p + e;
    const float rq = ss[2 * e] * kUp, rk = ss[2 * e + 1];
    uint32_t hi, lo;
    split2(y[0][e][0] * rq, y[0][e][1] * rq, hi, lo, one);
    *reinterpret_cast<uint32_t*>(&op.q_hi[t][2 * l]) = hi;
    *reinterpret_cast<uint32_t*>(&op.q_lo[t][2 * l]) = lo;
    split2(y[1][e][0] * rk, y[1][e][1] * rk, hi, lo, one);
    *reinterpret_cast<uint32_t*>(&op.k_hi[t][2 * l]) = hi;
    *reinterpret_cast<uint32_t*>(&op.k_lo[t][2 * l]) = lo;
    if constexpr (NSEG == 3) *reinterpret_cast<f32x2*>(&op.v[t][(2 * l) ^ vswz(t)]) = f32x2{y[2][e][0], y[2][e][1]};
  }
}

// bf16, consumer waves 2 and 3 in phase 2: conv + SiLU of the v channels (pair l) of
// chunk n for tokens 16 hv .. 16 hv + 15 (hv = w - 2), from the producers' staging rows:
// token tau of the chunk (tau >= -3) is row tau - 8 pp + 3 of producer wave
// pp = max(tau, 0) / 8.
__device__ __forceinline__ void conv_v(ChunkSmem<true>& sm, int n, int hv, int l) {
  constexpr int kR = 16 + kTaps - 1;
  Operands& op = sm.op[n & 1];
  const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sm.wt[2 * kD + 2 * l][0]);
  const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sm.wt[2 * kD + 2 * l + 1][0]);
  uint32_t xr[kR];
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const int tau = 16 * hv - (kTaps - 1) + i;
    const int pp = tau < 0 ? 0 : (tau >> 3);
    xr[i] = sm.stg.x[pp][2][tau - 8 * pp + (kTaps - 1)][l];
  }
  float x0[kR], x1[kR];
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    x0[i] = bf16_to_f32(xr[i] & 0xffffu);
    x1[i] = __uint_as_float(xr[i] & 0xffff0000u);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float u0 = w0[0] * x0[e], u1 = w1[0] * x1[e];
#pragma unroll
    for (int j = 1; j < kTaps; ++j) {
      u0 = fmaf(w0[j], x0[e + j], u0);
      u1 = fmaf(w1[j], x1[e + j], u1);
    }
    const int t = 16 * hv + e;
    *reinterpret_cast<f32x2*>(&op.v[t][(2 * l) ^ vswz(t)]) = f32x2{silu_l2e(u0), silu_l2e(u1)};
  }
}

// Epilogue of one 16 x 16 tile (tt, ss), x = K K^T (kk) or 2^15 Q K^T: K K^T (0, 0) -> T11,
// (1, 1) -> T22, (1, 0) -> A21; Q K^T -> P.
template <bool BF>
__device__ __forceinline__ void tile_epilogue(ChunkSmem<BF>& sm, const Operands& op, int l, int tt, int ss,
                                              bool is_kk, f32x4 x, float one) {
  const int q = l >> 4, c16 = l & 15;
  const int p = tt == 0 ? 0 : (ss == 1 ? 1 : 2);  // which K K^T block
  const int s = 16 * ss + c16;
  const double gs = op.g[s];
  float dec[4], bt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * tt + 4 * q + r;
    // exp(g_t - g_s) <= 1 for s <= t; the other entries are masked (argument clamped)
    dec[r] = (s <= t) ? __expf(fminf(static_cast<float>(op.g[t] - gs), 0.0f)) : 0.0f;
    bt[r] = op.beta[t];
  }
  if (!is_kk) {  // 2^15 P (q carries 2^15)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tt + 4 * q + r;
      uint32_t hi, lo;
      split1(dec[r] * x[r], hi, lo, one);
      sm.p_hi[t][s] = static_cast<uint16_t>(hi);
      sm.p_lo[t][s] = static_cast<uint16_t>(lo);
    }
  }
  if (is_kk && p == 2) {  // 2^15 A21
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t hi, lo;
      split1(bt[r] * dec[r] * x[r] * kUp, hi, lo, one);
      sm.a_hi[4 * q + r][c16] = static_cast<uint16_t>(hi);
      sm.a_lo[4 * q + r][c16] = static_cast<uint16_t>(lo);
    }
  }
  if (is_kk && p <= 1) {
    // L = A_pp (strictly lower): lsc[p][s][rho][kappa] = L[rho + 4 kappa][s]; this lane
    // holds rows t' = 4q + r (rho = r, kappa = q) of column c16
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.lsc[p][c16][r][q] = (4 * q + r > c16) ? bt[r] * dec[r] * x[r] : 0.0f;
    // the substitution reads what other lanes of the wave wrote (a wave's LDS accesses
    // complete in order; the fences keep the compiler from moving them)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // X = (I + L)^-1 by substitution: column j = l / 4 on the quad of lanes 4j .. 4j+3,
    // lane rho holding rows rho + 4 kappa. At step st the pivot x_st (lane st % 4, slot
    // st / 4) is final; a quad broadcast hands it to the quad and every row is updated
    // (rows at or above st have L[.][st] = 0).
    const int j = l >> 2, rho = l & 3;
    f32x4 lv[15];  // all columns of L this lane needs, read before the dependent steps
#pragma unroll
    for (int st = 0; st < 15; ++st) lv[st] = *reinterpret_cast<const f32x4*>(&sm.lsc[p][st][rho][0]);
    float xv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) xv[k] = (rho + 4 * k == j) ? 1.0f : 0.0f;
#pragma unroll
    for (int st = 0; st < 15; ++st) {
      float xs;
      switch (st & 3) {
        case 0: xs = dpp<0x00>(xv[st >> 2]); break;   // quad_perm [0,0,0,0]
        case 1: xs = dpp<0x55>(xv[st >> 2]); break;   // [1,1,1,1]
        case 2: xs = dpp<0xAA>(xv[st >> 2]); break;   // [2,2,2,2]
        default: xs = dpp<0xFF>(xv[st >> 2]); break;  // [3,3,3,3]
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) xv[k] = fmaf(-lv[st][k], xs, xv[k]);
    }
    // scale by 2^(15 - E), E the exponent of the largest |entry| (E >= 1: unit diagonal)
    float m = fmaxf(fmaxf(fabsf(xv[0]), fabsf(xv[1])), fmaxf(fabsf(xv[2]), fabsf(xv[3])));
    m = wave_max(m);
    int E;
    (void)frexpf(m, &E);
    const float up = ldexpf(1.0f, 15 - E);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t hi, lo;
      split1(xv[k] * up, hi, lo, one);
      sm.t_hi[p][rho + 4 * k][j] = static_cast<uint16_t>(hi);
      sm.t_lo[p][rho + 4 * k][j] = static_cast<uint16_t>(lo);
    }
    if (l == 0) sm.tscale[p] = ldexpf(1.0f, E - 15);
  }
}


// 16 x 16 tiles (tt, ss0 + i), i < np, of K K^T (kk) or Q K^T of chunk n (contraction over
// the 128 channels) and their epilogues. All fragments are read first, and each
// 32-channel block accumulates into its own registers (no long chain of dependent
// products).
template <bool BF>
__device__ __forceinline__ void produce_tiles(ChunkSmem<BF>& sm, int n, int l, int tt, int np, int ss0, bool kk,
                                              float one) {
  const Operands& op = sm.op[n & 1];
  const int q = l >> 4, c16 = l & 15;
  const uint16_t* ahp = kk ? &op.k_hi[0][0] : &op.q_hi[0][0];
  const uint16_t* alp = kk ? &op.k_lo[0][0] : &op.q_lo[0][0];
  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i >= np) break;
    u32x4 ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      ah[kb] = frag(ahp, kQKLd, 16 * tt + c16, 32 * kb, q);
      al[kb] = frag(alp, kQKLd, 16 * tt + c16, 32 * kb, q);
      if (kk && ss0 + i == tt) {  // diagonal K K^T tile: B holds the same rows as A
        bh[kb] = ah[kb];
        bl[kb] = al[kb];
      } else {
        bh[kb] = frag(&op.k_hi[0][0], kQKLd, 16 * (ss0 + i) + c16, 32 * kb, q);
        bl[kb] = frag(&op.k_lo[0][0], kQKLd, 16 * (ss0 + i) + c16, 32 * kb, q);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[i][kb] = mfma32x3(ah[kb], al[kb], bh[kb], bl[kb], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i >= np) break;
    const f32x4 x = (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
    tile_epilogue<BF>(sm, op, l, tt, ss0 + i, kk, x, one);
  }
}

// Phase 2 of producer wave p for chunk n:
//   p = 0: K K^T (0, 0) -> A11 -> T11 = (I + A11)^-1
//   p = 1: K K^T (1, 1) -> A22 -> T22
//   p = 2: K K^T (1, 0) -> A21 (times 2^15, split)
//   p = 3: Q K^T (0, 0) -> P
// (consumer waves 0 and 1 take Q K^T (1, 0) and (1, 1) after the outputs of chunk c).
template <bool BF>
__device__ __forceinline__ void produce_factors(ChunkSmem<BF>& sm, int n, int p, int l, float one) {
  produce_tiles<BF>(sm, n, l, p == 0 || p == 3 ? 0 : 1, 1, p == 1 ? 1 : 0, p <= 2, one);
}

// ---------------------------------------------------------------------------------
// consumer waves
// ---------------------------------------------------------------------------------

// The 16 outputs of a lane (rows 16 lt + 4q + r, columns 32w + 16jt + c16) as buffer
// stores at byte offset vo (the lane's row 4q and column) plus the row offset; bf16
// outputs are rounded to nearest even (a NaN stays a quiet NaN).
template <bool OUT_BF16>
__device__ __forceinline__ void store_rows(const float (&y)[2][4][2], __amdgpu_buffer_rsrc_t ors, int vo, int zr) {
  constexpr int esz = OUT_BF16 ? 2 : 4;
#pragma unroll
  for (int lt = 0; lt < 2; ++lt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ro = vo + (16 * lt + r) * zr * esz;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const float x = y[lt][r][jt];
        if constexpr (OUT_BF16) {
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, q = l >> 4, c16 = l & 15;
  // Workgroups are dealt to the 8 XCDs round robin by id. When the grid divides by 8,
  // consecutive (sequence, v-head) units share an XCD, so the G v-heads that read one
  // k-head's q and k rows find them in the same L2 (the rows are fetched from HBM once).
  const unsigned nwg = gridDim.x, x = blockIdx.x;
  const int u = static_cast<int>(nwg % 8 == 0 ? (x % 8) * (nwg / 8) + x / 8 : x);
  const int b = u / a.Hv;
  const int h = u - b * a.Hv;
  const int g = h / a.G;
  const int T = a.T;
  const int nchunks = (T + kC - 1) / kC;
  const bool consumer = w < 4;
  const int p = w - 4;  // producer index

  // ---- set-up: conv taps (log2(e)-scaled fp32) of the workgroup's channels; the upper
  // right tile of P (always 0)
  for (int u = tid; u < 3 * kD; u += kNT) {
    const long gc = u < kD ? static_cast<long>(g) * kD + u
                           : (u < 2 * kD ? static_cast<long>(a.Hk + g) * kD + (u - kD)
                                         : static_cast<long>(2 * a.Hk + h) * kD + (u - 2 * kD));
#pragma unroll
    for (int j = 0; j < kTaps; ++j) {
      const float wv = BF ? bf16_to_f32(static_cast<const uint16_t*>(a.conv_w)[gc * kTaps + j])
                          : static_cast<const float*>(a.conv_w)[gc * kTaps + j];
      sm.wt[u][j] = kLog2e * wv;
    }
  }
  for (int u = tid; u < 16 * 16; u += kNT) {
    sm.p_hi[u >> 4][16 + (u & 15)] = 0;
    sm.p_lo[u >> 4][16 + (u & 15)] = 0;
  }

  // consumers: wave w holds H[16 it + 4q + r][32 w + 16 jt + c16]
  float* hst = a.state + (static_cast<long>(b) * a.Hv + h) * (kD * kD);
  f32x4 hacc[8][2];
  float nw[2] = {0.0f, 0.0f};
  if (consumer) {
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hacc[it][jt][r] = hst[(16 * it + 4 * q + r) * kD + 32 * w + 16 * jt + c16];
    nw[0] = a.norm_w[32 * w + c16];
    nw[1] = a.norm_w[32 * w + 16 + c16];
  }
  const float A_exp = __expf(a.A_log[h]);
  const float dt_bias = a.dt_bias[h];
  const float rsd = 1.0f / sqrtf(static_cast<float>(kD));

  // producers (bf16): chunk 0's conv inputs by DMA and its gate inputs
  uint32_t gdt = 0, gbr = 0;
  if constexpr (BF) {
    if (!consumer && nchunks > 0) {
      if (p == kGateWave) load_gate_inputs<BF>(a, b, h, 0, l, gdt, gbr);
      for (int sg = 0; sg < 2; ++sg) stage_inputs(sm, a, b, g, h, 0, p, l, sg);
    }
  }
  __syncthreads();

  f32x4 oacc[2][2];  // consumers: O of the chunk (times 2^15), from phase 1 to phase 2

  // One pass of the two phases: the producers prepare chunk c + 1, the consumers (from
  // c = 0 on) process chunk c. The first pass (c = -1) only prepares chunk 0; it is a
  // separate instance so that the consumers' part of the loop has no condition.
  auto chunk_step = [&](const int c, auto first) {
    constexpr bool kFirst = decltype(first)::value;
    float one = 1.0f;
    asm volatile("" : "+s"(one));
    // lane indices re-derived per chunk (opaque to the optimiser), so that the many
    // lane-dependent LDS addresses are recomputed instead of held across the loop
    int tid_ = tid;
    asm volatile("" : "+v"(tid_));
    const int l = tid_ & 63, q = l >> 4, c16 = l & 15;
    const int n = c + 1;  // the chunk the producers prepare
    // ================= phase 1 =================
    if (consumer) {
      if constexpr (!kFirst) {
        const Operands& op = sm.op[c & 1];
        // K H0 and Q H0 for the wave's columns: rows t = 16 lt + 4q + r
        f32x4 kh[2][2], qh[2][2];
#pragma unroll
        for (int lt = 0; lt < 2; ++lt)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            kh[lt][jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            qh[lt][jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          u32x4 bh[2], bl[2];
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) bfrag(hacc[2 * kb][jt], hacc[2 * kb + 1][jt], bh[jt], bl[jt], one);
#pragma unroll
          for (int lt = 0; lt < 2; ++lt) {
            const u32x4 kah = frag(&op.k_hi[0][0], kQKLd, 16 * lt + c16, 32 * kb, q);
            const u32x4 kal = frag(&op.k_lo[0][0], kQKLd, 16 * lt + c16, 32 * kb, q);
            const u32x4 qah = frag(&op.q_hi[0][0], kQKLd, 16 * lt + c16, 32 * kb, q);
            const u32x4 qal = frag(&op.q_lo[0][0], kQKLd, 16 * lt + c16, 32 * kb, q);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              kh[lt][jt] = mfma32x3(kah, kal, bh[jt], bl[jt], kh[lt][jt]);
              qh[lt][jt] = mfma32x3(qah, qal, bh[jt], bl[jt], qh[lt][jt]);
            }
          }
        }
        // R = beta (v - gamma K H0) (v is stored as log2(e) v); O starts as gamma Q H0
        f32x4 R[2][2];
#pragma unroll
        for (int lt = 0; lt < 2; ++lt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * lt + 4 * q + r;
            const float gam = op.gam[t];
            const float bt = op.beta[t];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              const float v = op.v[t][(32 * w + 16 * jt + c16) ^ vswz(t)];
              R[lt][jt][r] = fmaf(-bt * gam, kh[lt][jt][r], bt * kLn2 * v);
              oacc[lt][jt][r] = gam * qh[lt][jt][r];
            }
          }
        // Delta1 = T11 R1; Delta2 = T22 (R2 - A21 Delta1)
        f32x4 delta[2][2];
        {
          const float ts1 = sm.tscale[0], ts2 = sm.tscale[1];
          const u32x2 t1h = *reinterpret_cast<const u32x2*>(&sm.t_hi[0][c16][4 * q]);
          const u32x2 t1l = *reinterpret_cast<const u32x2*>(&sm.t_lo[0][c16][4 * q]);
          const u32x2 t2h = *reinterpret_cast<const u32x2*>(&sm.t_hi[1][c16][4 * q]);
          const u32x2 t2l = *reinterpret_cast<const u32x2*>(&sm.t_lo[1][c16][4 * q]);
          const u32x2 a1h = *reinterpret_cast<const u32x2*>(&sm.a_hi[c16][4 * q]);
          const u32x2 a1l = *reinterpret_cast<const u32x2*>(&sm.a_lo[c16][4 * q]);
          const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            u32x2 rh, rl;
            split4(R[0][jt], rh, rl, one);
            delta[0][jt] = mfma16x3(t1h, t1l, rh, rl, zero) * ts1;
            split4(delta[0][jt], rh, rl, one);
            const f32x4 ad = mfma16x3(a1h, a1l, rh, rl, zero);
            f32x4 y2;
#pragma unroll
            for (int r = 0; r < 4; ++r) y2[r] = fmaf(-kDown, ad[r], R[1][jt][r]);
            split4(y2, rh, rl, one);
            delta[1][jt] = mfma16x3(t2h, t2l, rh, rl, zero) * ts2;
          }
        }
        // O += P Delta (both terms carry 2^15: P and q)
        {
          u32x4 dh[2], dl[2];
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) bfrag(delta[0][jt], delta[1][jt], dh[jt], dl[jt], one);
#pragma unroll
          for (int lt = 0; lt < 2; ++lt) {
            const u32x4 ph = frag(&sm.p_hi[0][0], kPLd, 16 * lt + c16, 0, q);
            const u32x4 pl = frag(&sm.p_lo[0][0], kPLd, 16 * lt + c16, 0, q);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) oacc[lt][jt] = mfma32x3(ph, pl, dh[jt], dl[jt], oacc[lt][jt]);
          }
        }
        // sums of O^2 over the wave's 32 columns, per row: the lane's 8 rows (i = 4 lt + r)
        // are summed over the 16 lanes of its row group as one transposed reduction; each
        // exchange halves the values a lane carries, and lane c16 ends with the total of
        // row i = c16 >> 1
        {
          float v8[8];
#pragma unroll
          for (int lt = 0; lt < 2; ++lt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              v8[4 * lt + r] = fmaf(oacc[lt][1][r], oacc[lt][1][r], oacc[lt][0][r] * oacc[lt][0][r]);
          const bool b3 = (c16 & 8) != 0, b2 = (c16 & 4) != 0, b1 = (c16 & 2) != 0;
          float v4[4], v2[2];
#pragma unroll
          for (int i = 0; i < 4; ++i)  // lanes c16 and c16 ^ 8 (row rotate by 8)
            v4[i] = (b3 ? v8[i + 4] : v8[i]) + dpp<0x128>(b3 ? v8[i] : v8[i + 4]);
#pragma unroll
          for (int i = 0; i < 2; ++i)  // lanes c16 and 7 - c16 of each half row (half-row mirror)
            v2[i] = (b2 ? v4[i + 2] : v4[i]) + dpp<0x141>(b2 ? v4[i] : v4[i + 2]);
          float v1 = (b1 ? v2[1] : v2[0]) + dpp<0x4E>(b1 ? v2[0] : v2[1]);  // lanes c16 ^ 2
          v1 += dpp<0xB1>(v1);                                                 // lanes c16 ^ 1
          const int i = c16 >> 1;
          if ((c16 & 1) == 0) sm.rsum[16 * (i >> 2) + 4 * q + (i & 3)][w] = v1;
        }
        // H = gamma_C H + K^T diag(exp(g_C - g)) Delta
        {
          const float gamC = op.gam[kC - 1];
#pragma unroll
          for (int lt = 0; lt < 2; ++lt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float f = op.dec[16 * lt + 4 * q + r];
#pragma unroll
              for (int jt = 0; jt < 2; ++jt) delta[lt][jt][r] *= f;
            }
          u32x4 eh[2], el[2];
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) bfrag(delta[0][jt], delta[1][jt], eh[jt], el[jt], one);
#pragma unroll
          for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) hacc[it][jt] *= gamC;
#pragma unroll
          for (int it = 0; it < 8; ++it) {
            const u32x4 ah = frag_t(&op.k_hi[0][0], 16 * it, q, c16);
            const u32x4 al = frag_t(&op.k_lo[0][0], 16 * it, q, c16);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) hacc[it][jt] = mfma32x3(ah, al, eh[jt], el[jt], hacc[it][jt]);
          }
        }
      }
    } else {
      if constexpr (BF) {
        if (n < nchunks) {
          // this wave's staged rows of chunk n have landed (its DMA was the last memory
          // operation it issued before the barrier)
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          const float dt = gate_input<BF>(gdt), br = gate_input<BF>(gbr);
          // memory operations in issue order: z rows of chunk c (2), v rows of chunk n (3;
          // consumer waves 2 and 3 convolve them in phase 2), gate inputs of chunk n + 1
          // (2, wave p = kGateWave), q and k rows of chunk n + 1 (3 per segment, each issued once
          // the segment's staged rows of chunk n are in registers)
          if (c >= 0) stage_z(sm, a, b, h, c, p, l);
          stage_inputs(sm, a, b, g, h, n, p, l, 2);
          if (p == kGateWave && n + 1 < nchunks) load_gate_inputs<BF>(a, b, h, n + 1, l, gdt, gbr);
          // the gates of chunk n come from phase 2 of the pass before (chunk 0: here)
          if constexpr (kFirst) {
            if (p == kGateWave) chunk_gates(T - n * kC, l, dt, br, A_exp, dt_bias, sm.op[n & 1]);
          }
          produce_conv<BF, 2>(
              sm, a, n, p, l,
              [&](int sg, float(&x0)[kRows], float(&x1)[kRows]) {
                uint32_t xr[kRows];
#pragma unroll
                for (int e = 0; e < kRows; ++e) xr[e] = sm.stg.x[p][sg][e][l];
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int e = 0; e < kRows; ++e) {
                  x0[e] = bf16_to_f32(xr[e] & 0xffffu);
                  x1[e] = __uint_as_float(xr[e] & 0xffff0000u);
                }
              },
              [&](int sg) {
                if (n + 1 < nchunks) stage_inputs(sm, a, b, g, h, n + 1, p, l, sg);
              },
              one);
          // the z rows of chunk c and the v rows of chunk n must have landed before the
          // barrier (the gate loads and the 6 q / k staging instructions may still be in
          // flight)
          if (n + 1 >= nchunks)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          else if (p == kGateWave)
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
          else
            asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        } else if (c >= 0) {
          stage_z(sm, a, b, h, c, p, l);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      } else {
        if (c >= 0) copy_z_f32(sm, a, b, h, c, p, l);
        if (n < nchunks) {
          F32Inputs xr;
          load_inputs_f32(a, b, g, h, n, p, l, xr);
          if (p == kGateWave) {
            uint32_t dt, br;
            load_gate_inputs<BF>(a, b, h, n, l, dt, br);
            chunk_gates(T - n * kC, l, gate_input<BF>(dt), gate_input<BF>(br), A_exp, dt_bias, sm.op[n & 1]);
          }
          produce_conv<BF, 3>(
              sm, a, n, p, l,
              [&](int sg, float(&x0)[kRows], float(&x1)[kRows]) {
#pragma unroll
                for (int e = 0; e < kRows; ++e) {
                  x0[e] = __uint_as_float(xr.x[e][sg][0]);
                  x1[e] = __uint_as_float(xr.x[e][sg][1]);
                }
              },
              [](int) {}, one);
        }
      }
    }
    lds_barrier();
    // ================= phase 2 =================
    if (consumer) {
      // Q K^T tiles (1, 0) and (1, 1) of the next chunk -> P (waves 0 and 1)
      if (w < 2 && n < nchunks) produce_tiles<BF>(sm, n, l, 1, 1, w, false, one);
      if constexpr (!kFirst) {
        // gated RMSNorm of o = O 2^-15 / sqrt(d), and the output rows
        const int t0 = c * kC, nt = min(kC, T - t0);
        float y[2][4][2];
#pragma unroll
        for (int lt = 0; lt < 2; ++lt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * lt + 4 * q + r;
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(&sm.rsum[t][0]);
            const float tot = (v4[0] + v4[1] + v4[2] + v4[3]) * (kDown * kDown * rsd * rsd);
            const float rr = __builtin_amdgcn_rsqf(tot * (1.0f / kD) + a.rms_eps) * (kDown * rsd);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              const int j = 32 * w + 16 * jt + c16;
              float zz;
              if constexpr (BF) {
                const int pos = (j >> 3) ^ zswz(t);
                zz = bf16_to_f32((sm.zr.z[t][4 * pos + ((j & 7) >> 1)] >> (16 * (j & 1))) & 0xffffu);
              } else {
                zz = sm.zr.z[t][j];
              }
              y[lt][r][jt] = oacc[lt][jt][r] * rr * nw[jt] * silu(zz);
            }
          }
        // The chunk's nt output rows form one buffer resource: rows past the end of the
        // sequence (last chunk) fall outside it and are not written (hardware range check).
        const int esz = a.out_bf16 ? 2 : 4;
        const int zr = a.Hv * kD;  // elements per token row
        const __amdgpu_buffer_rsrc_t ors = rows_rsrc(
            static_cast<char*>(a.out) + ((static_cast<long>(b) * T + t0) * zr + static_cast<long>(h) * kD) * esz,
            static_cast<uint32_t>(nt * zr * esz));
        const int vo = (4 * q * zr + 32 * w + c16) * esz;
        if (a.out_bf16)
          store_rows<true>(y, ors, vo, zr);
        else
          store_rows<false>(y, ors, vo, zr);
      }
      if constexpr (BF) {
        if (w >= 2 && n < nchunks) conv_v(sm, n, w - 2, l);
      }
    } else if (n < nchunks) {
      produce_factors<BF>(sm, n, p, l, one);
      // gates of chunk n + 1 (inputs loaded in phase 1) into the buffer of chunk c
      if constexpr (BF) {
        if (p == kGateWave && n + 1 < nchunks)
          chunk_gates(T - (n + 1) * kC, l, gate_input<BF>(gdt), gate_input<BF>(gbr), A_exp, dt_bias,
                      sm.op[(n + 1) & 1]);
      }
    }
    lds_barrier();
  };
  chunk_step(-1, std::true_type{});
  for (int c = 0; c < nchunks; ++c) chunk_step(c, std::false_type{});

  if (consumer) {
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hst[(16 * it + 4 * q + r) * kD + 32 * w + 16 * jt + c16] = hacc[it][jt][r];
  }
}

// Final conv state after T tokens: row j of the K-1 rows is element T + j of the
// sequence (old rows 0..K-2, x_0 .. x_{T-1}); a bit-exact copy. One thread per
// (sequence, channel); rows are visited in increasing order, so an old row is read
// before it is overwritten.
template <bool BF>
__global__ __launch_bounds__(256) void gdn_conv_state_tail(const KernelArgs a) {
  using raw_t = typename std::conditional<BF, uint16_t, uint32_t>::type;
  const long C = a.C;
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(a.B) * C) return;
  const long b = idx / C, c = idx - b * C;
  const int Km1 = a.K - 1;
  const long T = a.T;
  raw_t* cs = static_cast<raw_t*>(a.conv_state);
  const raw_t* x = static_cast<const raw_t*>(a.qkv);
  for (int j = 0; j < Km1; ++j) {
    const long e = T + j;  // element of the combined sequence
    const raw_t v = e < Km1 ? cs[(b * Km1 + e) * C + c] : x[(b * T + (e - Km1)) * C + c];
    cs[(b * Km1 + j) * C + c] = v;
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
