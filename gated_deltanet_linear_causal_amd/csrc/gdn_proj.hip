// Projections on either side of the GDN layer for CDNA4 (gfx950): the in_proj GEMVs
// of step 2 of the page "linear_attention.rs" (x_norm -> qkv, z, dt_raw, b_raw) and the
// out_proj GEMV of steps 9-11 (the gated output -> hidden). Both are
//   Y[m][n] = sum_k X[m][k] W[n][k]      X [M][K] bf16, W [N][K] bf16, fp32 accumulation,
// for up to four weight segments (W_s, Y_s, N_s) in one launch, so the four in_proj
// outputs come from one pass over x_norm.
//
// M <= 8 (decode at small batch) is weight-streaming: each wave takes NR output rows
// at a time, every lane reads 16-byte pieces of the rows (coalesced, K contiguous) and
// multiplies them with the M rows of X held in LDS; a wave reduction finishes each dot
// product. The bound is HBM: every weight byte is read once. Up to 32 rows with few
// output columns use a skinny MFMA kernel that splits K over the waves of a workgroup
// (see gdn_proj_skinny).
// Larger M uses MFMA (v_mfma_f32_16x16x32_bf16) on BM x BN tiles of Y, BK = 64, X and W
// tiles double-buffered in LDS. Operand fragments are 8 consecutive k per lane (a
// 16-byte LDS read) for both X and W: the product pairs A and B register slots of the
// same lane group and element, so any common k order gives the same sum.

#include <algorithm>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16, qnan = (u >> 16) | 0x40u;
  return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? qnan : rne);
}

__device__ __forceinline__ void put(const ProjSeg& s, long m, long n, float v) {
  if (s.y_bf16)
    static_cast<uint16_t*>(s.y)[m * s.n + n] = to_bf16(v);
  else
    static_cast<float*>(s.y)[m * s.n + n] = v;
}

// segment of global output row n (uniform across the caller)
__device__ __forceinline__ int seg_of(const ProjArgs& p, long n) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kMaxProjSegs; ++i)
    if (i < p.nseg && n >= p.seg[i].row0) s = i;
  return s;
}

// ----------------------------------------------------------------------------------
// M <= MT rows: weight streaming. Dynamic LDS: X as MT x K bf16 (rows >= M are zero).
// A wave takes NR output rows; each lane issues the loads of all its 16-byte pieces of
// those rows (CU pieces per row at a time, K/512 in all) before the first product.
// ----------------------------------------------------------------------------------
template <int MT, int NR, int CU>
__global__ __launch_bounds__(256) void gdn_proj_gemv(const ProjArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  const int K = p.K, K8 = K / 8;
  for (int i = threadIdx.x; i < MT * K8; i += 256) {
    const int m = i / K8, c = i - m * K8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (m < p.M) v = *reinterpret_cast<const u32x4*>(p.x + static_cast<long>(m) * K + 8 * c);
    *reinterpret_cast<u32x4*>(xs + static_cast<long>(m) * K + 8 * c) = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const long waves = static_cast<long>(gridDim.x) * 4;
  for (long r0 = (static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * NR; r0 < p.rows; r0 += waves * NR) {
    const uint16_t* wr[NR];
    bool live[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const long n = r0 + r;
      live[r] = n < p.rows;
      const ProjSeg s = p.seg[seg_of(p, live[r] ? n : r0)];
      wr[r] = s.w + (live[r] ? n - s.row0 : 0) * static_cast<long>(K);
    }
    float acc[NR][MT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
    for (int c0 = lane; c0 < K8; c0 += 64 * CU) {
      u32x4 wv[CU][NR];
#pragma unroll
      for (int u = 0; u < CU; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r)
          if (c0 + 64 * u < K8) wv[u][r] = *reinterpret_cast<const u32x4*>(wr[r] + 8 * (c0 + 64 * u));
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int c = c0 + 64 * u;
        if (c >= K8) break;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + static_cast<long>(m) * K + 8 * c);
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[r][m] = fmaf(lo_bf16(wv[u][r][e]), lo_bf16(xv[e]), acc[r][m]);
              acc[r][m] = fmaf(hi_bf16(wv[u][r][e]), hi_bf16(xv[e]), acc[r][m]);
            }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float v = acc[r][m];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        acc[r][m] = v;
      }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (!live[r]) continue;
        const long n = r0 + r;
        const ProjSeg s = p.seg[seg_of(p, n)];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < p.M) put(s, m, n - s.row0, acc[r][m]);
      }
    }
  }
}

// ----------------------------------------------------------------------------------
// MFMA tiles. Grid: x = N-tiles of all segments (tile0 of each segment), y = M-tiles.
// 4 waves as WM x WN, each a (BM/WM) x (BN/WN) block of 16x16 accumulator tiles; BK-deep
// stages of X and W double-buffered in LDS (rows padded by 8 bf16).
// ----------------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(256) void gdn_proj_mfma(const ProjArgs p) {
  static_assert(WM * WN == 4, "4 waves");
  constexpr int LD = BK + 8;
  constexpr int TI = BM / WM / 16, TJ = BN / WN / 16;  // 16x16 tiles per wave
  constexpr int PR = BK / 8;                          // 16-byte pieces per tile row
  constexpr int XC = BM * PR / 256, WC = BN * PR / 256;  // pieces per thread
  static_assert(XC >= 1 && WC >= 1 && TI >= 1 && TJ >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM][LD];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN][LD];

  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxProjSegs; ++i)
    if (i < p.nseg && static_cast<int>(blockIdx.x) >= p.seg[i].tile0) si = i;
  const ProjSeg s = p.seg[si];
  const long n0 = static_cast<long>(blockIdx.x - s.tile0) * BN;
  const long m0 = static_cast<long>(blockIdx.y) * BM;
  const int K = p.K;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, q = l >> 4, c16 = l & 15;
  const int wm = w / WN, wn = w % WN;

  // global -> register pieces: piece i of a tile is row i / PR, 8 bf16 at column 8 (i % PR)
  u32x4 xr[XC], wr_[WC];
  auto load = [&](int k0) {
#pragma unroll
    for (int c = 0; c < XC; ++c) {
      const int i = t + 256 * c, row = i / PR, col = 8 * (i % PR);
      const long m = m0 + row;
      xr[c] = m < p.M ? *reinterpret_cast<const u32x4*>(p.x + m * K + k0 + col) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < WC; ++c) {
      const int i = t + 256 * c, row = i / PR, col = 8 * (i % PR);
      const long n = n0 + row;
      wr_[c] = n < s.n ? *reinterpret_cast<const u32x4*>(s.w + n * K + k0 + col) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int c = 0; c < XC; ++c) {
      const int i = t + 256 * c;
      *reinterpret_cast<u32x4*>(&xs[buf][i / PR][8 * (i % PR)]) = xr[c];
    }
#pragma unroll
    for (int c = 0; c < WC; ++c) {
      const int i = t + 256 * c;
      *reinterpret_cast<u32x4*>(&ws[buf][i / PR][8 * (i % PR)]) = wr_[c];
    }
  };

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = K / BK;
  load(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);  // next stage in flight during the products
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      bf16x8 a[TI], bb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&xs[cur][wm * (BM / WM) + 16 * i + c16][32 * kk + 8 * q]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        bb[j] = *reinterpret_cast<const bf16x8*>(&ws[cur][wn * (BN / WN) + 16 * j + c16][32 * kk + 8 * q]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      stash(cur ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
    }
  }
  // accumulator tile (i, j): lane holds rows 4q + r, column c16
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const long n = n0 + wn * (BN / WN) + 16 * j + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long m = m0 + wm * (BM / WM) + 16 * i + 4 * q + r;
        if (m < p.M && n < s.n) put(s, m, n, acc[i][j][r]);
      }
    }
}

// ----------------------------------------------------------------------------------
// Skinny MFMA (M <= 16 TI): the weight stream with matrix cores. A workgroup of KW waves
// takes one BN = 16 TJ wide tile of outputs for all M rows; wave w covers k in
// [w K / KW, (w + 1) K / KW), and the KW partial tiles are summed through LDS at the end.
// Operands go from memory straight into MFMA fragments (no LDS staging): per 64-deep
// k-block, lane group q holds k0 + 16 q .. k0 + 16 q + 15 of its row (two 16-byte
// loads, one per MFMA step), so the four lane groups read a row's 128 bytes at once; A
// (X, small and reused from cache) and B (W, streamed once) use the same k order, which
// leaves every dot product unchanged. D k-blocks are in flight in registers. Rows of X
// past M and rows of W past the segment end are clamped to valid rows: they only feed
// outputs that are not stored.
// ----------------------------------------------------------------------------------
template <int TI, int TJ, int KW, int D>
__global__ __launch_bounds__(64 * KW) void gdn_proj_skinny(const ProjArgs p) {
  constexpr int BM = 16 * TI, BN = 16 * TJ, NT = 64 * KW;
  static_assert(KW * BM * BN * 4 <= 65536, "reduction buffer");
  __shared__ float red[KW][BM * BN];

  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxProjSegs; ++i)
    if (i < p.nseg && static_cast<int>(blockIdx.x) >= p.seg[i].tile0) si = i;
  const ProjSeg s = p.seg[si];
  const long n0 = static_cast<long>(blockIdx.x - s.tile0) * BN;
  const int m0 = static_cast<int>(blockIdx.y) * BM;  // row block
  const int K = p.K;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, q = l >> 4, c16 = l & 15;
  const int kw = K / KW, nkb = kw / 64;
  const long k0 = static_cast<long>(w) * kw + 16 * q;

  const uint16_t* xp[TI];
  const uint16_t* wp[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) xp[i] = p.x + static_cast<long>(min(m0 + 16 * i + c16, p.M - 1)) * K + k0;
#pragma unroll
  for (int j = 0; j < TJ; ++j) wp[j] = s.w + min(n0 + 16 * j + c16, s.n - 1) * K + k0;

  u32x4 xa[D][TI][2], wb[D][TJ][2];
  auto load = [&](int kb, int sl) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 2; ++e) wb[sl][j][e] = *reinterpret_cast<const u32x4*>(wp[j] + 64 * kb + 8 * e);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int e = 0; e < 2; ++e) xa[sl][i][e] = *reinterpret_cast<const u32x4*>(xp[i] + 64 * kb + 8 * e);
  };
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto mfma = [&](int sl) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[sl][i][e]),
                                                              __builtin_bit_cast(bf16x8, wb[sl][j][e]), acc[i][j], 0, 0, 0);
  };
  // the first D k-blocks (clamped to the last one when the slice is shorter, so that
  // every slot is loaded and the memory counter is the same on every path into the loop)
#pragma unroll
  for (int i = 0; i < D; ++i) load(min(i, nkb - 1), i);
  // k-block kb sits in register slot kb % D; unrolled by D so that slots are constants.
  // The steady state reloads every slot unconditionally: a conditional load there makes
  // the compiler rotate the slots through copies at the loop edge, which first waits for
  // every load in flight.
  int kb0 = 0;
  for (; kb0 + 2 * D <= nkb; kb0 += D) {
#pragma unroll
    for (int sl = 0; sl < D; ++sl) {
      mfma(sl);
      load(kb0 + sl + D, sl);
    }
  }
  // the last 2D - 1 or fewer k-blocks
#pragma unroll
  for (int sl = 0; sl < D; ++sl) {
    if (kb0 + sl < nkb) {
      mfma(sl);
      if (kb0 + sl + D < nkb) load(kb0 + sl + D, sl);
    }
  }
#pragma unroll
  for (int sl = 0; sl < D; ++sl)
    if (kb0 + D + sl < nkb) mfma(sl);
  // accumulator tile (i, j): lane holds rows 16 i + 4 q + r, column 16 j + c16
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[w][(16 * i + 4 * q + r) * BN + 16 * j + c16] = acc[i][j][r];
  __syncthreads();
  for (int e = t; e < BM * BN; e += NT) {
    float v = 0.0f;
#pragma unroll
    for (int u = 0; u < KW; ++u) v += red[u][e];
    const int m = e / BN;
    const long n = n0 + (e - m * BN);
    if (m0 + m < p.M && n < s.n) put(s, m0 + m, n, v);
  }
}

template <int TI, int TJ, int KW>
hipError_t launch_skinny(ProjArgs& p, int mblocks, hipStream_t st) {
  int tiles = 0;
  for (int i = 0; i < p.nseg; ++i) {
    p.seg[i].tile0 = tiles;
    tiles += static_cast<int>((p.seg[i].n + 16 * TJ - 1) / (16 * TJ));
  }
  gdn_proj_skinny<TI, TJ, KW, 3><<<dim3(tiles, mblocks), 64 * KW, 0, st>>>(p);
  return hipGetLastError();
}

// Row blocks and TI (16 rows per accumulator tile) from the row count. With fewer than
// 256 column tiles the rows are split into blocks until the grid covers the CUs: each
// workgroup then streams fewer X rows through its CU, and the row blocks of a column
// tile (workgroups t and t + tiles, on the same XCD when tiles is a multiple of 8) find
// its W rows in the shared L2.
template <int TJ, int KW>
hipError_t launch_skinny_m(ProjArgs& p, long ntiles, int cus, hipStream_t st) {
  int mb = 1;
  while (ntiles * mb < cus && 16 * mb < p.M) mb *= 2;
  const int rows = (p.M + mb - 1) / mb;
  if (rows <= 16) return launch_skinny<1, TJ, KW>(p, (p.M + 15) / 16, st);
  if (rows <= 32) return launch_skinny<2, TJ, KW>(p, (p.M + 31) / 32, st);
  if (rows <= 48) return launch_skinny<3, TJ, KW>(p, (p.M + 47) / 48, st);
  return launch_skinny<4, TJ, KW>(p, (p.M + 63) / 64, st);
}

// ----------------------------------------------------------------------------------
// Pipelined MFMA tiles for many rows (compute-bound). BM x BN tile per workgroup of
// WM x WN waves; 64-deep stages in a ring of S LDS slots, filled by direct-to-LDS DMA
// (global_load_lds_dwordx4: 64 lanes x 16 bytes into 1 KB of consecutive LDS), so S - 1
// stages of loads are in flight without registers. A stage holds BM rows of X and BN
// rows of W, 128 bytes (eight 16-byte cells) each; cell c of row r is stored at
// position c ^ (r & 7), so the eight rows that one fragment read touches per LDS cycle
// hit eight different bank groups. One DMA instruction fills 8 rows: lane i writes
// position i & 7 of row i >> 3 and so fetches cell (i & 7) ^ (i >> 3) of that row.
// Per stage: wait until this wave's DMA of the stage has landed (the memory counter,
// S - 2 later stages may still be in flight), an LDS-only barrier, then the DMA of
// stage + S - 1 into the slot every wave finished reading before the barrier, then the
// products (with the 256-row tiles, the DMA instructions go out between the products).
// No LDS store is issued in the loop, so nothing there waits for the DMA.
// Rows past M or the segment end are clamped to valid rows; they feed only outputs
// that are not stored.
// ----------------------------------------------------------------------------------
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// One DMA instruction: 16 bytes per lane from src into 1 KB of consecutive LDS at dst. A
// plain device function: the builtin has no host form, and a kernel that names it
// directly (or through a lambda or a function template) can lose its host launch stub.
__device__ __forceinline__ void dma16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
template <int BM, int BN, int S, int WM, int WN, int KB, bool ROT, bool IL>
__global__ __launch_bounds__(64 * WM * WN) void gdn_proj_pipe(const ProjArgs p) {
  constexpr int NW = WM * WN;           // waves
  constexpr int R = BM + BN;            // rows per stage
  constexpr int CPR = KB / 8;           // 16-byte cells per row of a stage
  constexpr int RPI = 64 / CPR;         // rows one DMA instruction fills (1 KB)
  constexpr int NI = R / RPI / NW;      // DMA instructions per wave per stage
  constexpr int TI = BM / WM / 16, TJ = BN / WN / 16;
  static_assert(KB % 64 == 0 && KB <= 512, "stage depth");
  static_assert(R % (RPI * NW) == 0 && TI >= 1 && TJ >= 1, "tile shape");
  static_assert((S - 2) * NI < 64, "memory counter range");
  __shared__ __attribute__((aligned(16))) uint16_t ring[S][R][KB];

  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by id, so XCD x takes
  // the column tiles nt = x, x + 8, ..., each with all its row blocks in a row. The
  // weight tile then comes from HBM once per column tile and the row blocks of the
  // activations are read by one XCD's workgroups, from its L2.
  const int id = static_cast<int>(blockIdx.x), xcd = id & 7, k = id >> 3, nmb = p.mblocks;
  const int nt = (k / nmb) * 8 + xcd;
  if (nt >= p.ntiles) return;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxProjSegs; ++i)
    if (i < p.nseg && nt >= p.seg[i].tile0) si = i;
  const ProjSeg s = p.seg[si];
  const long n0 = static_cast<long>(nt - s.tile0) * BN;
  const long m0 = static_cast<long>(k % nmb) * BM;
  const int K = p.K, nk = K / KB;
  // ROT: workgroup k takes the stages in the order k mod nk, ..., nk - 1, 0, ... (a
  // template flag: the wrap costs the short loop of the small tiles a few instructions)
  const int rot = ROT ? static_cast<int>(static_cast<unsigned>(k) % static_cast<unsigned>(nk)) : 0;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, q = l >> 4, c16 = l & 15;
  const int wm = w / WN, wn = w % WN;

  // this lane's DMA sources: instruction i of wave w fills rows RPI (NI w + i) .. + RPI - 1,
  // lane l position l % CPR of row l / CPR, with the global cell whose swizzled place that is
  const uint16_t* src[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = RPI * (NI * w + i) + l / CPR, cell = (l % CPR) ^ (r & 7);
    src[i] = r < BM ? p.x + min(m0 + r, static_cast<long>(p.M) - 1) * K + 8 * cell
                    : s.w + min(n0 + (r - BM), s.n - 1) * K + 8 * cell;
  }
  uint16_t* const ring0 = &ring[0][0][0] + 512 * NI * w;  // this wave's blocks of slot 0

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // the NI DMA instructions of stage j: 16 bytes per lane from src[i] + KB j into the
  // 1 KB blocks of this wave in ring slot j % S
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < nk)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        dma16(src[i] + static_cast<long>(KB) * (j + rot < nk ? j + rot : j + rot - nk), ring0 + j * (R * KB) + 512 * i);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's DMA of stage kt has landed once at most the S - 2 later stages are
    // outstanding (the memory counter drains in issue order)
    if (kt + S - 2 < nk)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 2) * NI));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    // the DMA of stage kt + S - 1 into the slot every wave finished reading before the
    // barrier: issued at once, or (IL) one instruction after every GAP products of this
    // stage, so that a wave does not stall on the memory pipe with its products unissued
    const bool more = kt + S - 1 < nk;
    const int jn = kt + S - 1;
    const long joff = static_cast<long>(KB) * (jn + rot < nk ? jn + rot : jn + rot - nk);
    uint16_t* const jdst = ring0 + (jn % S) * (R * KB);
    constexpr int NM = (KB / 32) * TI * TJ, GAP = NM / NI > 0 ? NM / NI : 1;
    if (!IL && more) {
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(src[i] + joff, jdst + 512 * i);
    }
    const uint16_t* st = &ring[kt % S][0][0];
#pragma unroll
    for (int kk = 0; kk < KB / 32; ++kk) {
      bf16x8 a[TI], bb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int r = wm * (BM / WM) + 16 * i + c16;
        a[i] = *reinterpret_cast<const bf16x8*>(st + KB * r + 8 * ((4 * kk + q) ^ (r & 7)));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int r = BM + wn * (BN / WN) + 16 * j + c16;
        bb[j] = *reinterpret_cast<const bf16x8*>(st + KB * r + 8 * ((4 * kk + q) ^ (r & 7)));
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
          const int idx = (kk * TI + i) * TJ + j;
          if (IL && idx % GAP == 0 && idx / GAP < NI && more) dma16(src[idx / GAP] + joff, jdst + 512 * (idx / GAP));
        }
    }
    if (IL && more) {  // instructions left over when there are more of them than products
#pragma unroll
      for (int i = NM; i < NI; ++i) dma16(src[i] + joff, jdst + 512 * i);
    }
  }
  // The tile leaves through LDS: the ring is free once every wave is past its last
  // products, so the accumulators go there as an fp32 BM x BN tile (lane: rows 4q + r,
  // column c16 of each 16 x 16 block), and the tile is stored row-wise in 16-byte pieces.
  __syncthreads();
  float* const tile = reinterpret_cast<float*>(&ring[0][0][0]);
  constexpr int TS = BN + 4;  // row stride in floats
  static_assert(BM * TS * 4 <= S * R * KB * 2, "output tile fits the ring");
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        tile[(wm * (BM / WM) + 16 * i + 4 * q + r) * TS + wn * (BN / WN) + 16 * j + c16] = acc[i][j][r];
  __syncthreads();
  // E output elements per 16-byte piece; a piece is stored whole when its columns are in
  // range and the segment's rows keep it 16-byte aligned, else element by element
  const int E = s.y_bf16 ? 8 : 4;
  const bool vec = (s.n % E) == 0 && (reinterpret_cast<uintptr_t>(s.y) & 15) == 0;
  const int pieces = BN / E;
  for (int e = t; e < BM * pieces; e += 64 * NW) {
    const int row = e / pieces, c0 = (e % pieces) * E;
    const long m = m0 + row, n = n0 + c0;
    if (m >= p.M || n >= s.n) continue;
    const float* v = tile + row * TS + c0;
    if (vec && n + E <= s.n) {
      u32x4 o;
      if (s.y_bf16) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          o[h] = static_cast<uint32_t>(to_bf16(v[2 * h])) | (static_cast<uint32_t>(to_bf16(v[2 * h + 1])) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(s.y) + m * s.n + n) = o;
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) o[h] = __float_as_uint(v[h]);
        *reinterpret_cast<u32x4*>(static_cast<float*>(s.y) + m * s.n + n) = o;
      }
    } else {
      for (int h = 0; h < E && n + h < s.n; ++h) put(s, m, n + h, v[h]);
    }
  }
}

template <int BM, int BN, int S, int WM = 2, int WN = 2, int KB = 64>
hipError_t launch_pipe(ProjArgs& p, hipStream_t st) {
  int tiles = 0;
  for (int i = 0; i < p.nseg; ++i) {
    p.seg[i].tile0 = tiles;
    tiles += static_cast<int>((p.seg[i].n + BN - 1) / BN);
  }
  p.ntiles = tiles;
  p.mblocks = static_cast<int>((p.M + BM - 1) / BM);
  // one workgroup per (column tile, row block), column tiles rounded up to a multiple of 8
  const dim3 grid(static_cast<unsigned>(((tiles + 7) / 8) * 8 * p.mblocks));
  // the 256-row tiles spread their DMA over the products (in_proj, hidden = 2048, at 512 /
  // 1024 rows: 41.0 / 80.8 -> 38.3 / 73.7 us); the smaller tiles, whose waves each issue
  // few products per stage, issue it at once (spread: in_proj at 64 / 256 rows 13.3 /
  // 25.1 -> 14.5 / 28.8 us)
  constexpr bool IL = BM >= 256;
  if (p.krot)
    gdn_proj_pipe<BM, BN, S, WM, WN, KB, true, IL><<<grid, 64 * WM * WN, 0, st>>>(p);
  else
    gdn_proj_pipe<BM, BN, S, WM, WN, KB, false, IL><<<grid, 64 * WM * WN, 0, st>>>(p);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN>
hipError_t launch_mfma(ProjArgs& p, hipStream_t st) {
  int tiles = 0;
  for (int i = 0; i < p.nseg; ++i) {
    p.seg[i].tile0 = tiles;
    tiles += static_cast<int>((p.seg[i].n + BN - 1) / BN);
  }
  const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>((p.M + BM - 1) / BM));
  gdn_proj_mfma<BM, BN, BK, WM, WN><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_gemv(const ProjArgs& p, hipStream_t st) {
  // Many rows (in_proj): a wave per row and no cap on the grid, so every wave's loads
  // go out in one pass (in_proj at B = 1 / 2: 11.7 / 12.5 -> 10.7 / 11.6 us against two
  // rows per wave on at most 1024 workgroups). Fewer rows: up to 1024 workgroups.
  const size_t lds = static_cast<size_t>(MT) * p.K * 2;
  if (p.rows >= 8192) {
    const unsigned grid = static_cast<unsigned>((p.rows + 3) / 4);
    gdn_proj_gemv<MT, 1, 4><<<grid, 256, lds, st>>>(p);
  } else {
    const unsigned grid = static_cast<unsigned>(std::min<long>((p.rows + 3) / 4, 1024));
    gdn_proj_gemv<MT, 1, 8><<<grid, 256, lds, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj(ProjArgs p, hipStream_t st) {
  long rows = 0;
  for (int i = 0; i < p.nseg; ++i) {
    p.seg[i].row0 = rows;
    rows += p.seg[i].n;
  }
  p.rows = rows;
  // Few output columns and a long K (the out_proj shape) at 3..32 rows: the skinny MFMA
  // kernel, K split over 8 waves, one 16-column tile per workgroup, 16 rows per workgroup
  // when that doubles the grid. Measured at hidden = 2048, K = 4096: 8.3 / 9.6 / 9.7 us at
  // 4 / 16 / 32 rows (32 rows in one block: 13.3 us), against 8.3 / 15.4 / 15.5 with the
  // weight-streaming and tiled paths. At 48 and 64 rows the split gave no gain over the
  // tiled kernel (13.3-13.5 us either way).
  if (p.M >= 3 && p.M <= 32 && rows <= 4096 && p.K % 512 == 0) return launch_skinny_m<1, 8>(p, (rows + 15) / 16, 256, st);
  // weight streaming for one or two rows, and for up to 8 rows when there are too few
  // output columns to give the MFMA tiles a full grid (X rows within the default LDS
  // allowance of 64 KB)
  const int mt = p.M <= 1 ? 1 : p.M <= 2 ? 2 : p.M <= 4 ? 4 : 8;
  if ((p.M <= 2 || (p.M <= 8 && rows < 8192)) && static_cast<long>(mt) * p.K * 2 <= 65536) {
    if (mt == 1) return launch_gemv<1>(p, st);
    if (mt == 2) return launch_gemv<2>(p, st);
    if (mt == 4) return launch_gemv<4>(p, st);
    return launch_gemv<8>(p, st);
  }
  // MFMA tiles: large tiles need fewer weight and LDS bytes per MFMA, small ones give
  // more workgroups; measured at hidden = 2048 and 12352 / 2048 output columns (in_proj /
  // out_proj), each rule below takes the fastest tile of its range
  auto tiles = [&](int bm, int bn) {
    long n = 0;
    for (int i = 0; i < p.nseg; ++i) n += (p.seg[i].n + bn - 1) / bn;
    return n * ((p.M + bm - 1) / bm);
  };
  // The DMA-ring workgroups stream their stages in staggered orders while the activations
  // are small (at most 2 MB), so that the workgroups running at once read different
  // slices of the weights: in_proj at 64 rows 14.2 -> 13.3 us, out_proj at 96 / 128 rows
  // 12.1 / 12.4 -> 11.7 / 12.0 us. Larger activations keep the common order, in which the
  // workgroups of an XCD read each activation slice together from its L2 (in_proj /
  // out_proj at 1024 rows: 70.6 / 27.8 us, staggered 73.7 / 39.2 us).
  p.krot = static_cast<long>(p.M) * p.K * 2 <= (2L << 20) ? 1 : 0;
  // A long contraction (the out_proj shape, K = H_v d_v = 4096) over few output columns
  // (at most 4096) takes deeper stages (below).
  const bool deep = p.K >= 4096 && p.K % 256 == 0 && rows <= 4096;
  // Otherwise 64-row blocks on 3-stage rings of 72 or 48 KB (two or three workgroups per
  // CU): 64 x 128 tiles while they make 257..448 workgroups, else 64 x 64 tiles where
  // 256-row blocks would pad two or more 64-row blocks and would still make 128 or more
  // workgroups. in_proj (hidden 2048) at 160 / 256 / 320 / 384 / 576 rows: 25.2 / 26.2 /
  // 36.3 / 36.8 / 66.6 -> 22.0 / 23.1 / 30.1 / 33.2 / 47.5 us (at 448 rows, one block
  // of padding, 64 x 64 measured 37.9 against 36.9 us).
  if (!deep) {
    const long t64 = tiles(64, 128);
    if (t64 > 256 && t64 <= 448) return launch_pipe<64, 128, 3>(p, st);
    if (tiles(256, 128) >= 128 && (p.M + 255) / 256 * 4 >= (p.M + 63) / 64 + 2) return launch_pipe<64, 64, 3>(p, st);
  }
  // many rows (in_proj at 512+): 256 x 128 tiles of 8 waves on a 3-stage DMA ring (144 KB
  // of LDS, one workgroup of two waves per SIMD per CU): 61.0 / 118.4 -> 47.8 / 95.6 us at
  // 512 / 1024 rows
  if (tiles(256, 128) >= 128) return launch_pipe<256, 128, 3, 4, 2>(p, st);
  // 128 x 128 tiles of 4 waves on a 4-stage ring (128 KB) when they still give 192
  // workgroups and their row blocks pad no more rows than 64-row blocks would (in_proj at
  // 256 rows, before the 64-row rings above: 28.9 -> 26.6 us)
  if (tiles(128, 128) >= 192 && (p.M + 127) / 128 * 2 == (p.M + 63) / 64) return launch_pipe<128, 128, 4>(p, st);
  // otherwise the largest of the 64 x 64, 32 x 64 and 32 x 32 rings (4 waves, 4 stages of
  // 64 / 48 / 32 KB) that gives at least 384 workgroups, so that the CUs whose tiles come
  // first are not the only ones streaming. in_proj at 4 / 16 / 64 rows: 12.2 / 12.2 /
  // 17.6 -> 10.9 / 11.1 / 14.3 us; out_proj at 256 / 320 / 384 rows: 23.5 / 32.7 / 33.1
  // -> 17.1 / 19.1 / 19.6 us (hidden = 2048)
  if (tiles(64, 64) >= 384) return launch_pipe<64, 64, 4>(p, st);
  if (tiles(32, 64) >= 384) return launch_pipe<32, 64, 4>(p, st);
  // The long contraction over few output columns (deep): 128-deep stages halve the
  // barriers and make each DMA instruction fetch 256 contiguous bytes of 4 rows. out_proj
  // (hidden = 2048) at 160 / 192 / 256 rows: 18.8 / 17.0 / 17.2 -> 15.2 / 15.8 / 16.2 us
  // against 64-deep stages (in_proj's 2048-long contraction gained nothing from them).
  if (deep && tiles(32, 32) >= 384) return launch_pipe<32, 32, 4, 2, 2, 128>(p, st);
  if (tiles(32, 32) >= 384) return launch_pipe<32, 32, 4>(p, st);
  // Up to 128 rows, 16 x 16 tiles of one wave on a ring of four 128-deep stages (32 KB,
  // up to five workgroups per CU): out_proj (hidden 2048) at 33 / 48 / 64 / 96 / 128 rows
  // 11.4 / 11.4 / 11.4 / 11.7 / 12.1 -> 10.1 / 10.1 / 10.1 / 11.0 / 11.7 us. Up to 64 rows
  // the stages keep the common order (staggered: 10.7 us at 33..64 rows, where each
  // column tile's four row blocks then stop sharing its weight rows in L2).
  if (deep && p.M <= 128) {
    if (p.M <= 64) p.krot = 0;
    return launch_pipe<16, 16, 4, 1, 1, 128>(p, st);
  }
  if (deep) return launch_pipe<32, 16, 4, 2, 1, 128>(p, st);
  // 64 x 64 ring with a full grid
  if (tiles(64, 64) >= 256) return launch_pipe<64, 64, 4>(p, st);
  // 32 x 32 tiles: 64-deep stages keep 8 workgroups per CU resident when the grid is
  // large; a small grid needs the deeper stages for bytes in flight
  if (tiles(32, 32) < 512 && p.K % 256 == 0) return launch_mfma<32, 32, 256, 2, 2>(p, st);
  return launch_mfma<32, 32, 64, 2, 2>(p, st);
}

}  // namespace gdn
