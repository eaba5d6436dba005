// Host side of libgdn.so: argument validation and kernel dispatch for the entry
// points declared in include/gdn.h. Every check runs before anything is enqueued, so
// an error return leaves every buffer untouched. No memory is allocated here.

#include "gdn.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <limits>

#include "gdn_internal.h"

namespace {

// A recurrent state larger than this cannot stay in MI355X's 256 MB Infinity Cache
// from one step to the next, so its loads and stores are marked non-temporal; smaller
// states keep the default policy and are re-read from the cache. Measured on MI355X
// (Qwen3.5-style layer, 2 MiB of state per sequence): the default policy is faster up
// to B = 128 (256 MiB), the streaming one from B = 160 (320 MiB) on.
#ifndef GDN_STREAM_STATE_BYTES
#define GDN_STREAM_STATE_BYTES (256ull << 20)
#endif
constexpr uint64_t kStreamStateBytes = GDN_STREAM_STATE_BYTES;

// Compute units of the current device, queried once per device (256 on MI355X).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// gdn_sequence takes the chunked MFMA form from this many tokens on, the token-by-token
// kernel below it. The chunked form runs one workgroup per (sequence, v-head) and CU
// for each chunk of 32 tokens, so its cost for T <= 32 is about one chunk per pass of
// the B x H_v workgroups over the CUs, whatever T is. Crossing points measured on
// MI355X (256 CUs, d = 128, K = 4, B x H_v = 128 ... 2048): T = 5 for one pass (B = 8,
// T = 8: 20.5 against 30.3 us), 9 to 10 for two passes, 13 to 14 from four passes on.
// Each threshold sits a token or so above its crossing point.
int32_t chunked_min_tokens(long units) {
  const long cus = device_cus();
  const long passes = (units + cus - 1) / cus;
  return passes <= 1 ? 6 : (passes <= 2 ? 10 : 14);
}

struct Buf {
  const void* p;
  size_t bytes;
  bool written;
  size_t align;
};

size_t elt(int32_t dtype) { return dtype == GDN_BF16 ? 2 : 4; }

bool valid_dtype(int32_t d) { return d == GDN_F32 || d == GDN_BF16; }

// Shape checks shared by all entry points. `need_heads` is false only for queries.
gdn_status_t check_shape(const gdn_shape_t* s) {
  if (!s) return GDN_ERR_NULL;
  if (s->batch < 0 || s->num_k_heads < 1 || s->num_v_heads < 1 || s->head_k_dim < 1 || s->head_v_dim < 1)
    return GDN_ERR_SHAPE;
  if (s->num_v_heads % s->num_k_heads != 0) return GDN_ERR_SHAPE;
  if (s->conv_kernel < 2 || s->conv_kernel > gdn::kMaxConvTaps) return GDN_ERR_SHAPE;
  if (!(std::isfinite(s->l2_eps) && s->l2_eps >= 0.0f) || !(std::isfinite(s->rms_eps) && s->rms_eps >= 0.0f))
    return GDN_ERR_SHAPE;
  if (!valid_dtype(s->act_dtype) || !valid_dtype(s->out_dtype)) return GDN_ERR_DTYPE;
  // grid = B * H_k workgroups; channel and state offsets are computed in 64 bits
  if (static_cast<int64_t>(s->batch) * s->num_k_heads > std::numeric_limits<int32_t>::max()) return GDN_ERR_SHAPE;
  const int64_t C = 2LL * s->num_k_heads * s->head_k_dim + static_cast<int64_t>(s->num_v_heads) * s->head_v_dim;
  if (C > std::numeric_limits<int32_t>::max()) return GDN_ERR_SHAPE;
  if (s->head_k_dim != s->head_v_dim) return GDN_ERR_UNSUPPORTED;
  const int d = s->head_k_dim;
  if (d != 32 && d != 64 && d != 128) return GDN_ERR_UNSUPPORTED;
  if (s->num_v_heads / s->num_k_heads > 64) return GDN_ERR_UNSUPPORTED;  // LDS holds G*d values
  return GDN_OK;
}

int heads_per_pass(const gdn_shape_t* s) { return (s->num_v_heads / s->num_k_heads) % 2 == 0 ? 2 : 1; }

// Null, alignment and overlap checks. Buffers with bytes == 0 are skipped.
gdn_status_t check_buffers(const Buf* bufs, int n) {
  for (int i = 0; i < n; ++i) {
    if (bufs[i].bytes == 0) continue;
    if (!bufs[i].p) return GDN_ERR_NULL;
  }
  for (int i = 0; i < n; ++i) {
    if (bufs[i].bytes == 0) continue;
    if (reinterpret_cast<uintptr_t>(bufs[i].p) % bufs[i].align != 0) return GDN_ERR_ALIGN;
  }
  for (int i = 0; i < n; ++i) {
    if (bufs[i].bytes == 0) continue;
    for (int j = i + 1; j < n; ++j) {
      if (bufs[j].bytes == 0) continue;
      if (!bufs[i].written && !bufs[j].written) continue;  // read-only pairs may share memory
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(bufs[i].p), a1 = a0 + bufs[i].bytes;
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(bufs[j].p), b1 = b0 + bufs[j].bytes;
      if (a0 < b1 && b0 < a1) return GDN_ERR_ALIAS;
    }
  }
  return GDN_OK;
}

struct Sizes {
  size_t B, Hk, Hv, d, K, C, ea, eo;
  explicit Sizes(const gdn_shape_t* s)
      : B(s->batch), Hk(s->num_k_heads), Hv(s->num_v_heads), d(s->head_k_dim), K(s->conv_kernel),
        C(2 * Hk * d + Hv * d), ea(elt(s->act_dtype)), eo(elt(s->out_dtype)) {}
  size_t conv_state() const { return B * (K - 1) * C * ea; }
  size_t state() const { return B * Hv * d * d * 4; }
  size_t conv_w() const { return C * K * ea; }
};

gdn::KernelArgs base_args(const gdn_shape_t* s) {
  gdn::KernelArgs a{};
  a.B = s->batch;
  a.Hk = s->num_k_heads;
  a.Hv = s->num_v_heads;
  a.G = s->num_v_heads / s->num_k_heads;
  a.K = s->conv_kernel;
  a.C = 2 * s->num_k_heads * s->head_k_dim + s->num_v_heads * s->head_v_dim;
  a.T = 1;
  a.l2_eps = s->l2_eps;
  a.rms_eps = s->rms_eps;
  a.act_bf16 = s->act_dtype == GDN_BF16;
  a.out_bf16 = s->out_dtype == GDN_BF16;
  const uint64_t state_bytes = static_cast<uint64_t>(s->batch) * s->num_v_heads * s->head_k_dim * s->head_v_dim * 4;
  a.stream_state = state_bytes > kStreamStateBytes;
  a.slots = nullptr;
  a.pool = s->batch;
  return a;
}

gdn_status_t launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// Trail of gdn_decode_verify (fp32): delta [B][T][H_v][d_v], then unit k
// [B][T][H_k][d_k], then alpha [B][T][H_v]. Both arrays of d-vectors start 16-byte
// aligned (d is a multiple of 32).
struct TrailLayout {
  size_t delta, k, alpha, bytes;  // byte offsets and total
  TrailLayout(const Sizes& z, size_t T)
      : delta(0), k(z.B * T * z.Hv * z.d * 4), alpha(k + z.B * T * z.Hk * z.d * 4), bytes(alpha + z.B * T * z.Hv * 4) {}
  void assign(gdn::KernelArgs& a, void* base) const {
    char* p = static_cast<char*>(base);
    a.trail_delta = reinterpret_cast<float*>(p + delta);
    a.trail_k = reinterpret_cast<float*>(p + k);
    a.trail_alpha = reinterpret_cast<float*>(p + alpha);
  }
};

}  // namespace

extern "C" {

int32_t gdn_abi_version(void) { return (1 << 16) | 4; }

const char* gdn_status_string(int32_t st) {
  switch (st) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "invalid shape or size";
    case GDN_ERR_DTYPE: return "invalid dtype";
    case GDN_ERR_ALIGN: return "misaligned buffer";
    case GDN_ERR_ALIAS: return "a written buffer overlaps another buffer";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    case GDN_ERR_UNSUPPORTED: return "shape has no compiled kernel (supported: d_k == d_v in {32, 64, 128})";
    case GDN_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

gdn_status_t gdn_conv_update(const gdn_shape_t* shape, void* conv1d_state, const void* qkv,
                             const void* conv1d_weight, float* qkv_act, void* stream) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  const Sizes z(shape);
  if (z.B == 0) return GDN_OK;
  const Buf bufs[] = {
      {conv1d_state, z.conv_state(), true, 16},
      {qkv, z.B * z.C * z.ea, false, 16},
      {conv1d_weight, z.conv_w(), false, 16},
      {qkv_act, z.B * z.C * 4, true, 16},
  };
  if ((st = check_buffers(bufs, 4)) != GDN_OK) return st;
  gdn::KernelArgs a = base_args(shape);
  a.conv_state = conv1d_state;
  a.qkv = qkv;
  a.qkv_bs = static_cast<long>(z.C);
  a.conv_w = conv1d_weight;
  a.qkv_act_out = qkv_act;
  (void)hipGetLastError();
  return launched(gdn::launch_step(gdn::kModeConv, shape->head_k_dim, heads_per_pass(shape), a,
                                   static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_recurrent_step(const gdn_shape_t* shape, float* state, const float* qkv_act,
                                const void* dt_raw, const void* b_raw, const float* A_log,
                                const float* dt_bias, void* y, void* stream) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  const Sizes z(shape);
  if (z.B == 0) return GDN_OK;
  const Buf bufs[] = {
      {state, z.state(), true, 16},
      {qkv_act, z.B * z.C * 4, false, 16},
      {dt_raw, z.B * z.Hv * z.ea, false, z.ea},
      {b_raw, z.B * z.Hv * z.ea, false, z.ea},
      {A_log, z.Hv * 4, false, 4},
      {dt_bias, z.Hv * 4, false, 4},
      {y, z.B * z.Hv * z.d * z.eo, true, 16},
  };
  if ((st = check_buffers(bufs, 7)) != GDN_OK) return st;
  gdn::KernelArgs a = base_args(shape);
  a.state = state;
  a.qkv_act_in = qkv_act;
  a.dt_raw = dt_raw;
  a.b_raw = b_raw;
  a.ab_bs = static_cast<long>(z.Hv);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.out = y;
  a.out_bs = static_cast<long>(z.Hv * z.d);
  (void)hipGetLastError();
  return launched(gdn::launch_step(gdn::kModeRec, shape->head_k_dim, heads_per_pass(shape), a,
                                   static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_decode_layer(const gdn_shape_t* shape, void* conv1d_state, float* state,
                              const void* qkv, const void* conv1d_weight, const void* dt_raw,
                              const void* b_raw, const void* z_in, const float* A_log,
                              const float* dt_bias, const float* norm_weight, void* out,
                              void* stream) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  const Sizes z(shape);
  if (z.B == 0) return GDN_OK;
  const Buf bufs[] = {
      {conv1d_state, z.conv_state(), true, 16},
      {state, z.state(), true, 16},
      {qkv, z.B * z.C * z.ea, false, 16},
      {conv1d_weight, z.conv_w(), false, 16},
      {dt_raw, z.B * z.Hv * z.ea, false, z.ea},
      {b_raw, z.B * z.Hv * z.ea, false, z.ea},
      {z_in, z.B * z.Hv * z.d * z.ea, false, 16},
      {A_log, z.Hv * 4, false, 4},
      {dt_bias, z.Hv * 4, false, 4},
      {norm_weight, z.d * 4, false, 16},
      {out, z.B * z.Hv * z.d * z.eo, true, 16},
  };
  if ((st = check_buffers(bufs, 11)) != GDN_OK) return st;
  gdn::KernelArgs a = base_args(shape);
  a.conv_state = conv1d_state;
  a.state = state;
  a.qkv = qkv;
  a.qkv_bs = static_cast<long>(z.C);
  a.conv_w = conv1d_weight;
  a.dt_raw = dt_raw;
  a.b_raw = b_raw;
  a.ab_bs = static_cast<long>(z.Hv);
  a.z = z_in;
  a.z_bs = static_cast<long>(z.Hv * z.d);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.norm_w = norm_weight;
  a.out = out;
  a.out_bs = static_cast<long>(z.Hv * z.d);
  (void)hipGetLastError();
  return launched(gdn::launch_step(gdn::kModeFused, shape->head_k_dim, heads_per_pass(shape), a,
                                   static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_decode_layer_debug(const gdn_shape_t* shape, void* conv1d_state, float* state, const void* qkv,
                                    const void* conv1d_weight, const void* dt_raw, const void* b_raw,
                                    const void* z_in, const float* A_log, const float* dt_bias,
                                    const float* norm_weight, void* out, float* qkv_act_tap, float* alpha_tap,
                                    float* beta_tap, float* y_tap, float* y_norm_tap, void* stream) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  const Sizes z(shape);
  if (z.B == 0) return GDN_OK;
  const size_t yb = z.B * z.Hv * z.d * 4;
  const Buf bufs[] = {
      {conv1d_state, z.conv_state(), true, 16},
      {state, z.state(), true, 16},
      {qkv, z.B * z.C * z.ea, false, 16},
      {conv1d_weight, z.conv_w(), false, 16},
      {dt_raw, z.B * z.Hv * z.ea, false, z.ea},
      {b_raw, z.B * z.Hv * z.ea, false, z.ea},
      {z_in, z.B * z.Hv * z.d * z.ea, false, 16},
      {A_log, z.Hv * 4, false, 4},
      {dt_bias, z.Hv * 4, false, 4},
      {norm_weight, z.d * 4, false, 16},
      {out, z.B * z.Hv * z.d * z.eo, true, 16},
      // taps: optional (a null tap is not written)
      {qkv_act_tap, qkv_act_tap ? z.B * z.C * 4 : 0, true, 4},
      {alpha_tap, alpha_tap ? z.B * z.Hv * 4 : 0, true, 4},
      {beta_tap, beta_tap ? z.B * z.Hv * 4 : 0, true, 4},
      {y_tap, y_tap ? yb : 0, true, 16},
      {y_norm_tap, y_norm_tap ? yb : 0, true, 16},
  };
  if ((st = check_buffers(bufs, 16)) != GDN_OK) return st;
  gdn::KernelArgs a = base_args(shape);
  a.conv_state = conv1d_state;
  a.state = state;
  a.qkv = qkv;
  a.qkv_bs = static_cast<long>(z.C);
  a.conv_w = conv1d_weight;
  a.dt_raw = dt_raw;
  a.b_raw = b_raw;
  a.ab_bs = static_cast<long>(z.Hv);
  a.z = z_in;
  a.z_bs = static_cast<long>(z.Hv * z.d);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.norm_w = norm_weight;
  a.out = out;
  a.out_bs = static_cast<long>(z.Hv * z.d);
  a.tap_act = qkv_act_tap;
  a.tap_alpha = alpha_tap;
  a.tap_beta = beta_tap;
  a.tap_y = y_tap;
  a.tap_y_norm = y_norm_tap;
  a.taps = 1;
  (void)hipGetLastError();
  return launched(gdn::launch_step(gdn::kModeFused, shape->head_k_dim, heads_per_pass(shape), a,
                                   static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_decode_layer_pooled(const gdn_shape_t* shape, int32_t pool_size, const int32_t* slots,
                                     void* conv1d_state_pool, float* state_pool, const void* qkv,
                                     const void* conv1d_weight, const void* dt_raw, const void* b_raw,
                                     const void* z_in, const float* A_log, const float* dt_bias,
                                     const float* norm_weight, void* out, void* stream) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (pool_size < 0) return GDN_ERR_SHAPE;
  const Sizes z(shape);
  if (z.B == 0) return GDN_OK;
  const size_t P = static_cast<size_t>(pool_size);
  const Buf bufs[] = {
      {slots, z.B * 4, false, 4},
      {conv1d_state_pool, P * (z.K - 1) * z.C * z.ea, true, 16},
      {state_pool, P * z.Hv * z.d * z.d * 4, true, 16},
      {qkv, z.B * z.C * z.ea, false, 16},
      {conv1d_weight, z.conv_w(), false, 16},
      {dt_raw, z.B * z.Hv * z.ea, false, z.ea},
      {b_raw, z.B * z.Hv * z.ea, false, z.ea},
      {z_in, z.B * z.Hv * z.d * z.ea, false, 16},
      {A_log, z.Hv * 4, false, 4},
      {dt_bias, z.Hv * 4, false, 4},
      {norm_weight, z.d * 4, false, 16},
      {out, z.B * z.Hv * z.d * z.eo, true, 16},
  };
  if ((st = check_buffers(bufs, 12)) != GDN_OK) return st;
  if (pool_size == 0) return GDN_OK;  // every slot is outside the pool: nothing to do
  gdn::KernelArgs a = base_args(shape);
  a.slots = slots;
  a.pool = pool_size;
  a.conv_state = conv1d_state_pool;
  a.state = state_pool;
  a.qkv = qkv;
  a.qkv_bs = static_cast<long>(z.C);
  a.conv_w = conv1d_weight;
  a.dt_raw = dt_raw;
  a.b_raw = b_raw;
  a.ab_bs = static_cast<long>(z.Hv);
  a.z = z_in;
  a.z_bs = static_cast<long>(z.Hv * z.d);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.norm_w = norm_weight;
  a.out = out;
  a.out_bs = static_cast<long>(z.Hv * z.d);
  (void)hipGetLastError();
  return launched(gdn::launch_step(gdn::kModeFused, shape->head_k_dim, heads_per_pass(shape), a,
                                   static_cast<hipStream_t>(stream)));
}

// A T-token call moves B x T rows of qkv, z and out; every buffer size computed from
// the shape stays below 2^62 bytes (so none of them wraps in 64 bits) when B x T times
// the largest of those rows does. Evaluated in 128 bits: B, T < 2^31, a row < 2^34 bytes.
bool sequence_fits(const gdn_shape_t* s, int32_t T) {
  const Sizes z(s);
  const size_t row = std::max(z.C * z.ea, z.Hv * z.d * std::max(z.ea, z.eo));
  const unsigned __int128 bytes = static_cast<unsigned __int128>(z.B) * static_cast<uint64_t>(T) * row;
  return bytes <= (static_cast<unsigned __int128>(1) << 62);
}

size_t gdn_sequence_workspace_bytes(const gdn_shape_t* shape, int32_t T) {
  if (check_shape(shape) != GDN_OK || T < 0 || !sequence_fits(shape, T)) return SIZE_MAX;
  return 0;
}

gdn_status_t gdn_sequence(const gdn_shape_t* shape, int32_t T, void* conv1d_state, float* state,
                          const void* qkv, const void* conv1d_weight, const void* dt_raw,
                          const void* b_raw, const void* z_in, const float* A_log,
                          const float* dt_bias, const float* norm_weight, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (T < 0 || !sequence_fits(shape, T)) return GDN_ERR_SHAPE;
  const Sizes z(shape);
  if (z.B == 0 || T == 0) return GDN_OK;
  const size_t need = gdn_sequence_workspace_bytes(shape, T);
  if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
  const size_t Tz = static_cast<size_t>(T);
  const Buf bufs[] = {
      {conv1d_state, z.conv_state(), true, 16},
      {state, z.state(), true, 16},
      {qkv, z.B * Tz * z.C * z.ea, false, 16},
      {conv1d_weight, z.conv_w(), false, 16},
      {dt_raw, z.B * Tz * z.Hv * z.ea, false, z.ea},
      {b_raw, z.B * Tz * z.Hv * z.ea, false, z.ea},
      {z_in, z.B * Tz * z.Hv * z.d * z.ea, false, 16},
      {A_log, z.Hv * 4, false, 4},
      {dt_bias, z.Hv * 4, false, 4},
      {norm_weight, z.d * 4, false, 16},
      {out, z.B * Tz * z.Hv * z.d * z.eo, true, 16},
      {workspace, need, true, 256},
  };
  if ((st = check_buffers(bufs, 12)) != GDN_OK) return st;
  gdn::KernelArgs a = base_args(shape);
  a.T = T;
  a.conv_state = conv1d_state;
  a.state = state;
  a.qkv = qkv;
  a.qkv_bs = static_cast<long>(Tz * z.C);
  a.qkv_ts = static_cast<long>(z.C);
  a.conv_w = conv1d_weight;
  a.dt_raw = dt_raw;
  a.b_raw = b_raw;
  a.ab_bs = static_cast<long>(Tz * z.Hv);
  a.ab_ts = static_cast<long>(z.Hv);
  a.z = z_in;
  a.z_bs = static_cast<long>(Tz * z.Hv * z.d);
  a.z_ts = static_cast<long>(z.Hv * z.d);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.norm_w = norm_weight;
  a.out = out;
  a.out_bs = static_cast<long>(Tz * z.Hv * z.d);
  a.out_ts = static_cast<long>(z.Hv * z.d);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = shape->head_k_dim, G = a.G;
  // the path is chosen before the error state is cleared, so that the launch check
  // below sees only the launch (the device query makes HIP calls of its own)
  const bool chunked = gdn::chunked_supported(d, a.K) && T >= chunked_min_tokens(static_cast<long>(z.B) * z.Hv);
  (void)hipGetLastError();
  if (chunked) return launched(gdn::launch_chunked_sequence(a, s));
  if (gdn::sequence_supported(G, a.K)) return launched(gdn::launch_sequence(d, G, a, s));
  // Shapes whose state or taps do not stay resident: one fused step launch per token.
  const size_t ea = z.ea, eo = z.eo;
  for (int32_t t = 0; t < T; ++t) {
    gdn::KernelArgs at = a;
    at.T = 1;
    at.qkv = static_cast<const char*>(qkv) + t * z.C * ea;
    at.dt_raw = static_cast<const char*>(dt_raw) + t * z.Hv * ea;
    at.b_raw = static_cast<const char*>(b_raw) + t * z.Hv * ea;
    at.z = static_cast<const char*>(z_in) + t * z.Hv * z.d * ea;
    at.out = static_cast<char*>(out) + t * z.Hv * z.d * eo;
    st = launched(gdn::launch_step(gdn::kModeFused, d, heads_per_pass(shape), at, s));
    if (st != GDN_OK) return st;
  }
  return GDN_OK;
}

size_t gdn_verify_trail_bytes(const gdn_shape_t* shape, int32_t T) {
  if (check_shape(shape) != GDN_OK || T < 0 || T > gdn::kMaxVerifyTokens) return SIZE_MAX;
  const Sizes z(shape);
  return TrailLayout(z, static_cast<size_t>(T)).bytes;
}

gdn_status_t gdn_decode_verify(const gdn_shape_t* shape, int32_t T, const void* conv1d_state,
                               const float* state, const void* qkv, const void* conv1d_weight,
                               const void* dt_raw, const void* b_raw, const void* z_in,
                               const float* A_log, const float* dt_bias, const float* norm_weight,
                               void* out, void* trail, size_t trail_bytes, void* stream) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (T < 0 || T > gdn::kMaxVerifyTokens) return GDN_ERR_SHAPE;
  const Sizes z(shape);
  if (z.B == 0 || T == 0) return GDN_OK;
  const size_t Tz = static_cast<size_t>(T);
  const TrailLayout tl(z, Tz);
  if (trail_bytes < tl.bytes) return GDN_ERR_WORKSPACE;
  const Buf bufs[] = {
      {conv1d_state, z.conv_state(), false, 16},
      {state, z.state(), false, 16},
      {qkv, z.B * Tz * z.C * z.ea, false, 16},
      {conv1d_weight, z.conv_w(), false, 16},
      {dt_raw, z.B * Tz * z.Hv * z.ea, false, z.ea},
      {b_raw, z.B * Tz * z.Hv * z.ea, false, z.ea},
      {z_in, z.B * Tz * z.Hv * z.d * z.ea, false, 16},
      {A_log, z.Hv * 4, false, 4},
      {dt_bias, z.Hv * 4, false, 4},
      {norm_weight, z.d * 4, false, 16},
      {out, z.B * Tz * z.Hv * z.d * z.eo, true, 16},
      {trail, tl.bytes, true, 16},
  };
  if ((st = check_buffers(bufs, 12)) != GDN_OK) return st;
  if (static_cast<int64_t>(shape->batch) * shape->num_v_heads > std::numeric_limits<int32_t>::max())
    return GDN_ERR_SHAPE;  // grid = B * H_v workgroups
  gdn::KernelArgs a = base_args(shape);
  a.T = T;
  a.conv_state = const_cast<void*>(conv1d_state);  // read only in this call
  a.state = const_cast<float*>(state);              // read only in this call
  a.qkv = qkv;
  a.qkv_bs = static_cast<long>(Tz * z.C);
  a.qkv_ts = static_cast<long>(z.C);
  a.conv_w = conv1d_weight;
  a.dt_raw = dt_raw;
  a.b_raw = b_raw;
  a.ab_bs = static_cast<long>(Tz * z.Hv);
  a.ab_ts = static_cast<long>(z.Hv);
  a.z = z_in;
  a.z_bs = static_cast<long>(Tz * z.Hv * z.d);
  a.z_ts = static_cast<long>(z.Hv * z.d);
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.norm_w = norm_weight;
  a.out = out;
  a.out_bs = static_cast<long>(Tz * z.Hv * z.d);
  a.out_ts = static_cast<long>(z.Hv * z.d);
  tl.assign(a, trail);
  (void)hipGetLastError();
  return launched(gdn::launch_verify(shape->head_k_dim, a, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_decode_commit(const gdn_shape_t* shape, int32_t T, const int32_t* accepted,
                               void* conv1d_state, float* state, const void* qkv, const void* trail,
                               size_t trail_bytes, void* stream) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (T < 0 || T > gdn::kMaxVerifyTokens) return GDN_ERR_SHAPE;
  const Sizes z(shape);
  if (z.B == 0 || T == 0) return GDN_OK;
  const size_t Tz = static_cast<size_t>(T);
  const TrailLayout tl(z, Tz);
  if (trail_bytes < tl.bytes) return GDN_ERR_WORKSPACE;
  const Buf bufs[] = {
      {accepted, z.B * 4, false, 4},
      {conv1d_state, z.conv_state(), true, 16},
      {state, z.state(), true, 16},
      {qkv, z.B * Tz * z.C * z.ea, false, 16},
      {trail, tl.bytes, false, 16},
  };
  if ((st = check_buffers(bufs, 5)) != GDN_OK) return st;
  if (static_cast<int64_t>(shape->batch) * shape->num_v_heads > std::numeric_limits<int32_t>::max())
    return GDN_ERR_SHAPE;
  gdn::KernelArgs a = base_args(shape);
  a.T = T;
  a.accepted = accepted;
  a.conv_state = conv1d_state;
  a.state = state;
  a.qkv = qkv;
  a.qkv_bs = static_cast<long>(Tz * z.C);
  a.qkv_ts = static_cast<long>(z.C);
  tl.assign(a, const_cast<void*>(trail));  // read only in this call
  (void)hipGetLastError();
  return launched(gdn::launch_commit(shape->head_k_dim, a, static_cast<hipStream_t>(stream)));
}

// Shared checks of the projections: bf16 activations, K a positive multiple of 64.
gdn_status_t check_proj(const gdn_shape_t* shape, int32_t hidden, int64_t K) {
  gdn_status_t st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (hidden < 1) return GDN_ERR_SHAPE;
  if (shape->act_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  // the contraction (hidden for in_proj, H_v d_v for out_proj) goes in 64-deep stages;
  // any number of output columns is fine (ragged tiles are stored element by element)
  if (K % 64 != 0) return GDN_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(shape->batch) + 31) / 32 > 65535) return GDN_ERR_SHAPE;  // grid rows
  return GDN_OK;
}

gdn_status_t gdn_in_proj(const gdn_shape_t* shape, int32_t hidden, const void* x_norm, const void* w_qkv,
                         const void* w_z, const void* w_a, const void* w_b, void* qkv, void* z_out, void* dt_raw,
                         void* b_raw, void* stream) {
  gdn_status_t st = check_proj(shape, hidden, hidden);
  if (st != GDN_OK) return st;
  const Sizes z(shape);
  if (z.B == 0) return GDN_OK;
  const size_t Hd = static_cast<size_t>(hidden), zd = z.Hv * z.d;
  const Buf bufs[] = {
      {x_norm, z.B * Hd * 2, false, 16},
      {w_qkv, z.C * Hd * 2, false, 16},
      {w_z, zd * Hd * 2, false, 16},
      {w_a, z.Hv * Hd * 2, false, 16},
      {w_b, z.Hv * Hd * 2, false, 16},
      {qkv, z.B * z.C * 2, true, 16},
      {z_out, z.B * zd * 2, true, 16},
      {dt_raw, z.B * z.Hv * 2, true, 2},
      {b_raw, z.B * z.Hv * 2, true, 2},
  };
  if ((st = check_buffers(bufs, 9)) != GDN_OK) return st;
  gdn::ProjArgs p{};
  p.M = shape->batch;
  p.K = hidden;
  p.x = static_cast<const uint16_t*>(x_norm);
  p.nseg = 4;
  const void* ws[4] = {w_qkv, w_z, w_a, w_b};
  void* ys[4] = {qkv, z_out, dt_raw, b_raw};
  const long ns[4] = {static_cast<long>(z.C), static_cast<long>(zd), static_cast<long>(z.Hv), static_cast<long>(z.Hv)};
  for (int i = 0; i < 4; ++i) {
    p.seg[i].w = static_cast<const uint16_t*>(ws[i]);
    p.seg[i].y = ys[i];
    p.seg[i].n = ns[i];
    p.seg[i].y_bf16 = 1;
  }
  (void)hipGetLastError();
  return launched(gdn::launch_proj(p, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_out_proj(const gdn_shape_t* shape, int32_t hidden, const void* gated, const void* w_out, void* y,
                          void* stream) {
  const int64_t K = static_cast<int64_t>(shape ? shape->num_v_heads : 0) * (shape ? shape->head_v_dim : 0);
  gdn_status_t st = check_proj(shape, hidden, K);
  if (st != GDN_OK) return st;
  const Sizes z(shape);
  if (z.B == 0) return GDN_OK;
  const size_t Hd = static_cast<size_t>(hidden), zd = z.Hv * z.d;
  const Buf bufs[] = {
      {gated, z.B * zd * 2, false, 16},
      {w_out, Hd * zd * 2, false, 16},
      {y, z.B * Hd * z.eo, true, 16},
  };
  if ((st = check_buffers(bufs, 3)) != GDN_OK) return st;
  gdn::ProjArgs p{};
  p.M = shape->batch;
  p.K = static_cast<int>(zd);
  p.x = static_cast<const uint16_t*>(gated);
  p.nseg = 1;
  p.seg[0].w = static_cast<const uint16_t*>(w_out);
  p.seg[0].y = y;
  p.seg[0].n = hidden;
  p.seg[0].y_bf16 = shape->out_dtype == GDN_BF16;
  (void)hipGetLastError();
  return launched(gdn::launch_proj(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
