// Streaming copy of the benchmark (libgdn_bench.so): the achievable-bandwidth reference
// for the HBM-bound kernels, and the kernel the HBM traffic counters are calibrated on.
// It moves data the way the decode kernel streams its state: 128-bit raw buffer loads
// and stores with the non-temporal (nt) cache policy, or the default policy. Each
// workgroup copies one 32 KiB block: every lane issues its eight 16-byte loads, then
// its eight stores (of the shapes measured on MI355X, grid-stride loops with 2-8 loads
// in flight and 1-8 workgroups per CU, one-shot blocks of 32-128 KiB, in place or not,
// this one was the fastest). Not part of the layer's ABI (include/gdn.h).

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
constexpr int kThreads = 256;
constexpr int kDepth = 8;                            // 16-byte transfers per lane
constexpr uint32_t kBlock = kThreads * kDepth * 16;  // bytes per workgroup (32 KiB)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  // raw-dword resource of the gfx9 family (word 3 = 0x00020000): accesses past `bytes`
  // read 0 and are not written
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

template <int AUX>
__global__ __launch_bounds__(kThreads) void stream_copy(const void* src, void* dst, uint32_t bytes) {
  const __amdgpu_buffer_rsrc_t rs = rsrc(src, bytes), rd = rsrc(dst, bytes);
  const uint32_t base = blockIdx.x * kBlock;
  u32x4 v[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i)
    v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + (i * kThreads + threadIdx.x) * 16, 0, AUX);
#pragma unroll
  for (int i = 0; i < kDepth; ++i)
    __builtin_amdgcn_raw_buffer_store_b128(v[i], rd, base + (i * kThreads + threadIdx.x) * 16, 0, AUX);
}

}  // namespace

// Copies `bytes` bytes (a multiple of 16) from src to dst (device pointers, not
// overlapping) on `stream`, with non-temporal loads and stores when nt != 0, in pieces
// of at most 1 GiB (a partial last block is cut by the buffer range check). Returns 0,
// or -1 for an invalid argument, -8 if a launch fails.
extern "C" int gdn_bench_stream_copy(const void* src, void* dst, uint64_t bytes, int nt, void* stream) {
  if (!src || !dst || bytes % 16 != 0) return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (uint64_t off = 0; off < bytes; off += (1ull << 30)) {
    const uint32_t n = static_cast<uint32_t>(bytes - off < (1ull << 30) ? bytes - off : (1ull << 30));
    const dim3 grid((n + kBlock - 1) / kBlock);
    const char* sp = static_cast<const char*>(src) + off;
    char* dp = static_cast<char*>(dst) + off;
    if (nt)
      stream_copy<2><<<grid, kThreads, 0, s>>>(sp, dp, n);
    else
      stream_copy<0><<<grid, kThreads, 0, s>>>(sp, dp, n);
    if (hipGetLastError() != hipSuccess) return -8;
  }
  return 0;
}
