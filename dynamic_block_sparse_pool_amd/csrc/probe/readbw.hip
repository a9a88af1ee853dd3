// Read-bandwidth probe for the benchmark: streams a device buffer once with 16-byte
// non-temporal loads (eight in flight per lane) and writes one word per workgroup, so nearly
// all of its traffic is HBM reads. It gives the achievable read-only ceiling that the
// selection kernels (which read Q and K once and write almost nothing) are compared with.
// Built into its own library, libdbsp_probe.so; the attention library does not contain it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4* __restrict__ src,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // one word per workgroup keeps the loads live; the value itself means nothing
  acc = __reduce_or_sync(~0ull, acc);
  if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Enqueue one read of `bytes` bytes (a multiple of 16, 16-byte aligned) at `src` on `stream`;
// `out` receives `grid` words (grid = workgroups, at least 1). Returns 0, or -1 for bad
// arguments, or -5 when the launch fails.
int32_t dbsp_probe_read(const void* src, uint64_t bytes, uint32_t* out, int32_t grid,
                        void* stream) {
  if (!src || !out || grid < 1 || (bytes & 15u) || ((uintptr_t)src & 15u)) return -1;
  read_stream_kernel<<<grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
