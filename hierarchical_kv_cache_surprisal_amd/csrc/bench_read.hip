// A plain streaming read of device memory, as a measured reference for the
// HBM roofline: what 16-byte vector loads over a buffer reach on this GPU,
// next to the 8 TB/s specification peak.  Built into its own library
// (libsekv_bench.so), used by the benchmark only; not part of the SeKV API.
//
//   int sekv_bench_read(const void* src, uint64_t bytes, uint32_t* sink,
//                       int32_t sink_len, int32_t grid, int32_t unroll,
//                       hipStream_t stream)
//
// src: device buffer of `bytes` (a multiple of 16, 16-byte aligned), read once.
// sink: device uint32 [sink_len] >= grid, written only if a checksum matches a
// value it never takes (keeps the loads live).  grid: workgroups of 256
// threads, each reading one contiguous slice; unroll: 4 or 8 loads of 16 bytes
// in flight per thread.  Returns 0, or -1 for bad arguments (nothing launched),
// or the HIP error of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int U>
__global__ __launch_bounds__(256) void k_read(const uint4* __restrict__ src, uint64_t n16, uint32_t* sink) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t lo = (uint64_t)blockIdx.x * per;
  const uint64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  uint64_t i = lo + threadIdx.x;
  // full rounds: every load in bounds, no lane condition
  for (; i + (uint64_t)(U - 1) * 256 < hi; i += 256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + (uint64_t)u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (; i < hi; i += 256) {
    const uint4 v = src[i];
    acc ^= v.x + v.y + v.z + v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int sekv_bench_read(const void* src, uint64_t bytes, uint32_t* sink, int32_t sink_len, int32_t grid,
                               int32_t unroll, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0 || grid < 1 ||
      grid > sink_len || (unroll != 4 && unroll != 8))
    return -1;
  const uint4* s = static_cast<const uint4*>(src);
  if (unroll == 4)
    hipLaunchKernelGGL(k_read<4>, dim3(grid), dim3(256), 0, stream, s, bytes / 16, sink);
  else
    hipLaunchKernelGGL(k_read<8>, dim3(grid), dim3(256), 0, stream, s, bytes / 16, sink);
  return (int)hipGetLastError();
}
