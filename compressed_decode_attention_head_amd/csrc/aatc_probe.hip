// A plain HBM read probe: the bandwidth that the decode-attention figures are compared with
// besides the vendor's peak.  It reads a buffer once with 16-byte vector loads and no other work
// (an XOR per load, kept live by one store per workgroup), the best case for any pass that must
// stream a cache of that size.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "aatc_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;               // independent loads in flight per thread and iteration
typedef unsigned u4 __attribute__((ext_vector_type(4)));

// Workgroup w reads the contiguous 16-byte units [w * per, (w + 1) * per) of the buffer.
__global__ __launch_bounds__(kThreads) void k_read_probe(const u4* __restrict__ src, int64_t units, int64_t per,
                                                          u4* __restrict__ sink) {
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * per;
  int64_t end = begin + per;
  if (end > units) end = units;
  u4 acc = {0u, 0u, 0u, 0u};
  int64_t i = begin + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
    u4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < end; i += kThreads) acc ^= src[i];
  __shared__ u4 red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u4 r = {0u, 0u, 0u, 0u};
    for (int t = 0; t < kThreads; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

extern "C" {

size_t aatc_probe_read_sink_bytes(void) { return static_cast<size_t>(AATC_PROBE_WORKGROUPS) * 16; }

aatc_status aatc_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  aatc::clear_error();
  if (!src || !sink) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(sink) & 15) || (bytes & 15) ||
      bytes == 0)
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "src, sink and bytes must be non-zero multiples of 16");
  const int64_t units = static_cast<int64_t>(bytes / 16);
  const int64_t per = (units + AATC_PROBE_WORKGROUPS - 1) / AATC_PROBE_WORKGROUPS;
  hipLaunchKernelGGL(k_read_probe, dim3(AATC_PROBE_WORKGROUPS), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u4*>(src), units, per, static_cast<u4*>(sink));
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return aatc::fail(AATC_ERR_HIP, "probe launch: %s", hipGetErrorString(err));
  return AATC_OK;
}

}  // extern "C"
