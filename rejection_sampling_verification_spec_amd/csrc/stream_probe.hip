// stream_probe.hip -- the streaming-read ceiling that the benchmark compares the
// row-statistics kernel with (a measurement kernel, not part of the verify step).
//
// Each workgroup reads one contiguous chunk of the buffer with the access
// pattern of the row-statistics kernel and none of its arithmetic: 256 threads,
// tiles of 8 16-byte non-temporal loads per thread, the next tile requested
// before the current one is consumed (two tiles in flight), an XOR fold, and one
// 32-bit word written per workgroup.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svprobe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kU = 8;

__device__ __forceinline__ void load_tile(const u32x4 *p, long t0, long v1, u32x4 *dst) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const long i = t0 + static_cast<long>(u) * kThreads + threadIdx.x;
    dst[u] = i < v1 ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ unsigned fold(const u32x4 *t) {
  unsigned a = 0;
#pragma unroll
  for (int u = 0; u < kU; ++u) a ^= t[u].x ^ t[u].y ^ t[u].z ^ t[u].w;
  return a;
}

__global__ __launch_bounds__(kThreads) void k_stream_read(const u32x4 *__restrict__ buf, long nvec, long chunk_vecs,
                                                          unsigned *__restrict__ out) {
  const long v0 = static_cast<long>(blockIdx.x) * chunk_vecs;
  const long v1 = v0 + chunk_vecs < nvec ? v0 + chunk_vecs : nvec;
  constexpr long kTile = static_cast<long>(kU) * kThreads;
  unsigned acc = 0;
  u32x4 a[kU], b[kU];
  if (v0 < v1) {
    load_tile(buf, v0, v1, a);
    for (long t0 = v0;;) {
      load_tile(buf, t0 + kTile, v1, b);
      acc ^= fold(a);
      t0 += kTile;
      if (t0 >= v1) break;
      load_tile(buf, t0 + kTile, v1, a);
      acc ^= fold(b);
      t0 += kTile;
      if (t0 >= v1) break;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) acc ^= __shfl_xor(acc, off);
  __shared__ unsigned sh[kThreads / 64];
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = sh[0] ^ sh[1] ^ sh[2] ^ sh[3];
}

}  // namespace

extern "C" int sv_stream_probe(const void *buf, size_t bytes, int groups, unsigned *out, void *stream,
                               void *events[2]) {
  if (!buf || !out || groups < 1 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return -1;
  const long nvec = static_cast<long>(bytes / 16);
  const long chunk = (nvec + groups - 1) / groups;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (events && events[0] && events[1])
    hipExtLaunchKernelGGL(k_stream_read, dim3(groups), dim3(kThreads), 0, st, static_cast<hipEvent_t>(events[0]),
                          static_cast<hipEvent_t>(events[1]), 0, static_cast<const u32x4 *>(buf), nvec, chunk, out);
  else
    hipLaunchKernelGGL(k_stream_read, dim3(groups), dim3(kThreads), 0, st, static_cast<const u32x4 *>(buf), nvec,
                       chunk, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
