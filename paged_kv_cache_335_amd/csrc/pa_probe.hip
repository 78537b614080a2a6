// Read-bandwidth probes: what this GPU's HBM delivers to a plain streaming
// read, and to a gather of fixed-size chunks in random order (the access
// pattern of a paged K/V read, where each block of a sequence sits somewhere
// else in the pool).  Measurement helpers for the benchmark; the decode
// path does not use them.  Contract: include/pa_probe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_probe.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef const u32x4 __attribute__((address_space(1)))* gvec;

constexpr int kThreads = 256;

__device__ __forceinline__ u32x4 ld_nt(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<gvec>(reinterpret_cast<uint64_t>(p)));
}

// Each workgroup reads chunk c = order[i] for i = blockIdx.x, blockIdx.x +
// gridDim.x, ...: chunk_bytes contiguous bytes at c * chunk_bytes, as
// 16-byte non-temporal loads, kUnroll in flight per thread.  XOR of
// everything read goes to sink[thread] so the loads stay live.
template <int kUnroll>
__global__ __launch_bounds__(kThreads) void gather_read_kernel(const uint8_t* __restrict__ buf,
                                                               const int32_t* __restrict__ order,
                                                               int32_t n_chunks,
                                                               uint32_t chunk_bytes,
                                                               uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint32_t per_pass = kThreads * 16 * kUnroll;
  for (int32_t i = blockIdx.x; i < n_chunks; i += gridDim.x) {
    const uint8_t* base = buf + (size_t)order[i] * chunk_bytes;
    for (uint32_t off = threadIdx.x * 16; off < chunk_bytes; off += per_pass) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t o = off + u * kThreads * 16;
        v[u] = o < chunk_bytes ? ld_nt(base + o) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
  }
  sink[blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

size_t pa_probe_sink_bytes(int32_t workgroups) {
  return workgroups > 0 ? (size_t)workgroups * kThreads * sizeof(uint32_t) : 0;
}

pa_status pa_probe_read(const void* buf, const int32_t* order, int32_t n_chunks,
                        uint32_t chunk_bytes, int32_t workgroups, int32_t loads_in_flight,
                        void* sink, void* stream) {
  if (!buf || !order || !sink || n_chunks <= 0 || workgroups <= 0) return PA_EINVAL;
  if (chunk_bytes == 0 || chunk_bytes % 16 != 0) return PA_EINVAL;
  const auto* b = static_cast<const uint8_t*>(buf);
  auto* k = static_cast<uint32_t*>(sink);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (loads_in_flight) {
    case 1: gather_read_kernel<1><<<workgroups, kThreads, 0, st>>>(b, order, n_chunks, chunk_bytes, k); break;
    case 2: gather_read_kernel<2><<<workgroups, kThreads, 0, st>>>(b, order, n_chunks, chunk_bytes, k); break;
    case 4: gather_read_kernel<4><<<workgroups, kThreads, 0, st>>>(b, order, n_chunks, chunk_bytes, k); break;
    case 8: gather_read_kernel<8><<<workgroups, kThreads, 0, st>>>(b, order, n_chunks, chunk_bytes, k); break;
    default: return PA_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_EHIP;
}

}  // extern "C"
