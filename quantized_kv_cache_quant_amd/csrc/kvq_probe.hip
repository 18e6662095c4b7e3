// Diagnostic streaming-read kernel (not part of the method): measures the
// HBM read rate this GPU delivers to a kernel of the attention call's shape,
// so that attention calls can be reported against a measured ceiling as
// well as against the nominal 8 TB/s.
//
// read_probe_kernel: one workgroup of 512 threads per part of the buffer;
// each thread keeps eight 16-byte nontemporal loads in flight (consecutive
// threads read consecutive 16-byte units, so every load instruction of a
// wavefront covers 1024 contiguous bytes) and folds what it read into one
// word, written to the sink so that no load can be dropped.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kUnroll = 8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* buf, uint64_t units,
                                                                    uint32_t* sink) {
  const uint64_t per = (units + gridDim.x - 1) / gridDim.x;
  const uint64_t b = (uint64_t)blockIdx.x * per;
  const uint64_t e = b + per < units ? b + per : units;
  uint32_t acc = 0;
  for (uint64_t i = b + threadIdx.x; i < e; i += (uint64_t)kProbeThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t k = i + (uint64_t)u * kProbeThreads;
      v[u] = k < e ? __builtin_nontemporal_load(buf + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(uint64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, uint64_t units, uint32_t* sink, int groups, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)groups), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(buf), units, sink);
  return hipGetLastError();
}

}  // namespace kvq
