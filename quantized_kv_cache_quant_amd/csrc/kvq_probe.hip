// Diagnostic kernels (not part of the method).  read_probe_kernel measures
// the HBM read rate this GPU delivers to a kernel of the attention call's
// shape, so that attention calls can be reported against a measured ceiling
// as well as against the nominal 8 TB/s; rw_probe_kernel moves the bytes of
// a flush (read a block's fp16 rows whole, then write its codes and
// metadata) with nothing else in the way, the ceiling of the flush.
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

// rw_probe_kernel: one workgroup of 256 threads per unit.  Thread t loads
// the unit's 16-byte words t, t + 256, ... (nr of them, all in flight
// together), folds them by XOR into one word w, then stores w + j as the
// unit's output word j for j = t, t + 256, ... < nw.
constexpr int kRwMaxLoads = 8;
__global__ __launch_bounds__(256) void rw_probe_kernel(const u32x4* src, u32x4* dst, int nr, int nw) {
  const u32x4* s = src + (uint64_t)blockIdx.x * nr * 256;
  u32x4 v[kRwMaxLoads];
#pragma unroll
  for (int i = 0; i < kRwMaxLoads; ++i) v[i] = i < nr ? s[threadIdx.x + 256 * i] : u32x4{0u, 0u, 0u, 0u};
  u32x4 acc = v[0];
#pragma unroll
  for (int i = 1; i < kRwMaxLoads; ++i) acc ^= v[i];
  u32x4* d = dst + (uint64_t)blockIdx.x * nw;
  for (int j = threadIdx.x; j < nw; j += 256) d[j] = acc + (unsigned)j;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, uint64_t units, uint32_t* sink, int groups, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)groups), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(buf), units, sink);
  return hipGetLastError();
}

hipError_t launch_rw_probe(const void* src, void* dst, uint64_t units, int read16, int write16, hipStream_t s) {
  if (read16 <= 0 || read16 % 256 != 0 || read16 / 256 > kRwMaxLoads || write16 < 0 || units == 0 ||
      units > 0x7fffffffu)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(rw_probe_kernel, dim3((unsigned)units), dim3(256), 0, s, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), read16 / 256, write16);
  return hipGetLastError();
}

}  // namespace kvq
