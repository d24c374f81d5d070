// Streaming read of a device buffer, for reporting a kernel's bandwidth
// against what this GPU's memory actually delivers to a plain read (a
// measurement helper, not part of the decode step).
//
// kReadProbeBlocks workgroups of 256 threads stride over the buffer in 16 B
// nontemporal loads, eight in flight per thread (the form that read fastest
// of those measured on this part: 6.8 TB/s over 4 GiB, against 5.6-6.1 TB/s
// for ordinary loads); each workgroup XOR-folds what it read into one 32-bit
// word, so no load can be dropped and the result can be checked against a
// host fold of the same bytes.
#include "common.h"
#include "launch.h"

namespace tidar {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* src, size_t n16, unsigned* sink) {
  __shared__ unsigned part[4];
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  constexpr int U = 8;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, unsigned* sink, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kReadProbeBlocks), dim3(256), 0, s, (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace tidar
