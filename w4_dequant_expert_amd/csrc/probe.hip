// Bandwidth probe for gfx950: a plain streaming read of a device buffer, the
// ceiling a weight-streaming kernel of the same size and launch path can
// reach.  Diagnostic only; nothing in the layer calls it.
#include "route.h"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;  // 16-byte loads in flight per thread

// Each thread reads kProbeUnroll 16-byte chunks (grid-strided) and folds them
// into one word; one word per workgroup is written so the loads stay live.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src,
                                                                   long long n16,
                                                                   uint32_t* __restrict__ sink) {
  const long long stride = static_cast<long long>(gridDim.x) * kProbeThreads;
  const long long i0 = static_cast<long long>(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (long long i = i0; i < n16; i += stride * kProbeUnroll) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[min(i + u * stride, n16 - 1)];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                             hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(workgroups)),
                     dim3(kProbeThreads), 0, stream, static_cast<const uint4*>(src),
                     static_cast<long long>(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace moe
