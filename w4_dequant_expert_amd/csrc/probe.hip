// Probes for gfx950: a plain streaming read of a device buffer (the ceiling a
// weight-streaming kernel of the same size and launch path can reach) and a
// loop of independent bf16 matrix instructions (the matrix-core throughput a
// launch shape reaches with no memory traffic).  Diagnostic only; nothing in
// the layer calls them.
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

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Eight independent accumulator chains per wave, so every MFMA issue finds its
// operands ready; the operands come from the lane index, not memory.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(static_cast<float>((lane + e) & 7) * 0.125f);
    b[e] = static_cast<__bf16>(static_cast<float>((lane * 3 + e) & 7) * 0.0625f);
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(256), 0,
                     stream, iters, sink);
  return hipGetLastError();
}

}  // namespace moe
