// Weight-layout kernels for gfx950: the one-time repack of groupwise-affine
// 4-bit matrices into the streaming layout the grouped GEMMs read, and the
// diagnostic expansion of a matrix to bfloat16 with the GEMMs' own
// reconstruction.  The packed layout is described next to its constants in
// moe_common.h; it is a byte permutation of the codes, scales and biases of
// ["Lily Beats MLX-LM 1.35x on Decode", "Model structure and three workload
// shapes"] (4-bit codes, one bfloat16 scale and bias per 64 weights).
#include "route.h"

namespace moe {

// One thread per (matrix, slice, step, lane): four code words, plus one
// (scale, bias) dword for the even lane groups.
__global__ __launch_bounds__(256) void pack_kernel(int nmat, int N, int K, int gate_up,
                                                   const uint8_t* __restrict__ q,
                                                   const uint16_t* __restrict__ s,
                                                   const uint16_t* __restrict__ b,
                                                   uint8_t* __restrict__ out) {
  const int nk = pack_steps(K);
  const int nsl = N / 16;
  const long long total = static_cast<long long>(nmat) * nsl * nk * 64;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int lane = static_cast<int>(idx % 64);
  long long rest = idx / 64;
  const int step = static_cast<int>(rest % nk);
  rest /= nk;
  const int slice = static_cast<int>(rest % nsl);
  const int mat = static_cast<int>(rest / nsl);
  const int r = lane & 15, g = lane >> 4;
  const int row = gate_up ? (r < 8 ? slice * 8 + r : N / 2 + slice * 8 + r - 8) : slice * 16 + r;

  const uint8_t* qm = q + static_cast<size_t>(mat) * N * (K / 2);
  const uint16_t* sm = s + static_cast<size_t>(mat) * N * (K / 64);
  const uint16_t* bm = b + static_cast<size_t>(mat) * N * (K / 64);
  uint8_t* blk = out + static_cast<size_t>(mat) * pack_bytes(N, K) +
                 (static_cast<size_t>(slice) * nk + step) * kPackBlock;

  // word j: inputs step*128 + 32j + 8g .. +7, nibbles regrouped in pair order
  uint32_t wv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k0 = step * kKS + 32 * j + 8 * g;
    uint32_t c = 0;
    if (k0 < K) c = *reinterpret_cast<const uint32_t*>(qm + static_cast<size_t>(row) * (K / 2) + k0 / 2);
    uint32_t p = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = (e & 1) ? 4 + (e >> 1) : (e >> 1);
      p |= ((c >> (4 * e)) & 0xFu) << (4 * pos);
    }
    wv[j] = p;
  }
  *reinterpret_cast<uint4*>(blk + lane * 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  if ((g & 1) == 0) {
    const int gg = g >> 1;                 // group of the step: inputs gg*64 .. +63
    const int grp = step * 2 + gg;
    uint32_t sb = 0;
    if (grp * 64 < K) {
      const size_t gi = static_cast<size_t>(row) * (K / 64) + grp;
      sb = static_cast<uint32_t>(sm[gi]) | (static_cast<uint32_t>(bm[gi]) << 16);
    }
    *reinterpret_cast<uint32_t*>(blk + kPackScales + (2 * r + gg) * 4) = sb;
  }
}

hipError_t launch_pack(int nmat, int N, int K, int gate_up, const uint8_t* q, const uint16_t* s,
                       const uint16_t* b, uint8_t* out, hipStream_t stream) {
  const long long total = static_cast<long long>(nmat) * (N / 16) * pack_steps(K) * 64;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
                     stream, nmat, N, K, gate_up, q, s, b, out);
  return hipGetLastError();
}

// Diagnostic expansion of a canonical-layout matrix: 8 weights per thread.
__global__ __launch_bounds__(256) void dequant_kernel(int rows, int K, const uint8_t* __restrict__ q,
                                                      const uint16_t* __restrict__ s,
                                                      const uint16_t* __restrict__ b,
                                                      uint16_t* __restrict__ out) {
  const int per_row = K / 8;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long long>(rows) * per_row) return;
  const int row = static_cast<int>(idx / per_row), c = static_cast<int>(idx % per_row);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(q + static_cast<size_t>(row) * (K / 2) + c * 4);
  const size_t gi = static_cast<size_t>(row) * (K / 64) + c / 8;
  const uint4 v = dequant8(w, bf16_to_f32(s[gi]), bf16_to_f32(b[gi]));
  *reinterpret_cast<uint4*>(out + static_cast<size_t>(row) * K + c * 8) = v;
}

hipError_t launch_dequant(int rows, int K, const uint8_t* q, const uint16_t* s, const uint16_t* b,
                          uint16_t* out, hipStream_t stream) {
  const long long n = static_cast<long long>(rows) * (K / 8);
  hipLaunchKernelGGL(dequant_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     stream, rows, K, q, s, b, out);
  return hipGetLastError();
}


// Diagnostic expansion of packed matrices back to the canonical [rows][K]
// order, through the packed addressing and the reconstruction the tall-tile
// GEMM uses (dequant8_pairs on one packed code word and its group's scale and
// bias).  One thread per (matrix, slice, step, lane, word): eight weights.
__global__ __launch_bounds__(256) void dequant_packed_kernel(int nmat, int N, int K, int gate_up,
                                                             const uint8_t* __restrict__ packed,
                                                             uint16_t* __restrict__ out) {
  const int nk = pack_steps(K);
  const int nsl = N / 16;
  const long long total = static_cast<long long>(nmat) * nsl * nk * 64 * 4;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int j = static_cast<int>(idx % 4);
  long long rest = idx / 4;
  const int lane = static_cast<int>(rest % 64);
  rest /= 64;
  const int step = static_cast<int>(rest % nk);
  rest /= nk;
  const int slice = static_cast<int>(rest % nsl);
  const int mat = static_cast<int>(rest / nsl);
  const int r = lane & 15, g = lane >> 4;
  const int k0 = step * kKS + 32 * j + 8 * g;
  if (k0 >= K) return;  // padding past K
  const int row = gate_up ? (r < 8 ? slice * 8 + r : N / 2 + slice * 8 + r - 8) : slice * 16 + r;
  const uint8_t* blk = packed + static_cast<size_t>(mat) * pack_bytes(N, K) +
                       (static_cast<size_t>(slice) * nk + step) * kPackBlock;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(blk + lane * 16 + 4 * j);
  const uint32_t sb = *reinterpret_cast<const uint32_t*>(blk + kPackScales + (2 * r + (j >> 1)) * 4);
  const uint4 v = dequant8_pairs(w, bf16_to_f32(sb & 0xFFFFu), bf16_to_f32(sb >> 16));
  *reinterpret_cast<uint4*>(out + (static_cast<size_t>(mat) * N + row) * K + k0) = v;
}

hipError_t launch_dequant_packed(int nmat, int N, int K, int gate_up, const uint8_t* packed,
                                 uint16_t* out, hipStream_t stream) {
  const long long total = static_cast<long long>(nmat) * (N / 16) * pack_steps(K) * 64 * 4;
  hipLaunchKernelGGL(dequant_packed_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                     dim3(256), 0, stream, nmat, N, K, gate_up, packed, out);
  return hipGetLastError();
}

}  // namespace moe
