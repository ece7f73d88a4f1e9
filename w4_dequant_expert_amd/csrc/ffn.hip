// Grouped expert GEMMs with fused groupwise-affine 4-bit reconstruction, the
// weighted top-k combine, and the diagnostic expansion kernel, for gfx950.
//
// ["Lily Beats MLX-LM 1.35x on Decode", "Prefill: fusing dequantisation and
// keeping routing GPU-resident"]: the grouped GEMM rebuilds the 4-bit weights
// one tile at a time next to the matrix units, accumulates in float32, and the
// expanded bfloat16 array is never written to memory.
//
// Work decomposition (one workgroup = 4 waves = one block of the map x one
// N tile):
//   - the block's activation rows (gathered through sorted_slot for the
//     gate/up GEMM, contiguous h rows for the down GEMM) are staged in LDS,
//     128 inputs at a time, and shared by the four waves;
//   - each wave owns a disjoint slice of output features and reconstructs
//     exactly the weights it multiplies: 16 bytes of codes per lane (32
//     consecutive inputs of one weight row) are loaded from HBM and turned into
//     the B operands of four v_mfma_f32_16x16x32_bf16 in registers, so no
//     reconstructed weight is ever re-read or written anywhere;
//   - SwiGLU is applied to the gate/up accumulators before h is stored.
// MFMA operand convention used throughout: for the 16x16x32 bf16 MFMA, lane l
// supplies row (l mod 16) of A and column (l mod 16) of B, each with eight
// consecutive elements of the reduction; this kernel gives lane l, in MFMA j
// of a 128-input step, the inputs 32*(l/16) + 8*j .. +7 for both operands, so
// A and B agree element for element.  Lane l receives D rows 4*(l/16)+i,
// column l mod 16.
#include "route.h"

namespace moe {

constexpr int kKS = 128;          // reduction inputs per step
constexpr int kLDA = kKS + 8;     // LDS row pitch in bf16 (16-byte pad against bank conflicts)

template <int M_MAX, bool GATE_UP>
__global__ __launch_bounds__(256) void w4_grouped_gemm_kernel(GemmArgs a,
                                                              const uint16_t* __restrict__ src,
                                                              uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[M_MAX * kLDA];
  __shared__ int s_tok[M_MAX];

  const int T = a.T, k = a.k;
  const int Sk = T * k;
  const int Rows = Sk + (a.n_shared ? T : 0);
  const int K = GATE_UP ? a.H : a.I;
  const int ntiles = GATE_UP ? (a.I + 127) / 128 : (a.H + 255) / 256;
  const int bid = blockIdx.x / ntiles, nt = blockIdx.x % ntiles;
  const int nblk = min(*a.n_blocks, a.max_blocks);
  if (bid >= nblk) return;

  const int4 blk = reinterpret_cast<const int4*>(a.blocks)[bid];
  const int G = blk.x, row0 = blk.y, rows = blk.z, tm = blk.w;
  if (G < 0 || G >= a.E + (a.n_shared ? 1 : 0) || rows < 1 || rows > tm || tm > M_MAX ||
      (tm & 15) || row0 < 0 || row0 + rows > Rows) {
    if (threadIdx.x == 0) status_set(a.status, MOE_STATUS_BAD_INDEX);
    return;
  }
  const BankView& bk = (G < a.E) ? a.routed : a.shared;
  const size_t ex = (G < a.E) ? static_cast<size_t>(G) : 0;
  const int Nw = GATE_UP ? 2 * a.I : a.H;  // weight rows of this matrix
  const uint8_t* Q = (GATE_UP ? bk.gu_q : bk.dn_q) + ex * Nw * (K / 2);
  const uint16_t* Sc = (GATE_UP ? bk.gu_s : bk.dn_s) + ex * Nw * (K / 64);
  const uint16_t* Bi = (GATE_UP ? bk.gu_b : bk.dn_b) + ex * Nw * (K / 64);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col0 = GATE_UP ? nt * 128 + wave * 32 : nt * 256 + wave * 64;
  const bool active = col0 < (GATE_UP ? a.I : a.H);
  int wrow[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    if (GATE_UP)
      wrow[ns] = (ns < 2 ? col0 + ns * 16 : a.I + col0 + (ns - 2) * 16) + (lane & 15);
    else
      wrow[ns] = col0 + ns * 16 + (lane & 15);
  }

  // token of every tile row (gate/up) ; -1 pads the tile
  if (GATE_UP) {
    for (int m = tid; m < tm; m += 256) {
      int tok = -1;
      if (m < rows) {
        const int r = row0 + m;
        tok = (r < Sk) ? a.sorted_slot[r] / k : r - Sk;
        if (tok < 0 || tok >= T) {
          status_set(a.status, MOE_STATUS_BAD_INDEX);
          tok = -1;
        }
      }
      s_tok[m] = tok;
    }
  }

  const int mtiles = tm >> 4;
  f32x4 acc[M_MAX / 16][4];
#pragma unroll
  for (int mt = 0; mt < M_MAX / 16; ++mt)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[mt][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < K; kb += kKS) {
    __syncthreads();
    for (int idx = tid; idx < tm * (kKS / 8); idx += 256) {
      const int m = idx / (kKS / 8), c = idx % (kKS / 8);
      const int kk = kb + c * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < rows && kk < K) {
        if (GATE_UP) {
          const int tok = s_tok[m];
          if (tok >= 0) v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(tok) * K + kk);
        } else {
          v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row0 + m) * K + kk);
        }
      }
      *reinterpret_cast<uint4*>(&As[m * kLDA + c * 8]) = v;
    }
    __syncthreads();
    if (!active) continue;

    const int kl = kb + (lane >> 4) * 32;  // this lane's 32 reduction inputs
    bf16x8 bfr[4][4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      if (kl < K) {
        const uint4 qv = *reinterpret_cast<const uint4*>(Q + static_cast<size_t>(wrow[ns]) * (K / 2) + kl / 2);
        const size_t gi = static_cast<size_t>(wrow[ns]) * (K / 64) + kl / 64;
        const float s = bf16_to_f32(Sc[gi]), b = bf16_to_f32(Bi[gi]);
        bfr[ns][0] = as_bf16x8(dequant8(qv.x, s, b));
        bfr[ns][1] = as_bf16x8(dequant8(qv.y, s, b));
        bfr[ns][2] = as_bf16x8(dequant8(qv.z, s, b));
        bfr[ns][3] = as_bf16x8(dequant8(qv.w, s, b));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[ns][j] = as_bf16x8(make_uint4(0, 0, 0, 0));
      }
    }
#pragma unroll
    for (int mt = 0; mt < M_MAX / 16; ++mt) {
      if (mt < mtiles) {
        const uint16_t* ap = &As[(mt * 16 + (lane & 15)) * kLDA + (lane >> 4) * 32];
        bf16x8 af[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = *reinterpret_cast<const bf16x8*>(ap + j * 8);
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[mt][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bfr[ns][j], acc[mt][ns], 0, 0, 0);
      }
    }
  }
  if (!active) return;

#pragma unroll
  for (int mt = 0; mt < M_MAX / 16; ++mt) {
    if (mt >= mtiles) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + (lane >> 4) * 4 + i;
      if (m >= rows) continue;
      const size_t r = static_cast<size_t>(row0 + m);
      if (GATE_UP) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
          const float g = acc[mt][ns][i], u = acc[mt][ns + 2][i];
          const float hv = g / (1.0f + __expf(-g)) * u;   // SwiGLU: silu(g) * u
          out[r * a.I + col0 + ns * 16 + (lane & 15)] = f32_to_bf16(hv);
        }
      } else {
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          out[r * a.H + col0 + ns * 16 + (lane & 15)] = f32_to_bf16(acc[mt][ns][i]);
      }
    }
  }
}

int gemm_m_max_for(int tile_m_max) {
  if (tile_m_max <= 64) return 64;
  if (tile_m_max <= 128) return 128;
  return 256;
}

template <bool GATE_UP>
static hipError_t launch_gemm(const GemmArgs& a, int m_max, const uint16_t* src, uint16_t* out,
                              hipStream_t stream) {
  const int ntiles = GATE_UP ? (a.I + 127) / 128 : (a.H + 255) / 256;
  const dim3 grid(static_cast<unsigned>(a.max_blocks) * ntiles), block(256);
  switch (m_max) {
    case 64:
      hipLaunchKernelGGL((w4_grouped_gemm_kernel<64, GATE_UP>), grid, block, 0, stream, a, src, out);
      break;
    case 128:
      hipLaunchKernelGGL((w4_grouped_gemm_kernel<128, GATE_UP>), grid, block, 0, stream, a, src, out);
      break;
    default:
      hipLaunchKernelGGL((w4_grouped_gemm_kernel<256, GATE_UP>), grid, block, 0, stream, a, src, out);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gate_up(const GemmArgs& a, int m_max, const uint16_t* x, uint16_t* h,
                          hipStream_t stream) {
  return launch_gemm<true>(a, m_max, x, h, stream);
}

hipError_t launch_down(const GemmArgs& a, int m_max, const uint16_t* h, uint16_t* y_slots,
                       hipStream_t stream) {
  return launch_gemm<false>(a, m_max, h, y_slots, stream);
}

// ---------------------------------------------------------------------------
// Weighted top-k combine: one thread per (token, 8 outputs); float32, slots in
// rank order, the shared expert last, one rounding to bfloat16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(int T, int H, int k, int n_shared,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const uint16_t* __restrict__ y_slots,
                                                      uint16_t* __restrict__ y,
                                                      uint32_t* __restrict__ status) {
  const int chunks = H / 8;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long long>(T) * chunks) return;
  const int t = static_cast<int>(idx / chunks), c = static_cast<int>(idx % chunks) * 8;
  const int Sk = T * k;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int pos = slot_pos[static_cast<size_t>(t) * k + j];
    if (pos < 0 || pos >= Sk) {
      status_set(status, MOE_STATUS_BAD_INDEX);
      continue;
    }
    const float w = topk_w[static_cast<size_t>(t) * k + j];
    const uint4 v = *reinterpret_cast<const uint4*>(y_slots + static_cast<size_t>(pos) * H + c);
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __builtin_fmaf(w, bf16_to_f32(p[i] & 0xFFFFu), acc[2 * i]);
      acc[2 * i + 1] = __builtin_fmaf(w, bf16_to_f32(p[i] >> 16), acc[2 * i + 1]);
    }
  }
  if (n_shared) {
    const uint4 v = *reinterpret_cast<const uint4*>(y_slots + static_cast<size_t>(Sk + t) * H + c);
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(p[i] & 0xFFFFu);
      acc[2 * i + 1] += bf16_to_f32(p[i] >> 16);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(y + static_cast<size_t>(t) * H + c) = o;
}

hipError_t launch_combine(int T, int H, int k, int n_shared, const float* topk_w,
                          const int32_t* slot_pos, const uint16_t* y_slots, uint16_t* y,
                          uint32_t* status, hipStream_t stream) {
  const long long n = static_cast<long long>(T) * (H / 8);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, T, H, k, n_shared, topk_w,
                     slot_pos, y_slots, y, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Diagnostic expansion with the GEMMs' own reconstruction: 8 weights per thread.
// ---------------------------------------------------------------------------
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

}  // namespace moe
