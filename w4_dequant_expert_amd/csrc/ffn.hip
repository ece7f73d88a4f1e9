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
constexpr int kSmallM = 32;       // tiles up to this height go to the small-tile kernel

// Raw operands of one reduction step for one wave: 16 bytes of codes (32
// inputs) and the group's scale and bias, for each of the wave's four
// 16-row weight slices.
struct CodeSlot {
  uint4 q[4];
  uint32_t s[4], b[4];
};

template <int M_MAX, bool GATE_UP>
__global__ __launch_bounds__(256) void w4_grouped_gemm_kernel(
    GemmArgs a, const uint16_t* __restrict__ src, uint16_t* __restrict__ out) {
  // A tile of the block, double-buffered over reduction steps
  __shared__ __attribute__((aligned(16))) uint16_t As[2][M_MAX * kLDA];
  __shared__ int s_tok[M_MAX];
  constexpr int AV = M_MAX / 16;  // 16-byte A chunks staged per thread per step

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
  if (tm <= kSmallM) return;  // a short block: the small-tile kernel owns it
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
  const uint8_t* qrow[4];
  const uint16_t* srow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    int wr;
    if (GATE_UP)
      wr = (ns < 2 ? col0 + ns * 16 : a.I + col0 + (ns - 2) * 16) + (lane & 15);
    else
      wr = col0 + ns * 16 + (lane & 15);
    if (!active) wr = 0;
    qrow[ns] = Q + static_cast<size_t>(wr) * (K / 2);
    srow[ns] = Sc + static_cast<size_t>(wr) * (K / 64);
    brow[ns] = Bi + static_cast<size_t>(wr) * (K / 64);
  }

  if (GATE_UP) {  // token of every tile row; -1 pads the tile
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
    __syncthreads();
  }

  const int nk = (K + kKS - 1) / kKS;
  const int mtiles = tm >> 4;
  const int lk = (lane >> 4) * 32;  // this lane's 32 inputs within a step

  // ---- operand movers ----------------------------------------------------
  auto load_codes = [&](int s, CodeSlot& cs) {
    const int kl = s * kKS + lk;
    if (!active || s >= nk || kl >= K) return;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      cs.q[ns] = *reinterpret_cast<const uint4*>(qrow[ns] + kl / 2);
      cs.s[ns] = srow[ns][kl / 64];
      cs.b[ns] = brow[ns][kl / 64];
    }
  };
  auto load_a = [&](int s, uint4 (&ar)[AV]) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int idx = tid + 256 * i;
      const int m = idx >> 4, c = idx & 15;
      const int kk = s * kKS + c * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (s < nk && m < rows && kk < K) {
        if (GATE_UP) {
          const int tok = s_tok[m];
          if (tok >= 0) v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(tok) * K + kk);
        } else {
          v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row0 + m) * K + kk);
        }
      }
      ar[i] = v;
    }
  };
  auto store_a = [&](int buf, const uint4 (&ar)[AV]) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int idx = tid + 256 * i;
      const int m = idx >> 4, c = idx & 15;
      if (m < tm) *reinterpret_cast<uint4*>(&As[buf][m * kLDA + c * 8]) = ar[i];
    }
  };

  f32x4 acc[M_MAX / 16][4];
#pragma unroll
  for (int mt = 0; mt < M_MAX / 16; ++mt)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[mt][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one reduction step: rebuild this step's weights from the ring slot, refill
  // the slot two steps ahead, run the MFMAs on the LDS buffer, move the next
  // step's A tile into the other buffer
  auto step = [&](int s, CodeSlot& cs, int buf, uint4 (&ar)[AV]) {
    if (active) {
      bf16x8 bfr[4][4];
      const bool live = s * kKS + lk < K;
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const float sc = bf16_to_f32(cs.s[ns]), bi = bf16_to_f32(cs.b[ns]);
        bfr[ns][0] = as_bf16x8(live ? dequant8(cs.q[ns].x, sc, bi) : make_uint4(0, 0, 0, 0));
        bfr[ns][1] = as_bf16x8(live ? dequant8(cs.q[ns].y, sc, bi) : make_uint4(0, 0, 0, 0));
        bfr[ns][2] = as_bf16x8(live ? dequant8(cs.q[ns].z, sc, bi) : make_uint4(0, 0, 0, 0));
        bfr[ns][3] = as_bf16x8(live ? dequant8(cs.q[ns].w, sc, bi) : make_uint4(0, 0, 0, 0));
      }
      load_codes(s + 2, cs);
#pragma unroll
      for (int mt = 0; mt < M_MAX / 16; ++mt) {
        if (mt < mtiles) {
          const uint16_t* ap = &As[buf][(mt * 16 + (lane & 15)) * kLDA + lk];
          bf16x8 af[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) af[j] = *reinterpret_cast<const bf16x8*>(ap + j * 8);
#pragma unroll
          for (int ns = 0; ns < 4; ++ns)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[mt][ns] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bfr[ns][j], acc[mt][ns], 0, 0, 0);
        }
      }
    }
    store_a(buf ^ 1, ar);
    load_a(s + 2, ar);
    __syncthreads();
  };

  // prologue: codes for steps 0 and 1 in flight, A(0) in LDS, A(1) in registers
  CodeSlot c0, c1;
  load_codes(0, c0);
  load_codes(1, c1);
  uint4 ar[AV];
  load_a(0, ar);
  store_a(0, ar);
  load_a(1, ar);
  __syncthreads();

  for (int s = 0; s < nk; s += 2) {
    step(s, c0, 0, ar);
    if (s + 1 < nk) step(s + 1, c1, 1, ar);
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

// ---------------------------------------------------------------------------
// Small-tile kernel: blocks of at most 32 rows (most experts of a prefill
// chunk), where the work is bound by streaming and rebuilding weights rather
// than by the matrix units.  Eight waves per workgroup; each wave owns two
// 16-wide MFMA column slices (32 weight rows), so a wave needs few registers
// and many waves per SIMD keep HBM loads in flight.  For gate/up, columns
// 0..7 of a slice are gate rows and 8..15 the matching up rows, so SwiGLU pairs
// lane n with lane n+8 in the epilogue.
// ---------------------------------------------------------------------------
struct SmallSlot {
  uint4 q[2];
  uint32_t sb[2];  // scale (low half) and bias (high half), bf16 bits
};

template <bool GATE_UP>
__global__ __launch_bounds__(512) void w4_gemm_small_kernel(GemmArgs a,
                                                            const uint16_t* __restrict__ src,
                                                            uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kSmallM * kLDA];
  __shared__ int s_tok[kSmallM];

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
  if (tm > kSmallM) return;  // a tall block: the big-tile kernel owns it
  if (G < 0 || G >= a.E + (a.n_shared ? 1 : 0) || rows < 1 || rows > tm || (tm & 15) ||
      row0 < 0 || row0 + rows > Rows) {
    if (threadIdx.x == 0) status_set(a.status, MOE_STATUS_BAD_INDEX);
    return;
  }
  const BankView& bk = (G < a.E) ? a.routed : a.shared;
  const size_t ex = (G < a.E) ? static_cast<size_t>(G) : 0;
  const int Nw = GATE_UP ? 2 * a.I : a.H;
  const uint8_t* Q = (GATE_UP ? bk.gu_q : bk.dn_q) + ex * Nw * (K / 2);
  const uint16_t* Sc = (GATE_UP ? bk.gu_s : bk.dn_s) + ex * Nw * (K / 64);
  const uint16_t* Bi = (GATE_UP ? bk.gu_b : bk.dn_b) + ex * Nw * (K / 64);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15;
  // output column of each slice (h column for gate/up, y column for down)
  int ocol[2];
  bool sl_on[2];
  int wrow[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (GATE_UP) {
      const int c8 = nt * 128 + (wave * 2 + sl) * 8;
      sl_on[sl] = c8 < a.I;
      ocol[sl] = c8 + (n & 7);
      wrow[sl] = sl_on[sl] ? ((n < 8) ? c8 + n : a.I + c8 + n - 8) : 0;
    } else {
      const int c16 = nt * 256 + (wave * 2 + sl) * 16;
      sl_on[sl] = c16 < a.H;
      ocol[sl] = c16 + n;
      wrow[sl] = sl_on[sl] ? c16 + n : 0;
    }
  }
  const bool active = sl_on[0];  // slice 1 is on only if slice 0 is

  if (GATE_UP) {
    if (tid < tm) {
      int tok = -1;
      if (tid < rows) {
        const int r = row0 + tid;
        tok = (r < Sk) ? a.sorted_slot[r] / k : r - Sk;
        if (tok < 0 || tok >= T) {
          status_set(a.status, MOE_STATUS_BAD_INDEX);
          tok = -1;
        }
      }
      s_tok[tid] = tok;
    }
    __syncthreads();
  }

  const int nk = (K + kKS - 1) / kKS;
  const int mtiles = tm >> 4;
  const int lk = (lane >> 4) * 32;

  auto load_codes = [&](int s, SmallSlot& cs) {
    const int kl = s * kKS + lk;
    if (!active || s >= nk || kl >= K) return;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      if (!sl_on[sl]) continue;
      cs.q[sl] = *reinterpret_cast<const uint4*>(Q + static_cast<size_t>(wrow[sl]) * (K / 2) + kl / 2);
      const size_t gi = static_cast<size_t>(wrow[sl]) * (K / 64) + kl / 64;
      cs.sb[sl] = static_cast<uint32_t>(Sc[gi]) | (static_cast<uint32_t>(Bi[gi]) << 16);
    }
  };
  // A staging: tm rows x 16 chunks of 16 bytes, one chunk per thread
  auto load_a = [&](int s) -> uint4 {
    const int m = tid >> 4, c = tid & 15;
    const int kk = s * kKS + c * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s < nk && m < rows && kk < K) {
      if (GATE_UP) {
        const int tok = s_tok[m];
        if (tok >= 0) v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(tok) * K + kk);
      } else {
        v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row0 + m) * K + kk);
      }
    }
    return v;
  };
  auto store_a = [&](int buf, uint4 v) {
    const int m = tid >> 4, c = tid & 15;
    if (m < tm) *reinterpret_cast<uint4*>(&As[buf][m * kLDA + c * 8]) = v;
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) acc[mt][sl] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int s, SmallSlot& cs, int buf, uint4& ar) {
    if (active) {
      bf16x8 bfr[2][4];
      const bool live = s * kKS + lk < K;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const float sc = bf16_to_f32(cs.sb[sl] & 0xFFFFu), bi = bf16_to_f32(cs.sb[sl] >> 16);
        const bool on = live && sl_on[sl];
        bfr[sl][0] = as_bf16x8(on ? dequant8(cs.q[sl].x, sc, bi) : make_uint4(0, 0, 0, 0));
        bfr[sl][1] = as_bf16x8(on ? dequant8(cs.q[sl].y, sc, bi) : make_uint4(0, 0, 0, 0));
        bfr[sl][2] = as_bf16x8(on ? dequant8(cs.q[sl].z, sc, bi) : make_uint4(0, 0, 0, 0));
        bfr[sl][3] = as_bf16x8(on ? dequant8(cs.q[sl].w, sc, bi) : make_uint4(0, 0, 0, 0));
      }
      load_codes(s + 2, cs);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        if (mt < mtiles) {
          const uint16_t* ap = &As[buf][(mt * 16 + n) * kLDA + lk];
          bf16x8 af[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) af[j] = *reinterpret_cast<const bf16x8*>(ap + j * 8);
#pragma unroll
          for (int sl = 0; sl < 2; ++sl)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[mt][sl] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bfr[sl][j], acc[mt][sl], 0, 0, 0);
        }
      }
    }
    store_a(buf ^ 1, ar);
    ar = load_a(s + 2);
    __syncthreads();
  };

  SmallSlot c0{}, c1{};
  load_codes(0, c0);
  load_codes(1, c1);
  uint4 ar = load_a(0);
  store_a(0, ar);
  ar = load_a(1);
  __syncthreads();
  for (int s = 0; s < nk; s += 2) {
    step(s, c0, 0, ar);
    if (s + 1 < nk) step(s + 1, c1, 1, ar);
  }
  if (!active) return;

#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    if (mt >= mtiles) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + (lane >> 4) * 4 + i;
      const size_t r = static_cast<size_t>(row0 + m);
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const float v = acc[mt][sl][i];
        if (GATE_UP) {
          const float u = __shfl_xor(v, 8, 64);  // lane n (< 8) holds gate, n + 8 the up value
          if (n < 8 && m < rows && sl_on[sl]) {
            const float hv = v / (1.0f + __expf(-v)) * u;   // SwiGLU: silu(g) * u
            out[r * a.I + ocol[sl]] = f32_to_bf16(hv);
          }
        } else if (m < rows && sl_on[sl]) {
          out[r * a.H + ocol[sl]] = f32_to_bf16(v);
        }
      }
    }
  }
}

// Tall-tile kernel variant for a tile height bound (0: no tile exceeds kSmallM).
int gemm_m_max_for(int tile_m_max) {
  if (tile_m_max <= kSmallM) return 0;
  if (tile_m_max <= 128) return 128;
  return 256;
}

template <bool GATE_UP>
static hipError_t launch_gemm(const GemmArgs& a, int m_max, const uint16_t* src, uint16_t* out,
                              hipStream_t stream) {
  const int ntiles = GATE_UP ? (a.I + 127) / 128 : (a.H + 255) / 256;
  const dim3 grid(static_cast<unsigned>(a.max_blocks) * ntiles);
  hipLaunchKernelGGL((w4_gemm_small_kernel<GATE_UP>), grid, dim3(512), 0, stream, a, src, out);
  switch (m_max) {
    case 0:
      break;  // every tile has at most kSmallM rows
    case 128:
      hipLaunchKernelGGL((w4_grouped_gemm_kernel<128, GATE_UP>), grid, dim3(256), 0, stream, a, src, out);
      break;
    default:
      hipLaunchKernelGGL((w4_grouped_gemm_kernel<256, GATE_UP>), grid, dim3(256), 0, stream, a, src, out);
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
