// Grouped expert GEMMs with fused groupwise-affine 4-bit reconstruction and the
// weighted top-k combine, for gfx950.
//
// ["Lily Beats MLX-LM 1.35x on Decode", "Prefill: fusing dequantisation and
// keeping routing GPU-resident"]: the grouped GEMM rebuilds the 4-bit weights
// one tile at a time next to the matrix units, accumulates in float32, and the
// expanded bfloat16 array is never written to memory.
//
// Work decomposition: one workgroup = one block of the block map x one N tile
// (128 h columns for gate/up, 256 output columns for down).  Within it:
//   - the block's activation rows (gathered through sorted_slot for gate/up,
//     contiguous h rows for down) are staged in LDS, 128 inputs at a time,
//     double-buffered, and shared by all waves of the workgroup;
//   - each wave owns whole 16-row weight slices; a lane loads 16 bytes of
//     packed codes (32 inputs of one weight row) plus its group's scale and
//     bias and rebuilds them in registers as the B operand of four
//     v_mfma_f32_16x16x32_bf16, so each reconstructed weight is used straight
//     from registers and never stored;
//   - codes are prefetched two steps ahead; all loads are unconditional so the
//     compiler's wait counts stay exact;
//   - SwiGLU is applied to the gate/up accumulators before h is stored (gate
//     and up outputs of a column are 8 lanes apart in the packed slices).
// Two kernels share this scheme: a small-tile kernel (blocks of <= 32 rows,
// eight light waves, high occupancy: streaming-bound work) and a tall-tile
// kernel (blocks of 48..128 rows, four waves holding 128-row accumulators:
// matrix-unit-bound work).  Each skips the blocks the other owns, so the host
// launches both without knowing the routing.
//
// MFMA operand convention: for the 16x16x32 bf16 MFMA, lane l supplies row
// (l mod 16) of A and column (l mod 16) of B with eight consecutive reduction
// elements; in MFMA j of a step, lane l carries inputs 32*(l/16) + 8*j .. +7
// for both operands.  Lane l receives D rows 4*(l/16)+i, column l mod 16.
#include "route.h"

namespace moe {

constexpr int kLDA = kKS + 8;     // LDS row pitch in bf16 (16-byte pad against bank conflicts)
constexpr int kSmallM = 32;       // tiles up to this height go to the small-tile kernel

// Raw operands of one step for one 16-row slice: 16 code bytes and the packed
// (scale, bias) dword.
struct SliceOps {
  uint4 q;
  uint32_t sb;
};

__device__ __forceinline__ void load_slice(const uint8_t* blk, int lane, SliceOps& o) {
  o.q = *reinterpret_cast<const uint4*>(blk + lane * 16);
  o.sb = *reinterpret_cast<const uint32_t*>(blk + kPackScales + (((lane >> 5) << 4) + (lane & 15)) * 4);
}

__device__ __forceinline__ void rebuild_slice(const SliceOps& o, bf16x8 (&b)[4]) {
  const float sc = bf16_to_f32(o.sb & 0xFFFFu), bi = bf16_to_f32(o.sb >> 16);
  b[0] = as_bf16x8(dequant8(o.q.x, sc, bi));
  b[1] = as_bf16x8(dequant8(o.q.y, sc, bi));
  b[2] = as_bf16x8(dequant8(o.q.z, sc, bi));
  b[3] = as_bf16x8(dequant8(o.q.w, sc, bi));
}

// Common per-workgroup setup: block entry, validation, the bank's packed matrix.
struct BlockInfo {
  int G, row0, rows, tm, nt;
  const uint8_t* P;  // packed matrix of this block's expert
};

template <bool GATE_UP>
__device__ __forceinline__ bool block_info(const GemmArgs& a, BlockInfo& bi) {
  const int ntiles = GATE_UP ? (a.I + 127) / 128 : (a.H + 255) / 256;
  const int bid = blockIdx.x / ntiles;
  bi.nt = blockIdx.x % ntiles;
  const int nblk = min(*a.n_blocks, a.max_blocks);
  if (bid >= nblk) return false;
  const int4 blk = reinterpret_cast<const int4*>(a.blocks)[bid];
  bi.G = blk.x;
  bi.row0 = blk.y;
  bi.rows = blk.z;
  bi.tm = blk.w;
  return true;
}

template <bool GATE_UP>
__device__ __forceinline__ bool block_valid(const GemmArgs& a, BlockInfo& bi, int m_max) {
  const int Rows = a.T * a.k + (a.n_shared ? a.T : 0);
  if (bi.G < 0 || bi.G >= a.E + (a.n_shared ? 1 : 0) || bi.rows < 1 || bi.rows > bi.tm ||
      bi.tm > m_max || (bi.tm & 15) || bi.row0 < 0 || bi.row0 + bi.rows > Rows) {
    if (threadIdx.x == 0) status_set(a.status, MOE_STATUS_BAD_INDEX);
    return false;
  }
  const BankView& bk = (bi.G < a.E) ? a.routed : a.shared;
  const size_t ex = (bi.G < a.E) ? static_cast<size_t>(bi.G) : 0;
  bi.P = GATE_UP ? bk.gu + ex * pack_bytes(2 * a.I, a.H) : bk.dn + ex * pack_bytes(a.H, a.I);
  return true;
}

// Token of every tile row of a gate/up block (-1 pads the tile).
__device__ __forceinline__ void block_tokens(const GemmArgs& a, const BlockInfo& bi, int* s_tok) {
  const int Sk = a.T * a.k;
  for (int m = threadIdx.x; m < bi.tm; m += blockDim.x) {
    int tok = -1;
    if (m < bi.rows) {
      const int r = bi.row0 + m;
      tok = (r < Sk) ? a.sorted_slot[r] / a.k : r - Sk;
      if (tok < 0 || tok >= a.T) {
        status_set(a.status, MOE_STATUS_BAD_INDEX);
        tok = -1;
      }
    }
    s_tok[m] = tok;
  }
}

// ---------------------------------------------------------------------------
// Small-tile kernel: blocks of at most 32 rows.  Eight waves, two slices each
// (a workgroup covers 16 slices), one A chunk per thread per step.
// ---------------------------------------------------------------------------
template <bool GATE_UP>
__global__ __launch_bounds__(512) void w4_gemm_small_kernel(GemmArgs a,
                                                            const uint16_t* __restrict__ src,
                                                            uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kSmallM * kLDA];
  __shared__ int s_tok[kSmallM];

  BlockInfo bi;
  if (!block_info<GATE_UP>(a, bi)) return;
  if (bi.tm > kSmallM) return;  // a tall block: the tall-tile kernel owns it
  if (!block_valid<GATE_UP>(a, bi, kSmallM)) return;

  const int K = GATE_UP ? a.H : a.I;
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  const int nk = pack_steps(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 15;
  const int lk = (lane >> 4) * 32;
  const int mtiles = bi.tm >> 4;
  const int row0 = bi.row0, rows = bi.rows;

  bool sl_on[2];
  const uint8_t* sbase[2];  // slice's first block
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int c = bi.nt * 16 + wave * 2 + sl;
    sl_on[sl] = c < nslices;
    sbase[sl] = bi.P + static_cast<size_t>(sl_on[sl] ? c : 0) * nk * kPackBlock;
  }
  const bool active = sl_on[0];

  if (GATE_UP) {
    block_tokens(a, bi, s_tok);
    __syncthreads();
  }

  // A staging: tm rows x 16 chunks of 16 bytes, one chunk per thread; rows
  // past the block read row 0 and are zeroed
  const int am = tid >> 4, ac = tid & 15;
  bool a_ok = am < rows;
  const uint16_t* arow;
  if (GATE_UP) {
    const int tok = a_ok ? s_tok[am] : -1;
    a_ok = tok >= 0;
    arow = src + static_cast<size_t>(a_ok ? tok : 0) * K;
  } else {
    arow = src + static_cast<size_t>(row0 + (a_ok ? am : 0)) * K;
  }
  auto load_a = [&](int s) -> uint4 {
    return *reinterpret_cast<const uint4*>(arow + min(s * kKS + ac * 8, K - 8));
  };
  auto store_a = [&](int buf, uint4 v, int s) {
    if (!(a_ok && s < nk && s * kKS + ac * 8 < K)) v = make_uint4(0, 0, 0, 0);
    // am < kSmallM always: unconditional, so no divergent branch disturbs the
    // wait counts of the code prefetch
    *reinterpret_cast<uint4*>(&As[buf][am * kLDA + ac * 8]) = v;
  };
  // steps past the end reload the last step (never used): no branch
  auto load_codes = [&](int s, SliceOps (&o)[2]) {
    const size_t off = static_cast<size_t>(min(s, nk - 1)) * kPackBlock;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) load_slice(sbase[sl] + off, lane, o[sl]);
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) acc[mt][sl] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int s, SliceOps (&o)[2], int buf, uint4& ar) {
    bf16x8 bfr[2][4];
    if (active) {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) rebuild_slice(o[sl], bfr[sl]);
    }
    load_codes(s + 2, o);
    if (active) {
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
    store_a(buf ^ 1, ar, s + 1);
    ar = load_a(s + 2);
    __syncthreads();
  };

  SliceOps c0[2], c1[2];
  load_codes(0, c0);
  load_codes(1, c1);
  uint4 ar = load_a(0);
  store_a(0, ar, 0);
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
        const int c = bi.nt * 16 + wave * 2 + sl;
        const float v = acc[mt][sl][i];
        if (GATE_UP) {
          const float u = __shfl_xor(v, 8, 64);  // lane n (< 8) holds gate, n + 8 the up value
          if (n < 8 && m < rows && sl_on[sl]) {
            const float hv = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;  // silu(g) * u
            out[r * a.I + c * 8 + n] = f32_to_bf16(hv);
          }
        } else if (m < rows && sl_on[sl]) {
          out[r * a.H + c * 16 + n] = f32_to_bf16(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tall-tile kernel: blocks of 48..128 rows.  Four waves, four slices each,
// every wave holding all of the block's tile rows of accumulators.  The block
// body is instantiated per tile height (MT = 3..8 row tiles of 16), so its
// step loop has no per-row-tile branches, and the weights of step s+1 are
// rebuilt between the MFMAs of step s (two B buffers): the VALU work of the
// reconstruction overlaps the matrix units instead of preceding them.
// ---------------------------------------------------------------------------
constexpr int kTallM = 128;

template <int MT, bool GATE_UP>
__device__ __forceinline__ void tall_block(const GemmArgs& a, const BlockInfo& bi,
                                           const uint16_t* __restrict__ src,
                                           uint16_t* __restrict__ out,
                                           uint16_t (*As)[kTallM * kLDA], const int* s_tok) {
  const int K = GATE_UP ? a.H : a.I;
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  const int nk = pack_steps(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 15;
  const int lk = (lane >> 4) * 32;
  const int row0 = bi.row0, rows = bi.rows;

  const int c_first = bi.nt * 16 + wave * 4;
  const bool active = c_first < nslices;  // a wave's four slices are all on or all off
  const uint8_t* sbase = bi.P + static_cast<size_t>(active ? c_first : 0) * nk * kPackBlock;
  const size_t sstride = static_cast<size_t>(nk) * kPackBlock;

  // A staging: chunk i of this thread is tile row (tid + 256 i) / 16 and
  // 16-byte column tid % 16; rows past the block read row 0 and are zeroed.
  const int ac = tid & 15;
  int arow[MT];  // source row (token for gate/up, h row for down); -1 = pad
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = (tid + 256 * i) >> 4;
    int r = -1;
    if (m < rows) r = GATE_UP ? s_tok[m] : row0 + m;
    arow[i] = r;
  }
  auto load_a = [&](int s, uint4 (&ar)[MT]) {
    const int kk = min(s * kKS + ac * 8, K - 8);
#pragma unroll
    for (int i = 0; i < MT; ++i)
      ar[i] = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(max(arow[i], 0)) * K + kk);
  };
  auto store_a = [&](int buf, uint4 (&ar)[MT], int s) {
    const bool kin = s < nk && s * kKS + ac * 8 < K;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = (tid + 256 * i) >> 4;
      const uint4 v = (arow[i] >= 0 && kin) ? ar[i] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&As[buf][m * kLDA + ac * 8]) = v;
    }
  };
  auto load_codes = [&](int s, SliceOps (&o)[4]) {
    const size_t off = static_cast<size_t>(min(s, nk - 1)) * kPackBlock;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) load_slice(sbase + ns * sstride + off, lane, o[ns]);
  };
  // rebuild word w (0..15: slice w/4, 32-bit word w%4) of a code slot
  auto rebuild_word = [&](const SliceOps (&o)[4], bf16x8 (&b)[4][4], int w) {
    const SliceOps& so = o[w >> 2];
    const float sc = bf16_to_f32(so.sb & 0xFFFFu), bi2 = bf16_to_f32(so.sb >> 16);
    const uint32_t q = (w & 3) == 0 ? so.q.x : (w & 3) == 1 ? so.q.y : (w & 3) == 2 ? so.q.z : so.q.w;
    b[w >> 2][w & 3] = as_bf16x8(dequant8(q, sc, bi2));
  };

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[mt][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int WPER = (16 + MT - 1) / MT;  // rebuilt words per row tile
  // One step: MFMAs of step s on bcur; in between, rebuild step s+1 (slot
  // cnext) into bnext; then refill cnext with the codes of step s+3.
  auto step = [&](int s, bf16x8 (&bcur)[4][4], bf16x8 (&bnext)[4][4], SliceOps (&cnext)[4],
                  int buf, uint4 (&ar)[MT]) {
    if (active) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint16_t* ap = &As[buf][(mt * 16 + n) * kLDA + lk];
        bf16x8 af[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = *reinterpret_cast<const bf16x8*>(ap + j * 8);
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[mt][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bcur[ns][j], acc[mt][ns], 0, 0, 0);
#pragma unroll
        for (int w = mt * WPER; w < (mt + 1) * WPER && w < 16; ++w) rebuild_word(cnext, bnext, w);
      }
    }
    load_codes(s + 3, cnext);
    store_a(buf ^ 1, ar, s + 1);
    load_a(s + 2, ar);
    __syncthreads();
  };

  SliceOps c0[4], c1[4];
  bf16x8 b0[4][4], b1[4][4];
  load_codes(0, c0);
  load_codes(1, c1);
  uint4 ar[MT];
  load_a(0, ar);
  store_a(0, ar, 0);
  load_a(1, ar);
#pragma unroll
  for (int w = 0; w < 16; ++w) rebuild_word(c0, b0, w);
  load_codes(2, c0);
  __syncthreads();
  for (int s = 0; s < nk; s += 2) {
    step(s, b0, b1, c1, 0, ar);
    if (s + 1 < nk) step(s + 1, b1, b0, c0, 1, ar);
  }
  if (!active) return;

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + (lane >> 4) * 4 + i;
      const size_t r = static_cast<size_t>(row0 + m);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const int c = c_first + ns;
        const float v = acc[mt][ns][i];
        if (GATE_UP) {
          const float u = __shfl_xor(v, 8, 64);
          if (n < 8 && m < rows) {
            const float hv = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;  // silu(g) * u
            out[r * a.I + c * 8 + n] = f32_to_bf16(hv);
          }
        } else if (m < rows) {
          out[r * a.H + c * 16 + n] = f32_to_bf16(v);
        }
      }
    }
  }
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) void w4_gemm_tall_kernel(GemmArgs a,
                                                           const uint16_t* __restrict__ src,
                                                           uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTallM * kLDA];
  __shared__ int s_tok[kTallM];

  BlockInfo bi;
  if (!block_info<GATE_UP>(a, bi)) return;
  if (bi.tm <= kSmallM) return;  // a short block: the small-tile kernel owns it
  if (!block_valid<GATE_UP>(a, bi, kTallM)) return;
  if (GATE_UP) {
    block_tokens(a, bi, s_tok);
    __syncthreads();
  }
  switch (bi.tm >> 4) {
    case 3: tall_block<3, GATE_UP>(a, bi, src, out, As, s_tok); break;
    case 4: tall_block<4, GATE_UP>(a, bi, src, out, As, s_tok); break;
    case 5: tall_block<5, GATE_UP>(a, bi, src, out, As, s_tok); break;
    case 6: tall_block<6, GATE_UP>(a, bi, src, out, As, s_tok); break;
    case 7: tall_block<7, GATE_UP>(a, bi, src, out, As, s_tok); break;
    default: tall_block<8, GATE_UP>(a, bi, src, out, As, s_tok); break;
  }
}

// ---------------------------------------------------------------------------
// Short-batch kernel (every block at most 16 rows: decode and batches of up
// to 16 tokens).  The weight stream is spread over the whole chip: a
// workgroup of four waves covers 4/KS slices of one block, and each wave
// handles one slice over 1/KS of the input steps.  A wave issues all loads of
// a chunk of steps (codes, scale/bias words and its activation fragments,
// read straight from memory in the MFMA layout) before its first multiply;
// the KS partial sums of a slice are then added in LDS in wave order.
// ---------------------------------------------------------------------------
constexpr int kGemvRows = 16;   // rows per block this kernel accepts
constexpr int kGemvChunk = 4;   // steps whose loads are in flight together

template <int KS, bool GATE_UP>
__global__ __launch_bounds__(256) void w4_gemv_kernel(GemmArgs a, const uint16_t* __restrict__ src,
                                                      uint16_t* __restrict__ out) {
  constexpr int SPW = 4 / KS;  // slices per workgroup
  __shared__ f32x4 red[4][64];

  const int K = GATE_UP ? a.H : a.I;
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  const int ntiles = (nslices + SPW - 1) / SPW;
  const int bid = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
  const int nblk = min(*a.n_blocks, a.max_blocks);
  if (bid >= nblk) return;
  BlockInfo bi;
  {
    const int4 blk = reinterpret_cast<const int4*>(a.blocks)[bid];
    bi.G = blk.x;
    bi.row0 = blk.y;
    bi.rows = blk.z;
    bi.tm = blk.w;
    bi.nt = 0;
  }
  if (bi.rows > kGemvRows) {  // the host launches this kernel only when T <= 16
    if (threadIdx.x == 0) status_set(a.status, MOE_STATUS_BAD_INDEX);
    return;
  }
  if (!block_valid<GATE_UP>(a, bi, 1 << 30)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int ws = wave / KS, wk = wave % KS;
  const bool c_ok = tile * SPW + ws < nslices;
  const int c = min(tile * SPW + ws, nslices - 1);  // a clamped slice computes, never stores
  const int nk = pack_steps(K);
  const int s_begin = wk * nk / KS, s_end = (wk + 1) * nk / KS;
  const uint8_t* sbase = bi.P + static_cast<size_t>(c) * nk * kPackBlock;

  // source row of MFMA row r = lane % 16 (-1: no row); this load goes first,
  // so that waiting for it leaves the weight loads below in flight
  const int r = lane & 15;
  const int Sk = a.T * a.k;
  const int rr = bi.row0 + min(r, bi.rows - 1);
  int srow = GATE_UP ? ((rr < Sk) ? a.sorted_slot[rr] : rr) : rr;

  auto load_w = [&](int s0, SliceOps (&o)[kGemvChunk]) {
#pragma unroll
    for (int u = 0; u < kGemvChunk; ++u)
      load_slice(sbase + static_cast<size_t>(min(s0 + u, max(s_end - 1, 0))) * kPackBlock, lane, o[u]);
  };
  SliceOps o0[kGemvChunk];
  load_w(s_begin, o0);

  if (GATE_UP) {
    srow = (rr < Sk) ? srow / a.k : rr - Sk;
    if (srow < 0 || srow >= a.T) {
      status_set(a.status, MOE_STATUS_BAD_INDEX);
      srow = 0;
    }
  }
  // Rows past the block read the block's last row: an MFMA row only reaches
  // its own output row, and those are never stored.
  const uint16_t* arow = src + static_cast<size_t>(srow) * K;
  const int kq = (lane >> 4) * 32;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto chunk = [&](int s0, const SliceOps (&o)[kGemvChunk]) {
    uint4 av[kGemvChunk][4];
#pragma unroll
    for (int u = 0; u < kGemvChunk; ++u) {
      const int s = min(s0 + u, s_end - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        av[u][j] = *reinterpret_cast<const uint4*>(arow + min(s * kKS + kq + 8 * j, K - 8));
    }
#pragma unroll
    for (int u = 0; u < kGemvChunk; ++u) {
      // Steps past the wave's range and inputs past K multiply zeros (the
      // mask is opaque to the compiler, so the loads above stay unconditional
      // and their wait counts exact); the weights there are finite.
      bf16x8 b[4];
      rebuild_slice(o[u], b);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t mk = (s0 + u < s_end && (s0 + u) * kKS + kq + 8 * j < K) ? ~0u : 0u;
        asm("" : "+v"(mk));
        const uint4 v = make_uint4(av[u][j].x & mk, av[u][j].y & mk, av[u][j].z & mk, av[u][j].w & mk);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(v), b[j], acc, 0, 0, 0);
      }
    }
  };
  // the first chunk is peeled, so its weight loads (issued above) are not
  // loop-carried and nothing waits for them before the activation loads
  if (s_begin < s_end) chunk(s_begin, o0);
  for (int s0 = s_begin + kGemvChunk; s0 < s_end; s0 += kGemvChunk) {
    SliceOps o1[kGemvChunk];
    load_w(s0, o1);
    chunk(s0, o1);
  }

  if (KS > 1) {
    red[wave][lane] = acc;
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int q = 1; q < KS; ++q) acc += red[wave + q][lane];
  }
  if (!c_ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = (lane >> 4) * 4 + i;
    const int n = lane & 15;
    const size_t row = static_cast<size_t>(bi.row0 + m);
    const float v = acc[i];
    if (GATE_UP) {
      const float u = __shfl_xor(v, 8, 64);  // lane n (< 8) holds gate, n + 8 the up value
      if (n < 8 && m < bi.rows) {
        const float hv = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;  // silu(g) * u
        out[row * a.I + c * 8 + n] = f32_to_bf16(hv);
      }
    } else if (m < bi.rows) {
      out[row * a.H + c * 16 + n] = f32_to_bf16(v);
    }
  }
}

template <bool GATE_UP>
static hipError_t launch_gemv(const GemmArgs& a, const uint16_t* src, uint16_t* out,
                              hipStream_t stream) {
  const int K = GATE_UP ? a.H : a.I;
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  const int nk = pack_steps(K);
  // about four steps per wave: split the inputs of a slice over up to four waves
  const int ks = nk >= 16 ? 4 : nk >= 8 ? 2 : 1;
  const int spw = 4 / ks;
  const dim3 grid(static_cast<unsigned>(a.max_blocks) * ((nslices + spw - 1) / spw));
  if (ks == 4)
    hipLaunchKernelGGL((w4_gemv_kernel<4, GATE_UP>), grid, dim3(256), 0, stream, a, src, out);
  else if (ks == 2)
    hipLaunchKernelGGL((w4_gemv_kernel<2, GATE_UP>), grid, dim3(256), 0, stream, a, src, out);
  else
    hipLaunchKernelGGL((w4_gemv_kernel<1, GATE_UP>), grid, dim3(256), 0, stream, a, src, out);
  return hipGetLastError();
}

// Tall-tile kernel variant for a tile height bound (0: no tile exceeds kSmallM).
int gemm_m_max_for(int tile_m_max) { return tile_m_max <= kSmallM ? 0 : 128; }

template <bool GATE_UP>
static hipError_t launch_gemm(const GemmArgs& a, int m_max, const uint16_t* src, uint16_t* out,
                              hipStream_t stream) {
  if (a.T <= kGemvRows) return launch_gemv<GATE_UP>(a, src, out, stream);
  const int ntiles = GATE_UP ? (a.I + 127) / 128 : (a.H + 255) / 256;
  const dim3 grid(static_cast<unsigned>(a.max_blocks) * ntiles);
  hipLaunchKernelGGL((w4_gemm_small_kernel<GATE_UP>), grid, dim3(512), 0, stream, a, src, out);
  if (m_max)
    hipLaunchKernelGGL((w4_gemm_tall_kernel<GATE_UP>), grid, dim3(256), 0, stream, a, src, out);
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
  // The shared row and, eight slots at a time, the slot positions, weights and
  // rows are loaded with clamped indices before any is used, so each group of
  // loads is in flight together.
  const uint4 vsh = *reinterpret_cast<const uint4*>(
      y_slots + static_cast<size_t>(n_shared ? Sk + t : 0) * H + c);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  auto group = [&](int j0) {
    int pos[8];
    float w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t sj = static_cast<size_t>(t) * k + min(j0 + u, k - 1);
      pos[u] = slot_pos[sj];
      w[u] = topk_w[sj];
    }
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = (pos[u] >= 0 && pos[u] < Sk) ? pos[u] : 0;
      v[u] = *reinterpret_cast<const uint4*>(y_slots + static_cast<size_t>(p) * H + c);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u >= k) break;
      if (pos[u] < 0 || pos[u] >= Sk) {
        status_set(status, MOE_STATUS_BAD_INDEX);
        continue;
      }
      const uint32_t p[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(w[u], bf16_to_f32(p[i] & 0xFFFFu), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(w[u], bf16_to_f32(p[i] >> 16), acc[2 * i + 1]);
      }
    }
  };
  group(0);  // peeled: nothing waits for the shared row before it
  for (int j0 = 8; j0 < k; j0 += 8) group(j0);
  if (n_shared) {
    const uint32_t p[4] = {vsh.x, vsh.y, vsh.z, vsh.w};
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

}  // namespace moe
