// Grouped expert GEMMs with fused groupwise-affine 4-bit reconstruction and the
// weighted top-k combine, for gfx950.
//
// ["Lily Beats MLX-LM 1.35x on Decode", "Prefill: fusing dequantisation and
// keeping routing GPU-resident"]: the grouped GEMM rebuilds the 4-bit weights
// one tile at a time next to the matrix units, accumulates in float32, and the
// expanded bfloat16 array is never written to memory.
//
// Work decomposition: one workgroup = one block of the block map x one N tile
// (a run of 16-row weight slices).  Within it:
//   - the block's activation rows (gathered through sorted_slot for gate/up,
//     contiguous h rows for down) are staged in LDS, 128 inputs at a time
//     (all of them at once in the down kernel for I <= 512), and shared by
//     all waves of the workgroup;
//   - each wave owns whole 16-row weight slices; a lane loads 16 bytes of
//     packed codes (four runs of 8 inputs of one weight row) plus the scale
//     and bias of the step's two groups, and the codes become MFMA B operands
//     in registers, so no reconstructed weight is ever stored;
//   - codes are prefetched ahead; all loads are unconditional so the
//     compiler's wait counts stay exact;
//   - SwiGLU is applied to the gate/up accumulators before h is stored (gate
//     and up outputs of a column are 8 lanes apart in the packed slices);
//     outputs leave through an LDS tile as 16-byte runs of rows.
// Four kernels share this scheme: a small-tile kernel (blocks of <= 32 rows,
// high occupancy, the scale applied after the product: streaming-bound work),
// its down variant with the block's activations resident in LDS (I <= 512),
// a tall-tile kernel (blocks of 48..128 rows, waves holding 128-row
// accumulators over rebuilt bf16 weights: matrix-unit-bound work) and a
// short-batch kernel for at most 16 tokens.  The small and tall kernels each
// skip the blocks the other owns, so the host launches both without knowing
// the routing (for large batches, where nearly every row is in a tall block,
// only the tall kernel, which then takes the short blocks too).  A launch
// covers every block, only the routed ones, or only the shared expert's
// (whose blocks follow from T alone, so that launch reads no routing tables).
//
// MFMA operand convention: for the 16x16x32 bf16 MFMA, lane l supplies row
// (l mod 16) of A and column (l mod 16) of B with eight consecutive reduction
// elements; in MFMA j of a step, lane l carries inputs 32*j + 8*(l/16) .. +7
// for both operands, so MFMAs 0, 1 cover the step's first input group and
// MFMAs 2, 3 its second.  Lane l receives D rows 4*(l/16)+i, column l mod 16.
#include "route.h"

namespace moe {

constexpr int kSmallM = 32;       // tiles up to this height go to the small-tile kernel
// Waves (two slices each) per small-tile workgroup.  Four waves give four
// workgroups per CU at the kernel's register budget, the same sixteen waves
// as two eight-wave workgroups but with finer-grained scheduling.
constexpr int kSmallWaves = 4;
// 16-row weight slices per small-tile wave.  One slice a wave halves the
// registers (five or six waves per SIMD) but doubles the activation-fragment
// reads per slice and was slower (gate/up 92 against 79 us at 512 tokens).
constexpr int kSmallSlices = 2;

// Workgroup barrier for LDS data whose copies the caller has already waited
// for.  A plain __syncthreads() would also wait for every copy into LDS still
// in flight (the prefetch of later steps); the asm's memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N), leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Raw operands of one step for one 16-row slice: the lane's four code words
// (word j for MFMA j) and the (scale, bias) dwords of its row for the step's
// two input groups.
struct SliceOps {
  uint4 q;
  uint2 sb;
};

// blk is wave-uniform: with an unsigned 32-bit lane offset the loads take
// the scalar-base form (no 64-bit address arithmetic per lane and step).
__device__ __forceinline__ void load_slice(const uint8_t* blk, int lane, SliceOps& o) {
  const uint32_t l = static_cast<uint32_t>(lane);
  o.q = *reinterpret_cast<const uint4*>(blk + l * 16u);
  o.sb = *reinterpret_cast<const uint2*>(blk + kPackScales + (l & 15u) * 8u);
}

// Scale after the product.  Within one input group g of a weight row,
//   sum_k a_k (q_k s + b) = s * sum_k a_k (128 + q_k) + (b - 128 s) * sum_k a_k,
// and 128 + q (q = 0..15) is a bfloat16 with the code in its low mantissa
// bits: OR-ing the two codes of a pair-order nibble pair into 0x4300 (128.0)
// gives the MFMA operand with two VALU operations per pair of weights.  The
// matrix core then forms P = sum a (128 + q) and X = sum a (a ones operand)
// per group, and two float32 FMAs per output apply the group's scale and
// bias.  This replaces the per-weight convert, FMA and round of a rebuild
// whenever a rebuilt weight would feed only one or two 16-row tiles.
// The identity is exact; the float32 products and sums round differently
// from a bfloat16 rebuild, well inside the layer's tolerance (X and P are
// exact products summed in float32, and |P s| exceeds the result by about the
// ratio 128 / |q - 8| at most).
// The mask and the exponent pattern are passed in registers: with literal
// constants the compiler splits each v_and_or_b32 into an AND and an OR.
struct PairConsts {
  uint32_t mask, magic;
};

__device__ __forceinline__ PairConsts pair_consts() {
  PairConsts k{0x000F000Fu, 0x43004300u};
  asm("" : "+v"(k.mask));
  asm("" : "+v"(k.magic));
  return k;
}

__device__ __forceinline__ bf16x8 codes_plus128(uint32_t w, const PairConsts& k) {
  u32x4 r;
  r.x = (w & k.mask) | k.magic;
  r.y = ((w >> 4) & k.mask) | k.magic;
  r.z = ((w >> 8) & k.mask) | k.magic;
  r.w = ((w >> 12) & k.mask) | k.magic;
  return __builtin_bit_cast(bf16x8, r);
}

// MFMA operand of eight bfloat16 ones.
__device__ __forceinline__ bf16x8 bf16_ones() {
  const u32x4 r = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  return __builtin_bit_cast(bf16x8, r);
}

// Scale s and the folded bias b - 128 s of a packed (scale, bias) dword.
__device__ __forceinline__ void group_affine(uint32_t sb, float& s, float& c) {
  s = __uint_as_float(sb << 16);
  c = __builtin_fmaf(-128.0f, s, __uint_as_float(sb & 0xFFFF0000u));
}

// Common per-workgroup setup: block entry, validation, the bank's packed matrix.
struct BlockInfo {
  int G, row0, rows, tm, nt;
  const uint8_t* P;  // packed matrix of this block's expert
};

// Workgroups are dealt to the eight XCDs round-robin (workgroup i runs on
// XCD i mod 8).  Blocks (in the order below) are dealt the same way -- block
// b to XCD b mod 8 --
// with all N tiles of a block, which read the same activation rows, on the
// block's XCD so that they share its L2: workgroup i takes block
// 8 * ((i / 8) / ntiles) + i mod 8 and N tile (i / 8) mod ntiles.  The grid
// holds ceil(blocks / 8) * 8 * ntiles workgroups.
constexpr int kXcds = 8;

// N tiles of a block when a workgroup covers spw slices.
template <bool GATE_UP>
__host__ __device__ inline int n_tiles(const GemmArgs& a, int spw) {
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  return (nslices + spw - 1) / spw;
}

template <bool GATE_UP>
__device__ __forceinline__ bool block_info(const GemmArgs& a, BlockInfo& bi, int spw) {
  const int ntiles = n_tiles<GATE_UP>(a, spw);
  const int r = blockIdx.x / kXcds;
  int bid = kXcds * (r / ntiles) + blockIdx.x % kXcds;
  bi.nt = r % ntiles;
  // routed blocks only: the grid starts after the shared blocks
  if (a.shared_mode == 1) bid += a.n_shared_blocks;
  // The shared expert's blocks, last in the map, are dealt first: they all
  // stream the same weights, and started together with the routed blocks
  // they no longer form the last, partly filled round of workgroups alone.
  // Their entries follow from T and the tile bounds (the shared group always
  // holds T rows), so those workgroups load nothing to find their block.
  const int nsh = a.n_shared_blocks;
  if (bid < nsh) {
    const int bs = a.T / nsh, rem = a.T % nsh;
    bi.G = a.E;
    bi.row0 = a.T * a.k + bid * bs + min(bid, rem);
    bi.rows = bs + (bid < rem ? 1 : 0);
    bi.tm = (bs + (rem > 0 ? 1 : 0) + a.tile_gran - 1) / a.tile_gran * a.tile_gran;
    return true;
  }
  if (a.shared_mode == 2) return false;  // shared blocks only: no routing tables are read
  // A routed block: its entry is loaded together with the map length (the
  // index is in bounds either way), not after it.
  const int rb = bid - nsh;
  const int4 blk = reinterpret_cast<const int4*>(a.blocks)[min(rb, a.max_blocks - 1)];
  const int nblk = min(*a.n_blocks, a.max_blocks);
  if (rb >= nblk - nsh) return false;
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
// Small-tile kernel: blocks of at most 32 rows, MT = 1 or 2 row tiles of 16.
// WAVES waves, SW slices each (a workgroup covers SW * WAVES slices of one
// block); each thread stages MT * 16 * 16 / (64 WAVES) activation chunks per
// step.
//
// The folded bias term of the scale-after identity, sum over the groups g of
// c[n][g] X_g[m] (X_g[m] the sum of row m's activations over group g), is a
// product over the groups: four groups at a time it is one float32 MFMA
// (16x16x4: A[m][k] = X_g[m], B[k][n] = c[n][g] for the k-th group of the
// window), in place of one FMA per output and group.  For that each lane
// keeps the X and c of one group of every window of four: lane l, l/16 = q,
// keeps group 4w + q.  X comes from the matrix core transposed (ones times
// the activation fragment, so lane l receives X_g[l mod 16]), which is
// already the A layout of the float32 MFMA; c[n][g] is the lane's own
// column's.  Two steps make one window.  X depends only on the activations:
// one wave forms each (group, row tile) pair and the others read it from LDS
// (small_block), or the whole block's X is formed once (the resident-
// activation down kernel).
// ---------------------------------------------------------------------------

// One step of the small-tile product for SW slices and MT row tiles: the
// slices' 128 + q operands, per tile and group the P of each slice on the
// matrix core, P s into the accumulators and this lane's c for its group of
// the window (wpos: the window place of the step's first group, 0 or 2; the
// window's first group clears the other lanes' entries, so a step that is not
// computed contributes nothing).  The window's X comes from the caller.
// frag(mt, g, h) is the address of this lane's 16 bytes of activations for
// row tile mt, group g of the step and half h (the step's inputs
// 64 g + 32 h + 8 (lane / 16) .. +7 of row 16 mt + lane % 16).
template <int SW, int MT, typename Frag>
__device__ __forceinline__ void small_step_math(const SliceOps (&o)[SW], const Frag& frag,
                                                int wpos, int q4, const PairConsts& pk,
                                                f32x4 (&acc)[MT][SW], float (&ck)[SW]) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  uint32_t qw[SW][4];
  float gs[SW][2], gc[SW][2];
#pragma unroll
  for (int sl = 0; sl < SW; ++sl) {
    qw[sl][0] = o[sl].q.x;
    qw[sl][1] = o[sl].q.y;
    qw[sl][2] = o[sl].q.z;
    qw[sl][3] = o[sl].q.w;
    group_affine(o[sl].sb.x, gs[sl][0], gc[sl][0]);
    group_affine(o[sl].sb.y, gs[sl][1], gc[sl][1]);
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int wg = wpos + g;  // the group's place in its window
    bf16x8 bq[SW][2];
#pragma unroll
    for (int sl = 0; sl < SW; ++sl) {
      bq[sl][0] = codes_plus128(qw[sl][2 * g], pk);
      bq[sl][1] = codes_plus128(qw[sl][2 * g + 1], pk);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(frag(mt, g, 0));
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(frag(mt, g, 1));
#pragma unroll
      for (int sl = 0; sl < SW; ++sl) {
        f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bq[sl][0], zero, 0, 0, 0);
        P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bq[sl][1], P, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][sl][i] = __builtin_fmaf(P[i], gs[sl][g], acc[mt][sl][i]);
      }
    }
#pragma unroll
    for (int sl = 0; sl < SW; ++sl) ck[sl] = (q4 == wg) ? gc[sl][g] : (wg == 0 ? 0.0f : ck[sl]);
  }
}

// The window's bias terms, sum over its four groups of X_g[m] c[n][g].
template <int SW, int MT>
__device__ __forceinline__ void small_window_bias(f32x4 (&acc)[MT][SW], const float (&xk)[MT],
                                                  const float (&ck)[SW]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int sl = 0; sl < SW; ++sl)
      acc[mt][sl] = __builtin_amdgcn_mfma_f32_16x16x4f32(xk[mt], ck[sl], acc[mt][sl], 0, 0, 0);
}

// Rounds a small-tile workgroup's outputs into the LDS tile (row pitch TP,
// OC columns per slice; gate/up: SwiGLU first, lane n < 8 holds the gate and
// n + 8 the up value of column n).
template <int WAVES, int SW, bool GATE_UP, int MT, int TP>
__device__ __forceinline__ void small_tile_out(const f32x4 (&acc)[MT][SW], uint16_t* tile, int wave,
                                               int n, int q4) {
  constexpr int OC = GATE_UP ? 8 : 16;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + q4 * 4 + i;
#pragma unroll
      for (int sl = 0; sl < SW; ++sl) {
        const int col = (wave * SW + sl) * OC + n;
        const float v = acc[mt][sl][i];
        if (GATE_UP) {
          const float u = __shfl_xor(v, 8, 64);
          if (n < 8) {
            const float hv = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;  // silu(g) * u
            tile[m * TP + col] = f32_to_bf16(hv);
          }
        } else {
          tile[m * TP + col] = f32_to_bf16(v);
        }
      }
    }
  }
}

template <int WAVES, int SW, bool GATE_UP, int MT>
__device__ __forceinline__ void small_block(const GemmArgs& a, const BlockInfo& bi,
                                            const uint16_t* __restrict__ src,
                                            uint16_t* __restrict__ out,
                                            uint16_t* As0, uint16_t* As1, int* s_tok, float* Xw) {
  static_assert(MT == 1 || MT == 2, "16 or 32 rows");
  static_assert(WAVES == 4, "each wave computes one (group, row tile) pair of the transposed X");
  const int K = GATE_UP ? a.H : a.I;
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  const int nk = pack_steps(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 15;
  const int q4 = lane >> 4;
  const int lk = q4 * 8;
  const int row0 = bi.row0, rows = bi.rows;

  bool sl_on[SW];
  const uint8_t* sbase[SW];  // slice's first block
#pragma unroll
  for (int sl = 0; sl < SW; ++sl) {
    const int c = bi.nt * (SW * WAVES) + wave * SW + sl;
    sl_on[sl] = c < nslices;
    sbase[sl] = bi.P + static_cast<size_t>(sl_on[sl] ? c : 0) * nk * kPackBlock;
  }
  const bool active = sl_on[0];

  // steps past the end reload the last step (never used): no branch
  auto load_codes = [&](int s, SliceOps (&o)[SW]) {
    const size_t off = static_cast<size_t>(min(s, nk - 1)) * kPackBlock;
#pragma unroll
    for (int sl = 0; sl < SW; ++sl) load_slice(sbase[sl] + off, lane, o[sl]);
  };
  // The codes of step 0 do not depend on the block's tokens: they are in
  // flight while the token list is gathered.
  SliceOps c0[SW], c1[SW];
  load_codes(0, c0);
  if (GATE_UP) {
    block_tokens(a, bi, s_tok);
    __syncthreads();
  }

  // Activation staging by direct copies into LDS (global_load_lds): each
  // copy instruction moves four rows (1 KB), lane l's 16 bytes landing at
  // byte 16 l of it; rows are 256 bytes with their 16-byte chunks XOR-swizzled
  // by the row (chunk c of row r at c ^ (r mod 16)), so the 16 rows one MFMA
  // fragment read covers fall in different banks.  Copy p of wave w moves rows
  // 4 (p WAVES + w) .. +3.  Rows past the block copy the block's last row and
  // inputs past K copy the row's last inputs: such rows only reach output rows
  // that are never stored, and inputs past K meet codes with scale and bias 0.
  constexpr int NPASS = MT * 16 / (4 * WAVES);
  static_assert(NPASS >= 1 && NPASS * 4 * WAVES == MT * 16, "whole copies");
  const int pc = lane & 15;
  const uint16_t* arow[NPASS];
  int alc[NPASS];  // this lane's logical chunk
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int r = 4 * (p * WAVES + wave) + (lane >> 4);
    alc[p] = pc ^ (r & 15);
    const int mm = min(r, rows - 1);
    if (GATE_UP) {
      arow[p] = src + static_cast<size_t>(max(s_tok[mm], 0)) * K;
    } else {
      arow[p] = src + static_cast<size_t>(row0 + mm) * K;
    }
  }
  auto issue_a = [&](int s, int buf) {
    const int s0 = min(s, nk - 1) * kKS;
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
    {
      const uint16_t* gp = arow[p] + min(s0 + alc[p] * 8, K - 8);
      uint8_t* lp = reinterpret_cast<uint8_t*>((buf ? As1 : As0) + (p * WAVES + wave) * 512);
      __builtin_amdgcn_global_load_lds(gp, lp, 16, 0, 0);
    }
  };
  f32x4 acc[MT][SW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int sl = 0; sl < SW; ++sl) acc[mt][sl] = f32x4{0.f, 0.f, 0.f, 0.f};
  float xk[MT], ck[SW];  // this lane's group of the current window of four

  // Per step: operands 128 + q of both slices and their groups' affine
  // terms; per 16-row tile and group, P per slice and the transposed X on
  // the matrix core, then P s into the accumulators and the lane's X and c
  // kept for the window's bias product.
  bf16x8 ones = bf16_ones();
  asm volatile("" : "+v"(ones));  // kept in registers, not rebuilt at every use
  const PairConsts pk = pair_consts();
  // Step s: the copies of step s+1 go into the other buffer (read in step
  // s-1, released by the barrier that ended it); the step's products; the
  // codes of step s+2 into the registers the products have read; then a wait
  // for the copies only (the codes stay in flight) and a barrier that does
  // not drain global loads.
  // The transposed X of each (group, row tile) pair of a step is computed by
  // one wave (wave w: group w mod 2, row tile (w / 2) mod MT) and shared
  // through Xw[window parity][group of the window][row]; a step past the end
  // stores zeros.  The window's reads follow the barrier of its second step,
  // and the next writes to the same half come two steps later, after another
  // barrier.
  const int gx = wave & 1, mtx = (wave >> 1) % MT;
  auto step = [&](int s, SliceOps (&o)[SW], int buf) {
    const uint16_t* tb = buf ? As1 : As0;
    auto frag = [&](int mt, int g, int hh) {
      const int r = mt * 16 + n;
      return tb + r * kKS + (((q4 + 8 * g + 4 * hh) ^ n) << 3);
    };
    // X first: its LDS store then comes before the step's copies are issued,
    // so it need not wait for them
    __builtin_amdgcn_sched_barrier(0);
    {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const bf16x8 ax0 = *reinterpret_cast<const bf16x8*>(frag(mtx, gx, 0));
      const bf16x8 ax1 = *reinterpret_cast<const bf16x8*>(frag(mtx, gx, 1));
      f32x4 X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ax0, zero, 0, 0, 0);
      X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ax1, X, 0, 0, 0);
      if (lane < 16)
        Xw[((s >> 1) & 1) * (4 * kSmallM) + (2 * buf + gx) * kSmallM + mtx * 16 + lane] =
            s < nk ? X[0] : 0.0f;
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_a(s + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    if (active && s < nk) small_step_math<SW, MT>(o, frag, 2 * buf, q4, pk, acc, ck);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(s + 2, o);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 * SW>();  // the copies of step s+1 (the codes of step s+2 stay in flight)
    lds_barrier();
  };

  issue_a(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_codes(1, c1);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<2 * SW>();  // the copies of step 0 (and the codes of step 0)
  lds_barrier();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xk[mt] = 0.0f;
#pragma unroll
  for (int sl = 0; sl < SW; ++sl) ck[sl] = 0.0f;
  int s = 0;
  do {  // nk >= 1: no guard in front of the loop, so no load sinks into it
    step(s, c0, 0);
    step(s + 1, c1, 1);  // past the end: loads clamped, no compute
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xk[mt] = Xw[((s >> 1) & 1) * (4 * kSmallM) + q4 * kSmallM + mt * 16 + n];
    small_window_bias<SW, MT>(acc, xk, ck);
    s += 2;
  } while (s < nk);

  // Epilogue through LDS (free after the last step's barrier): each wave
  // writes its outputs, rounded to bfloat16, into a [MT*16][OC * SW * WAVES]
  // tile, and the workgroup then stores whole 16-byte runs of output rows.
  // A lane's own outputs are one 2-byte column entry per row, which as
  // global stores cost one memory instruction per 2 bytes.
  constexpr int OC = GATE_UP ? 8 : 16;  // output columns per slice
  constexpr int TW = OC * SW * WAVES;   // output columns of the tile
  constexpr int TP = TW + 8;            // LDS row pitch (bf16): rows 4 apart fall 16 banks apart
  uint16_t* tile = As0;  // at least kSmallM * (16 * SW * WAVES + 8) elements
  if (active) small_tile_out<WAVES, SW, GATE_UP, MT, TP>(acc, tile, wave, n, q4);
  __syncthreads();
  // 8-column runs: the tile's columns past the matrix (a partial last N tile)
  // and its rows past the block are not stored
  constexpr int RUNS = TW / 8;
  const int ldo = GATE_UP ? a.I : a.H;
  const int col0 = bi.nt * TW;
  const int ncols = min(TW, (GATE_UP ? a.I : a.H) - col0);
  for (int idx = tid; idx < rows * RUNS; idx += 64 * WAVES) {
    const int m = idx / RUNS, run = idx % RUNS;
    if (run * 8 < ncols)
      *reinterpret_cast<uint4*>(out + static_cast<size_t>(row0 + m) * ldo + col0 + run * 8) =
          *reinterpret_cast<const uint4*>(&tile[m * TP + run * 8]);
  }
}

// ---------------------------------------------------------------------------
// Down GEMM, blocks of at most 32 rows, when I <= 512: the block's whole
// activation tile (its h rows, every input) fits in LDS.  It is staged once;
// the workgroup then computes NTW consecutive N tiles, streaming only codes,
// with no barrier between steps and the codes of the next two steps -- across
// tile boundaries too -- always in flight.  The per-step product is the
// small-tile kernel's.
// ---------------------------------------------------------------------------
constexpr int kResK = 512;             // largest K (= I) the resident-activation kernel takes
constexpr int kResLDA = kResK + 8;     // its LDS row pitch (bf16)
constexpr long long kResTargetWgs = 2048;  // grid size the tile grouping keeps
constexpr int kResDepth = 2;           // steps of codes in flight per wave (four measured slower)

template <int WAVES, int SW, int MT, int DEPTH>
__device__ __forceinline__ void down_resident_block(const GemmArgs& a, const BlockInfo& bi, int ntw,
                                                    const uint16_t* __restrict__ src,
                                                    uint16_t* __restrict__ out, uint16_t* As,
                                                    uint16_t* Os, float* Xs) {
  constexpr int SPT = SW * WAVES;        // slices per N tile
  constexpr int TW = 16 * SPT;           // output columns per N tile
  constexpr int TP = TW + 8;             // output tile pitch (bf16)
  constexpr int RUNS = TW / 8;
  const int K = a.I;
  const int nk = pack_steps(K);          // 1..4
  static_assert(DEPTH == 2 || DEPTH == 4, "steps in flight: whole windows of two");
  const int nkp = (nk + DEPTH - 1) / DEPTH * DEPTH;  // steps per tile, padded to whole prefetch rounds
  const int nslices = a.H / 16;
  const int ntiles = (nslices + SPT - 1) / SPT;
  const int t0 = bi.nt * ntw, t1 = min(t0 + ntw, ntiles);
  const int F = (t1 - t0) * nkp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 15, q4 = lane >> 4, lk = q4 * 8;
  const int row0 = bi.row0, rows = bi.rows;

  // the block's h rows: MT*16 rows x 64 chunks of 8 inputs; rows past the
  // block and inputs past K are zeros.  Issued before the first codes, so
  // that waiting for them leaves the codes in flight.
  constexpr int NA = MT * 16 * (kResK / 8) / (64 * WAVES);
  static_assert(NA * 64 * WAVES == MT * 16 * (kResK / 8), "whole passes");
  const int kc = K / 8;
  uint4 av[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int idx = tid + i * 64 * WAVES;
    const int m = idx >> 6, ch = idx & 63;
    av[i] = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row0 + min(m, rows - 1)) * K +
                                            min(ch, kc - 1) * 8);
  }
  // codes of flattened step f: tile t0 + f / nkp, step f % nkp; padding steps
  // and steps past the last tile reload a valid block (never used)
  auto load_codes = [&](int f, SliceOps (&o)[SW]) {
    const int ff = min(f, F - 1);
    const int t = t0 + ff / nkp, st = min(ff % nkp, nk - 1);
#pragma unroll
    for (int sl = 0; sl < SW; ++sl) {
      const int c = min(t * SPT + wave * SW + sl, nslices - 1);
      load_slice(bi.P + (static_cast<size_t>(c) * nk + st) * kPackBlock, lane, o[sl]);
    }
  };
  SliceOps cq[DEPTH][SW];  // the codes of the next DEPTH steps
  __builtin_amdgcn_sched_barrier(0);  // each step's loads in the order the loop keeps
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    load_codes(d, cq[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int idx = tid + i * 64 * WAVES;
    const int m = idx >> 6, ch = idx & 63;
    uint4 w = av[i];
    if (!(m < rows && ch < kc)) w = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&As[m * kResLDA + ch * 8]) = w;
  }
  __syncthreads();

  bf16x8 ones = bf16_ones();
  asm volatile("" : "+v"(ones));
  const PairConsts pk = pair_consts();
  // X_g[m], the row sums of the resident rows over each group of 64 inputs,
  // once per workgroup (the same two products per (row tile, group) that the
  // small-tile step runs, so the same values), spread over the waves; every
  // N tile and every wave then reads them from Xs[m][g]
  constexpr int NG = kResK / 64;
  {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int ng = 2 * nk;
    for (int p = wave; p < MT * ng; p += WAVES) {
      const int mt = p / ng, g = p % ng;
      const uint16_t* a0p = &As[(mt * 16 + n) * kResLDA + 64 * g + lk];
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(a0p);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(a0p + 32);
      f32x4 X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, a0, zero, 0, 0, 0);
      X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, a1, X, 0, 0, 0);
      if (lane < 16) Xs[(mt * 16 + lane) * NG + g] = X[0];
    }
  }
  __syncthreads();
  f32x4 acc[MT][SW];
  float xk[MT], ck[SW];
  int f = 0;
  for (int t = t0; t < t1; ++t) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      xk[mt] = 0.0f;
#pragma unroll
      for (int sl = 0; sl < SW; ++sl) acc[mt][sl] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int sl = 0; sl < SW; ++sl) ck[sl] = 0.0f;
    const bool act = t * SPT + wave * SW < nslices;
    for (int s = 0; s < nkp; s += DEPTH, f += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        if (act && s + d < nk) {
          const uint16_t* ar = &As[n * kResLDA + (s + d) * kKS + lk];
          auto frag = [&](int mt, int g, int hh) { return ar + mt * 16 * kResLDA + 64 * g + 32 * hh; };
          small_step_math<SW, MT>(cq[d], frag, 2 * (d & 1), q4, pk, acc, ck);
        }
        load_codes(f + d + DEPTH, cq[d]);
        if (d & 1) {
          // this lane's group of the window: 4 window + q4 (steps past K: none)
          const int g = 2 * (s + d - 1) + q4;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) xk[mt] = g < 2 * nk ? Xs[(mt * 16 + n) * NG + g] : 0.0f;
          small_window_bias<SW, MT>(acc, xk, ck);
        }
      }
    }
    // epilogue of tile t through one of two LDS tiles (the other may still be
    // read by the previous tile's stores)
    uint16_t* tile = Os + ((t - t0) & 1) * (kSmallM * TP);
    if (act) small_tile_out<WAVES, SW, false, MT, TP>(acc, tile, wave, n, q4);
    __syncthreads();
    const int col0 = t * TW;
    const int ncols = min(TW, a.H - col0);
    constexpr int SR = MT * 16 * RUNS / (64 * WAVES);  // runs per thread (a fixed count)
#pragma unroll
    for (int i = 0; i < SR; ++i) {
      const int idx = tid + i * 64 * WAVES;
      const int m = idx / RUNS, run = idx % RUNS;
      if (m < rows && run * 8 < ncols)
        *reinterpret_cast<uint4*>(out + static_cast<size_t>(row0 + m) * a.H + col0 + run * 8) =
            *reinterpret_cast<const uint4*>(&tile[m * TP + run * 8]);
    }
  }
}

template <int WAVES, int SW, int MODE>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(3))) void w4_down_resident_kernel(
    GemmArgs a, const uint16_t* __restrict__ src, uint16_t* __restrict__ out, int ntw) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kSmallM * kResLDA];
  __shared__ __attribute__((aligned(16))) uint16_t Os[2 * kSmallM * (16 * SW * WAVES + 8)];
  __shared__ float Xs[kSmallM * (kResK / 64)];
  BlockInfo bi;
  if (!block_info<false>(a, bi, SW * WAVES * ntw)) return;
  if (bi.tm > kSmallM) return;  // a tall block: the tall-tile kernel owns it
  if (!block_valid<false>(a, bi, kSmallM)) return;
  if (bi.tm <= 16)
    down_resident_block<WAVES, SW, 1, kResDepth>(a, bi, ntw, src, out, As, Os, Xs);
  else
    down_resident_block<WAVES, SW, 2, kResDepth>(a, bi, ntw, src, out, As, Os, Xs);
}

// MODE: the blocks the launch computes (GemmArgs::shared_mode: 0 all, 1 the
// routed ones, 2 the shared expert's), a kernel of its own per mode so that
// traces tell the launches apart.
template <int WAVES, int SW, bool GATE_UP, int MODE>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(4))) void w4_gemm_small_kernel(
    GemmArgs a, const uint16_t* __restrict__ src, uint16_t* __restrict__ out) {
  // two staging buffers of 32 rows x 128 inputs, distinct arrays so that the
  // compiler can tell a read of one from a copy into the other; the first
  // also holds the output tile (32 rows x 136)
  __shared__ __attribute__((aligned(1024))) uint16_t As0[kSmallM * (kKS + 8)];
  __shared__ __attribute__((aligned(1024))) uint16_t As1[kSmallM * kKS];
  __shared__ int s_tok[kSmallM];
  __shared__ float Xw[2 * 4 * kSmallM];

  BlockInfo bi;
  if (!block_info<GATE_UP>(a, bi, SW * WAVES)) return;
  if (bi.tm > kSmallM) return;  // a tall block: the tall-tile kernel owns it
  if (!block_valid<GATE_UP>(a, bi, kSmallM)) return;
  if (bi.tm <= 16)
    small_block<WAVES, SW, GATE_UP, 1>(a, bi, src, out, As0, As1, s_tok, Xw);
  else
    small_block<WAVES, SW, GATE_UP, 2>(a, bi, src, out, As0, As1, s_tok, Xw);
}

// ---------------------------------------------------------------------------
// Tall-tile kernel (blocks of 48..128 rows, and every block for large
// batches): MT = 1..4 row tiles of 32 rows on v_mfma_f32_32x32x16_bf16 (on
// gfx950 the 32x32 form delivers twice the 16x16 form's throughput).  A
// workgroup of four waves covers 16 slices; each wave owns two 32-column
// tiles and all of the block's rows, so each rebuilt weight feeds MT MFMAs
// and each activation fragment read from LDS feeds 2 MT.
//   - Only two activation buffers live in LDS (64 KB) and the weight codes go
//     straight into registers, so two workgroups share a CU.  Each SIMD then
//     holds waves of two workgroups whose step barriers, prologues and
//     epilogues fall at different times, and one workgroup's waits are covered
//     by the other's work (an eight-wave workgroup holding the whole LDS kept
//     all of a CU's waves in lock-step and was about 10 % slower).
//   - Step s issues the codes of step s+1 (registers), then the activations of
//     step s+1 (copied from memory straight into LDS with global_load_lds,
//     into the buffer step s-1 read, free after step s's barrier).  Before the
//     last k-chunk of step s, all but the last NCP loads done means the codes
//     of step s+1 have landed; at the start of step s+1 everything is waited
//     for.  The step barrier is an s_barrier without the fence that would also
//     drain copies still in flight.
//   - A row's sixteen 16-byte chunks are stored XOR-swizzled by the row index,
//     so rows need no padding and the 32-row MFMA reads are conflict-free.
//   - The weights of k-chunk j+1 are rebuilt while the MFMAs of chunk j run.
// MFMA operand convention (32x32x16): lane l supplies row l mod 32 of A and
// column l mod 32 of B with eight consecutive reduction elements; in k-chunk
// j of a step (j = 0..7) lane l carries inputs 16j + 8*(l/32) .. +7.  Lane l
// receives D column l mod 32, rows 8*(i/4) + 4*(l/32) + (i mod 4), i = 0..15.
// ---------------------------------------------------------------------------
constexpr int kTallM = 128;
constexpr int kTallBuf = kTallM * kKS * 2;  // bytes of one staged activation step

typedef float f32x16 __attribute__((ext_vector_type(16)));

// One step's codes of a 32-column tile for one lane: eight code words (k-chunk
// j in q[j]) and the scale/bias words of the step's two input groups.
struct TileCodes {
  uint32_t q[8];
  uint32_t sb[2];
};

constexpr int kT4Waves = 4;
constexpr int kT4Threads = kT4Waves * kWave;

struct RawCodes {
  uint4 ce, co;
  uint2 g;
};

template <int MT, int CT, bool GATE_UP>
__device__ __forceinline__ void tall4_block(const GemmArgs& a, const BlockInfo& bi,
                                            const uint16_t* __restrict__ src,
                                            uint16_t* __restrict__ out, uint8_t* As0, uint8_t* As1,
                                            int* s_tok) {
  constexpr int NCP = 2 * MT;  // activation copies per wave per step (4 rows each)
  const int K = GATE_UP ? a.H : a.I;
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  const int nk = pack_steps(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int row0 = bi.row0, rows = bi.rows;

  // CT 32-column tiles (two slices each) per wave; nslices is even, so a
  // tile's two slices are both in or both out
  const int c_first = bi.nt * (2 * CT * kT4Waves) + wave * 2 * CT;
  const size_t sstride = static_cast<size_t>(nk) * kPackBlock;

  // Lane l reads column n = l mod 32 of each of its 32-column tiles: row
  // n mod 16 of slice n/16; k-chunk j holds inputs 16j + 8h .. +7 (h = l/32),
  // word j/2 of the 16 bytes at (16 (2 (j mod 2) + h) + row) * 16 of the
  // packed block.
  const int h = lane >> 5, nrow = lane & 15, nsl = (lane >> 4) & 1;
  const uint8_t* cbase[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    cbase[ct] = bi.P + static_cast<size_t>(min(c_first + 2 * ct, nslices - 2) + nsl) * sstride;
  auto load_codes = [&](int s, RawCodes (&rc)[CT]) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const uint8_t* blk = cbase[ct] + static_cast<size_t>(min(s, nk - 1)) * kPackBlock;
      rc[ct].ce = *reinterpret_cast<const uint4*>(blk + (16 * h + nrow) * 16);
      rc[ct].co = *reinterpret_cast<const uint4*>(blk + (16 * h + nrow) * 16 + 512);
      rc[ct].g = *reinterpret_cast<const uint2*>(blk + kPackScales + nrow * 8);
    }
  };
  auto to_tile = [&](const RawCodes& rc, TileCodes& tc) {
    tc.q[0] = rc.ce.x; tc.q[1] = rc.co.x;
    tc.q[2] = rc.ce.y; tc.q[3] = rc.co.y;
    tc.q[4] = rc.ce.z; tc.q[5] = rc.co.z;
    tc.q[6] = rc.ce.w; tc.q[7] = rc.co.w;
    tc.sb[0] = rc.g.x;
    tc.sb[1] = rc.g.y;
  };
  auto rebuild_j = [&](const TileCodes& tc, int j) -> bf16x8 {
    const uint32_t sbw = tc.sb[j >> 2];
    return as_bf16x8(dequant8_pairs(tc.q[j], bf16_to_f32(sbw & 0xFFFFu), bf16_to_f32(sbw >> 16)));
  };

  // Activation copies: copy i of wave w moves tile rows 4q .. 4q+3, q = 4i + w,
  // into LDS bytes [1024 q, 1024 q + 1024); lane -> row 4q + lane/16, stored
  // chunk lane % 16, which holds the row's chunk (lane % 16) ^ (row % 16).
  const int cg = (lane & 15) ^ ((4 * wave + (lane >> 4)) & 15);
  const uint16_t* arow[NCP];  // set once the block's tokens are known
  auto issue_a = [&](int s, uint8_t* buf) {
    const int kk = min(min(s, nk - 1) * kKS + cg * 8, K - 8);
#pragma unroll
    for (int i = 0; i < NCP; ++i)
      __builtin_amdgcn_global_load_lds(arow[i] + kk, buf + (kT4Waves * i + wave) * 1024, 16, 0, 0);
  };
  const bool ktail = (K % kKS) != 0;
  auto zero_tail = [&](int s, uint8_t* buf) {
    if (ktail && s == nk - 1 && s * kKS + cg * 8 >= K) {
#pragma unroll
      for (int i = 0; i < NCP; ++i)
        *reinterpret_cast<uint4*>(buf + (kT4Waves * i + wave) * 1024 + lane * 16) =
            make_uint4(0, 0, 0, 0);
    }
  };
  const int arow_l = lane & 31;
  int aoff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) aoff[j] = arow_l * (kKS * 2) + (((2 * j + h) ^ (arow_l & 15)) * 16);

  f32x16 acc[CT][MT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[ct][mt][i] = 0.0f;

  bf16x8 bq[2][CT];
  TileCodes tc[CT];
  auto step = [&](int s, uint8_t* acur, uint8_t* anew, RawCodes (&rnext)[CT]) {
    wait_vmcnt<0>();  // activations of step s (and everything before)
    zero_tail(s, acur);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    load_codes(s + 1, rnext);
    issue_a(s + 1, anew);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 af[2][MT];
    auto read_a = [&](int j, bf16x8 (&f)[MT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        f[mt] = *reinterpret_cast<const bf16x8*>(acur + mt * 32 * (kKS * 2) + aoff[j]);
    };
    read_a(0, af[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < 7) read_a(j + 1, af[(j + 1) & 1]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[ct][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j & 1][mt], bq[j & 1][ct],
                                                               acc[ct][mt], 0, 0, 0);
      if (j < 7) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          bq[(j + 1) & 1][ct] = rebuild_j(tc[ct], j + 1);
          // The operand of the MFMAs above stays live past the rebuild, so
          // the rebuild writes other registers and need not wait for those
          // MFMAs to read theirs.
          asm volatile("" ::"v"(bq[j & 1][ct]));
        }
      } else {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<NCP>();  // codes of step s+1
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          to_tile(rnext[ct], tc[ct]);
          bq[0][ct] = rebuild_j(tc[ct], 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The codes of step 0 do not depend on the block's tokens: they are in
  // flight while the token list is gathered.
  RawCodes r0[CT], r1[CT];
  load_codes(0, r0);
  if (GATE_UP) {
    block_tokens(a, bi, s_tok);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int r = min(4 * (kT4Waves * i + wave) + (lane >> 4), rows - 1);
    const int srow = GATE_UP ? max(s_tok[r], 0) : row0 + r;
    arow[i] = src + static_cast<size_t>(srow) * K;
  }
  issue_a(0, As0);
  wait_vmcnt<0>();
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    to_tile(r0[ct], tc[ct]);
    bq[0][ct] = rebuild_j(tc[ct], 0);
  }
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    step(s, As0, As1, r1);
    step(s + 1, As1, As0, r0);
  }
  if (s < nk) step(s, As0, As1, r1);
  wait_vmcnt<0>();  // the last step's spare copies land before the LDS is released
  lds_barrier();    // and every wave has read its last activations

  // Epilogue through LDS, as in the small-tile kernel: rows 0..63 of the
  // [tm][TW] bfloat16 output tile go to As0, rows 64..127 to As1, each row's
  // 16-byte runs XOR-swizzled by bits 2..3 of the row so that the two rows
  // one write instruction covers (4 apart, 16 banks apart after the swizzle)
  // do not collide; then the workgroup stores 16-byte runs of output rows.
  constexpr int OC = GATE_UP ? 8 : 16;     // output columns per slice
  constexpr int TW = OC * 2 * CT * kT4Waves;
  constexpr int RUNS = TW / 8;
  static_assert(64 * TW * 2 <= kTallBuf && RUNS % 16 == 0, "half a tile fits one buffer");
  auto tile_off = [](int lr, int col) {  // bf16 offset of (row lr of a half, column col)
    return lr * TW + (((col >> 3) ^ (((lr >> 2) & 3) << 2)) << 3) + (col & 7);
  };
  const int n16 = lane & 15;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int ctile = c_first + 2 * ct;
    if (ctile >= nslices) break;
    const int col = (ctile - bi.nt * (2 * CT * kT4Waves) + nsl) * OC + n16;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint16_t* half = reinterpret_cast<uint16_t*>(mt < 2 ? As0 : As1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int lr = (mt & 1) * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        const float v = acc[ct][mt][i];
        if (GATE_UP) {
          const float u = __shfl_xor(v, 8, 64);  // lane n (mod 16 < 8) holds gate, n + 8 up
          if (n16 < 8) {
            const float hv = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;  // silu(g) * u
            half[tile_off(lr, col)] = f32_to_bf16(hv);
          }
        } else {
          half[tile_off(lr, col)] = f32_to_bf16(v);
        }
      }
    }
  }
  lds_barrier();
  // 8-column runs; columns past the matrix and rows past the block are not stored
  const int ldo = GATE_UP ? a.I : a.H;
  const int col0 = bi.nt * TW;
  const int ncols = min(TW, ldo - col0);
  for (int idx = tid; idx < rows * RUNS; idx += kT4Threads) {
    const int m = idx / RUNS, run = idx % RUNS;
    if (run * 8 < ncols) {
      const uint16_t* half = reinterpret_cast<const uint16_t*>(m < 64 ? As0 : As1);
      *reinterpret_cast<uint4*>(out + static_cast<size_t>(row0 + m) * ldo + col0 + run * 8) =
          *reinterpret_cast<const uint4*>(&half[tile_off(m & 63, run * 8)]);
    }
  }
}

constexpr int kT4CT = 2;  // 32-column tiles per wave of the tall-tile kernel

template <bool GATE_UP>
__device__ __forceinline__ void tall4_entry(const GemmArgs& a, const uint16_t* __restrict__ src,
                                            uint16_t* __restrict__ out, uint8_t* As0, uint8_t* As1,
                                            int* s_tok, float* Xw) {
  BlockInfo bi;
  if (!block_info<GATE_UP>(a, bi, 2 * kT4CT * kT4Waves)) return;
  if (bi.tm <= kSmallM && !a.tall_all) return;  // a short block: the small-tile kernel owns it
  if (bi.tm > kTallM) return;  // a block of more than 128 rows: the 256-row kernel owns it
  if (!block_valid<GATE_UP>(a, bi, kTallM)) return;
  if (bi.tm <= kSmallM) {
    // A short block in a launch that takes every block: the small-tile
    // product (scale after the product), whose cost per weight does not
    // depend on the tile height, over the workgroup's 16 slices as two
    // 8-slice halves.  Rebuilding weights for a single 32-row tile would cost
    // as much vector work as for four.
    static_assert(kSmallM * (kKS + 8) * 2 <= kTallBuf, "the small-tile buffers fit");
    static_assert(2 * kT4CT * kT4Waves == 2 * kSmallSlices * kSmallWaves && kT4Waves == kSmallWaves,
                  "a tall workgroup's slices are two small-tile halves");
    for (int p = 0; p < 2; ++p) {
      BlockInfo half = bi;
      half.nt = 2 * bi.nt + p;
      if (p) __syncthreads();  // the first half's output tile has been stored
      if (half.tm <= 16)
        small_block<kSmallWaves, kSmallSlices, GATE_UP, 1>(a, half, src, out, reinterpret_cast<uint16_t*>(As0),
                                                           reinterpret_cast<uint16_t*>(As1), s_tok, Xw);
      else
        small_block<kSmallWaves, kSmallSlices, GATE_UP, 2>(a, half, src, out, reinterpret_cast<uint16_t*>(As0),
                                                           reinterpret_cast<uint16_t*>(As1), s_tok, Xw);
    }
    return;
  }
  switch ((bi.tm + 31) >> 5) {
    case 1: tall4_block<1, kT4CT, GATE_UP>(a, bi, src, out, As0, As1, s_tok); break;
    case 2: tall4_block<2, kT4CT, GATE_UP>(a, bi, src, out, As0, As1, s_tok); break;
    case 3: tall4_block<3, kT4CT, GATE_UP>(a, bi, src, out, As0, As1, s_tok); break;
    default: tall4_block<4, kT4CT, GATE_UP>(a, bi, src, out, As0, As1, s_tok); break;
  }
}

template <bool GATE_UP>
__global__ __launch_bounds__(kT4Threads) __attribute__((amdgpu_waves_per_eu(2))) void w4_gemm_tall4_kernel(
    GemmArgs a, const uint16_t* __restrict__ src, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t As0[kTallBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[kTallBuf];
  __shared__ int s_tok[kTallM];
  __shared__ float Xw[2 * 4 * kSmallM];
  tall4_entry<GATE_UP>(a, src, out, As0, As1, s_tok, Xw);
}

// The same kernel for the launches that compute only the routed blocks and only
// the shared expert's blocks (kernels of their own, so that traces tell the
// launches apart).
template <bool GATE_UP>
__global__ __launch_bounds__(kT4Threads) __attribute__((amdgpu_waves_per_eu(2))) void w4_gemm_tall4_routed_kernel(
    GemmArgs a, const uint16_t* __restrict__ src, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t As0[kTallBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[kTallBuf];
  __shared__ int s_tok[kTallM];
  __shared__ float Xw[2 * 4 * kSmallM];
  tall4_entry<GATE_UP>(a, src, out, As0, As1, s_tok, Xw);
}

template <bool GATE_UP>
__global__ __launch_bounds__(kT4Threads) __attribute__((amdgpu_waves_per_eu(2))) void w4_gemm_tall4_shared_kernel(
    GemmArgs a, const uint16_t* __restrict__ src, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t As0[kTallBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[kTallBuf];
  __shared__ int s_tok[kTallM];
  __shared__ float Xw[2 * 4 * kSmallM];
  tall4_entry<GATE_UP>(a, src, out, As0, As1, s_tok, Xw);
}

// ---------------------------------------------------------------------------
// Tall-tile kernel for blocks of 160..256 rows: MT = 5..8 row tiles of 32 on
// v_mfma_f32_32x32x16_bf16 with ONE 32-column tile per wave, so that each
// rebuilt weight feeds MT (up to eight) MFMAs -- half the rebuild work per
// MFMA of the four-row-tile kernel, whose rebuild is what keeps the matrix
// core waiting there.  A workgroup of four waves covers 8 slices.
//   - The activation tile of up to 256 rows is staged in LDS one half-step (64
//     inputs, 128 bytes a row) at a time, in two buffers of 32 KB, so two
//     workgroups still share a CU.  Half-step hs+1 is copied (global_load_lds)
//     into the buffer half-step hs-1 read while half-step hs computes.
//   - A row's eight 16-byte chunks are stored XOR-swizzled by (row / 2) mod 8:
//     with 128-byte rows, sixteen consecutive rows then cover every LDS bank
//     once, so the 32-row MFMA reads are conflict-free.
//   - The weight codes of a step are loaded into registers one step ahead
//     (at its first half-step) and rebuilt one k-chunk ahead of the MFMAs.
// Half-steps entirely past K (K mod 128 = 64) are skipped.
// ---------------------------------------------------------------------------
constexpr int kTall8M = 256;
constexpr int kHalfK = 64;                            // inputs per staged half-step
constexpr int kTall8Buf = kTall8M * kHalfK * 2;       // bytes of one staged half-step
static_assert(kTall8Buf == kTallBuf, "both tall kernels stage 32 KB buffers");

template <int MT, bool GATE_UP>
__device__ __forceinline__ void tall8_block(const GemmArgs& a, const BlockInfo& bi,
                                            const uint16_t* __restrict__ src,
                                            uint16_t* __restrict__ out, uint8_t* As0, uint8_t* As1,
                                            int* s_tok) {
  constexpr int NCP = MT;  // activation copies per wave per half-step (8 rows each)
  const int K = GATE_UP ? a.H : a.I;
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  const int nk = pack_steps(K);
  const int nh = 2 * nk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int row0 = bi.row0, rows = bi.rows;

  // one 32-column tile (two slices) per wave; nslices is even, so both
  // slices of a tile are in or both out
  const int c_first = bi.nt * (2 * kT4Waves) + wave * 2;
  const size_t sstride = static_cast<size_t>(nk) * kPackBlock;
  // lane l reads column n = l mod 32 of the tile: row n mod 16 of slice n/16;
  // k-chunk j of a step holds inputs 16j + 8h .. +7 (h = l/32)
  const int h = lane >> 5, nrow = lane & 15, nsl = (lane >> 4) & 1;
  const uint8_t* cbase = bi.P + static_cast<size_t>(min(c_first, nslices - 2) + nsl) * sstride;
  auto load_codes = [&](int s, RawCodes& rc) {
    const uint8_t* blk = cbase + static_cast<size_t>(min(s, nk - 1)) * kPackBlock;
    rc.ce = *reinterpret_cast<const uint4*>(blk + (16 * h + nrow) * 16);
    rc.co = *reinterpret_cast<const uint4*>(blk + (16 * h + nrow) * 16 + 512);
    rc.g = *reinterpret_cast<const uint2*>(blk + kPackScales + nrow * 8);
  };
  auto to_tile = [&](const RawCodes& rc, TileCodes& tc) {
    tc.q[0] = rc.ce.x; tc.q[1] = rc.co.x;
    tc.q[2] = rc.ce.y; tc.q[3] = rc.co.y;
    tc.q[4] = rc.ce.z; tc.q[5] = rc.co.z;
    tc.q[6] = rc.ce.w; tc.q[7] = rc.co.w;
    tc.sb[0] = rc.g.x;
    tc.sb[1] = rc.g.y;
  };
  auto rebuild_j = [&](const TileCodes& tc, int j) -> bf16x8 {
    const uint32_t sbw = tc.sb[j >> 2];
    return as_bf16x8(dequant8_pairs(tc.q[j], bf16_to_f32(sbw & 0xFFFFu), bf16_to_f32(sbw >> 16)));
  };

  // Activation copies: copy i of wave w moves tile rows 8q .. 8q+7, q = 4i + w,
  // into LDS bytes [1024 q, 1024 q + 1024); lane -> row 8q + lane/8, stored at
  // chunk position lane % 8, which holds the row's chunk (lane % 8) ^ ((row /
  // 2) mod 8).  (row / 2) mod 8 is the same for every copy of a lane.
  const int rsub = lane >> 3;
  const int cg = (lane & 7) ^ (((8 * wave + rsub) >> 1) & 7);
  const uint16_t* arow[NCP];  // each copy's source row, set once the block's tokens are known
  auto issue_a = [&](int hs, uint8_t* buf) {
    const int kk = min(min(hs, nh - 1) * kHalfK + cg * 8, K - 8);
#pragma unroll
    for (int i = 0; i < NCP; ++i)
      __builtin_amdgcn_global_load_lds(arow[i] + kk, buf + (kT4Waves * i + wave) * 1024, 16, 0, 0);
  };
  // MFMA A reads: row l mod 32 of a row tile, chunk 2j + h of the half-step
  const int arow_l = lane & 31;
  int aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aoff[j] = arow_l * (kHalfK * 2) + (((2 * j + h) ^ ((arow_l >> 1) & 7)) * 16);

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.0f;

  bf16x8 bq[2];
  TileCodes tc;
  RawCodes rnext;
  // Issue order: the first half-step of step s issues the copies of half-step
  // 2s+1, then the codes of step s+1 (three loads); the second issues the
  // copies of 2s+2.  So the second half-step can wait for its activations
  // with the codes still in flight, and the codes are waited for only before
  // the step's last k-chunk rebuilds the next step's first weights.
  constexpr int kCodeLoads = 3;
  auto half = [&](int hs, uint8_t* acur, uint8_t* anew) {
    const bool first = (hs & 1) == 0;
    if (first) wait_vmcnt<0>();           // activations of half-step hs
    else wait_vmcnt<kCodeLoads>();        // activations of half-step hs; codes may fly on
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_a(hs + 1, anew);
    if (first) load_codes((hs >> 1) + 1, rnext);
    __builtin_amdgcn_sched_barrier(0);
    if (hs * kHalfK >= K) {  // past K: nothing to multiply (uniform)
      if (!first) {
        wait_vmcnt<NCP>();  // codes of the next step
        to_tile(rnext, tc);
        bq[0] = rebuild_j(tc, 0);
      }
      return;
    }
    bf16x8 af[2][MT];
    auto read_a = [&](int j, bf16x8 (&f)[MT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        f[mt] = *reinterpret_cast<const bf16x8*>(acur + mt * 32 * (kHalfK * 2) + aoff[j]);
    };
    read_a(0, af[0]);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = (first ? 0 : 4) + jj;  // k-chunk within the step
      if (jj < 3) read_a(jj + 1, af[(jj + 1) & 1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[jj & 1][mt], bq[j & 1], acc[mt], 0, 0, 0);
      if (j < 7) {
        bq[(j + 1) & 1] = rebuild_j(tc, j + 1);
        // the operand of the MFMAs above stays live past the rebuild (other
        // registers, no wait for those MFMAs to read theirs)
        asm volatile("" ::"v"(bq[j & 1]));
      } else {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<NCP>();  // codes of the next step
        __builtin_amdgcn_sched_barrier(0);
        to_tile(rnext, tc);
        bq[0] = rebuild_j(tc, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The codes of step 0 do not depend on the block's tokens: they are in
  // flight while the token list is gathered.
  RawCodes r0;
  load_codes(0, r0);
  if (GATE_UP) {
    block_tokens(a, bi, s_tok);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int r = min(8 * (kT4Waves * i + wave) + rsub, rows - 1);
    const int srow = GATE_UP ? max(s_tok[r], 0) : row0 + r;
    arow[i] = src + static_cast<size_t>(srow) * K;
  }
  issue_a(0, As0);
  wait_vmcnt<0>();
  to_tile(r0, tc);
  bq[0] = rebuild_j(tc, 0);
  int hs = 0;
  for (; hs + 1 < nh; hs += 2) {
    half(hs, As0, As1);
    half(hs + 1, As1, As0);
  }
  wait_vmcnt<0>();  // the last half-step's spare copies land before the LDS is released

  if (c_first >= nslices) return;
  const int c = c_first + nsl;
  const int n16 = lane & 15;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      const size_t r = static_cast<size_t>(row0 + m);
      const float v = acc[mt][i];
      if (GATE_UP) {
        const float u = __shfl_xor(v, 8, 64);  // lane n (mod 16 < 8) holds gate, n + 8 up
        if (n16 < 8 && m < rows) {
          const float hv = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;  // silu(g) * u
          out[r * a.I + c * 8 + n16] = f32_to_bf16(hv);
        }
      } else if (m < rows) {
        out[r * a.H + c * 16 + n16] = f32_to_bf16(v);
      }
    }
  }
}

template <bool GATE_UP>
__global__ __launch_bounds__(kT4Threads) __attribute__((amdgpu_waves_per_eu(2))) void w4_gemm_tall8_kernel(
    GemmArgs a, const uint16_t* __restrict__ src, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t As0[kTall8Buf];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[kTall8Buf];
  __shared__ int s_tok[kTall8M];
  BlockInfo bi;
  if (!block_info<GATE_UP>(a, bi, 2 * kT4Waves)) return;
  if (bi.tm <= kTallM) return;  // the four-row-tile kernel owns it
  if (!block_valid<GATE_UP>(a, bi, kTall8M)) return;
  switch ((bi.tm + 31) >> 5) {
    case 5: tall8_block<5, GATE_UP>(a, bi, src, out, As0, As1, s_tok); break;
    case 6: tall8_block<6, GATE_UP>(a, bi, src, out, As0, As1, s_tok); break;
    case 7: tall8_block<7, GATE_UP>(a, bi, src, out, As0, As1, s_tok); break;
    default: tall8_block<8, GATE_UP>(a, bi, src, out, As0, As1, s_tok); break;
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

// The short-batch kernel's pieces, shared with the batch-1 down-and-combine
// kernel: the codes of kGemvChunk steps of one slice (steps past s_end reload
// the last one), and one chunk's products (steps past s_end and inputs past K
// multiply zeros; the weights there are finite) with the scale applied after
// the product, as in the small-tile kernel.
__device__ __forceinline__ void gemv_load_w(const uint8_t* sbase, int s0, int s_end, int lane,
                                            SliceOps (&o)[kGemvChunk]) {
#pragma unroll
  for (int u = 0; u < kGemvChunk; ++u)
    load_slice(sbase + static_cast<size_t>(min(s0 + u, max(s_end - 1, 0))) * kPackBlock, lane, o[u]);
}

__device__ __forceinline__ void gemv_chunk(const uint16_t* arow, int K, int kq, int s0, int s_end,
                                           const SliceOps (&o)[kGemvChunk], const bf16x8& ones,
                                           const PairConsts& pk, f32x4& acc) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  uint4 av[kGemvChunk][4];
#pragma unroll
  for (int u = 0; u < kGemvChunk; ++u) {
    const int s = min(s0 + u, s_end - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      av[u][j] = *reinterpret_cast<const uint4*>(arow + min(s * kKS + 32 * j + kq, K - 8));
  }
#pragma unroll
  for (int u = 0; u < kGemvChunk; ++u) {
    // The mask is opaque to the compiler, so the loads above stay
    // unconditional and their wait counts exact.
    const uint32_t qw[4] = {o[u].q.x, o[u].q.y, o[u].q.z, o[u].q.w};
    float gs[2], gc[2];
    group_affine(o[u].sb.x, gs[0], gc[0]);
    group_affine(o[u].sb.y, gs[1], gc[1]);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      bf16x8 am[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * g + jj;
        uint32_t mk = (s0 + u < s_end && (s0 + u) * kKS + 32 * j + kq < K) ? ~0u : 0u;
        asm("" : "+v"(mk));
        am[jj] = as_bf16x8(make_uint4(av[u][j].x & mk, av[u][j].y & mk, av[u][j].z & mk, av[u][j].w & mk));
      }
      f32x4 X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[0], ones, zero, 0, 0, 0);
      X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[1], ones, X, 0, 0, 0);
      f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[0], codes_plus128(qw[2 * g], pk), zero, 0, 0, 0);
      P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[1], codes_plus128(qw[2 * g + 1], pk), P, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(P[i], gs[g], __builtin_fmaf(X[i], gc[g], acc[i]));
    }
  }
}

// ONE: a single-token batch, where every gate/up row reads x row 0, so the
// activation loads need not wait for the slot-to-token lookup.
template <int KS, bool GATE_UP, bool ONE>
__global__ __launch_bounds__(256) void w4_gemv_kernel(GemmArgs a, const uint16_t* __restrict__ src,
                                                      uint16_t* __restrict__ out) {
  constexpr int SPW = 4 / KS;  // slices per workgroup
  __shared__ f32x4 red[4][64];

  const int K = GATE_UP ? a.H : a.I;
  const int nslices = GATE_UP ? a.I / 8 : a.H / 16;
  const int ntiles = (nslices + SPW - 1) / SPW;
  const int bid = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
  BlockInfo bi;
  bi.nt = 0;
  if (a.shared_mode == 2) {  // the shared expert only: one block of all T rows
    bi.G = a.E;
    bi.row0 = a.T * a.k;
    bi.rows = a.T;
    bi.tm = (a.T + a.tile_gran - 1) / a.tile_gran * a.tile_gran;
  } else {
    // bid < max_blocks (grid size): the entry is loaded together with the map
    // length, not after it; the routed-only launch stops before the shared block
    const int4 blk = reinterpret_cast<const int4*>(a.blocks)[bid];
    const int nblk = min(*a.n_blocks, a.max_blocks) - (a.shared_mode == 1 ? a.n_shared_blocks : 0);
    if (bid >= nblk) return;
    bi.G = blk.x;
    bi.row0 = blk.y;
    bi.rows = blk.z;
    bi.tm = blk.w;
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
  int srow = (GATE_UP && !ONE) ? ((rr < Sk) ? a.sorted_slot[rr] : rr) : rr;

  SliceOps o0[kGemvChunk];
  gemv_load_w(sbase, s_begin, s_end, lane, o0);

  if (GATE_UP && ONE) {
    srow = 0;
  } else if (GATE_UP) {
    srow = (rr < Sk) ? srow / a.k : rr - Sk;
    if (srow < 0 || srow >= a.T) {
      status_set(a.status, MOE_STATUS_BAD_INDEX);
      srow = 0;
    }
  }
  // Rows past the block read the block's last row: an MFMA row only reaches
  // its own output row, and those are never stored.
  const uint16_t* arow = src + static_cast<size_t>(srow) * K;
  const int kq = (lane >> 4) * 8;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = bf16_ones();
  const PairConsts pk = pair_consts();
  // the first chunk is peeled, so its weight loads (issued above) are not
  // loop-carried and nothing waits for them before the activation loads
  if (s_begin < s_end) gemv_chunk(arow, K, kq, s_begin, s_end, o0, ones, pk, acc);
  for (int s0 = s_begin + kGemvChunk; s0 < s_end; s0 += kGemvChunk) {
    SliceOps o1[kGemvChunk];
    gemv_load_w(sbase, s0, s_end, lane, o1);
    gemv_chunk(arow, K, kq, s0, s_end, o1, ones, pk, acc);
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
  const int nb = a.shared_mode == 2 ? 1 : a.max_blocks - (a.shared_mode == 1 ? a.n_shared_blocks : 0);
  if (nb <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nb) * ((nslices + spw - 1) / spw));
#define MOE_GEMV(KS, ONE) \
  hipLaunchKernelGGL((w4_gemv_kernel<KS, GATE_UP, ONE>), grid, dim3(256), 0, stream, a, src, out)
  if constexpr (GATE_UP) {
    const bool one = a.T == 1;
    if (ks == 4) {
      if (one) MOE_GEMV(4, true); else MOE_GEMV(4, false);
    } else if (ks == 2) {
      if (one) MOE_GEMV(2, true); else MOE_GEMV(2, false);
    } else {
      if (one) MOE_GEMV(1, true); else MOE_GEMV(1, false);
    }
  } else {
    if (ks == 4) MOE_GEMV(4, false);
    else if (ks == 2) MOE_GEMV(2, false);
    else MOE_GEMV(1, false);
  }
#undef MOE_GEMV
  return hipGetLastError();
}

// Tall-tile kernel variant for a tile height bound (0: no tile exceeds kSmallM).
int gemm_m_max_for(int tile_m_max) {
  return tile_m_max <= kSmallM ? 0 : tile_m_max <= kTallM ? kTallM : kTall8M;
}

// N tiles per workgroup of the resident-activation down kernel: whole tiles,
// enough of them that the block's staging is amortised, few enough that the
// grid still holds about two workgroups per slot (three per CU).
static int down_resident_ntw(const GemmArgs& a, long long blocks8) {
  const int ntiles = n_tiles<false>(a, kSmallSlices * kSmallWaves);
  int ntw = 1;
  while (ntw * 2 <= ntiles && blocks8 * ((ntiles + 2 * ntw - 1) / (2 * ntw)) >= kResTargetWgs) ntw *= 2;
  return ntw;
}

template <int MODE>
static void launch_down_resident(const GemmArgs& a, long long blocks8, const uint16_t* src,
                                 uint16_t* out, hipStream_t stream) {
  const int ntw = down_resident_ntw(a, blocks8);
  const dim3 grid(static_cast<unsigned>(blocks8 * n_tiles<false>(a, kSmallSlices * kSmallWaves * ntw)));
  hipLaunchKernelGGL((w4_down_resident_kernel<kSmallWaves, kSmallSlices, MODE>), grid,
                     dim3(64 * kSmallWaves), 0, stream, a, src, out, ntw);
}

template <bool GATE_UP>
static hipError_t launch_gemm(const GemmArgs& a, int m_max, const uint16_t* src, uint16_t* out,
                              hipStream_t stream) {
  if (a.T <= kGemvRows) return launch_gemv<GATE_UP>(a, src, out, stream);
  // When tall tiles are allowed and an expert averages at least kSmallM rows,
  // nearly all rows sit in tall blocks; the few short blocks then run in the
  // tall-tile kernel too (one 32-row tile), where they fill its last round of
  // workgroups instead of occupying a launch of their own that the chip
  // cannot fill.
  GemmArgs ga = a;
  ga.tall_all = m_max && static_cast<long long>(a.T) * a.k >= static_cast<long long>(kSmallM) * a.E;
  const int nsh = a.n_shared_blocks;
  if (a.shared_mode == 2) {  // the shared expert only: its tile height is known here
    if (nsh <= 0) return hipSuccess;
    const int tm = ((a.T + nsh - 1) / nsh + a.tile_gran - 1) / a.tile_gran * a.tile_gran;
    const long long b8 = (nsh + kXcds - 1) / kXcds * kXcds;
    if (tm <= kSmallM && !ga.tall_all && !GATE_UP && a.I <= kResK) {
      launch_down_resident<2>(ga, b8, src, out, stream);
    } else if (tm <= kSmallM && !ga.tall_all) {
      hipLaunchKernelGGL((w4_gemm_small_kernel<kSmallWaves, kSmallSlices, GATE_UP, 2>),
                         dim3(static_cast<unsigned>(b8 * n_tiles<GATE_UP>(a, kSmallSlices * kSmallWaves))),
                         dim3(64 * kSmallWaves), 0, stream, ga, src, out);
    } else if (tm > kTallM) {
      hipLaunchKernelGGL((w4_gemm_tall8_kernel<GATE_UP>),
                         dim3(static_cast<unsigned>(b8 * n_tiles<GATE_UP>(a, 2 * kT4Waves))),
                         dim3(kT4Threads), 0, stream, ga, src, out);
    } else {
      hipLaunchKernelGGL((w4_gemm_tall4_shared_kernel<GATE_UP>),
                         dim3(static_cast<unsigned>(b8 * n_tiles<GATE_UP>(a, 2 * kT4CT * kT4Waves))),
                         dim3(kT4Threads), 0, stream, ga, src, out);
    }
    return hipGetLastError();
  }
  const int nb = a.max_blocks - (a.shared_mode == 1 ? nsh : 0);
  if (nb <= 0) return hipSuccess;
  const long long blocks8 = (nb + kXcds - 1) / kXcds * kXcds;
  const bool routed_only = a.shared_mode == 1;
  if (!ga.tall_all && !GATE_UP && a.I <= kResK) {
    if (routed_only)
      launch_down_resident<1>(ga, blocks8, src, out, stream);
    else
      launch_down_resident<0>(ga, blocks8, src, out, stream);
  } else if (!ga.tall_all) {
    const dim3 grid_small(static_cast<unsigned>(blocks8 * n_tiles<GATE_UP>(a, kSmallSlices * kSmallWaves)));
    if (routed_only)
      hipLaunchKernelGGL((w4_gemm_small_kernel<kSmallWaves, kSmallSlices, GATE_UP, 1>), grid_small,
                         dim3(64 * kSmallWaves), 0, stream, ga, src, out);
    else
      hipLaunchKernelGGL((w4_gemm_small_kernel<kSmallWaves, kSmallSlices, GATE_UP, 0>), grid_small,
                         dim3(64 * kSmallWaves), 0, stream, ga, src, out);
  }
  if (m_max > kTallM) {  // blocks of 160..256 rows first: they hold most of the work
    const dim3 grid8(static_cast<unsigned>(blocks8 * n_tiles<GATE_UP>(a, 2 * kT4Waves)));
    hipLaunchKernelGGL((w4_gemm_tall8_kernel<GATE_UP>), grid8, dim3(kT4Threads), 0, stream, ga, src, out);
  }
  if (m_max) {
    const dim3 grid(static_cast<unsigned>(blocks8 * n_tiles<GATE_UP>(a, 2 * kT4CT * kT4Waves)));
    if (routed_only)
      hipLaunchKernelGGL((w4_gemm_tall4_routed_kernel<GATE_UP>), grid, dim3(kT4Threads), 0, stream, ga, src, out);
    else
      hipLaunchKernelGGL((w4_gemm_tall4_kernel<GATE_UP>), grid, dim3(kT4Threads), 0, stream, ga, src, out);
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
  // one token per workgroup (ceil(H/8 / 256) workgroups per token): the
  // token's slot positions and weights are workgroup-uniform, scalar loads
  const int chunks = H / 8;
  const int cg = (chunks + 255) / 256;
  const int t = static_cast<int>(blockIdx.x / static_cast<unsigned>(cg));
  const int ci = static_cast<int>(blockIdx.x % static_cast<unsigned>(cg)) * 256 + static_cast<int>(threadIdx.x);
  if (t >= T || ci >= chunks) return;
  const int c = ci * 8;
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
  const long long n = static_cast<long long>(T) * ((H / 8 + 255) / 256);
  const dim3 grid(static_cast<unsigned>(n));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, T, H, k, n_shared, topk_w,
                     slot_pos, y_slots, y, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Batch-1 down GEMM with the combine in its epilogue.  With one token every
// block of the map holds one row -- the routed slots in expert order, then
// the shared expert's -- and block b's row is y_slots row b.  A workgroup
// owns one 16-column slice of the output and gives each block one wave, which
// runs the short-batch product over all of I (the same steps, in the same
// order, as the down launch of w4_gemv_kernel with one wave per slice),
// stores its row of the slice to y_slots rounded to bfloat16 as that launch
// does, and keeps it in LDS.  Then sixteen lanes combine the slots as
// combine_kernel does: float32 fused multiply-adds in rank order, the shared
// expert's row added last, one rounding to bfloat16.  y_slots and y are
// bit-identical to the two launches; one launch and y_slots' read-back go.
// ---------------------------------------------------------------------------
constexpr int kFusedMaxBlocks = 16;

__global__ __launch_bounds__(64 * kFusedMaxBlocks) void w4_down_combine_one_kernel(
    GemmArgs a, const float* __restrict__ topk_w, const int32_t* __restrict__ slot_pos,
    const uint16_t* __restrict__ h, uint16_t* __restrict__ y_slots, uint16_t* __restrict__ y) {
  __shared__ float s_ys[kFusedMaxBlocks][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int c = blockIdx.x;          // 16-column slice of the output
  const int nb = a.k + a.n_shared;   // blocks of a one-token map (the block size is 64 nb)
  // the combine's slot positions and weights (thread j: slot j), loaded
  // first so that the products cover their latency, kept in LDS below
  __shared__ int s_pos[kFusedMaxBlocks];
  __shared__ float s_w[kFusedMaxBlocks];
  int pj = 0;
  float wj = 0.0f;
  if (tid < a.k) {
    pj = slot_pos[tid];
    wj = topk_w[tid];
  }
  {
    // the entry is loaded together with the map length (wave < nb <= max_blocks)
    const int4 blk = reinterpret_cast<const int4*>(a.blocks)[wave];
    const int nblk = min(*a.n_blocks, a.max_blocks);
    BlockInfo bi;
    bi.nt = 0;
    bi.G = blk.x;
    bi.row0 = blk.y;
    bi.rows = blk.z;
    bi.tm = blk.w;
    if (nblk == nb && bi.rows == 1 && bi.row0 == wave && block_valid<false>(a, bi, 1 << 30)) {
      const int nk = pack_steps(a.I);
      const uint8_t* sbase = bi.P + static_cast<size_t>(c) * nk * kPackBlock;
      const uint16_t* arow = h + static_cast<size_t>(bi.row0) * a.I;
      const int kq = (lane >> 4) * 8;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const bf16x8 ones = bf16_ones();
      const PairConsts pk = pair_consts();
      SliceOps o0[kGemvChunk];
      gemv_load_w(sbase, 0, nk, lane, o0);
      gemv_chunk(arow, a.I, kq, 0, nk, o0, ones, pk, acc);
      for (int s0 = kGemvChunk; s0 < nk; s0 += kGemvChunk) {
        SliceOps o1[kGemvChunk];
        gemv_load_w(sbase, s0, nk, lane, o1);
        gemv_chunk(arow, a.I, kq, s0, nk, o1, ones, pk, acc);
      }
      if (lane < 16) {  // MFMA row 0 (the block's row), column lane
        const uint16_t v = f32_to_bf16(acc[0]);
        y_slots[static_cast<size_t>(bi.row0) * a.H + c * 16 + lane] = v;
        s_ys[wave][lane] = bf16_to_f32(v);
      }
    } else {
      if (lane == 0) status_set(a.status, MOE_STATUS_BAD_INDEX);
      if (lane < 16) s_ys[wave][lane] = 0.0f;
    }
  }
  if (tid < a.k) {
    s_pos[tid] = pj;
    s_w[tid] = wj;
  }
  __syncthreads();
  if (tid < 16) {
    float acc = 0.0f;
    for (int j = 0; j < a.k; ++j) {
      const int p = s_pos[j];
      if (p < 0 || p >= a.k) {
        status_set(a.status, MOE_STATUS_BAD_INDEX);
        continue;
      }
      acc = __builtin_fmaf(s_w[j], s_ys[p][tid], acc);
    }
    if (a.n_shared) acc += s_ys[a.k][tid];
    y[c * 16 + tid] = f32_to_bf16(acc);
  }
}

bool down_combine_fused(const GemmArgs& a) {
  // one token, at most kFusedMaxBlocks blocks, and a down GEMM that the
  // short-batch launch runs with one wave per slice (fewer than 8 steps)
  return a.T == 1 && a.k + a.n_shared <= kFusedMaxBlocks && pack_steps(a.I) < 8 && a.H % 16 == 0;
}

hipError_t launch_down_combine_one(const GemmArgs& a, const float* topk_w, const int32_t* slot_pos,
                                   const uint16_t* h, uint16_t* y_slots, uint16_t* y,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(w4_down_combine_one_kernel, dim3(static_cast<unsigned>(a.H / 16)),
                     dim3(64 * (a.k + a.n_shared)), 0, stream, a, topk_w, slot_pos, h, y_slots, y);
  return hipGetLastError();
}

}  // namespace moe
