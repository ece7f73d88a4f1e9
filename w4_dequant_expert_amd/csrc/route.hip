// GPU-resident routing for the MoE expert layer on gfx950: router scores,
// top-k with renormalised softmax weights, the expert histogram, one exclusive
// scan, the stable scatter and the tile block map.  Everything stays on the
// device: the grouped GEMMs read the block map and its length from memory, so
// nothing returns to the host between the router and the GEMMs ["Lily Beats
// MLX-LM 1.35x on Decode", "Prefill: fusing dequantisation and keeping routing
// GPU-resident"; "Introduction: Revolutionizing Local AI Inference on Apple
// Silicon", "Optimizing Prefill Operations"].
//
// Three kernels on one stream:
//   K1 router scores (float32, fixed evaluation order) and clearing of the
//      token bitmask;
//   K2 top-k and weights, one wave per token with DPP and row-swap
//      reductions; every selection sets its token's bit in a [token word]
//      [expert] bitmask with an atomic OR (order-independent, hence
//      deterministic);
//   K3 one workgroup: per-expert popcount prefixes over the bitmask give the
//      histogram and every slot's stable rank, then the exclusive scan, the
//      block map and the scatter.
// A token selects an expert at most once, so ordering an expert's slots by
// token is the same as ordering them by slot id: the rank of slot (t, j) in
// its expert e is the number of tokens before t that selected e.
#include "route.h"

#include <math.h>

namespace moe {

// ---------------------------------------------------------------------------
// K1: router scores.  A wave computes a tile of TW tokens x EW experts; lane m
// owns partial m of every one of its outputs: a float32 fma chain over inputs
// h = m, m+64, m+128, ...  The 64 partials of each output are combined by a
// transposed butterfly across the lanes whose pairing is exactly the tree
// p[i] += p[i+s], s = 32..1, so every score has one fixed evaluation order
// that a host implementation reproduces bit for bit.  x (as float32,
// transposed) and the router weights are staged through LDS, CH chunks of 64
// inputs at a time.
// ---------------------------------------------------------------------------
constexpr int kTW = 8, kEW = 8;  // per-lane tile: 64 outputs
constexpr int kShortT = 16;      // batches up to this size use the short-batch kernel

template <int WT, int WE, int CH, bool VEC>
__global__ __launch_bounds__(WT * WE * 64) void router_scores_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, uint32_t* __restrict__ bits,
    int nbits, uint32_t* __restrict__ status) {
  constexpr int NT = WT * WE * 64;
  constexpr int RT = kTW * WT, RE = kEW * WE;  // workgroup tile
  constexpr int PT = RT + 4, PE = RE + 4;      // padded LDS rows
  __shared__ float xs[CH][64][PT];  // x chunk, transposed: [input][token]
  __shared__ float ws[CH][64][PE];  // router chunk: [input][expert]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wt = wave % WT, we = wave / WT;
  const int t0 = blockIdx.x * RT, e0 = blockIdx.y * RE;

  {  // clear the token bitmask of K2 and the status word (stream-ordered before K2)
    const long long gid = (static_cast<long long>(blockIdx.y) * gridDim.x + blockIdx.x) * NT + tid;
    const long long gsz = static_cast<long long>(gridDim.x) * gridDim.y * NT;
    for (long long i = gid; i < nbits; i += gsz) bits[i] = 0u;
    if (gid == 0 && status) *status = 0u;
  }

  float acc[kTW * kEW];
#pragma unroll
  for (int o = 0; o < kTW * kEW; ++o) acc[o] = 0.0f;

  // Staging with fixed per-thread counts, so every load of a chunk is issued
  // before any of them is waited for; the next chunk is loaded into registers
  // while the current one is multiplied.
  constexpr int XN = RT * CH * 8;          // 16-byte x loads per chunk
  constexpr int WN = CH * 64 * (RE / 4);   // 16-byte router loads per chunk
  constexpr int XI = (XN + NT - 1) / NT, WI = (WN + NT - 1) / NT;
  const int nchunk = H / 64;
  uint4 xr[XI];
  u32x4 wrg[WI];  // router values as raw bits (native vectors: they stay in registers)
  // Loads are unconditional, with clamped indices, so that all of a chunk's
  // loads are in flight together: a clamped token row or chunk only feeds
  // outputs that are never stored or chunks that are never multiplied.
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      // consecutive lanes take consecutive tokens, so the transposed LDS
      // writes below fall in different banks
      const int idx = min(tid + i * NT, XN - 1);
      const int t = idx % RT, part = idx / RT;
      const int c = part / 8, m = (part % 8) * 8;
      const int gt = min(t0 + t, T - 1), hc = min(c0 + c, nchunk - 1);
      xr[i] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(gt) * H + hc * 64 + m);
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int idx = min(tid + i * NT, WN - 1);
      const int row = idx / (RE / 4), col = (idx % (RE / 4)) * 4;
      const int c = row / 64, m = row % 64;
      const int h = min(c0 + c, nchunk - 1) * 64 + m;
      const float* src = wr + static_cast<size_t>(h) * E;
      if constexpr (VEC) {  // E % 4 == 0 and 16-byte rows: a clamped column stays in the row
        wrg[i] = *reinterpret_cast<const u32x4*>(src + min(e0 + col, E - 4));
      } else {
        const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
        wrg[i] = u32x4{s32[min(e0 + col, E - 1)], s32[min(e0 + col + 1, E - 1)],
                       s32[min(e0 + col + 2, E - 1)], s32[min(e0 + col + 3, E - 1)]};
      }
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int idx = tid + i * NT;
      if (XN % NT == 0 || idx < XN) {
        const int t = idx % RT, part = idx / RT;
        const int c = part / 8, m = (part % 8) * 8;
        const uint32_t wv[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xs[c][m + 2 * q][t] = bf16_to_f32(wv[q] & 0xFFFFu);
          xs[c][m + 2 * q + 1][t] = bf16_to_f32(wv[q] >> 16);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int idx = tid + i * NT;
      if (WN % NT == 0 || idx < WN) {
        const int row = idx / (RE / 4), col = (idx % (RE / 4)) * 4;
        *reinterpret_cast<u32x4*>(&ws[row / 64][row % 64][col]) = wrg[i];
      }
    }
  };

  load_chunk(0);
  for (int c0 = 0; c0 < nchunk; c0 += CH) {
    __syncthreads();  // the previous chunk's reads are done
    store_chunk();
    __syncthreads();
    load_chunk(c0 + CH);  // in flight during the multiply below
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c0 + c >= nchunk) break;
      float xv[kTW], wv[kEW];
      const float4 xa = *reinterpret_cast<const float4*>(&xs[c][lane][wt * kTW]);
      const float4 xb = *reinterpret_cast<const float4*>(&xs[c][lane][wt * kTW + 4]);
      const float4 wa = *reinterpret_cast<const float4*>(&ws[c][lane][we * kEW]);
      const float4 wb = *reinterpret_cast<const float4*>(&ws[c][lane][we * kEW + 4]);
      xv[0] = xa.x; xv[1] = xa.y; xv[2] = xa.z; xv[3] = xa.w;
      xv[4] = xb.x; xv[5] = xb.y; xv[6] = xb.z; xv[7] = xb.w;
      wv[0] = wa.x; wv[1] = wa.y; wv[2] = wa.z; wv[3] = wa.w;
      wv[4] = wb.x; wv[5] = wb.y; wv[6] = wb.z; wv[7] = wb.w;
#pragma unroll
      for (int i = 0; i < kTW; ++i)
#pragma unroll
        for (int j = 0; j < kEW; ++j) acc[i * kEW + j] = __builtin_fmaf(xv[i], wv[j], acc[i * kEW + j]);
    }
  }

  // Transposed butterfly: at distance s the lane with bit s clear keeps the
  // lower half of its outputs and the partner keeps the upper half; each adds
  // its partner's copy.  Tree index of lane L is L mod 2s, so the pairing is
  // p[i] + p[i+s].  After s = 1 lane L holds output L.
  // At s = 32 and 16 one v_permlane32_swap / v_permlane16_swap of the pair
  // (acc[i], acc[i+s]) leaves, in every lane, its own kept value in one
  // register and the partner's in the other, so the level is one swap and one
  // add per output (the same sum: addition commutes).
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i]), __float_as_uint(acc[i + 32]),
                                                    false, false);
    acc[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i]), __float_as_uint(acc[i + 16]),
                                                    false, false);
    acc[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) {
    const bool upper = (lane & s) != 0;
#pragma unroll
    for (int i = 0; i < s; ++i) {
      const float send = upper ? acc[i] : acc[i + s];
      const float keep = upper ? acc[i + s] : acc[i];
      const float recv = __shfl_xor(send, s, 64);
      acc[i] = keep + recv;
    }
  }
  const int ti = lane / kEW, ej = lane % kEW;
  const int t = t0 + wt * kTW + ti, e = e0 + we * kEW + ej;
  if (t < T && e < E) {
    float l = acc[0];
    if (bias) l = l + bias[e];
    logits[static_cast<size_t>(t) * E + e] = l;
  }
}

// ---------------------------------------------------------------------------
// K1 for short batches (decode): the same scores in the same evaluation order,
// with the work spread over the router matrix instead of over tokens, so that
// its 4*H*E bytes stream through many compute units at once.  A workgroup owns
// 16 experts; thread (m, e) runs the fma chain of partial m of expert e for
// every token, reading each of its router weights once.  The 64 partials of a
// (token, expert) then meet in LDS, where one thread applies the tree
// p[i] += p[i+s], s = 32..1, and adds the bias.
// ---------------------------------------------------------------------------
constexpr int kShortHC = 2048;           // inputs of x staged per pass
constexpr int kShortIU = kShortHC / 64;  // chain steps per pass

template <int TT>  // batch bucket: T <= TT; rows T..TT-1 are computed and dropped
__global__ __launch_bounds__(1024) void router_scores_short_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, uint32_t* __restrict__ bits,
    int nbits, uint32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[TT][kShortHC];
  __shared__ float ps[TT][64][17];

  const int tid = threadIdx.x, lane = tid & 63;
  const int es = lane & 15, m = (tid >> 6) * 4 + (lane >> 4);
  const int e = blockIdx.x * 16 + es, ec = min(e, E - 1);

  {  // clear the token bitmask of K2 and the status word
    for (int i = blockIdx.x * 1024 + tid; i < nbits; i += gridDim.x * 1024) bits[i] = 0u;
    if (blockIdx.x == 0 && tid == 0 && status) *status = 0u;
  }

  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;

  for (int c = 0; c < H; c += kShortHC) {
    const int ni = min(kShortHC, H - c) / 64;  // chain steps of this pass
    float wv[kShortIU];
#pragma unroll
    for (int i = 0; i < kShortIU; ++i)
      wv[i] = wr[static_cast<size_t>(c + min(i, ni - 1) * 64 + m) * E + ec];
    // x[0..T)[c .. c + 64 ni) as bfloat16, XU 16-byte chunks per thread and pass
    constexpr int XU = (TT * kShortHC / 8 + 1023) / 1024;
    const int nq = T * ni * 8;
    uint4 xv[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int q = min(tid + u * 1024, nq - 1);
      const int t = q / (ni * 8), cc = q % (ni * 8);
      xv[u] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + c + cc * 8);
    }
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int q = tid + u * 1024;
      if (q < nq) {
        const int t = q / (ni * 8), cc = q % (ni * 8);
        *reinterpret_cast<uint4*>(&xs[t][cc * 8]) = xv[u];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kShortIU; ++i) {
      if (i < ni) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
          acc[t] = __builtin_fmaf(bf16_to_f32(xs[t][i * 64 + m]), wv[i], acc[t]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) ps[t][m][es] = acc[t];
  __syncthreads();
  // The tree, one level at a time across the threads of partial m < s2:
  // level s2 reads entries s2 .. 2 s2 - 1, which it does not write.
#pragma unroll
  for (int s2 = 32; s2 >= 1; s2 >>= 1) {
    if (m < s2) {
#pragma unroll
      for (int t = 0; t < TT; ++t) ps[t][m][es] = ps[t][m][es] + ps[t][m + s2][es];
    }
    __syncthreads();
  }
  if (tid < T * 16) {
    const int t = tid >> 4, j = tid & 15;
    const int eo = blockIdx.x * 16 + j;
    if (eo < E) {
      float l = ps[t][0][j];
      if (bias) l = l + bias[eo];
      logits[static_cast<size_t>(t) * E + eo] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// K1 for short batches with E <= 256, spread over eight times as many
// workgroups.  The tree's first three levels (s = 32, 16, 8) only ever add
// partials whose indices agree mod 8, so the 64 partials of an output split
// into eight classes m = q (mod 8) that reduce independently: workgroup
// (expert chunk, q) runs the chains of the eight partials of class q for 16
// experts and every token, reduces them with those three levels in LDS, and
// writes the class sum to part[q][t][e].  The last three levels (s = 4, 2, 1)
// over the eight class sums and the bias are applied by route_short_kernel,
// so the evaluation order is exactly that of the full tree.  Only the inputs
// h = q (mod 8) are staged, as float32.
// ---------------------------------------------------------------------------
constexpr int kClasses = 8;

template <int TT>  // batch bucket: T <= TT; rows T..TT-1 are computed and dropped
__global__ __launch_bounds__(128) void router_partials_short_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    float* __restrict__ part, uint32_t* __restrict__ status) {
  __shared__ float xs[TT][kShortHC / kClasses];
  __shared__ float ps[TT][kClasses][17];

  const int tid = threadIdx.x;
  const int q = blockIdx.x % kClasses;
  const int es = tid & 15, mi = tid >> 4;  // partial m = q + 8 mi
  const int m = q + kClasses * mi;
  const int e = (blockIdx.x / kClasses) * 16 + es, ec = min(e, E - 1);
  if (blockIdx.x == 0 && tid == 0) *status = 0u;

  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;

  for (int c = 0; c < H; c += kShortHC) {
    const int ni = min(kShortHC, H - c) / 64;  // chain steps of this pass
    float wv[kShortIU];
#pragma unroll
    for (int i = 0; i < kShortIU; ++i)
      wv[i] = wr[static_cast<size_t>(c + min(i, ni - 1) * 64 + m) * E + ec];
    // x[t][c + 8 j + q], j < 8 ni: XU values per thread, all loads in flight together
    constexpr int XU = TT * (kShortHC / kClasses) / 128;
    const int nv = T * ni * 8;
    uint16_t xv[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int v = min(tid + u * 128, nv - 1);
      const int t = v / (ni * 8), j = v % (ni * 8);
      xv[u] = x[static_cast<size_t>(t) * H + c + 8 * j + q];
    }
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int v = tid + u * 128;
      if (v < nv) xs[v / (ni * 8)][v % (ni * 8)] = bf16_to_f32(xv[u]);
    }
    __syncthreads();
    // chain step i of partial m reads input c + 64 i + m = c + 8 (8 i + mi) + q
#pragma unroll
    for (int i = 0; i < kShortIU; ++i) {
      if (i < ni) {
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = __builtin_fmaf(xs[t][8 * i + mi], wv[i], acc[t]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) ps[t][mi][es] = acc[t];
  __syncthreads();
  // levels s = 32, 16, 8 of the tree: partial m + s is index mi + s / 8
#pragma unroll
  for (int s2 = 4; s2 >= 1; s2 >>= 1) {
    if (mi < s2) {
#pragma unroll
      for (int t = 0; t < TT; ++t) ps[t][mi][es] = ps[t][mi][es] + ps[t][mi + s2][es];
    }
    __syncthreads();
  }
  for (int i = tid; i < T * 16; i += 128) {
    const int t = i >> 4, j = i & 15;
    const int eo = (blockIdx.x / kClasses) * 16 + j;
    if (eo < E) part[(static_cast<size_t>(q) * T + t) * E + eo] = ps[t][0][j];
  }
}

// Score of (t, e) from its eight class sums: the tree's levels s = 4, 2, 1,
// then the bias.
__device__ __forceinline__ float score_from_classes(const float* __restrict__ part, int T, int E,
                                                    int t, int e, const float* __restrict__ bias) {
  float p[kClasses];
#pragma unroll
  for (int i = 0; i < kClasses; ++i) p[i] = part[(static_cast<size_t>(i) * T + t) * E + e];
#pragma unroll
  for (int s = kClasses / 2; s >= 1; s >>= 1)
#pragma unroll
    for (int i = 0; i < s; ++i) p[i] = p[i] + p[i + s];
  return bias ? p[0] + bias[e] : p[0];
}

// ---------------------------------------------------------------------------
// K2: top-k and weights.  A token is served by one wave; lane l holds the
// scores of experts l, l+64, l+128...  Every score becomes a 64-bit key: an
// order-preserving image of the float32 score in the high word and the
// complemented expert index in the low word, so that a larger key means a
// higher score or, between equal scores, a lower expert index (the selection
// order), and no two keys are equal.  Round j takes each lane's largest key
// below the previous round's winner and the wave maximum of those: four DPP
// exchanges within each 16-lane row (row mirror, half-row mirror, quad swaps
// by 2 and by 1, which pair every lane with every other through the
// butterfly), then the rows pairwise.  The rounds are branch-free.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t max_step(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(dpp<CTRL>(static_cast<int>(v)));
  const uint32_t hi = static_cast<uint32_t>(dpp<CTRL>(static_cast<int>(v >> 32)));
  const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
  return o > v ? o : v;
}

template <int CTRL>
__device__ __forceinline__ float sum_step(float v) {
  return v + __int_as_float(dpp<CTRL>(__float_as_int(v)));
}

constexpr int kRowMirror = 0x140, kHalfMirror = 0x141;
constexpr int kQuadSwap2 = 0x4E, kQuadSwap1 = 0xB1;  // quad_perm [2,3,0,1] and [1,0,3,2]

// Order-preserving map of a float32 (not NaN, -0 already folded into +0) to
// an unsigned integer, and back.
__device__ __forceinline__ uint32_t float_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// The same exchange across the four rows of a wave: lane l and lane l ^ 16
// (v_permlane16_swap), then l ^ 32 (v_permlane32_swap).  Swapping a register
// with itself leaves, in every lane, its own value and its partner's in the
// two results, in some order; max and + do not care which.
__device__ __forceinline__ uint64_t max_rows16(uint64_t v) {
  const auto lo = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(v >> 32), static_cast<uint32_t>(v >> 32),
                                                   false, false);
  const uint64_t a = (static_cast<uint64_t>(hi[0]) << 32) | lo[0];
  const uint64_t b = (static_cast<uint64_t>(hi[1]) << 32) | lo[1];
  return a > b ? a : b;
}
__device__ __forceinline__ uint64_t max_rows32(uint64_t v) {
  const auto lo = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(v >> 32), static_cast<uint32_t>(v >> 32),
                                                   false, false);
  const uint64_t a = (static_cast<uint64_t>(hi[0]) << 32) | lo[0];
  const uint64_t b = (static_cast<uint64_t>(hi[1]) << 32) | lo[1];
  return a > b ? a : b;
}
__device__ __forceinline__ float sum_rows(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Top-k of token t for one wave (lane l holds the scores of experts l, l+64,
// ...): writes the token's indices and weights (t < T) and returns the expert
// this lane selected (rank l; -1 where l >= k).  A round's local maximum is a
// tree over the lane's VPL keys (depth log2 VPL, not a chain), then the wave
// maximum over four DPP steps within the rows and two row swaps.
template <int VPL>  // scores per lane: E <= 64 * VPL
__device__ __forceinline__ int topk_wave(int T, int E, int k, const float* __restrict__ logits,
                                         int t, int32_t* __restrict__ topk_idx,
                                         float* __restrict__ topk_w, uint32_t* __restrict__ status) {
  static_assert((VPL & (VPL - 1)) == 0, "a power of two");
  const int lane = threadIdx.x & 63;
  const bool tok_ok = t < T;
  const int tt = tok_ok ? t : T - 1;  // waves past T work on a real token and store nothing

  // every load is issued unconditionally (clamped index), all in flight together
  float val[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) val[v] = logits[static_cast<size_t>(tt) * E + min(lane + 64 * v, E - 1)];
  bool saw_nan = false;
  uint64_t key[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane + 64 * v;
    const float sc = val[v];
    saw_nan |= (e < E) && (sc != sc);
    const float f = (sc == sc) ? sc + 0.0f : -INFINITY;  // NaN ranks as -inf; -0 as +0
    const uint64_t kk = (static_cast<uint64_t>(float_order(f)) << 32) | static_cast<uint32_t>(~e);
    key[v] = (e < E) ? kk : 0ull;  // 0 is below every real key
  }

  uint64_t prev = ~0ull;
  uint64_t sel = 0;  // this lane's selection: rank lane
  for (int j = 0; j < k; ++j) {
    uint64_t m[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) m[v] = key[v] < prev ? key[v] : 0ull;
#pragma unroll
    for (int w = VPL / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int v = 0; v < w; ++v) m[v] = m[v + w] > m[v] ? m[v + w] : m[v];
    uint64_t best = m[0];
    best = max_step<kRowMirror>(best);
    best = max_step<kHalfMirror>(best);
    best = max_step<kQuadSwap2>(best);
    best = max_step<kQuadSwap1>(best);
    best = max_rows16(best);
    best = max_rows32(best);
    prev = best;
    sel = (j == lane) ? best : sel;
  }
  const float sv = order_float(static_cast<uint32_t>(sel >> 32));
  const int se = static_cast<int>(~static_cast<uint32_t>(sel));

  // weights: exp(l_j - l_max) / sum over the selected (the softmax
  // denominator over all experts cancels in the renormalisation)
  const float top = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sv)));
  const float ex = (lane < k) ? __expf(sv - top) : 0.0f;
  float den = ex;
  den = sum_step<kRowMirror>(den);
  den = sum_step<kHalfMirror>(den);
  den = sum_step<kQuadSwap2>(den);
  den = sum_step<kQuadSwap1>(den);
  den = sum_rows(den);
  if (tok_ok && lane < k) {
    topk_idx[static_cast<size_t>(t) * k + lane] = se;
    topk_w[static_cast<size_t>(t) * k + lane] = ex / den;
  }
  if (saw_nan && tok_ok) status_set(status, MOE_STATUS_NAN_LOGIT);
  return (tok_ok && lane < k) ? se : -1;
}

template <int VPL>  // scores per lane: E <= 64 * VPL
__global__ __launch_bounds__(256) void router_topk_kernel(int T, int E, int k,
                                                          const float* __restrict__ logits,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          uint32_t* __restrict__ bits,
                                                          uint32_t* __restrict__ status) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);  // one token per wave
  if (t >= T) return;  // wave-uniform; the kernel has no barrier
  const int se = topk_wave<VPL>(T, E, k, logits, t, topk_idx, topk_w, status);
  if (se >= 0) atomicOr(&bits[static_cast<size_t>(t >> 5) * E + se], 1u << (t & 31));
}

// ---------------------------------------------------------------------------
// K3: one workgroup of 1024 threads.
// ---------------------------------------------------------------------------
__device__ int block_exclusive_scan(int v, int* tmp /* >= 17 ints */, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int s = tmp[w];
      tmp[w] = run;
      run += s;
    }
    tmp[16] = run;
  }
  __syncthreads();
  const int r = tmp[wave] + inc - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

// Histogram -> offsets (exclusive scan) and the tile block map, for a
// workgroup of 1024 threads; thread e < E holds the count of expert e.
// Leaves the counts and offsets in s_cnt / s_off (index E: the shared group).
__device__ void finish_tables(int T, int E, int k, int n_shared, int tile_m_max, int tile_gran,
                              int cnt, int* s_cnt, int* s_off, int* s_bstart, int* tmp,
                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ blocks, int32_t* __restrict__ n_blocks,
                              int max_blocks, uint32_t* __restrict__ status, bool write = true) {
  const int tid = threadIdx.x;
  const int S = T * k;
  int total = 0;
  const int off = block_exclusive_scan((tid < E) ? cnt : 0, tmp, &total);
  if (tid < E) {
    if (write) {
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    s_off[tid] = off;
    s_cnt[tid] = cnt;
  }
  if (tid == 0) {
    if (write) offsets[E] = total;
    s_off[E] = S;
    s_cnt[E] = n_shared ? T : 0;
    if (write && total != S) status_set(status, MOE_STATUS_BAD_INDEX);
  }
  __syncthreads();
  if (!write) return;  // only the offsets are needed

  // block map: blocks per group, scanned into each group's first block.
  // Thread g scans group g (g < 1024); with 1024 routed experts and a shared
  // expert there are 1025 groups, and the last one (the shared group, index
  // E = 1024) follows the scan: its first block is the scan's total.
  const int groups = E + (n_shared ? 1 : 0);
  const int scanned = min(groups, 1024);
  int nb = 0;
  if (tid < scanned) {
    const int c = s_cnt[tid];
    nb = (c + tile_m_max - 1) / tile_m_max;
  }
  int nb_total = 0;
  const int bstart = block_exclusive_scan(nb, tmp, &nb_total);
  if (tid < scanned) s_bstart[tid] = bstart;
  if (tid == 0) {
    for (int g = scanned; g < groups; ++g) {  // at most one group
      s_bstart[g] = nb_total;
      nb_total += (s_cnt[g] + tile_m_max - 1) / tile_m_max;
    }
    s_bstart[groups] = nb_total;
    if (nb_total > max_blocks) status_set(status, MOE_STATUS_BLOCK_OVERFLOW);
    *n_blocks = min(nb_total, max_blocks);
  }
  __syncthreads();
  nb_total = s_bstart[groups];  // thread 0 may have added the last group
  const int nwrite = min(nb_total, max_blocks);
  for (int b = tid; b < nwrite; b += 1024) {
    int lo = 0, hi = groups - 1;  // last group whose first block is <= b
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_bstart[mid] <= b) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int c = s_cnt[g];
    const int ng = s_bstart[g + 1] - s_bstart[g];
    const int i = b - s_bstart[g];
    const int bs = c / ng, rem = c % ng;
    const int rows = bs + (i < rem ? 1 : 0);
    const int first = (g < E ? s_off[g] : S) + i * bs + min(i, rem);
    const int tallest = bs + (rem > 0 ? 1 : 0);
    const int tm = (tallest + tile_gran - 1) / tile_gran * tile_gran;
    reinterpret_cast<int4*>(blocks)[b] = make_int4(g, first, rows, tm);
  }

}

// Tables for batches of at most 16 tokens (E <= 256), in one wave and with no
// workgroup barrier.  A group then holds at most 16 rows, never more than one
// tile (tile_m_max >= 16), so each non-empty expert has exactly one block and
// the shared group one.  Lane l owns experts 4l .. 4l+3; a single wave scan of
// (block count << 16 | row count) gives every expert's offset and block index
// (row counts total at most 16 * kMaxK, so the low half never carries).
__device__ void short_tables_wave(int T, int E, int k, int n_shared, int tile_gran,
                                  const uint32_t* s_bits, int* s_off,
                                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                  int32_t* __restrict__ blocks, int32_t* __restrict__ n_blocks,
                                  int max_blocks, uint32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int S = T * k;
  int c[4];
  int packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    c[i] = (e < E) ? __popc(s_bits[e]) : 0;
    packed += (c[i] > 0 ? (1 << 16) : 0) + c[i];
  }
  // inclusive wave scan on DPP: shifts by 1, 2, 4, 8 within each 16-lane
  // row (lanes shifted in from outside the row read 0), then each row's total
  // broadcast into the next rows (row_bcast:15 into rows 1 and 3, row_bcast:31
  // into rows 2 and 3)
  int inc = packed;
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x111, 0xF, 0xF, true);  // row_shr:1
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x112, 0xF, 0xF, true);  // row_shr:2
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x114, 0xF, 0xF, true);  // row_shr:4
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x118, 0xF, 0xF, true);  // row_shr:8
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x142, 0xA, 0xF, false);  // row_bcast:15
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x143, 0xC, 0xF, false);  // row_bcast:31
  const int tot = __builtin_amdgcn_readlane(inc, 63);
  const int total = tot & 0xFFFF, nb_routed = tot >> 16;
  int run = inc - packed;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    const int off = run & 0xFFFF, b = run >> 16;
    if (e < E) {
      counts[e] = c[i];
      offsets[e] = off;
      s_off[e] = off;
    }
    if (c[i] > 0 && b < max_blocks)
      reinterpret_cast<int4*>(blocks)[b] =
          make_int4(e, off, c[i], (c[i] + tile_gran - 1) / tile_gran * tile_gran);
    run += (c[i] > 0 ? (1 << 16) : 0) + c[i];
  }
  if (lane == 0) {
    const int nb_total = nb_routed + (n_shared ? 1 : 0);
    offsets[E] = total;
    s_off[E] = S;
    if (total != S) status_set(status, MOE_STATUS_BAD_INDEX);
    if (nb_total > max_blocks) status_set(status, MOE_STATUS_BLOCK_OVERFLOW);
    *n_blocks = min(nb_total, max_blocks);
    if (n_shared && nb_routed < max_blocks)
      reinterpret_cast<int4*>(blocks)[nb_routed] =
          make_int4(E, S, T, (T + tile_gran - 1) / tile_gran * tile_gran);
  }
}

constexpr int kScatterU = 16;  // slots per thread per scatter pass

__global__ __launch_bounds__(1024) void route_scan_kernel(
    int T, int E, int k, int n_shared, int tile_m_max, int tile_gran,
    const uint32_t* __restrict__ bits, int32_t* __restrict__ pref, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, const int32_t* __restrict__ topk_idx,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos, int32_t* __restrict__ blocks,
    int32_t* __restrict__ n_blocks, int max_blocks, uint32_t* __restrict__ status) {
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_bstart[kMaxE + 2];
  __shared__ int s_cnt[kMaxE + 1];
  __shared__ int s_part[1024];
  __shared__ int tmp[17];
  const int tid = threadIdx.x;
  const int S = T * k;
  const int W = (T + 31) / 32;

  // Per-expert prefix popcounts over the token words: thread (e, q) of the
  // tpe threads of expert e counts words [q*W/tpe, (q+1)*W/tpe).
  const int tpe = max(1, 1024 / E);
  const int e = tid % E, q = tid / E;
  const bool scanner = tid < E * tpe;
  const int w0 = scanner ? static_cast<int>(static_cast<long long>(q) * W / tpe) : 0;
  const int w1 = scanner ? static_cast<int>(static_cast<long long>(q + 1) * W / tpe) : 0;
  // words are read eight at a time with clamped indices, so each batch of
  // loads is in flight together
  int part = 0;
  for (int w = w0; w < w1; w += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = bits[static_cast<size_t>(min(w + u, w1 - 1)) * E + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) part += (w + u < w1) ? __popc(v[u]) : 0;
  }
  s_part[tid] = part;
  __syncthreads();
  int cnt = 0;
  if (scanner) {
    int base = 0;
    for (int p = 0; p < tpe; ++p) {
      const int v = s_part[p * E + e];
      if (p < q) base += v;
      cnt += v;
    }
    int run = base;
    for (int w = w0; w < w1; w += 8) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = bits[static_cast<size_t>(min(w + u, w1 - 1)) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (w + u < w1) {
          pref[static_cast<size_t>(w + u) * E + e] = run;
          run += __popc(v[u]);
        }
      }
    }
  }
  finish_tables(T, E, k, n_shared, tile_m_max, tile_gran, cnt, s_cnt, s_off, s_bstart, tmp, counts,
                offsets, blocks, n_blocks, max_blocks, status);

  // stable scatter: row = expert offset + tokens before t that chose e;
  // kScatterU slots per thread per pass, their loads issued together
  for (int s0 = tid; s0 < S; s0 += kScatterU * 1024) {
    int ex[kScatterU];
#pragma unroll
    for (int u = 0; u < kScatterU; ++u) ex[u] = topk_idx[min(s0 + u * 1024, S - 1)];
    uint32_t wbits[kScatterU];
    int wpref[kScatterU];
#pragma unroll
    for (int u = 0; u < kScatterU; ++u) {
      const int t = min(s0 + u * 1024, S - 1) / k;
      const int e = min(max(ex[u], 0), E - 1);
      const size_t wi = static_cast<size_t>(t >> 5) * E + e;
      wbits[u] = bits[wi];
      wpref[u] = pref[wi];
    }
#pragma unroll
    for (int u = 0; u < kScatterU; ++u) {
      const int s = s0 + u * 1024;
      if (s >= S) continue;
      if (ex[u] < 0 || ex[u] >= E) {
        status_set(status, MOE_STATUS_BAD_INDEX);
        continue;
      }
      const int t = s / k;
      const int pos = s_off[ex[u]] + wpref[u] + __popc(wbits[u] & ((1u << (t & 31)) - 1u));
      if (pos < 0 || pos >= S) {
        status_set(status, MOE_STATUS_BAD_INDEX);
        continue;
      }
      sorted_slot[pos] = s;
      slot_pos[s] = pos;
    }
  }
}

// ---------------------------------------------------------------------------
// K3 when the token bitmask fits in LDS (ceil(T/32) * E <= kScanLdsWords):
// the bitmask is read once, coalesced; the per-expert prefixes, the scan, the
// block map and the scatter ranks all come from LDS, and the slot experts for
// the scatter are loaded at the start, so the kernel makes two rounds of
// global loads instead of four.
// ---------------------------------------------------------------------------
constexpr int kScanLdsWords = 16384;
constexpr int kScanLoads = kScanLdsWords / 1024;

__global__ __launch_bounds__(1024) void route_scan_lds_kernel(
    int T, int E, int k, int n_shared, int tile_m_max, int tile_gran,
    const uint32_t* __restrict__ bits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, const int32_t* __restrict__ topk_idx,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos, int32_t* __restrict__ blocks,
    int32_t* __restrict__ n_blocks, int max_blocks, uint32_t* __restrict__ status) {
  __shared__ uint32_t s_bits[kScanLdsWords];  // [word][expert]
  __shared__ int s_pref[kScanLdsWords];       // tokens before each word, per expert
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_bstart[kMaxE + 2];
  __shared__ int s_cnt[kMaxE + 1];
  __shared__ int s_part[1024];
  __shared__ int tmp[17];
  const int tid = threadIdx.x;
  const int S = T * k;
  const int W = (T + 31) / 32;
  const int nw = W * E;
  // Every workgroup builds the same prefixes and offsets from the bitmask;
  // workgroup 0 writes the tables, and each scatters its own range of slots.
  const int slo = static_cast<int>(static_cast<long long>(blockIdx.x) * S / gridDim.x);
  const int shi = static_cast<int>(static_cast<long long>(blockIdx.x + 1) * S / gridDim.x);

  // the first scatter round's slot experts, then the whole bitmask
  // (only the rounds this launch needs: the conditions are uniform, so no
  // wave issues a load whose every lane would be clamped)
  int ex[kScatterU];
#pragma unroll
  for (int u = 0; u < kScatterU; ++u)
    ex[u] = (slo + u * 1024 < shi) ? topk_idx[min(slo + tid + u * 1024, S - 1)] : 0;
  uint32_t bv[kScanLoads];
#pragma unroll
  for (int u = 0; u < kScanLoads; ++u) bv[u] = (u * 1024 < nw) ? bits[min(tid + u * 1024, nw - 1)] : 0u;
#pragma unroll
  for (int u = 0; u < kScanLoads; ++u)
    if (tid + u * 1024 < nw) s_bits[tid + u * 1024] = bv[u];
  __syncthreads();

  // per-expert prefix popcounts: thread (e, q) of the tpe threads of expert e
  // covers words [q*W/tpe, (q+1)*W/tpe)
  const int tpe = max(1, 1024 / E);
  const int e = tid % E, q = tid / E;
  const bool scanner = tid < E * tpe;
  const int w0 = scanner ? q * W / tpe : 0;
  const int w1 = scanner ? (q + 1) * W / tpe : 0;
  int part = 0;
  for (int w = w0; w < w1; ++w) part += __popc(s_bits[w * E + e]);
  s_part[tid] = part;
  __syncthreads();
  int cnt = 0;
  if (scanner) {
    int base = 0;
    for (int p = 0; p < tpe; ++p) {
      const int v = s_part[p * E + e];
      if (p < q) base += v;
      cnt += v;
    }
    int run = base;
    for (int w = w0; w < w1; ++w) {
      s_pref[w * E + e] = run;
      run += __popc(s_bits[w * E + e]);
    }
  }
  finish_tables(T, E, k, n_shared, tile_m_max, tile_gran, cnt, s_cnt, s_off, s_bstart, tmp, counts,
                offsets, blocks, n_blocks, max_blocks, status, blockIdx.x == 0);
  __syncthreads();  // s_pref complete

  // stable scatter: row = expert offset + tokens before t that chose e
  for (int s0 = slo + tid; s0 < shi; s0 += kScatterU * 1024) {
    if (s0 != slo + tid) {
#pragma unroll
      for (int u = 0; u < kScatterU; ++u) ex[u] = topk_idx[min(s0 + u * 1024, S - 1)];
    }
#pragma unroll
    for (int u = 0; u < kScatterU; ++u) {
      const int sl = s0 + u * 1024;
      if (sl >= shi) continue;
      if (ex[u] < 0 || ex[u] >= E) {
        status_set(status, MOE_STATUS_BAD_INDEX);
        continue;
      }
      const int t = sl / k;
      const int wi = (t >> 5) * E + ex[u];
      const int pos = s_off[ex[u]] + s_pref[wi] + __popc(s_bits[wi] & ((1u << (t & 31)) - 1u));
      if (pos < 0 || pos >= S) {
        status_set(status, MOE_STATUS_BAD_INDEX);
        continue;
      }
      sorted_slot[pos] = sl;
      slot_pos[sl] = pos;
    }
  }
}

// ---------------------------------------------------------------------------
// K2+K3 for short batches (T <= 16): one workgroup does the top-k of every
// token (one wave a token), the histogram and ranks from a per-expert token
// bitmask kept in LDS, the scan, the block map and the scatter, with no
// global round trip in between.
// ---------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(1024) void route_short_kernel(
    int T, int E, int k, int n_shared, int tile_m_max, int tile_gran,
    const float* __restrict__ part, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ blocks, int32_t* __restrict__ n_blocks,
    int max_blocks, uint32_t* __restrict__ status) {
  __shared__ uint32_t s_bits[kMaxE];         // bit t: token t selected expert e
  __shared__ int s_sel[kShortT * kMaxK];     // expert of slot t*k + j
  __shared__ int s_off[16 * VPL + 1];
  __shared__ float s_logit[kShortT * 16 * VPL];
  const int tid = threadIdx.x;
  const int S = T * k;
  for (int e = tid; e < E; e += 1024) s_bits[e] = 0u;
  // scores from the class sums of router_partials_short_kernel (exported too)
  for (int i = tid; i < T * E; i += 1024) {
    const float l = score_from_classes(part, T, E, i / E, i % E, bias);
    s_logit[i] = l;
    logits[i] = l;
  }
  __syncthreads();
  if ((tid >> 6) < T) {  // one wave per token (wave-uniform): the waves past T only wait
    const int t = tid >> 6, r = tid & 63;
    const int se = topk_wave<VPL / 4>(T, E, k, s_logit, t, topk_idx, topk_w, status);
    if (se >= 0) {
      s_sel[t * k + r] = se;
      atomicOr(&s_bits[se], 1u << t);
    }
  }
  __syncthreads();
  if (tid < 64)
    short_tables_wave(T, E, k, n_shared, tile_gran, s_bits, s_off, counts, offsets, blocks,
                      n_blocks, max_blocks, status);
  __syncthreads();
  // stable scatter: row = expert offset + tokens before t that chose e
  for (int sl = tid; sl < S; sl += 1024) {
    const int t = sl / k, e = s_sel[sl];
    const int pos = s_off[e] + __popc(s_bits[e] & ((1u << t) - 1u));
    sorted_slot[pos] = sl;
    slot_pos[sl] = pos;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_route(const moe_dims& d, const uint16_t* x, const float* wr, const float* bias,
                        const RouteBuffers& rb, hipStream_t stream) {
  const int T = d.T, E = d.E, k = d.k;
  const int nbits = ((T + 31) / 32) * E;
  // 16-byte router loads only when every row start is 16-byte aligned
  const int vec_wr = (E % 4 == 0) && (reinterpret_cast<uintptr_t>(wr) % 16 == 0);
  if (T <= kShortT && E <= 256) {  // decode-sized batches: class sums, then one workgroup
    const dim3 g((E + 15) / 16 * kClasses);
#define MOE_PART(TT)                                                                              \
  hipLaunchKernelGGL(router_partials_short_kernel<TT>, g, dim3(128), 0, stream, T, d.H, E, x, wr, \
                     rb.part, rb.status)
    if (T <= 1) MOE_PART(1);
    else if (T <= 2) MOE_PART(2);
    else if (T <= 4) MOE_PART(4);
    else if (T <= 8) MOE_PART(8);
    else MOE_PART(16);
#undef MOE_PART
    hipLaunchKernelGGL((route_short_kernel<16>), dim3(1), dim3(1024), 0, stream, T, E, k,
                       d.n_shared, d.tile_m_max, d.tile_gran, rb.part, bias, rb.logits,
                       rb.topk_idx, rb.topk_w, rb.counts, rb.offsets, rb.sorted_slot, rb.slot_pos,
                       rb.blocks, rb.n_blocks, rb.max_blocks, rb.status);
    return hipGetLastError();
  }
  if (T <= kShortT) {  // decode-sized batches with more experts: spread over the router matrix
    const dim3 g((E + 15) / 16);
#define MOE_SHORT(TT)                                                                      \
  hipLaunchKernelGGL(router_scores_short_kernel<TT>, g, dim3(1024), 0, stream, T, d.H, E, x, wr, \
                     bias, rb.logits, rb.bits, nbits, rb.status)
    if (T <= 1) MOE_SHORT(1);
    else if (T <= 2) MOE_SHORT(2);
    else if (T <= 4) MOE_SHORT(4);
    else if (T <= 8) MOE_SHORT(8);
    else MOE_SHORT(16);
#undef MOE_SHORT
  } else if (T >= 1024) {  // 32 x 32 tiles, 16 waves
    const dim3 g1((T + 31) / 32, (E + 31) / 32);
    if (vec_wr)
      hipLaunchKernelGGL((router_scores_kernel<4, 4, 2, true>), g1, dim3(1024), 0, stream, T,
                         d.H, E, x, wr, bias, rb.logits, rb.bits, nbits, rb.status);
    else
      hipLaunchKernelGGL((router_scores_kernel<4, 4, 2, false>), g1, dim3(1024), 0, stream, T,
                         d.H, E, x, wr, bias, rb.logits, rb.bits, nbits, rb.status);
  } else {  // 16 x 16 tiles, 4 waves: more workgroups for short batches
    const dim3 g1((T + 15) / 16, (E + 15) / 16);
    if (vec_wr)
      hipLaunchKernelGGL((router_scores_kernel<2, 2, 4, true>), g1, dim3(256), 0, stream, T,
                         d.H, E, x, wr, bias, rb.logits, rb.bits, nbits, rb.status);
    else
      hipLaunchKernelGGL((router_scores_kernel<2, 2, 4, false>), g1, dim3(256), 0, stream, T,
                         d.H, E, x, wr, bias, rb.logits, rb.bits, nbits, rb.status);
  }
  const dim3 g2((T + 3) / 4);
  if (E <= 256)
    hipLaunchKernelGGL((router_topk_kernel<4>), g2, dim3(256), 0, stream, T, E, k, rb.logits,
                       rb.topk_idx, rb.topk_w, rb.bits, rb.status);
  else
    hipLaunchKernelGGL((router_topk_kernel<16>), g2, dim3(256), 0, stream, T, E, k, rb.logits,
                       rb.topk_idx, rb.topk_w, rb.bits, rb.status);
  if (static_cast<long long>((T + 31) / 32) * E <= kScanLdsWords) {
    // the scatter spread over up to eight workgroups (one per 2048 slots)
    const int gs = max(1, min(8, T * k / 2048));
    hipLaunchKernelGGL(route_scan_lds_kernel, dim3(gs), dim3(1024), 0, stream, T, E, k, d.n_shared,
                       d.tile_m_max, d.tile_gran, rb.bits, rb.counts, rb.offsets, rb.topk_idx,
                       rb.sorted_slot, rb.slot_pos, rb.blocks, rb.n_blocks, rb.max_blocks,
                       rb.status);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, T, E, k, d.n_shared,
                     d.tile_m_max, d.tile_gran, rb.bits, rb.pref, rb.counts, rb.offsets,
                     rb.topk_idx, rb.sorted_slot, rb.slot_pos, rb.blocks, rb.n_blocks,
                     rb.max_blocks, rb.status);
  return hipGetLastError();
}

}  // namespace moe
