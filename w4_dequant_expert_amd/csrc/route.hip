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
//   K2 top-k and weights, 16 lanes per token with DPP row reductions; every
//      selection sets its token's bit in a [token word][expert] bitmask with
//      an atomic OR (order-independent, hence deterministic);
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

template <int WT, int WE, int CH>
__global__ __launch_bounds__(WT * WE * 64) void router_scores_kernel(
    int T, int H, int E, int vec_wr, const uint16_t* __restrict__ x, const float* __restrict__ wr,
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
  float4 wrg[WI];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      // consecutive lanes take consecutive tokens, so the transposed LDS
      // writes below fall in different banks
      const int idx = tid + i * NT;
      const int t = idx % RT, part = idx / RT;
      const int c = part / 8, m = (part % 8) * 8;
      const int gt = t0 + t, hc = c0 + c;
      xr[i] = make_uint4(0, 0, 0, 0);
      if (idx < XN && gt < T && hc < nchunk)
        xr[i] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(gt) * H + hc * 64 + m);
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / (RE / 4), col = (idx % (RE / 4)) * 4;
      const int c = row / 64, m = row % 64;
      const int h = (c0 + c) * 64 + m;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (idx < WN && c0 + c < nchunk) {
        const float* src = wr + static_cast<size_t>(h) * E + e0 + col;
        if (vec_wr && e0 + col + 3 < E) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          if (e0 + col + 0 < E) v.x = src[0];
          if (e0 + col + 1 < E) v.y = src[1];
          if (e0 + col + 2 < E) v.z = src[2];
          if (e0 + col + 3 < E) v.w = src[3];
        }
      }
      wrg[i] = v;
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int idx = tid + i * NT;
      if (idx < XN) {
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
      if (idx < WN) {
        const int row = idx / (RE / 4), col = (idx % (RE / 4)) * 4;
        *reinterpret_cast<float4*>(&ws[row / 64][row % 64][col]) = wrg[i];
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
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
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
// K2: top-k and weights.  A token is served by one 16-lane row of a wave
// (four tokens per wave); lane r holds the scores of experts r, r+16, r+32...
// Each of the k rounds takes the lane-local best unselected expert and reduces
// across the row with four DPP exchanges (row mirror, half-row mirror, quad
// swaps by 2 and by 1, which pair every lane with every other through the
// butterfly), ordering by higher score and then lower expert index.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& be) {
  const float ov = __int_as_float(dpp<CTRL>(__float_as_int(bv)));
  const int oe = dpp<CTRL>(be);
  if (better(ov, oe, bv, be)) {
    bv = ov;
    be = oe;
  }
}

template <int CTRL>
__device__ __forceinline__ float sum_step(float v) {
  return v + __int_as_float(dpp<CTRL>(__float_as_int(v)));
}

constexpr int kRowMirror = 0x140, kHalfMirror = 0x141;
constexpr int kQuadSwap2 = 0x4E, kQuadSwap1 = 0xB1;  // quad_perm [2,3,0,1] and [1,0,3,2]

template <int VPL>  // scores per lane: E <= 16 * VPL
__global__ __launch_bounds__(256) void router_topk_kernel(int T, int E, int k,
                                                          const float* __restrict__ logits,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          uint32_t* __restrict__ bits,
                                                          uint32_t* __restrict__ status) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = lane & 15;
  const int t = blockIdx.x * 16 + (tid >> 4);
  const bool tok_ok = t < T;
  const int tt = tok_ok ? t : 0;  // rows past T work on token 0 and store nothing

  float val[VPL];
  bool saw_nan = false;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = r + 16 * v;
    float s = -INFINITY;
    if (e < E) {
      s = logits[static_cast<size_t>(tt) * E + e];
      if (s != s) {
        saw_nan = true;
        s = -INFINITY;
      }
    }
    val[v] = s;
  }
  uint64_t taken = 0;
  float sel_v[2] = {-INFINITY, -INFINITY};  // selections r and r + 16 of this token
  int sel_e[2] = {0, 0};
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = r + 16 * v;
      if (e < E && !((taken >> v) & 1ull) && better(val[v], e, bv, be)) {
        bv = val[v];
        be = e;
      }
    }
    argmax_step<kRowMirror>(bv, be);
    argmax_step<kHalfMirror>(bv, be);
    argmax_step<kQuadSwap2>(bv, be);
    argmax_step<kQuadSwap1>(bv, be);
    if ((be & 15) == r) taken |= 1ull << (be >> 4);
    if (j == r) {
      sel_v[0] = bv;
      sel_e[0] = be;
    }
    if (j == r + 16) {
      sel_v[1] = bv;
      sel_e[1] = be;
    }
  }
  // weights: exp(l_j - l_max) / sum over the selected (the softmax
  // denominator over all experts cancels in the renormalisation)
  const float top = __int_as_float(__shfl(__float_as_int(sel_v[0]), lane & ~15, 64));
  float ex[2];
  float den = 0.0f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = r + 16 * q;
    ex[q] = (j < k) ? __expf(sel_v[q] - top) : 0.0f;
    den += ex[q];
  }
  den = sum_step<kRowMirror>(den);
  den = sum_step<kHalfMirror>(den);
  den = sum_step<kQuadSwap2>(den);
  den = sum_step<kQuadSwap1>(den);
  if (tok_ok) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = r + 16 * q;
      if (j < k) {
        topk_idx[static_cast<size_t>(t) * k + j] = sel_e[q];
        topk_w[static_cast<size_t>(t) * k + j] = ex[q] / den;
        atomicOr(&bits[static_cast<size_t>(t >> 5) * E + sel_e[q]], 1u << (t & 31));
      }
    }
  }
  if (saw_nan && tok_ok) status_set(status, MOE_STATUS_NAN_LOGIT);
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
  int part = 0;
  for (int w = w0; w < w1; ++w) part += __popc(bits[static_cast<size_t>(w) * E + e]);
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
      pref[static_cast<size_t>(w) * E + e] = run;
      run += __popc(bits[static_cast<size_t>(w) * E + e]);
    }
  }
  int total = 0;
  const int off = block_exclusive_scan((tid < E) ? cnt : 0, tmp, &total);
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = off;
    s_off[tid] = off;
    s_cnt[tid] = cnt;
  }
  if (tid == 0) {
    offsets[E] = total;
    s_off[E] = S;
    s_cnt[E] = n_shared ? T : 0;
    if (total != S) status_set(status, MOE_STATUS_BAD_INDEX);
  }
  __syncthreads();

  // block map: blocks per group, scanned into each group's first block
  const int groups = E + (n_shared ? 1 : 0);
  int nb = 0;
  if (tid < groups) {
    const int c = s_cnt[tid];
    nb = (c + tile_m_max - 1) / tile_m_max;
  }
  int nb_total = 0;
  const int bstart = block_exclusive_scan(nb, tmp, &nb_total);
  if (tid < groups) s_bstart[tid] = bstart;
  if (tid == 0) {
    s_bstart[groups] = nb_total;
    if (nb_total > max_blocks) status_set(status, MOE_STATUS_BLOCK_OVERFLOW);
    *n_blocks = min(nb_total, max_blocks);
  }
  __syncthreads();
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

  // stable scatter: row = expert offset + tokens before t that chose e; four
  // slots per thread per pass so their loads overlap
  for (int s0 = tid; s0 < S; s0 += 4 * 1024) {
    int ex[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + u * 1024;
      ex[u] = (s < S) ? topk_idx[s] : 0;
    }
    uint32_t wbits[4];
    int wpref[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + u * 1024;
      const int t = (s < S) ? s / k : 0;
      const int e = min(max(ex[u], 0), E - 1);
      const size_t wi = static_cast<size_t>(t >> 5) * E + e;
      wbits[u] = bits[wi];
      wpref[u] = pref[wi];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
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
hipError_t launch_route(const moe_dims& d, const uint16_t* x, const float* wr, const float* bias,
                        const RouteBuffers& rb, hipStream_t stream) {
  const int T = d.T, E = d.E, k = d.k;
  const int nbits = ((T + 31) / 32) * E;
  // 16-byte router loads only when every row start is 16-byte aligned
  const int vec_wr = (E % 4 == 0) && (reinterpret_cast<uintptr_t>(wr) % 16 == 0);
  if (T >= 1024) {  // 32 x 32 tiles, 16 waves
    const dim3 g1((T + 31) / 32, (E + 31) / 32);
    hipLaunchKernelGGL((router_scores_kernel<4, 4, 2>), g1, dim3(1024), 0, stream, T, d.H, E,
                       vec_wr, x, wr, bias, rb.logits, rb.bits, nbits, rb.status);
  } else {  // 16 x 16 tiles, 4 waves: more workgroups for short batches
    const dim3 g1((T + 15) / 16, (E + 15) / 16);
    hipLaunchKernelGGL((router_scores_kernel<2, 2, 4>), g1, dim3(256), 0, stream, T, d.H, E,
                       vec_wr, x, wr, bias, rb.logits, rb.bits, nbits, rb.status);
  }
  const dim3 g2((T + 15) / 16);
  if (E <= 256)
    hipLaunchKernelGGL((router_topk_kernel<16>), g2, dim3(256), 0, stream, T, E, k, rb.logits,
                       rb.topk_idx, rb.topk_w, rb.bits, rb.status);
  else
    hipLaunchKernelGGL((router_topk_kernel<64>), g2, dim3(256), 0, stream, T, E, k, rb.logits,
                       rb.topk_idx, rb.topk_w, rb.bits, rb.status);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, T, E, k, d.n_shared,
                     d.tile_m_max, d.tile_gran, rb.bits, rb.pref, rb.counts, rb.offsets,
                     rb.topk_idx, rb.sorted_slot, rb.slot_pos, rb.blocks, rb.n_blocks,
                     rb.max_blocks, rb.status);
  return hipGetLastError();
}

}  // namespace moe
