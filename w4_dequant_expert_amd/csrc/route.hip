// GPU-resident routing for the MoE expert layer on gfx950: router scores,
// top-k with renormalised softmax weights, per-workgroup histograms with
// wavefront ballot ranks, one exclusive scan, the stable scatter and the tile
// block map.  Everything stays on the device: the grouped GEMMs read the block
// map and its length from memory, so nothing returns to the host between the
// router and the GEMMs ["Lily Beats MLX-LM 1.35x on Decode", "Prefill: fusing
// dequantisation and keeping routing GPU-resident"].
#include "route.h"

#include <float.h>
#include <math.h>

namespace moe {

// ---------------------------------------------------------------------------
// K1: router scores.  Workgroup tile: kRT tokens x kRE experts, 16 waves of
// 8 tokens x 8 experts.  Within a wave, lane m owns partial m of every one of
// its 64 outputs: a float32 fma chain over inputs h = m, m+64, m+128, ...  The
// 64 partials of each output are then combined by a transposed butterfly over
// the lanes whose pairing is exactly the tree p[i] += p[i+s], s = 32..1, so
// every score has one fixed, host-reproducible evaluation order.  x and the
// router weights are staged through LDS in chunks of kCH x 64 inputs.
// ---------------------------------------------------------------------------
constexpr int kTW = 8, kEW = 8;         // per-lane tile
constexpr int kWT = 4, kWE = 4;         // waves per workgroup (tokens x experts)
constexpr int kRT = kTW * kWT;          // 32 tokens per workgroup
constexpr int kRE = kEW * kWE;          // 32 experts per workgroup
constexpr int kCH = 2;                  // 64-input chunks per LDS stage
constexpr int kPadT = kRT + 4, kPadE = kRE + 4;

__global__ __launch_bounds__(1024) void router_scores_kernel(int T, int H, int E, int vec_wr,
                                                             const uint16_t* __restrict__ x,
                                                             const float* __restrict__ wr,
                                                             const float* __restrict__ bias,
                                                             float* __restrict__ logits,
                                                             uint32_t* __restrict__ status) {
  __shared__ float xs[kCH][64][kPadT];  // x chunk, transposed: [input][token]
  __shared__ float ws[kCH][64][kPadE];  // router chunk: [input][expert]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wt = wave % kWT, we = wave / kWT;
  const int t0 = blockIdx.x * kRT, e0 = blockIdx.y * kRE;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0 && status) *status = 0u;

  float acc[kTW * kEW];
#pragma unroll
  for (int o = 0; o < kTW * kEW; ++o) acc[o] = 0.0f;

  const int nchunk = H / 64;
  for (int c0 = 0; c0 < nchunk; c0 += kCH) {
    __syncthreads();
    for (int idx = tid; idx < kRT * kCH * 8; idx += 1024) {  // stage x, 8 bf16 per load
      const int t = idx / (kCH * 8), part = idx % (kCH * 8);
      const int c = part / 8, m = (part % 8) * 8;
      const int gt = t0 + t, hc = c0 + c;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gt < T && hc < nchunk)
        v = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(gt) * H + hc * 64 + m);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[c][m + 2 * i][t] = bf16_to_f32(wv[i] & 0xFFFFu);
        xs[c][m + 2 * i + 1][t] = bf16_to_f32(wv[i] >> 16);
      }
    }
    for (int idx = tid; idx < kCH * 64 * (kRE / 4); idx += 1024) {  // stage router weights
      const int row = idx / (kRE / 4), col = (idx % (kRE / 4)) * 4;
      const int c = row / 64, m = row % 64;
      const int h = (c0 + c) * 64 + m;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + c < nchunk) {
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
      *reinterpret_cast<float4*>(&ws[c][m][col]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kCH; ++c) {
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
// K2: top-k, weights, and the workgroup's histogram with stable local ranks.
// One wave selects for one token at a time: k rounds of a butterfly arg-max
// over the token's scores (higher score first, equal scores by lower expert).
// Then the workgroup's <= 256 slots are ranked within their expert in slot
// order: a ballot per expert-index bit finds the lanes of a wave that chose
// the same expert, popcount below the lane gives the rank inside the wave,
// and the waves add their counts to an LDS histogram one after another.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

__global__ __launch_bounds__(256) void router_topk_kernel(
    int T, int E, int k, int tpb, const float* __restrict__ logits, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ local_rank, int32_t* __restrict__ partial,
    uint32_t* __restrict__ status) {
  __shared__ int sel[256];
  __shared__ int hist[kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tbase = blockIdx.x * tpb;
  for (int e = tid; e < E; e += 256) hist[e] = 0;

  const int nc = (E + 63) / 64;
  bool saw_nan = false;
  for (int tt = wave; tt < tpb; tt += 4) {
    const int t = tbase + tt;
    if (t >= T) break;
    float val[kMaxE / 64];
#pragma unroll
    for (int c = 0; c < kMaxE / 64; ++c) {
      const int e = lane + 64 * c;
      float v = -INFINITY;
      if (c < nc && e < E) {
        v = logits[static_cast<size_t>(t) * E + e];
        if (v != v) {
          saw_nan = true;
          v = -INFINITY;
        }
      }
      val[c] = v;
    }
    uint32_t taken = 0;
    float my_v = -INFINITY;  // score of selection number `lane`
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int c = 0; c < kMaxE / 64; ++c) {
        const int e = lane + 64 * c;
        if (c < nc && e < E && !((taken >> c) & 1u) && better(val[c], e, bv, be)) {
          bv = val[c];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oe = __shfl_xor(be, off, 64);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (lane == j) my_v = bv;
      if (lane == 0) {
        sel[tt * k + j] = be;
        topk_idx[static_cast<size_t>(t) * k + j] = be;
      }
    }
    // weights: exp(l_j - l_max) / sum over the selected (the softmax
    // denominator over all experts cancels in the renormalisation)
    const float top = __shfl(my_v, 0, 64);
    float ex = (lane < k) ? __expf(my_v - top) : 0.0f;
    float den = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);
    if (lane < k) topk_w[static_cast<size_t>(t) * k + lane] = ex / den;
  }
  if (saw_nan) status_set(status, MOE_STATUS_NAN_LOGIT);
  __syncthreads();

  const int nslot = min(tpb, T - tbase) * k;
  const bool valid = tid < nslot;
  const int e = valid ? sel[tid] : 0;
  uint64_t match = __ballot(valid);
  for (int b = 0; (1 << b) < E; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    match &= bit ? bb : ~bb;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank_in_wave = __popcll(match & below);
  const int cnt_in_wave = __popcll(match);
  int rank = 0;
  for (int w = 0; w < 4; ++w) {
    if (wave == w && valid) rank = hist[e] + rank_in_wave;
    __syncthreads();
    if (wave == w && valid && rank_in_wave == 0) hist[e] += cnt_in_wave;
    __syncthreads();
  }
  if (valid) local_rank[static_cast<size_t>(tbase) * k + tid] = rank;
  for (int x = tid; x < E; x += 256) partial[static_cast<size_t>(blockIdx.x) * E + x] = hist[x];
}

// ---------------------------------------------------------------------------
// K3: one workgroup: per-expert totals and per-(workgroup, expert) bases, the
// exclusive scan into offsets, the block map, and the stable scatter.
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
    int T, int E, int k, int n_shared, int tile_m_max, int tile_gran, int nwg, int tpb,
    int32_t* __restrict__ partial, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ local_rank,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos, int32_t* __restrict__ blocks,
    int32_t* __restrict__ n_blocks, int max_blocks, uint32_t* __restrict__ status) {
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_bstart[kMaxE + 2];
  __shared__ int s_cnt[kMaxE + 1];
  __shared__ int tmp[17];
  const int tid = threadIdx.x;
  const int S = T * k;

  // per expert: running sum over the routing workgroups (in workgroup order)
  int cnt = 0;
  if (tid < E) {
    int g = 0;
    for (; g + 4 <= nwg; g += 4) {
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = partial[static_cast<size_t>(g + u) * E + tid];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        partial[static_cast<size_t>(g + u) * E + tid] = cnt;
        cnt += c[u];
      }
    }
    for (; g < nwg; ++g) {
      const int c = partial[static_cast<size_t>(g) * E + tid];
      partial[static_cast<size_t>(g) * E + tid] = cnt;
      cnt += c;
    }
  }
  int total = 0;
  const int off = block_exclusive_scan(tid < E ? cnt : 0, tmp, &total);
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
    const int base = c / ng, rem = c % ng;
    const int rows = base + (i < rem ? 1 : 0);
    const int first = (g < E ? s_off[g] : S) + i * base + min(i, rem);
    const int tallest = base + (rem > 0 ? 1 : 0);
    const int tm = (tallest + tile_gran - 1) / tile_gran * tile_gran;
    reinterpret_cast<int4*>(blocks)[b] = make_int4(g, first, rows, tm);
  }

  // stable scatter: row = offset of the expert + slots of earlier routing
  // workgroups + rank inside this slot's workgroup
  for (int s = tid; s < S; s += 1024) {
    const int e = topk_idx[s];
    if (e < 0 || e >= E) {
      status_set(status, MOE_STATUS_BAD_INDEX);
      continue;
    }
    const int g = (s / k) / tpb;
    const int pos = s_off[e] + partial[static_cast<size_t>(g) * E + e] + local_rank[s];
    if (pos < 0 || pos >= S) {
      status_set(status, MOE_STATUS_BAD_INDEX);
      continue;
    }
    sorted_slot[pos] = s;
    slot_pos[s] = pos;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_route(const moe_dims& d, const uint16_t* x, const float* wr, const float* bias,
                        const RouteBuffers& rb, hipStream_t stream) {
  const int T = d.T, E = d.E, k = d.k;
  dim3 g1((T + kRT - 1) / kRT, (E + kRE - 1) / kRE);
  // 16-byte router loads only when every row start is 16-byte aligned
  const int vec_wr = (E % 4 == 0) && (reinterpret_cast<uintptr_t>(wr) % 16 == 0);
  hipLaunchKernelGGL(router_scores_kernel, g1, dim3(1024), 0, stream, T, d.H, E, vec_wr, x, wr,
                     bias, rb.logits, rb.status);
  const int tpb = route_tokens_per_wg(k);
  const int nwg = (T + tpb - 1) / tpb;
  hipLaunchKernelGGL(router_topk_kernel, dim3(nwg), dim3(256), 0, stream, T, E, k, tpb,
                     rb.logits, rb.topk_idx, rb.topk_w, rb.local_rank, rb.partial, rb.status);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, T, E, k, d.n_shared,
                     d.tile_m_max, d.tile_gran, nwg, tpb, rb.partial, rb.counts, rb.offsets,
                     rb.topk_idx, rb.local_rank, rb.sorted_slot, rb.slot_pos, rb.blocks,
                     rb.n_blocks, rb.max_blocks, rb.status);
  return hipGetLastError();
}

}  // namespace moe
