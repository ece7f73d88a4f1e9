// Gated DeltaNet recurrent scan for gfx950 with the state in registers.
//
// ["Lily Beats MLX-LM 1.35x on Decode", "Prefill: fusing dequantisation and
// keeping routing GPU-resident"]: the recurrent state of a Gated DeltaNet
// layer stays on chip for the whole scan, each simdgroup carrying one column
// of it, instead of an intermediate of 256 MiB per layer going through memory.
// The recurrence is the gated delta rule (Yang, Kautz, Hatamizadeh, ICLR
// 2025); per value head, with state rows s_j (value dimension j, length dk):
//     a_t = s_j . k_t
//     s_j <- alpha_t s_j + beta_t (v_t[j] - alpha_t a_t) k_t
//     o_t[j] = s_j . q_t
// which is row j of S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
// and o_t = S_t q_t.  Rows are independent: only dot products over dk couple
// the elements of one row.
//
// Mapping on gfx950: a state row is spread over one 16-lane DPP row of a wave
// (8 float32 elements per lane), so a wave carries 4 rows and both dot
// products of a token reduce with four DPP adds and no LDS.  A workgroup of
// four waves carries 16 rows of one head; 32 heads x 128 rows fill 256
// workgroups, one per compute unit.  The inputs of a head (k, q, and for the
// workgroup's rows v, with alpha = exp(g), beta and k.q per token) are staged
// in LDS in chunks of 32 tokens, widened to float32 once, double-buffered:
// the next chunk's global loads are issued before the current chunk's tokens
// run.  The state is read once at the start and written once at the end.
//
// Evaluation order: tokens go in pairs, both read from the state before the
// pair (pair_step below): four dot products of the state (with k and q of both
// tokens), four independent reductions, a few scalar operations with the
// head's per-token products (k.q, and k_t.k_{t+1}, k_t.q_{t+1} across the
// pair), then one update of the state for both tokens.  The products of k and
// q are one dot product each per token, shared by every row of the head, and
// are formed while the chunk is staged.
#include "route.h"
#include "gdn_scan.h"

namespace moe {
namespace {

constexpr int kD = 128;                   // dk = dv
constexpr int kC = 32;                    // tokens per staged chunk
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

static_assert(kC * kD / 8 == 2 * kThreads, "k and q chunks: two 16-byte loads per thread");

// Layout of the state over a workgroup, for R float32 elements per lane: a
// state row spreads over L = 128 / R lanes (one DPP row of 16 at R = 8, two
// at R = 4), a wave carries 64 / L rows, a workgroup of four waves Rows rows,
// and a head takes RowBlocks workgroups.
template <int R>
struct Cfg {
  static constexpr int L = kD / R;
  static constexpr int RowsPerWave = 64 / L;
  static constexpr int Rows = RowsPerWave * kWaves;
  static constexpr int RowBlocks = kD / Rows;
  static constexpr int VPieces = Rows / 8;  // 16-byte pieces of v per token
  static_assert(R % 4 == 0 && (L == 16 || L == 32), "a state row spans one or two DPP rows");
  static_assert(kC * VPieces <= 64, "v chunk: at most one 16-byte load per lane of wave 0");
};

// Per-token scalars of a head, shared by all its rows, one 32-byte record per
// token pair (t, t+1), t even: alpha_t = exp(g_t), beta_t, k_t.q_t,
// k_t.k_{t+1}, k_t.q_{t+1}, alpha_{t+1}, beta_{t+1}, k_{t+1}.q_{t+1}.  A pair
// reads its record with two 16-byte reads and uses every value.
struct PairMeta {
  float v[8];
};

// Where token t's alpha, beta and k.q start in its pair's record.
__device__ __forceinline__ int meta_slot(int t) { return (t & 1) ? 5 : 0; }

__device__ __attribute__((aligned(16))) const float kZeros[8] = {};

// v is stored by state row, so a token pair is one 8-byte read; rows are
// padded by two floats so the rows of one wave fall in different banks.
constexpr int kVPitch = kC + 2;

template <int ROWS>
struct Stage {
  float k[kC][kD];
  float q[kC][kD];
  float v[ROWS][kVPitch];
  PairMeta meta[kC / 2];
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row, the same bits in every lane (each step
// adds two equal-order partial sums, and addition commutes).
__device__ __forceinline__ float sum16(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

// Sum over the L lanes of a state row.  For two DPP rows, one
// v_permlane16_swap of x with itself leaves row 2i's sums in one result and
// row 2i+1's in the other, in every lane of both rows.
template <int L>
__device__ __forceinline__ float row_sum(float x) {
  x = sum16(x);
  if constexpr (L == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

__device__ __forceinline__ void widen8(uint4 w, float* f) {
  f[0] = __uint_as_float(w.x << 16);
  f[1] = __uint_as_float(w.x & 0xFFFF0000u);
  f[2] = __uint_as_float(w.y << 16);
  f[3] = __uint_as_float(w.y & 0xFFFF0000u);
  f[4] = __uint_as_float(w.z << 16);
  f[5] = __uint_as_float(w.z & 0xFFFF0000u);
  f[6] = __uint_as_float(w.w << 16);
  f[7] = __uint_as_float(w.w & 0xFFFF0000u);
}

// Global loads of one chunk, held in registers until the chunk's LDS buffer
// is free.  Every thread loads two 16-byte pieces of k and the same two of q
// (tokens tid/16 and 16 + tid/16, elements 8*(tid%16) .. +7), one 16-byte
// piece of v (wave 0 lane l < 32 * VPieces: token l / VPieces, rows
// 8 * (l % VPieces) .. +7 of the workgroup) and one float of g (lanes 0..31,
// token lane) or beta (lanes 32..63, token lane-32); only wave 0's v and
// wave 1's g and beta are stored.  The loads carry no condition (addresses are
// clamped into the sequence), so no branch separates them from the token loop
// and its waits stay exact.
struct ChunkRegs {
  uint4 k[2], q[2];
  uint4 v;
  float gb;
};

template <int R>
__device__ __forceinline__ void load_chunk(ChunkRegs& cr, int t0, int T, int Hk, int Hv, int kh,
                                           int h, int row0, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const float* __restrict__ g,
                                           const float* __restrict__ beta) {
  constexpr int P = Cfg<R>::VPieces;
  const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int seg = tid + u * kThreads;
    const int t = min(t0 + seg / 16, T - 1);  // past T: a valid token, never used
    const size_t off = (static_cast<size_t>(t) * Hk + kh) * kD + (seg % 16) * 8;
    cr.k[u] = *reinterpret_cast<const uint4*>(k + off);
    cr.q[u] = *reinterpret_cast<const uint4*>(q + off);
  }
  const int lv = lane % (kC * P);
  const int tv = min(t0 + lv / P, T - 1);
  cr.v = *reinterpret_cast<const uint4*>(v + (static_cast<size_t>(tv) * Hv + h) * kD + row0 +
                                         (lv % P) * 8);
  const int tg = min(t0 + (lane % 32), T - 1);
  const float* src = lane < 32 ? g : beta;
  cr.gb = src[static_cast<size_t>(tg) * Hv + h];
}

template <int R>
__device__ __forceinline__ void store_chunk(const ChunkRegs& cr, Stage<Cfg<R>::Rows>& st) {
  constexpr int P = Cfg<R>::VPieces;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int seg = tid + u * kThreads;
    const int t = seg / 16, e0 = (seg % 16) * 8;
    float kf[8], qf[8];
    widen8(cr.k[u], kf);
    widen8(cr.q[u], qf);
    // Token t's partner in the pair step, t ^ 1, sits 16 lanes away.
    float kq = 0.0f, kk1 = 0.0f, kq1 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kn = __shfl_xor(kf[e], 16, 64);
      const float qn = __shfl_xor(qf[e], 16, 64);
      kq = __builtin_fmaf(kf[e], qf[e], kq);
      kk1 = __builtin_fmaf(kf[e], kn, kk1);
      kq1 = __builtin_fmaf(kf[e], qn, kq1);
    }
    // the 16 pieces of token t sit in the 16 lanes of one DPP row
    kq = sum16(kq);
    kk1 = sum16(kk1);
    kq1 = sum16(kq1);
    *reinterpret_cast<float4*>(&st.k[t][e0]) = make_float4(kf[0], kf[1], kf[2], kf[3]);
    *reinterpret_cast<float4*>(&st.k[t][e0 + 4]) = make_float4(kf[4], kf[5], kf[6], kf[7]);
    *reinterpret_cast<float4*>(&st.q[t][e0]) = make_float4(qf[0], qf[1], qf[2], qf[3]);
    *reinterpret_cast<float4*>(&st.q[t][e0 + 4]) = make_float4(qf[4], qf[5], qf[6], qf[7]);
    if ((seg % 16) == 0) {
      float* m = st.meta[t / 2].v;
      m[meta_slot(t) + 2] = kq;
      if ((t & 1) == 0) {  // k_t.k_{t+1} and k_t.q_{t+1} for the pair (t, t+1)
        m[3] = kk1;
        m[4] = kq1;
      }
    }
  }
  if (wave == 0 && lane < kC * P) {
    float vf[8];
    widen8(cr.v, vf);
    const int t = lane / P, r0 = (lane % P) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.v[r0 + i][t] = vf[i];
  } else if (wave == 1) {
    const int t = lane % 32;
    float* m = st.meta[t / 2].v + meta_slot(t);
    if (lane < 32)
      m[0] = expf(cr.gb);
    else
      m[1] = cr.gb;
  }
}

// Which elements of a state row a lane holds: R/4 groups of four, group i
// being elements 4 L i + 4 sub .. +3.  One 16-byte LDS read of group i by the
// L lanes of a row then covers 4 L consecutive floats, free of bank conflicts.
template <int R>
__device__ __forceinline__ int elem_base(int i, int sub) {
  return 4 * Cfg<R>::L * i + 4 * sub;
}

template <int R>
__device__ __forceinline__ void load_row(float* dst, const float* row, int sub) {
#pragma unroll
  for (int i = 0; i < R / 4; ++i) {
    const float4 a = *reinterpret_cast<const float4*>(row + elem_base<R>(i, sub));
    dst[4 * i] = a.x;
    dst[4 * i + 1] = a.y;
    dst[4 * i + 2] = a.z;
    dst[4 * i + 3] = a.w;
  }
}

// One token through the lane's R state elements of row r: both dot products
// on the state before the update, one reduction each over the row's lanes,
// then the update.  Lane u of the row keeps the token's output in oreg.
template <int R>
__device__ __forceinline__ void token_step(const Stage<Cfg<R>::Rows>& st, int t, int u, int sub,
                                           int r, float* s, float& oreg) {
  float kv[R], qv[R];
  load_row<R>(kv, st.k[t], sub);
  load_row<R>(qv, st.q[t], sub);
  float a = 0.0f, b = 0.0f;
#pragma unroll
  for (int e = 0; e < R; ++e) {
    a = __builtin_fmaf(s[e], kv[e], a);
    b = __builtin_fmaf(s[e], qv[e], b);
  }
  a = row_sum<Cfg<R>::L>(a);
  b = row_sum<Cfg<R>::L>(b);
  // t is even here (a run's odd last token): alpha_t, beta_t, k_t.q_t, k_t.k_{t+1}
  const float4 mt = *reinterpret_cast<const float4*>(st.meta[t / 2].v);
  const float cf = mt.y * (st.v[r][t] - mt.x * a);
  const float out = __builtin_fmaf(mt.x, b, cf * mt.z);
#pragma unroll
  for (int e = 0; e < R; ++e) s[e] = __builtin_fmaf(cf, kv[e], mt.x * s[e]);
  oreg = (sub == u) ? out : oreg;
}

// Operands of a token pair (t, t+1) for one lane: its k and q elements of both
// tokens, both v of its row and the head's per-token scalars.
template <int R>
struct PairOps {
  float k1[R], q1[R], k2[R], q2[R];
  float2 v;
  float4 m1, m2;  // the pair's record
};

template <int R>
__device__ __forceinline__ void load_pair(PairOps<R>& p, const Stage<Cfg<R>::Rows>& st, int t,
                                          int sub, int r) {
  load_row<R>(p.k1, st.k[t], sub);
  load_row<R>(p.q1, st.q[t], sub);
  load_row<R>(p.k2, st.k[t + 1], sub);
  load_row<R>(p.q2, st.q[t + 1], sub);
  p.v = *reinterpret_cast<const float2*>(&st.v[r][t]);
  p.m1 = *reinterpret_cast<const float4*>(st.meta[t / 2].v);
  p.m2 = *reinterpret_cast<const float4*>(st.meta[t / 2].v + 4);
}

// Two tokens from one read of the state s (before both updates).  With the
// state's dot products against k_t, q_t, k_{t+1} and q_{t+1}, the head's
// scalars k_t.q_t, k_t.k_{t+1}, k_t.q_{t+1} and k_{t+1}.q_{t+1} give both
// tokens exactly as two single steps would (up to rounding):
//   c1 = beta1 (v1 - alpha1 s.k1),            o1 = alpha1 s.q1 + c1 k1.q1
//   s1.k2 = alpha1 s.k2 + c1 k1.k2,           s1.q2 = alpha1 s.q2 + c1 k1.q2
//   c2 = beta2 (v2 - alpha2 s1.k2),           o2 = alpha2 s1.q2 + c2 k2.q2
//   s <- alpha1 alpha2 s + alpha2 c1 k1 + c2 k2
// Four independent dot products and reductions instead of two dependent
// pairs, and three operations per state element for two tokens instead of four.
template <int R>
__device__ __forceinline__ void pair_step(const PairOps<R>& p, int u, int sub, float* s,
                                          float& oreg) {
  float a1 = 0.0f, b1 = 0.0f, a2 = 0.0f, b2 = 0.0f;
#pragma unroll
  for (int e = 0; e < R; ++e) {
    a1 = __builtin_fmaf(s[e], p.k1[e], a1);
    b1 = __builtin_fmaf(s[e], p.q1[e], b1);
    a2 = __builtin_fmaf(s[e], p.k2[e], a2);
    b2 = __builtin_fmaf(s[e], p.q2[e], b2);
  }
  a1 = row_sum<Cfg<R>::L>(a1);
  b1 = row_sum<Cfg<R>::L>(b1);
  a2 = row_sum<Cfg<R>::L>(a2);
  b2 = row_sum<Cfg<R>::L>(b2);
  const float al1 = p.m1.x, be1 = p.m1.y, kq11 = p.m1.z, kk12 = p.m1.w, kq12 = p.m2.x;
  const float al2 = p.m2.y, be2 = p.m2.z, kq22 = p.m2.w;
  const float c1 = be1 * (p.v.x - al1 * a1);
  const float o1 = __builtin_fmaf(al1, b1, c1 * kq11);
  const float s1k2 = __builtin_fmaf(al1, a2, c1 * kk12);
  const float s1q2 = __builtin_fmaf(al1, b2, c1 * kq12);
  const float c2 = be2 * (p.v.y - al2 * s1k2);
  const float o2 = __builtin_fmaf(al2, s1q2, c2 * kq22);
  const float dec = al1 * al2, w1 = al2 * c1;
#pragma unroll
  for (int e = 0; e < R; ++e)
    s[e] = __builtin_fmaf(c2, p.k2[e], __builtin_fmaf(w1, p.k1[e], dec * s[e]));
  oreg = (sub == u) ? o1 : oreg;
  oreg = (sub == u + 1) ? o2 : oreg;
}

// s_waitcnt immediate (gfx9 encoding) that waits for every vector memory load:
// vmcnt 0, expcnt 7 and lgkmcnt 15 (no wait on those).
constexpr int kWaitAllVmem = 0x0F70;

template <int R>
__global__ __launch_bounds__(kThreads) void gdn_scan_kernel(
    int T, int Hk, int Hv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    const float* state_in, float* state_out, uint16_t* __restrict__ o) {
  using C = Cfg<R>;
  constexpr int L = C::L, ROWS = C::Rows;
  __shared__ Stage<ROWS> stage[2];
  __shared__ float obuf[2][kC][ROWS];

  // Workgroup -> (head, row block).  The hardware deals workgroups to the 8
  // XCDs round-robin; when the heads divide evenly, the row blocks of a head
  // land on one XCD and share its L2 for the head's k and q.
  const int wg = blockIdx.x;
  int h, rb;
  if (Hv % 8 == 0) {
    const int xcd = wg % 8, slot = wg / 8;
    rb = slot % C::RowBlocks;
    h = (slot / C::RowBlocks) * 8 + xcd;
  } else {
    h = wg / C::RowBlocks;
    rb = wg % C::RowBlocks;
  }
  const int kh = h / (Hv / Hk);
  const int row0 = rb * ROWS;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rw = lane / L, sub = lane % L;
  const int r = wave * C::RowsPerWave + rw;
  const size_t srow = (static_cast<size_t>(h) * kD + row0 + r) * kD;   // state row r

  // Initial state, loaded without a branch (a null state_in reads zeros), so
  // that no merge point leaves these loads pending into the token loop.
  // (A global-address-space pointer: a generic one would make these flat
  // loads, which the compiler must then wait for on every LDS read.)
  typedef const f32x4 __attribute__((address_space(1)))* gf4;
  float s[R];
#pragma unroll
  for (int i = 0; i < R / 4; ++i) {
    const gf4 src = (gf4)(state_in ? state_in + srow + elem_base<R>(i, sub) : kZeros);
    const f32x4 a = *src;
    s[4 * i] = a.x;
    s[4 * i + 1] = a.y;
    s[4 * i + 2] = a.z;
    s[4 * i + 3] = a.w;
  }

  const int nchunks = (T + kC - 1) / kC;
  ChunkRegs cr;
  if (nchunks > 0) {
    load_chunk<R>(cr, 0, T, Hk, Hv, kh, h, row0, q, k, v, g, beta);
    store_chunk<R>(cr, stage[0]);
  }
  // The initial state and the first chunk are in registers or LDS from here
  // on; said explicitly, since the compiler's wait tracking loses count across
  // the branches above and would otherwise wait for every load in flight
  // inside the token loop.
  __builtin_amdgcn_s_waitcnt(kWaitAllVmem);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * kC;
    const int n = min(kC, T - t0);
    if (c + 1 < nchunks) load_chunk<R>(cr, t0 + kC, T, Hk, Hv, kh, h, row0, q, k, v, g, beta);

    const Stage<ROWS>& st = stage[c & 1];
    // Tokens in runs of L: lane sub keeps the output of token tb + sub (a
    // select, not a branch), and the run's outputs go to LDS in one store.
    for (int tb = 0; tb < n; tb += L) {
      float oreg = 0.0f;
      if (n - tb >= L) {
        // L/2 pairs; the next pair's operands are read from LDS while the
        // current pair computes
        PairOps<R> cur, nxt;
        load_pair<R>(cur, st, tb, sub, r);
#pragma unroll
        for (int pr = 0; pr < L / 2; ++pr) {
          if (pr + 1 < L / 2) load_pair<R>(nxt, st, tb + 2 * pr + 2, sub, r);
          pair_step<R>(cur, 2 * pr, sub, s, oreg);
          if (pr + 1 < L / 2) cur = nxt;
        }
      } else {
        const int m = n - tb;
        int u = 0;
        for (; u + 1 < m; u += 2) {
          PairOps<R> p;
          load_pair<R>(p, st, tb + u, sub, r);
          pair_step<R>(p, u, sub, s, oreg);
        }
        if (u < m) token_step<R>(st, tb + u, u, sub, r, s, oreg);
      }
      obuf[c & 1][tb + sub][r] = oreg;  // entries past n are never written out
    }

    if (c + 1 < nchunks) store_chunk<R>(cr, stage[(c + 1) & 1]);
    __syncthreads();

    // outputs of the chunk: token tid / (ROWS/2), rows 2 * (tid % (ROWS/2))
    // and +1 as one bf16 pair
    {
      constexpr int PP = ROWS / 2;
      const int t = tid / PP, p = tid % PP;
      if (t < n) {
        const uint32_t pr = pack_bf16x2(obuf[c & 1][t][2 * p], obuf[c & 1][t][2 * p + 1]);
        *reinterpret_cast<uint32_t*>(o + (static_cast<size_t>(t0 + t) * Hv + h) * kD + row0 + 2 * p) = pr;
      }
    }
  }

  if (state_out) {
#pragma unroll
    for (int i = 0; i < R / 4; ++i)
      *reinterpret_cast<float4*>(state_out + srow + elem_base<R>(i, sub)) =
          make_float4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
  }
}

// Elements per lane of the shipped layout.
constexpr int kShipR = 8;

}  // namespace

hipError_t launch_gdn_scan(int T, int n_k_heads, int n_v_heads, const uint16_t* q,
                          const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                          const float* state_in, float* state_out, uint16_t* o, hipStream_t stream) {
  hipLaunchKernelGGL(gdn_scan_kernel<kShipR>,
                     dim3(static_cast<unsigned>(n_v_heads * Cfg<kShipR>::RowBlocks)), dim3(kThreads),
                     0, stream, T, n_k_heads, n_v_heads, q, k, v, g, beta, state_in, state_out, o);
  return hipGetLastError();
}

}  // namespace moe

namespace {
bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int validate_gdn_dims(const gdn_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->dk != 128 || d->dv != 128) return MOE_EINVAL;
  if (d->T < 0 || d->T > (1 << 24)) return MOE_EINVAL;
  if (d->n_k_heads < 1 || d->n_v_heads < d->n_k_heads || d->n_v_heads > 1024 ||
      d->n_v_heads % d->n_k_heads)
    return MOE_EINVAL;
  return MOE_OK;
}

int validate_gdn(const gdn_dims* d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const float* g, const float* beta, const float* state_in, const float* state_out,
                 const uint16_t* o) {
  int rc = validate_gdn_dims(d);
  if (rc) return rc;
  if (d->T > 0 && (!q || !k || !v || !g || !beta || !o)) return MOE_EINVAL;
  if ((q && !aligned_to(q, 16)) || (k && !aligned_to(k, 16)) || (v && !aligned_to(v, 16)) ||
      (o && !aligned_to(o, 16)) || (g && !aligned_to(g, 4)) || (beta && !aligned_to(beta, 4)) ||
      (state_in && !aligned_to(state_in, 16)) || (state_out && !aligned_to(state_out, 16)))
    return MOE_EALIGN;
  return MOE_OK;
}
}  // namespace

extern "C" int gdn_scan(const gdn_dims* d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* g, const float* beta, const float* state_in, float* state_out,
                        uint16_t* o, void* stream) {
  int rc = validate_gdn(d, q, k, v, g, beta, state_in, state_out, o);
  if (rc) return rc;
  if (d->T == 0 && !state_out) return MOE_OK;
  if ((rc = moe::check_device())) return rc;
  (void)hipGetLastError();
  const hipError_t e = moe::launch_gdn_scan(d->T, d->n_k_heads, d->n_v_heads, q, k, v, g, beta,
                                            state_in, state_out, o, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

extern "C" size_t gdn_scan_chunked_ws_bytes(const gdn_dims* d) {
  if (validate_gdn_dims(d)) return 0;
  return moe::gdn_chunked_ws_bytes(d->T, d->n_v_heads);
}

extern "C" int gdn_scan_chunked(const gdn_dims* d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const float* g, const float* beta,
                                const float* state_in, float* state_out, uint16_t* o, void* ws,
                                size_t ws_bytes, void* stream) {
  int rc = validate_gdn(d, q, k, v, g, beta, state_in, state_out, o);
  if (rc) return rc;
  const size_t need = moe::gdn_chunked_ws_bytes(d->T, d->n_v_heads);
  if (need && !ws) return MOE_EINVAL;
  if (ws && !aligned_to(ws, 256)) return MOE_EALIGN;
  if (ws_bytes < need) return MOE_EWS;
  if (d->T == 0 && !state_out) return MOE_OK;
  if ((rc = moe::check_device())) return rc;
  (void)hipGetLastError();
  const hipError_t e = moe::launch_gdn_scan_chunked(d->T, d->n_k_heads, d->n_v_heads, q, k, v, g,
                                                    beta, state_in, state_out, o,
                                                    static_cast<float*>(ws),
                                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
