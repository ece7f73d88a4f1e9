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
// Evaluation order: both dot products of token t use the state before its
// update, and the output is formed as o = alpha (s.q) + c (k.q) with
// c = beta (v[j] - alpha (s.k)), which equals (alpha s + c k).q.  The two
// reductions are then independent, so they interleave; k.q is one dot
// product per token, shared by every row of the head.
#include "route.h"
#include "gdn_scan.h"

namespace moe {
namespace {

constexpr int kD = 128;                   // dk = dv
constexpr int kC = 32;                    // tokens per staged chunk
constexpr int kR = 8;                     // state elements per lane
constexpr int kL = kD / kR;               // lanes per state row: one DPP row
constexpr int kRowsPerWave = 64 / kL;     // 4
constexpr int kWaves = 4;
constexpr int kRows = kRowsPerWave * kWaves;  // 16 rows per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBlocks = kD / kRows;    // 8 workgroups per head

static_assert(kC * kD / 8 == 2 * kThreads, "k and q chunks: two 16-byte loads per thread");
static_assert(kC * kRows / 8 == 64, "v chunk: one 16-byte load per lane of wave 0");

struct Meta {
  float alpha, beta, kq, pad;
};

__device__ __attribute__((aligned(16))) const float kZeros[kR] = {};

struct Stage {
  float k[kC][kD];
  float q[kC][kD];
  float v[kC][kRows];
  Meta meta[kC];
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
// piece of v (token lane/2, rows 8*(lane%2) .. +7 of the workgroup) and one
// float of g (lanes 0..31, token lane) or beta (lanes 32..63, token lane-32);
// only wave 0's v and wave 1's g and beta are stored.  The loads carry no
// condition (addresses are clamped into the sequence), so no branch separates
// them from the token loop and its waits stay exact.
struct ChunkRegs {
  uint4 k[2], q[2];
  uint4 v;
  float gb;
};

__device__ __forceinline__ void load_chunk(ChunkRegs& cr, int t0, int T, int Hk, int Hv, int kh,
                                           int h, int row0, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const float* __restrict__ g,
                                           const float* __restrict__ beta) {
  const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int seg = tid + u * kThreads;
    const int t = min(t0 + seg / 16, T - 1);  // past T: a valid token, never used
    const size_t off = (static_cast<size_t>(t) * Hk + kh) * kD + (seg % 16) * 8;
    cr.k[u] = *reinterpret_cast<const uint4*>(k + off);
    cr.q[u] = *reinterpret_cast<const uint4*>(q + off);
  }
  const int tv = min(t0 + lane / 2, T - 1);
  cr.v = *reinterpret_cast<const uint4*>(v + (static_cast<size_t>(tv) * Hv + h) * kD + row0 +
                                         (lane % 2) * 8);
  const int tg = min(t0 + (lane % 32), T - 1);
  const float* src = lane < 32 ? g : beta;
  cr.gb = src[static_cast<size_t>(tg) * Hv + h];
}

__device__ __forceinline__ void store_chunk(const ChunkRegs& cr, Stage& st) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int seg = tid + u * kThreads;
    const int t = seg / 16, e0 = (seg % 16) * 8;
    float kf[8], qf[8];
    widen8(cr.k[u], kf);
    widen8(cr.q[u], qf);
    float kq = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) kq = __builtin_fmaf(kf[e], qf[e], kq);
    // the 16 pieces of token t sit in the 16 lanes of one DPP row
    kq = sum16(kq);
    *reinterpret_cast<float4*>(&st.k[t][e0]) = make_float4(kf[0], kf[1], kf[2], kf[3]);
    *reinterpret_cast<float4*>(&st.k[t][e0 + 4]) = make_float4(kf[4], kf[5], kf[6], kf[7]);
    *reinterpret_cast<float4*>(&st.q[t][e0]) = make_float4(qf[0], qf[1], qf[2], qf[3]);
    *reinterpret_cast<float4*>(&st.q[t][e0 + 4]) = make_float4(qf[4], qf[5], qf[6], qf[7]);
    if ((seg % 16) == 0) st.meta[t].kq = kq;
  }
  if (wave == 0) {
    float vf[8];
    widen8(cr.v, vf);
    const int t = lane / 2, r0 = (lane % 2) * 8;
    *reinterpret_cast<float4*>(&st.v[t][r0]) = make_float4(vf[0], vf[1], vf[2], vf[3]);
    *reinterpret_cast<float4*>(&st.v[t][r0 + 4]) = make_float4(vf[4], vf[5], vf[6], vf[7]);
  } else if (wave == 1) {
    const int t = lane % 32;
    if (lane < 32)
      st.meta[t].alpha = expf(cr.gb);
    else
      st.meta[t].beta = cr.gb;
  }
}

// One token through the lane's 8 state elements of row r: both dot products
// on the state before the update, one reduction each over the row's 16 lanes,
// then the update.  Lane u of the row keeps the token's output in oreg.
__device__ __forceinline__ void token_step(const Stage& st, int t, int u, int sub, int r, float* s,
                                           float& oreg) {
  const float4 k0 = *reinterpret_cast<const float4*>(&st.k[t][sub * kR]);
  const float4 k1 = *reinterpret_cast<const float4*>(&st.k[t][sub * kR + 4]);
  const float4 q0 = *reinterpret_cast<const float4*>(&st.q[t][sub * kR]);
  const float4 q1 = *reinterpret_cast<const float4*>(&st.q[t][sub * kR + 4]);
  const float kv[kR] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
  const float qv[kR] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  float a = 0.0f, b = 0.0f;
#pragma unroll
  for (int e = 0; e < kR; ++e) {
    a = __builtin_fmaf(s[e], kv[e], a);
    b = __builtin_fmaf(s[e], qv[e], b);
  }
  a = sum16(a);
  b = sum16(b);
  const Meta mt = st.meta[t];
  const float cf = mt.beta * (st.v[t][r] - mt.alpha * a);
  const float out = __builtin_fmaf(mt.alpha, b, cf * mt.kq);
#pragma unroll
  for (int e = 0; e < kR; ++e) s[e] = __builtin_fmaf(cf, kv[e], mt.alpha * s[e]);
  oreg = (sub == u) ? out : oreg;
}

// s_waitcnt immediate (gfx9 encoding) that waits for every vector memory load:
// vmcnt 0, expcnt 7 and lgkmcnt 15 (no wait on those).
constexpr int kWaitAllVmem = 0x0F70;

__global__ __launch_bounds__(kThreads) void gdn_scan_kernel(
    int T, int Hk, int Hv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    const float* state_in, float* state_out, uint16_t* __restrict__ o) {
  __shared__ Stage stage[2];
  __shared__ float obuf[2][kC][kRows];

  // Workgroup -> (head, row block).  The hardware deals workgroups to the 8
  // XCDs round-robin; when the heads divide evenly, the 8 row blocks of a head
  // land on one XCD and share its L2 for the head's k and q.
  const int wg = blockIdx.x;
  int h, rb;
  if (Hv % 8 == 0) {
    const int xcd = wg % 8, slot = wg / 8;
    rb = slot % kRowBlocks;
    h = (slot / kRowBlocks) * 8 + xcd;
  } else {
    h = wg / kRowBlocks;
    rb = wg % kRowBlocks;
  }
  const int kh = h / (Hv / Hk);
  const int row0 = rb * kRows;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rw = lane / kL, sub = lane % kL;
  const int r = wave * kRowsPerWave + rw;
  const size_t srow = (static_cast<size_t>(h) * kD + row0 + r) * kD + sub * kR;

  // Initial state, loaded without a branch (a null state_in reads zeros), so
  // that no merge point leaves these loads pending into the token loop.
  // (A global-address-space pointer: a generic one would make these flat
  // loads, which the compiler must then wait for on every LDS read.)
  typedef const f32x4 __attribute__((address_space(1)))* gf4;
  const gf4 s_src = (gf4)(state_in ? state_in + srow : kZeros);
  const f32x4 s_lo = s_src[0];
  const f32x4 s_hi = s_src[1];
  float s[kR] = {s_lo.x, s_lo.y, s_lo.z, s_lo.w, s_hi.x, s_hi.y, s_hi.z, s_hi.w};

  const int nchunks = (T + kC - 1) / kC;
  ChunkRegs cr;
  if (nchunks > 0) {
    load_chunk(cr, 0, T, Hk, Hv, kh, h, row0, q, k, v, g, beta);
    store_chunk(cr, stage[0]);
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
    if (c + 1 < nchunks) load_chunk(cr, t0 + kC, T, Hk, Hv, kh, h, row0, q, k, v, g, beta);

    const Stage& st = stage[c & 1];
    // Tokens in runs of 16: lane sub keeps the output of token tb + sub (a
    // select, not a branch), and the run's outputs go to LDS in one store.
    for (int tb = 0; tb < n; tb += kL) {
      float oreg = 0.0f;
      if (n - tb >= kL) {
#pragma unroll
        for (int u = 0; u < kL; ++u) token_step(st, tb + u, u, sub, r, s, oreg);
      } else {
        for (int u = 0; u < n - tb; ++u) token_step(st, tb + u, u, sub, r, s, oreg);
      }
      obuf[c & 1][tb + sub][r] = oreg;  // entries past n are never written out
    }

    if (c + 1 < nchunks) store_chunk(cr, stage[(c + 1) & 1]);
    __syncthreads();

    // outputs of the chunk: token tid/8, rows 2*(tid%8) and +1 as one bf16 pair
    {
      const int t = tid / 8, p = tid % 8;
      if (t < n) {
        const uint32_t pr = pack_bf16x2(obuf[c & 1][t][2 * p], obuf[c & 1][t][2 * p + 1]);
        *reinterpret_cast<uint32_t*>(o + (static_cast<size_t>(t0 + t) * Hv + h) * kD + row0 + 2 * p) = pr;
      }
    }
  }

  if (state_out) {
    *reinterpret_cast<float4*>(state_out + srow) = make_float4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<float4*>(state_out + srow + 4) = make_float4(s[4], s[5], s[6], s[7]);
  }
}

}  // namespace

hipError_t launch_gdn_scan(int T, int n_k_heads, int n_v_heads, const uint16_t* q,
                          const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                          const float* state_in, float* state_out, uint16_t* o, hipStream_t stream) {
  hipLaunchKernelGGL(gdn_scan_kernel, dim3(static_cast<unsigned>(n_v_heads * kRowBlocks)),
                     dim3(kThreads), 0, stream, T, n_k_heads, n_v_heads, q, k, v, g, beta,
                     state_in, state_out, o);
  return hipGetLastError();
}

}  // namespace moe

namespace {
bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
}  // namespace

extern "C" int gdn_scan(const gdn_dims* d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* g, const float* beta, const float* state_in, float* state_out,
                        uint16_t* o, void* stream) {
  if (!d) return MOE_EINVAL;
  if (d->dk != 128 || d->dv != 128) return MOE_EINVAL;
  if (d->T < 0 || d->T > (1 << 24)) return MOE_EINVAL;
  if (d->n_k_heads < 1 || d->n_v_heads < d->n_k_heads || d->n_v_heads > 1024 ||
      d->n_v_heads % d->n_k_heads)
    return MOE_EINVAL;
  if (d->T > 0 && (!q || !k || !v || !g || !beta || !o)) return MOE_EINVAL;
  if ((q && !aligned_to(q, 16)) || (k && !aligned_to(k, 16)) || (v && !aligned_to(v, 16)) ||
      (o && !aligned_to(o, 16)) || (g && !aligned_to(g, 4)) || (beta && !aligned_to(beta, 4)) ||
      (state_in && !aligned_to(state_in, 16)) || (state_out && !aligned_to(state_out, 16)))
    return MOE_EALIGN;
  if (d->T == 0 && !state_out) return MOE_OK;
  int rc = moe::check_device();
  if (rc) return rc;
  (void)hipGetLastError();
  const hipError_t e = moe::launch_gdn_scan(d->T, d->n_k_heads, d->n_v_heads, q, k, v, g, beta,
                                            state_in, state_out, o, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
