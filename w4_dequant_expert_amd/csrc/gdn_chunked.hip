// Gated DeltaNet scan for gfx950 in chunked form, on the matrix cores.
//
// The same recurrence as gdn.hip (["Lily Beats MLX-LM 1.35x on Decode",
// "Prefill: fusing dequantisation and keeping routing GPU-resident"]; the
// gated delta rule of Yang, Kautz, Hatamizadeh, ICLR 2025), regrouped over
// chunks of C = 32 tokens the way the Gated DeltaNet paper parallelises it.
// Within a chunk, with G_t the running sum of g over the chunk's tokens,
// gamma_t = exp(G_t) and S_0 the state before the chunk:
//   A_ts  = beta_t exp(G_t - G_s) k_t.k_s  for s < t      (strictly lower)
//   T     = (I + A)^-1                                      (unit lower)
//   U     = T diag(beta) V - T diag(beta gamma) K S_0^T     (C x dv)
//   O     = diag(gamma) Q S_0^T + (M o Q K^T) U,  M_ts = exp(G_t - G_s), s <= t
//   S_C   = gamma_C S_0 + U^T diag(exp(G_C - G_t)) K
// where U's row t is beta_t (v_t - alpha_t S_{t-1} k_t), the vector by which
// token t writes k_t into the state.  Unrolling the token recurrence gives
// exactly these sums, so the result is the token-by-token scan up to rounding.
//
// Two kernels:
//   - gdn_chunk_prep_kernel, one workgroup per (value head, chunk), all in
//     parallel: everything that does not depend on the state (A, T, the
//     products T diag(beta gamma) K and T diag(beta), M o QK^T, the decays),
//     written to a caller-provided workspace;
//   - gdn_chunk_scan_kernel, one workgroup per (value head, 16 state rows):
//     the state rows stay in LDS for the whole sequence, and each chunk is
//     four products on the matrix cores (v_mfma_f32_16x16x4_f32, exact
//     float32 products with float32 sums).
// The state never goes through memory between chunks, as in the
// register-resident scan; the intermediates written are per chunk and
// independent of the state.
//
// MFMA operand layout (16x16x4, float32), verified on the device: lane l
// supplies A[l % 16][l / 16] and B[l / 16][l % 16] and receives
// D[4 (l / 16) + r][l % 16], r = 0..3.  Over the k steps of a product the
// four k positions of a step can be any four indices, as long as A and B
// agree; the kernels give lane group l / 16 a contiguous run of k so that each
// lane's operands are consecutive floats in LDS.
#include "route.h"
#include "gdn_scan.h"

namespace moe {
namespace {

constexpr int kCD = 128;         // dk = dv
constexpr int kCC = 32;          // tokens per chunk
constexpr int kCRows = 16;       // state rows per scan workgroup
constexpr int kCThreads = 256;
constexpr int kP = kCD + 4;      // LDS pitch of 128-wide rows (floats): 16 rows fall in 16 banks
constexpr int kPc = kCC + 1;     // LDS pitch of 32-wide rows

// Workspace record of one (value head, chunk), float32:
constexpr int kRecW = 0;                       // [32][128] T diag(beta gamma) K
constexpr int kRecB = kRecW + kCC * kCD;       // [32][32]  T diag(beta)
constexpr int kRecM = kRecB + kCC * kCC;       // [32][32]  M o Q K^T (lower, diagonal included)
constexpr int kRecGam = kRecM + kCC * kCC;     // [32]      gamma_t
constexpr int kRecDec = kRecGam + kCC;         // [32]      exp(G_last - G_t)
constexpr int kRecGC = kRecDec + kCC;          // [4]       gamma of the chunk's last token, 0, 0, 0
constexpr int kRecFloats = ((kRecGC + 4) + 63) / 64 * 64;   // 256-byte records

typedef float f32x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4c mfma4(float a, float b, f32x4c c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void widen8c(uint4 w, float* f) {
  f[0] = __uint_as_float(w.x << 16);
  f[1] = __uint_as_float(w.x & 0xFFFF0000u);
  f[2] = __uint_as_float(w.y << 16);
  f[3] = __uint_as_float(w.y & 0xFFFF0000u);
  f[4] = __uint_as_float(w.z << 16);
  f[5] = __uint_as_float(w.z & 0xFFFF0000u);
  f[6] = __uint_as_float(w.w << 16);
  f[7] = __uint_as_float(w.w & 0xFFFF0000u);
}

// Loads 4 N consecutive floats of LDS (16-byte aligned) into registers.
template <int N>
__device__ __forceinline__ void lds_row(float* dst, const float* src) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float4 a = reinterpret_cast<const float4*>(src)[i];
    dst[4 * i] = a.x;
    dst[4 * i + 1] = a.y;
    dst[4 * i + 2] = a.z;
    dst[4 * i + 3] = a.w;
  }
}

// 16 x 16 tile of X Y^T over 128 columns: lane l supplies X[l % 16][32 (l/16) + ks]
// and Y[l % 16][32 (l/16) + ks] from its rows; four independent accumulator
// chains keep the matrix core busy.
__device__ __forceinline__ f32x4c tile_xyT(const float* xrow, const float* yrow) {
  float xa[32], ya[32];
  lds_row<8>(xa, xrow);
  lds_row<8>(ya, yrow);
  f32x4c acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4c{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) acc[ks & 3] = mfma4(xa[ks], ya[ks], acc[ks & 3]);
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// 16 x 16 tile over 32 k: lane l supplies A[.][8 (l/16) + ks] and B from 8
// consecutive floats each; two chains.
__device__ __forceinline__ f32x4c tile_k32(const float* arow, const float* brow, f32x4c init) {
  float aa[8], bb[8];
  lds_row<2>(aa, arow);
  lds_row<2>(bb, brow);
  f32x4c acc0 = init, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 8; ks += 2) {
    acc0 = mfma4(aa[ks], bb[ks], acc0);
    acc1 = mfma4(aa[ks + 1], bb[ks + 1], acc1);
  }
  return acc0 + acc1;
}

constexpr int kPt = kCC + 4;     // LDS pitch of 32-wide rows read as 16-byte pieces

// ---------------------------------------------------------------------------
// Prep: one workgroup per (value head h, chunk c).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCThreads) void gdn_chunk_prep_kernel(
    int T, int Hk, int Hv, int nchunks, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const float* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float Ks[kCC][kP];
  __shared__ __attribute__((aligned(16))) float Qs[kCC][kP];
  __shared__ float KK[kCC][kPc];
  __shared__ float QK[kCC][kPc];
  __shared__ __attribute__((aligned(16))) float At[kCC][kPt];   // A transposed: At[s][t] = A_ts
  __shared__ __attribute__((aligned(16))) float Tm[kCC][kPt];
  __shared__ float Gs[kCC], Bs[kCC], BG[kCC];

  const int h = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
  const int kh = h / (Hv / Hk);
  const int t0 = c * kCC, n = min(kCC, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane % 16, gq = lane / 16;
  float* rec = ws + (static_cast<size_t>(h) * nchunks + c) * kRecFloats;

  // k and q rows of the chunk, float32; rows past the sequence are zero
  {
    const int t = tid / 8, e0 = (tid % 8) * 16;
    const bool ok = t < n;
    const size_t off = (static_cast<size_t>(t0 + (ok ? t : 0)) * Hk + kh) * kCD + e0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint4 wk = *reinterpret_cast<const uint4*>(k + off + 8 * u);
      uint4 wq = *reinterpret_cast<const uint4*>(q + off + 8 * u);
      if (!ok) wk = wq = make_uint4(0, 0, 0, 0);
      float fk[8], fq[8];
      widen8c(wk, fk);
      widen8c(wq, fq);
      float* kd = &Ks[t][e0 + 8 * u];
      float* qd = &Qs[t][e0 + 8 * u];
      reinterpret_cast<float4*>(kd)[0] = make_float4(fk[0], fk[1], fk[2], fk[3]);
      reinterpret_cast<float4*>(kd)[1] = make_float4(fk[4], fk[5], fk[6], fk[7]);
      reinterpret_cast<float4*>(qd)[0] = make_float4(fq[0], fq[1], fq[2], fq[3]);
      reinterpret_cast<float4*>(qd)[1] = make_float4(fq[4], fq[5], fq[6], fq[7]);
    }
  }
  if (tid < kCC) {
    const bool ok = tid < n;
    Gs[tid] = ok ? g[static_cast<size_t>(t0 + tid) * Hv + h] : 0.0f;
    Bs[tid] = ok ? beta[static_cast<size_t>(t0 + tid) * Hv + h] : 0.0f;
  }
  __syncthreads();
  if (tid == 0) {  // running sum of g, left to right
    float acc = 0.0f;
    for (int t = 0; t < kCC; ++t) {
      acc += Gs[t];
      Gs[t] = acc;
    }
  }

  // K K^T and Q K^T, lower block tiles (0,0), (1,0), (1,1) of each: wave w
  // takes tiles w and w + 4 of the six.
  for (int tile = wave; tile < 6; tile += 4) {
    const bool isq = tile >= 3;
    const int tt = tile % 3;
    const int I = tt == 0 ? 0 : 1, J = tt == 2 ? 1 : 0;
    const float* xrow = isq ? &Qs[I * 16 + i16][32 * gq] : &Ks[I * 16 + i16][32 * gq];
    const f32x4c acc = tile_xyT(xrow, &Ks[J * 16 + i16][32 * gq]);
    float (*dst)[kPc] = isq ? QK : KK;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[I * 16 + 4 * gq + r][J * 16 + i16] = acc[r];
  }
  __syncthreads();

  // A (strictly lower, stored transposed) and M o QK^T (lower with the diagonal)
  for (int e = tid; e < kCC * kCC; e += kCThreads) {
    const int t = e / kCC, s = e % kCC;
    const float d = (s <= t) ? expf(Gs[t] - Gs[s]) : 0.0f;
    At[s][t] = (s < t) ? Bs[t] * d * KK[t][s] : 0.0f;
    rec[kRecM + e] = (s <= t) ? d * QK[t][s] : 0.0f;
  }
  if (tid < kCC) BG[tid] = Bs[tid] * expf(Gs[tid]);
  __syncthreads();

  // T = (I + A)^-1 in 16 x 16 blocks: T11 = (I + A11)^-1, T22 = (I + A22)^-1
  // by forward substitution (lanes 0-15 of wave 0 one column of T11 each,
  // lanes 16-31 one of T22), right-looking: once x_t is final it is taken out
  // of every later row, p_u -= A_ut x_t, so the rows' updates are independent.
  // Then T21 = -T22 A21 T11 and T12 = 0.
  if (wave == 0 && lane < kCC) {
    const int base = lane < 16 ? 0 : 16, j = base + lane % 16;
    float p[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) p[u] = (base + u == j) ? 1.0f : 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float x = p[t];
      Tm[base + t][j] = x;
      float col[16];
      lds_row<4>(col, &At[base + t][base]);   // A_ut for the block's rows u (zero for u <= t)
#pragma unroll
      for (int u = t + 1; u < 16; ++u) p[u] = __builtin_fmaf(-col[u], x, p[u]);
    }
  }
  __syncthreads();
  {
    const int i = tid / 16, j = tid % 16;   // X = A21 T11, kept in KK
    float x = 0.0f;
#pragma unroll
    for (int s = 0; s < 16; ++s) x = __builtin_fmaf(At[s][16 + i], Tm[s][j], x);
    KK[i][j] = x;
  }
  __syncthreads();
  {
    const int i = tid / 16, j = tid % 16;   // T21 = -T22 X
    float y = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) y = __builtin_fmaf(Tm[16 + i][16 + kk], KK[kk][j], y);
    Tm[16 + i][j] = -y;
    Tm[i][16 + j] = 0.0f;
  }
  __syncthreads();

  // T diag(beta) to the record; gamma, the decays to the chunk's end
  const float Glast = Gs[kCC - 1];
  for (int e = tid; e < kCC * kCC; e += kCThreads) {
    const int t = e / kCC, s = e % kCC;
    rec[kRecB + e] = Tm[t][s] * Bs[s];
  }
  if (tid < kCC) {
    rec[kRecGam + tid] = expf(Gs[tid]);
    rec[kRecDec + tid] = expf(Glast - Gs[tid]);
  }
  if (tid == 0) {
    rec[kRecGC] = expf(Glast);
    rec[kRecGC + 1] = rec[kRecGC + 2] = rec[kRecGC + 3] = 0.0f;
  }

  // W = T diag(beta gamma) K: 2 x 8 tiles of 16 x 16, k = the chunk's tokens;
  // wave w takes output column tiles 2w and 2w+1 of both row tiles.
#pragma unroll
  for (int I = 0; I < 2; ++I) {
    float ta[8];
    lds_row<2>(ta, &Tm[I * 16 + i16][8 * gq]);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ta[ks] *= BG[8 * gq + ks];
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const int N = 2 * wave + nn;
      f32x4c acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 8; ks += 2) {
        acc0 = mfma4(ta[ks], Ks[8 * gq + ks][N * 16 + i16], acc0);
        acc1 = mfma4(ta[ks + 1], Ks[8 * gq + ks + 1][N * 16 + i16], acc1);
      }
      const f32x4c acc = acc0 + acc1;
#pragma unroll
      for (int r = 0; r < 4; ++r) rec[kRecW + (I * 16 + 4 * gq + r) * kCD + N * 16 + i16] = acc[r];
    }
  }
}

// ---------------------------------------------------------------------------
// Scan: one workgroup per (value head, 16 state rows); the rows stay in LDS.
// Operands sit in LDS so that each lane's k run is 16-byte pieces:
// W and Q by token (k = dk), K transposed and decayed (k = token), Bm and Mq
// by token (k = token), V transposed, U transposed.
// ---------------------------------------------------------------------------
struct __attribute__((aligned(16))) ChunkBuf {
  float W[kCC][kP];      // T diag(beta gamma) K
  float Q[kCC][kP];      // q rows, float32
  float KT[kCD][kPt];    // KT[i][t] = exp(G_last - G_t) k_t[i]
  float Bm[kCC][kPt];    // T diag(beta)
  float Mq[kCC][kPt];    // M o Q K^T
  float VT[kCRows][kPt]; // VT[j][t] = v_t[row0 + j]
  float gam[kCC];
  float gC[4];
};

constexpr int kSThreads = 512;   // scan workgroup: eight waves, two per SIMD

// Global loads of one chunk held in registers until the buffer is free.
// Thread tid: the record's W floats 8 tid .. +7; Bm and Mq floats 4 (tid % 256)
// .. +3 (threads < 256 Bm, the others Mq); q elements 8 (tid % 16) .. +7 of
// token tid / 16; k elements 8 (tid / 32) .. +7 of token tid % 32; threads
// < 32: v rows row0 .. +15 of token tid, gamma and the decay of token tid.
// (Clang vector types, not HIP's float4/uint4 classes: with those the
// compiler kept this struct in memory and placed it in LDS, a round trip
// through LDS for every staged value.)
typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));
struct ScanRegs {
  f32x4c w0, w1;
  f32x4c bmq;
  u32x4c q, k;
  u32x4c v0, v1;
  float gam, dec, gC;
};

__device__ __forceinline__ uint4 as_uint4(u32x4c a) { return make_uint4(a.x, a.y, a.z, a.w); }

__device__ __forceinline__ void scan_load(ScanRegs& R, const float* __restrict__ rec, int t0, int T,
                                          int Hk, int Hv, int kh, int h, int row0,
                                          const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ v) {
  const int tid = threadIdx.x;
  R.w0 = reinterpret_cast<const f32x4c*>(rec + kRecW + 8 * tid)[0];
  R.w1 = reinterpret_cast<const f32x4c*>(rec + kRecW + 8 * tid)[1];
  R.bmq = reinterpret_cast<const f32x4c*>(rec + (tid < 256 ? kRecB : kRecM))[tid % 256];
  {
    const int t = min(t0 + tid / 16, T - 1);
    R.q = *reinterpret_cast<const u32x4c*>(q + (static_cast<size_t>(t) * Hk + kh) * kCD + (tid % 16) * 8);
  }
  {
    const int t = min(t0 + tid % 32, T - 1);
    R.k = *reinterpret_cast<const u32x4c*>(k + (static_cast<size_t>(t) * Hk + kh) * kCD + (tid / 32) * 8);
    const size_t voff = (static_cast<size_t>(t) * Hv + h) * kCD + row0;
    R.v0 = *reinterpret_cast<const u32x4c*>(v + voff);
    R.v1 = *reinterpret_cast<const u32x4c*>(v + voff + 8);
  }
  R.gam = rec[kRecGam + (tid % kCC)];
  R.dec = rec[kRecDec + (tid % kCC)];
  R.gC = rec[kRecGC];
}

__device__ __forceinline__ void scan_store(const ScanRegs& R, ChunkBuf& B, int t0, int T) {
  const int tid = threadIdx.x;
  {
    const int t = tid / 16, e0 = (tid % 16) * 8;
    *reinterpret_cast<f32x4c*>(&B.W[t][e0]) = R.w0;
    *reinterpret_cast<f32x4c*>(&B.W[t][e0 + 4]) = R.w1;
  }
  {
    const int i = tid % 256, t = i / 8, s0 = (i % 8) * 4;
    *reinterpret_cast<f32x4c*>(tid < 256 ? &B.Bm[t][s0] : &B.Mq[t][s0]) = R.bmq;
  }
  {  // q rows past the sequence are zero
    const int t = tid / 16, e0 = (tid % 16) * 8;
    float f[8];
    widen8c(t0 + t < T ? as_uint4(R.q) : make_uint4(0, 0, 0, 0), f);
    reinterpret_cast<float4*>(&B.Q[t][e0])[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(&B.Q[t][e0])[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
  {  // k transposed and decayed; consecutive lanes write consecutive tokens
    const int t = tid % 32, i0 = (tid / 32) * 8;
    const float dec = (t0 + t < T) ? R.dec : 0.0f;
    float f[8];
    widen8c(as_uint4(R.k), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) B.KT[i0 + e][t] = f[e] * dec;
  }
  if (tid < kCC) {
    const bool ok = t0 + tid < T;
    float f[8];
    widen8c(as_uint4(R.v0), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) B.VT[e][tid] = ok ? f[e] : 0.0f;
    widen8c(as_uint4(R.v1), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) B.VT[8 + e][tid] = ok ? f[e] : 0.0f;
    B.gam[tid] = R.gam;
  }
  if (tid == 0) B.gC[0] = R.gC;
}

// 16 x 16 tile of X Y^T over 64 of the 128 columns (half kh): lane l supplies
// X[l % 16][64 kh + 16 (l/16) + ks] and Y[..][same]; two chains.
__device__ __forceinline__ f32x4c tile_xyT_half(const float* xrow, const float* yrow) {
  float xa[16], ya[16];
  lds_row<4>(xa, xrow);
  lds_row<4>(ya, yrow);
  f32x4c acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 16; ks += 2) {
    acc0 = mfma4(xa[ks], ya[ks], acc0);
    acc1 = mfma4(xa[ks + 1], ya[ks + 1], acc1);
  }
  return acc0 + acc1;
}

// s_waitcnt immediate (gfx9 encoding) that waits for every vector memory load.
constexpr int kWaitAllVmemC = 0x0F70;

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// not for its global loads, so the next chunk's loads stay in flight across
// it (a full __syncthreads would drain them at the first barrier after they
// are issued).  The memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void lds_barrier_c() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Work of a chunk over the eight waves (wave w runs on SIMD w % 4), each
// 16 x 16 tile split into halves of its 128-long sum where needed:
//   phase 1  w 0-3: W S^T, row tile w & 1, half w >> 1;  w 4-7: Q S^T likewise;
//            w 2, 3 also T diag(beta) V for row tile w & 1;
//   combine  w 2, 3: U = T diag(beta) V - both halves of W S^T;
//            w 4, 5: R = both halves of Q S^T;
//   phase 2  w 4, 5: outputs diag(gamma) R + (M o QK^T) U;
//            all: the state update for columns 16 w .. 16 w + 15.
// Every SIMD carries 56 matrix instructions per chunk.
__global__ __launch_bounds__(kSThreads) void gdn_chunk_scan_kernel(
    int T, int Hk, int Hv, int nchunks, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ ws,
    const float* state_in, float* state_out, uint16_t* __restrict__ o) {
  __shared__ ChunkBuf buf;                                          // the next chunk waits in registers
  __shared__ __attribute__((aligned(16))) float Sx[kCRows][kP];    // the workgroup's state rows
  __shared__ __attribute__((aligned(16))) float UxT[kCRows][kPt];  // U of the chunk, transposed
  __shared__ __attribute__((aligned(16))) float4 Part[8][64];      // half-sum tiles, per wave and lane

  constexpr int kRB = kCD / kCRows;       // workgroups per head
  const int wg = blockIdx.x;
  int h, rb;
  if (Hv % 8 == 0) {  // the row blocks of a head on one XCD (shared L2)
    const int xcd = wg % 8, slot = wg / 8;
    rb = slot % kRB;
    h = (slot / kRB) * 8 + xcd;
  } else {
    h = wg / kRB;
    rb = wg % kRB;
  }
  const int kh = h / (Hv / Hk);
  const int row0 = rb * kCRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane % 16, gq = lane / 16;
  const float* recs = ws + static_cast<size_t>(h) * nchunks * kRecFloats;

  // state rows in: thread tid covers row tid / 32, columns 4 (tid % 32) .. +3
  {
    const int r = tid / 32, e0 = (tid % 32) * 4;
    const size_t off = (static_cast<size_t>(h) * kCD + row0 + r) * kCD + e0;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (state_in) a = *reinterpret_cast<const float4*>(state_in + off);
    *reinterpret_cast<float4*>(&Sx[r][e0]) = a;
  }
  ScanRegs R;
  if (nchunks > 0) {
    scan_load(R, recs, 0, T, Hk, Hv, kh, h, row0, q, k, v);
    scan_store(R, buf, 0, T);
  }
  __builtin_amdgcn_s_waitcnt(kWaitAllVmemC);
  __syncthreads();

  const int I = wave & 1;                  // row tile of the chunk's tokens
  const int half = (wave >> 1) & 1;        // half of the 128-long sums
  const bool is_u = wave < 4;              // W S^T (for U) or Q S^T (for R)
  const f32x4c zero = {0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * kCC;
    const int n = min(kCC, T - t0);
    if (c + 1 < nchunks)
      scan_load(R, recs + static_cast<size_t>(c + 1) * kRecFloats, t0 + kCC, T, Hk, Hv, kh, h, row0,
                q, k, v);
    const ChunkBuf& B = buf;

    // operands of phase 2 that do not depend on U, read now so that phase 2
    // waits only for U: this wave's decayed K columns, its state tile, and
    // (waves 4, 5) the rows of M o QK^T
    // (Vector values, not arrays: an array kept live across the barriers'
    // memory clobbers would be placed in LDS by the compiler.)
    const int col = 16 * wave;
    const f32x4c kt0 = *reinterpret_cast<const f32x4c*>(&B.KT[col + i16][8 * gq]);
    const f32x4c kt1 = *reinterpret_cast<const f32x4c*>(&B.KT[col + i16][8 * gq + 4]);
    f32x4c sinit;
#pragma unroll
    for (int r = 0; r < 4; ++r) sinit[r] = Sx[4 * gq + r][col + i16];
    f32x4c mq0 = zero, mq1 = zero;
    if (wave == 4 || wave == 5) {
      mq0 = *reinterpret_cast<const f32x4c*>(&B.Mq[I * 16 + i16][8 * gq]);
      mq1 = *reinterpret_cast<const f32x4c*>(&B.Mq[I * 16 + i16][8 * gq + 4]);
    }
    const float gC = B.gC[0];

    // phase 1: half sums (and T diag(beta) V on waves 2, 3)
    const int k0 = 64 * half + 16 * gq;
    const float* xrow = is_u ? &B.W[I * 16 + i16][k0] : &B.Q[I * 16 + i16][k0];
    const f32x4c part = tile_xyT_half(xrow, &Sx[i16][k0]);
    f32x4c bv = zero;
    if (wave == 2 || wave == 3) bv = tile_k32(&B.Bm[I * 16 + i16][8 * gq], &B.VT[i16][8 * gq], zero);
    Part[wave][lane] = make_float4(part[0], part[1], part[2], part[3]);
    lds_barrier_c();

    // combine: U (waves 2, 3) and R (waves 4, 5)
    f32x4c rr = zero;
    if (wave == 2 || wave == 3) {
      const float4 p0 = Part[wave - 2][lane];
      *reinterpret_cast<float4*>(&UxT[i16][I * 16 + 4 * gq]) =
          make_float4(bv[0] - (p0.x + part[0]), bv[1] - (p0.y + part[1]), bv[2] - (p0.z + part[2]),
                      bv[3] - (p0.w + part[3]));
    } else if (wave == 4 || wave == 5) {
      const float4 p1 = Part[wave + 2][lane];
      rr = f32x4c{part[0] + p1.x, part[1] + p1.y, part[2] + p1.z, part[3] + p1.w};
    }
    lds_barrier_c();

    // phase 2: outputs (waves 4, 5) and the state update (all)
    const f32x4c ua0 = *reinterpret_cast<const f32x4c*>(&UxT[i16][8 * gq]);
    const f32x4c ua1 = *reinterpret_cast<const f32x4c*>(&UxT[i16][8 * gq + 4]);
    if (wave == 4 || wave == 5) {
      f32x4c mu0 = zero, mu1 = zero;
#pragma unroll
      for (int ks = 0; ks < 4; ks += 2) {
        mu0 = mfma4(mq0[ks], ua0[ks], mu0);
        mu1 = mfma4(mq0[ks + 1], ua0[ks + 1], mu1);
        mu0 = mfma4(mq1[ks], ua1[ks], mu0);
        mu1 = mfma4(mq1[ks + 1], ua1[ks + 1], mu1);
      }
      const f32x4c mu = mu0 + mu1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = I * 16 + 4 * gq + r;
        const float out = __builtin_fmaf(B.gam[t], rr[r], mu[r]);
        if (t < n)
          o[(static_cast<size_t>(t0 + t) * Hv + h) * kCD + row0 + i16] = f32_to_bf16(out);
      }
    }
    {
      f32x4c st0 = gC * sinit, st1 = zero;
#pragma unroll
      for (int ks = 0; ks < 4; ks += 2) {
        st0 = mfma4(ua0[ks], kt0[ks], st0);
        st1 = mfma4(ua0[ks + 1], kt0[ks + 1], st1);
        st0 = mfma4(ua1[ks], kt1[ks], st0);
        st1 = mfma4(ua1[ks + 1], kt1[ks + 1], st1);
      }
      const f32x4c st = st0 + st1;
#pragma unroll
      for (int r = 0; r < 4; ++r) Sx[4 * gq + r][col + i16] = st[r];
    }
    lds_barrier_c();  // every read of this chunk's buffer is done
    if (c + 1 < nchunks) {
      scan_store(R, buf, t0 + kCC, T);
      lds_barrier_c();
    }
  }

  if (state_out) {
    const int r = tid / 32, e0 = (tid % 32) * 4;
    const size_t off = (static_cast<size_t>(h) * kCD + row0 + r) * kCD + e0;
    *reinterpret_cast<float4*>(state_out + off) = *reinterpret_cast<const float4*>(&Sx[r][e0]);
  }
}

}  // namespace

size_t gdn_chunked_ws_bytes(int T, int n_v_heads) {
  const size_t nchunks = (static_cast<size_t>(T) + kCC - 1) / kCC;
  return nchunks * n_v_heads * kRecFloats * sizeof(float);
}

hipError_t launch_gdn_scan_chunked(int T, int n_k_heads, int n_v_heads, const uint16_t* q,
                                   const uint16_t* k, const uint16_t* v, const float* g,
                                   const float* beta, const float* state_in, float* state_out,
                                   uint16_t* o, float* ws, hipStream_t stream) {
  const int nchunks = (T + kCC - 1) / kCC;
  if (nchunks > 0) {
    hipLaunchKernelGGL(gdn_chunk_prep_kernel, dim3(static_cast<unsigned>(n_v_heads * nchunks)),
                       dim3(kCThreads), 0, stream, T, n_k_heads, n_v_heads, nchunks, q, k, g, beta, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gdn_chunk_scan_kernel, dim3(static_cast<unsigned>(n_v_heads * (kCD / kCRows))),
                     dim3(kSThreads), 0, stream, T, n_k_heads, n_v_heads, nchunks, q, k, v, ws,
                     state_in, state_out, o);
  return hipGetLastError();
}

}  // namespace moe
