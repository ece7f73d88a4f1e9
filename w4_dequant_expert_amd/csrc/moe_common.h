// Device helpers shared by the gfx950 kernels of the W4 MoE expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_w4.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two float32 -> packed bfloat16 pair (low half = a), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  return static_cast<uint16_t>(pack_bf16x2(a, 0.0f) & 0xFFFFu);
}

// Reconstruct eight consecutive 4-bit weights of one row (one 32-bit word of
// packed codes, element i in bits 4i..4i+3) that share one group's scale s and
// bias b: w_i = bf16(fma(q_i, s, b)).  Returns the eight bfloat16 values in
// element order, packed two per 32-bit word (element 2p in the low half).
//   - even elements sit in the low nibble of each byte, odd ones in the high
//     nibble; masking gives one code per byte, v_cvt_f32_ubyteN widens it
//     exactly;
//   - one float32 fused multiply-add per weight, then one round to bfloat16.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float s, float b) {
  uint32_t ev = w & 0x0F0F0F0Fu;          // codes 0,2,4,6, one per byte
  uint32_t od = (w >> 4) & 0x0F0F0F0Fu;   // codes 1,3,5,7
  // Opaque to the optimiser, so that each byte below widens with one
  // v_cvt_f32_ubyteN instead of a field extract plus a conversion.
  asm("" : "+v"(ev));
  asm("" : "+v"(od));
  const float f0 = __builtin_fmaf(static_cast<float>(ev & 0xFFu), s, b);
  const float f1 = __builtin_fmaf(static_cast<float>(od & 0xFFu), s, b);
  const float f2 = __builtin_fmaf(static_cast<float>((ev >> 8) & 0xFFu), s, b);
  const float f3 = __builtin_fmaf(static_cast<float>((od >> 8) & 0xFFu), s, b);
  const float f4 = __builtin_fmaf(static_cast<float>((ev >> 16) & 0xFFu), s, b);
  const float f5 = __builtin_fmaf(static_cast<float>((od >> 16) & 0xFFu), s, b);
  const float f6 = __builtin_fmaf(static_cast<float>(ev >> 24), s, b);
  const float f7 = __builtin_fmaf(static_cast<float>(od >> 24), s, b);
  uint4 r;
  r.x = pack_bf16x2(f0, f1);
  r.y = pack_bf16x2(f2, f3);
  r.z = pack_bf16x2(f4, f5);
  r.w = pack_bf16x2(f6, f7);
  return r;
}

// dequant8 for a code word in pair order (as stored in the packed layout):
// the same eight weights, in element order.
__device__ __forceinline__ uint4 dequant8_pairs(uint32_t w, float s, float b) {
  uint32_t ev = w & 0x0F0F0F0Fu;          // elements 0, 4, 1, 5 (bytes 0..3)
  uint32_t od = (w >> 4) & 0x0F0F0F0Fu;   // elements 2, 6, 3, 7
  asm("" : "+v"(ev));
  asm("" : "+v"(od));
  const float f0 = __builtin_fmaf(static_cast<float>(ev & 0xFFu), s, b);
  const float f4 = __builtin_fmaf(static_cast<float>((ev >> 8) & 0xFFu), s, b);
  const float f1 = __builtin_fmaf(static_cast<float>((ev >> 16) & 0xFFu), s, b);
  const float f5 = __builtin_fmaf(static_cast<float>(ev >> 24), s, b);
  const float f2 = __builtin_fmaf(static_cast<float>(od & 0xFFu), s, b);
  const float f6 = __builtin_fmaf(static_cast<float>((od >> 8) & 0xFFu), s, b);
  const float f3 = __builtin_fmaf(static_cast<float>((od >> 16) & 0xFFu), s, b);
  const float f7 = __builtin_fmaf(static_cast<float>(od >> 24), s, b);
  uint4 r;
  r.x = pack_bf16x2(f0, f1);
  r.y = pack_bf16x2(f2, f3);
  r.z = pack_bf16x2(f4, f5);
  r.w = pack_bf16x2(f6, f7);
  return r;
}

// Wave-uniform copy of a value the compiler cannot prove uniform.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ void status_set(uint32_t* status, uint32_t bits) {
  if (status) atomicOr(status, bits);
}

// ---------------------------------------------------------------------------
// Packed weight layout (written once by moe_w4_pack, read by the GEMMs).
//
// A matrix of N output rows and K inputs is cut into N/16 slices of 16 rows
// and ceil(K/128) steps of 128 inputs.  Each (slice, step) is one contiguous
// block of kPackBlock bytes, blocks ordered slice-major:
//   bytes [0, 1024): lane l (0..63) of a wave finds at l*16 four code words
//     of row (l mod 16) of the slice; word j holds the eight inputs
//     step*128 + 32j + 8*(l/16) .. +7, in pair order (below);
//   bytes [1024, 1152): 32 dwords; dword 2r + g holds the scale (low half)
//     and bias (high half) of row r for inputs step*128 + g*64 .. +63.
// Pair order: nibble t of a code word holds element 2t and nibble t+4 holds
// element 2t+1 (t = 0..3), so that masking the word shifted by 4t with
// 0x000F000F puts elements 2t and 2t+1 in the two halves of one dword.
// Inputs past K are code 0 with scale 0 and bias 0 (they rebuild to +0).
// Gate/up matrices interleave gate and up rows: slice c holds gate rows
// 8c..8c+7 as rows 0..7 and the matching up rows I+8c.. as rows 8..15, so a
// lane's gate and up outputs sit 8 lanes apart.  Down matrices are straight:
// slice c holds rows 16c..16c+15.
// A 16x16x32 MFMA over inputs 32j .. 32j+31 of a step takes word j of every
// lane as its B operand; both of the step's scale groups are whole MFMAs.
// ---------------------------------------------------------------------------
constexpr int kKS = 128;             // inputs per step
constexpr int kPackBlock = 1152;     // bytes per (slice, step) block
constexpr int kPackScales = 1024;    // offset of the scale/bias dwords

__host__ __device__ inline int pack_steps(int K) { return (K + kKS - 1) / kKS; }
__host__ __device__ inline size_t pack_bytes(int N, int K) {
  return static_cast<size_t>(N / 16) * pack_steps(K) * kPackBlock;
}

// Packed matrices of one expert bank (device) as seen by the kernels.
struct BankView {
  const uint8_t* gu;  // [n][pack_bytes(2I, H)]
  const uint8_t* dn;  // [n][pack_bytes(H, I)]
};

}  // namespace moe
