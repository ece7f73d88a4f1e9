// Internal launch interface of the routing, GEMM, combine and scan kernels.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

// MOE_OK when the current device is a gfx950 (checked once per device and
// cached), MOE_EDEVICE otherwise or when the query fails.
int check_device();

struct RouteBuffers {
  float* logits;         // [T][E]
  int32_t* topk_idx;     // [T][k]
  float* topk_w;         // [T][k]
  int32_t* counts;       // [E]
  int32_t* offsets;      // [E+1]
  int32_t* sorted_slot;  // [T*k]
  int32_t* slot_pos;     // [T*k]
  int32_t* blocks;       // [max_blocks][4]
  int32_t* n_blocks;     // [1]
  uint32_t* bits;        // [ceil(T/32)][E] token bitmask per expert   (workspace)
  int32_t* pref;         // [ceil(T/32)][E] tokens before each word     (workspace)
  float* part;           // [8][T][E] router class sums, T <= 16 and E <= 256 (workspace)
  uint32_t* status;
  int max_blocks;
};

hipError_t launch_route(const moe_dims& d, const uint16_t* x, const float* wr, const float* bias,
                        const RouteBuffers& rb, hipStream_t stream);

struct GemmArgs {
  int T, H, I, E, k, n_shared, max_blocks;
  const int32_t* blocks;
  const int32_t* n_blocks;
  const int32_t* sorted_slot;
  BankView routed, shared;
  uint32_t* status;
  int n_shared_blocks;  // blocks of the shared expert (the last ones of the map)
  int tile_gran;        // tile heights are multiples of this
  int tall_all;         // set by the launcher: the tall-tile kernel takes every block
  int shared_mode;      // 0: every block; 1: the routed blocks only; 2: the shared blocks only
};

// M_MAX: largest tile height the chosen kernel variant accepts (64, 128, 256).
int gemm_m_max_for(int tile_m_max);
hipError_t launch_gate_up(const GemmArgs& a, int m_max, const uint16_t* x, uint16_t* h,
                          hipStream_t stream);
hipError_t launch_down(const GemmArgs& a, int m_max, const uint16_t* h, uint16_t* y_slots,
                       hipStream_t stream);
hipError_t launch_combine(int T, int H, int k, int n_shared, const float* topk_w,
                          const int32_t* slot_pos, const uint16_t* y_slots, uint16_t* y,
                          uint32_t* status, hipStream_t stream);
// Batch 1: the down GEMM and the combine in one launch (when down_combine_fused).
bool down_combine_fused(const GemmArgs& a);
hipError_t launch_down_combine_one(const GemmArgs& a, const float* topk_w, const int32_t* slot_pos,
                                   const uint16_t* h, uint16_t* y_slots, uint16_t* y,
                                   hipStream_t stream);
hipError_t launch_dequant(int rows, int K, const uint8_t* q, const uint16_t* s, const uint16_t* b,
                          uint16_t* out, hipStream_t stream);
hipError_t launch_dequant_packed(int nmat, int N, int K, int gate_up, const uint8_t* packed,
                                 uint16_t* out, hipStream_t stream);
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                             hipStream_t stream);
hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t stream);
hipError_t launch_gdn_scan(int T, int n_k_heads, int n_v_heads, const uint16_t* q,
                          const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                          const float* state_in, float* state_out, uint16_t* o, hipStream_t stream);
size_t gdn_chunked_ws_bytes(int T, int n_v_heads);
hipError_t launch_gdn_scan_chunked(int T, int n_k_heads, int n_v_heads, const uint16_t* q,
                                   const uint16_t* k, const uint16_t* v, const float* g,
                                   const float* beta, const float* state_in, float* state_out,
                                   uint16_t* o, float* ws, hipStream_t stream);
hipError_t launch_pack(int nmat, int N, int K, int gate_up, const uint8_t* q, const uint16_t* s,
                       const uint16_t* b, uint8_t* out, hipStream_t stream);

}  // namespace moe
