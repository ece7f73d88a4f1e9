// Host driver for the sanitizer build of the C ABI's host half (argument
// validation, workspace layout, block bound, packed sizes).  It links the
// library's api.hip against the stub launchers below, which record that they
// were reached and enqueue nothing, so it runs without a GPU.  Test
// infrastructure only.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "moe_w4.h"
#include "route.h"

namespace moe {
static int g_launches = 0;
hipError_t launch_route(const moe_dims&, const uint16_t*, const float*, const float*,
                        const RouteBuffers&, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
int gemm_m_max_for(int tile_m_max) { return tile_m_max <= 32 ? 0 : (tile_m_max <= 128 ? 128 : 256); }
hipError_t launch_gate_up(const GemmArgs&, int, const uint16_t*, uint16_t*, hipStream_t) {
  ++g_launches; return hipErrorInvalidValue;
}
hipError_t launch_down(const GemmArgs&, int, const uint16_t*, uint16_t*, hipStream_t) {
  ++g_launches; return hipErrorInvalidValue;
}
hipError_t launch_combine(int, int, int, int, const float*, const int32_t*, const uint16_t*,
                          uint16_t*, uint32_t*, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
bool down_combine_fused(const GemmArgs& a) { return a.T == 1; }
hipError_t launch_down_combine_one(const GemmArgs&, const float*, const int32_t*, const uint16_t*,
                                   uint16_t*, uint16_t*, hipStream_t) {
  ++g_launches; return hipErrorInvalidValue;
}
hipError_t launch_dequant(int, int, const uint8_t*, const uint16_t*, const uint16_t*, uint16_t*,
                          hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_dequant_packed(int, int, int, int, const uint8_t*, uint16_t*, hipStream_t) {
  ++g_launches; return hipErrorInvalidValue;
}
hipError_t launch_read_probe(const void*, size_t, uint32_t*, int, hipStream_t) {
  ++g_launches; return hipErrorInvalidValue;
}
hipError_t launch_mfma_probe(int, int, float*, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_gdn_scan(int, int, int, const uint16_t*, const uint16_t*, const uint16_t*,
                           const float*, const float*, const float*, float*, uint16_t*, hipStream_t) {
  ++g_launches; return hipErrorInvalidValue;
}
hipError_t launch_pack(int, int, int, int, const uint8_t*, const uint16_t*, const uint16_t*,
                       uint8_t*, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
}  // namespace moe

static int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

// Stand-in "device" memory: host buffers that the host half only checks for
// alignment and never dereferences.
alignas(256) static unsigned char g_mem[1 << 16];

static moe_dims dims(int T, int E, int k, int shared, int tm, int gran) {
  moe_dims d;
  d.T = T; d.H = 256; d.I = 128; d.E = E; d.k = k; d.n_shared = shared;
  d.tile_m_max = tm; d.tile_gran = gran;
  return d;
}

static moe_route_out route_out(size_t ws_bytes) {
  moe_route_out r;
  memset(&r, 0, sizeof r);
  r.topk_idx = reinterpret_cast<int32_t*>(g_mem + 0);
  r.topk_w = reinterpret_cast<float*>(g_mem + 256);
  r.counts = reinterpret_cast<int32_t*>(g_mem + 512);
  r.offsets = reinterpret_cast<int32_t*>(g_mem + 768);
  r.sorted_slot = reinterpret_cast<int32_t*>(g_mem + 1024);
  r.slot_pos = reinterpret_cast<int32_t*>(g_mem + 1280);
  r.blocks = reinterpret_cast<int32_t*>(g_mem + 1536);
  r.n_blocks = reinterpret_cast<int32_t*>(g_mem + 1792);
  r.status = reinterpret_cast<uint32_t*>(g_mem + 2048);
  r.logits = nullptr;
  r.ws = g_mem + 4096;
  r.ws_bytes = ws_bytes;
  return r;
}

int main() {
  CHECK(moe_abi_version() == MOE_W4_ABI_VERSION);
  for (int c = -8; c <= 2; ++c) CHECK(moe_strerror(c) != nullptr && strlen(moe_strerror(c)) > 0);

  // dimension sweep: bounds, workspace and block bound stay defined and the
  // workspace never shrinks as T grows
  const int Es[] = {1, 2, 8, 255, 256, 257, 300, 1023, 1024, 1025};
  const int tms[] = {0, 15, 16, 32, 48, 128, 240, 256, 272};
  for (int E : Es)
    for (int k : {1, 2, 8, 32, 33})
      for (int shared : {0, 1, 2})
        for (int tm : tms)
          for (int gran : {8, 16, 32}) {
            size_t prev_ws = 0;
            for (int T : {0, 1, 2, 15, 16, 17, 31, 32, 33, 511, 512, 2048, 2049, 16384, 1 << 20, (1 << 20) + 1}) {
              moe_dims d = dims(T, E, k, shared, tm, gran);
              const int32_t mb = moe_max_blocks(&d);
              const size_t ws = moe_route_ws_bytes(&d);
              const bool valid = E <= 1024 && k <= 32 && k <= E && shared <= 1 && tm >= 16 &&
                                 tm <= 256 && (gran == 16 || gran == 32) && tm % gran == 0 &&
                                 T <= (1 << 20);
              CHECK(valid ? (mb >= 0 && (T == 0 || ws > 0)) : (mb == -1 && ws == 0));
              if (valid) {
                CHECK(ws >= prev_ws);
                prev_ws = ws;
                const long long S = static_cast<long long>(T) * k;
                CHECK(mb >= (S + tm - 1) / tm);
              }
            }
          }
  CHECK(moe_max_blocks(nullptr) == -1);
  CHECK(moe_route_ws_bytes(nullptr) == 0);
  moe_dims bad = dims(4, 8, 2, 1, 32, 16);
  bad.H = 100;
  CHECK(moe_max_blocks(&bad) == -1);
  bad = dims(4, 8, 2, 1, 32, 16);
  bad.I = 0;
  CHECK(moe_route_ws_bytes(&bad) == 0);

  // packed sizes
  for (int rows : {-16, 0, 8, 16, 48, 1 << 20, (1 << 20) + 16})
    for (int K : {-64, 0, 32, 64, 128, 192, 2048, 1 << 16, (1 << 16) + 64}) {
      const size_t n = moe_w4_packed_bytes(rows, K);
      const bool ok = rows > 0 && rows % 16 == 0 && rows <= (1 << 20) && K > 0 && K % 64 == 0 &&
                      K <= (1 << 16);
      CHECK(ok ? n >= static_cast<size_t>(rows) * K / 2 : n == 0);
    }

  // entry points: every rejection happens before a launch
  const uint16_t* x = reinterpret_cast<const uint16_t*>(g_mem + 8192);
  const float* wr = reinterpret_cast<const float*>(g_mem + 12288);
  moe_dims d = dims(4, 8, 2, 1, 32, 16);
  const size_t need = moe_route_ws_bytes(&d);
  moe_route_out r = route_out(need);
  CHECK(moe_route(nullptr, x, wr, nullptr, &r, nullptr) == MOE_EINVAL);
  CHECK(moe_route(&d, nullptr, wr, nullptr, &r, nullptr) == MOE_EINVAL);
  CHECK(moe_route(&d, x, nullptr, nullptr, &r, nullptr) == MOE_EINVAL);
  CHECK(moe_route(&d, x, wr, nullptr, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_route(&d, x + 1, wr, nullptr, &r, nullptr) == MOE_EALIGN);
  {
    moe_route_out r2 = route_out(need - 1);
    CHECK(moe_route(&d, x, wr, nullptr, &r2, nullptr) == MOE_EWS);
    r2 = route_out(need);
    r2.blocks = reinterpret_cast<int32_t*>(g_mem + 1540);
    CHECK(moe_route(&d, x, wr, nullptr, &r2, nullptr) == MOE_EALIGN);
    r2 = route_out(need);
    r2.ws = nullptr;
    CHECK(moe_route(&d, x, wr, nullptr, &r2, nullptr) == MOE_EINVAL);
    r2 = route_out(need);
    r2.status = nullptr;
    CHECK(moe_route_no_alloc(&d, x, wr, nullptr, &r2, nullptr) == MOE_EINVAL);
  }
  {
    moe_dims big = dims(1 << 20, 1024, 8, 1, 128, 16);
    CHECK(moe_route_no_alloc(&big, x, wr, nullptr, &r, nullptr) == MOE_EWS);
  }
  moe_dims d0 = dims(0, 8, 2, 1, 32, 16);
  CHECK(moe_route(&d0, x, wr, nullptr, &r, nullptr) == MOE_OK);
  CHECK(moe_route_no_alloc(&d0, x, wr, nullptr, &r, nullptr) == MOE_OK);

  const moe_w4_bank bank{g_mem + 16384, g_mem + 20480};
  const moe_w4_bank bad_bank{g_mem + 16385, g_mem + 20480};
  const moe_w4_bank null_bank{nullptr, g_mem + 20480};
  uint16_t* h = reinterpret_cast<uint16_t*>(g_mem + 24576);
  uint16_t* ys = reinterpret_cast<uint16_t*>(g_mem + 28672);
  uint16_t* y = reinterpret_cast<uint16_t*>(g_mem + 32768);
  CHECK(moe_w4_gate_up(&d, x, &r, &bank, nullptr, h, nullptr) == MOE_EINVAL);  // shared bank missing
  CHECK(moe_w4_gate_up(&d, x, &r, &bad_bank, &bank, h, nullptr) == MOE_EALIGN);
  CHECK(moe_w4_gate_up(&d, x, &r, &null_bank, &bank, h, nullptr) == MOE_EINVAL);
  CHECK(moe_w4_gate_up(&d, x, &r, &bank, &bank, h + 1, nullptr) == MOE_EALIGN);
  CHECK(moe_w4_gate_up(&d0, x, &r, &bank, &bank, h, nullptr) == MOE_OK);
  CHECK(moe_w4_down(&d, &r, &bank, &bank, nullptr, ys, nullptr) == MOE_EINVAL);
  CHECK(moe_w4_down(&d, &r, &bank, &bank, h, ys + 4, nullptr) == MOE_EALIGN);
  CHECK(moe_w4_down(&d0, &r, &bank, &bank, h, ys, nullptr) == MOE_OK);
  CHECK(moe_grouped_w4_ffn(&d, x, &r, &bank, &bank, h, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_grouped_w4_ffn(&d, x + 2, &r, &bank, &bank, h, ys, nullptr) == MOE_EALIGN);
  CHECK(moe_grouped_w4_ffn(&d0, x, &r, &bank, &bank, h, ys, nullptr) == MOE_OK);
  CHECK(moe_routed_w4_ffn(&d, x, &r, nullptr, h, ys, nullptr) == MOE_EINVAL);
  CHECK(moe_routed_w4_ffn(&d0, x, &r, &bank, h, ys, nullptr) == MOE_OK);
  {
    moe_dims dn = dims(4, 8, 2, 0, 32, 16);
    CHECK(moe_shared_w4_ffn(&dn, x, &bank, h, ys, nullptr) == MOE_EINVAL);  // no shared expert
  }
  CHECK(moe_shared_w4_ffn(&d, x, &bad_bank, h, ys, nullptr) == MOE_EALIGN);
  CHECK(moe_shared_w4_ffn(&d0, x, &bank, h, ys, nullptr) == MOE_OK);
  CHECK(moe_combine(&d, nullptr, ys, y, nullptr) == MOE_EINVAL);
  CHECK(moe_combine(&d, &r, ys, y + 1, nullptr) == MOE_EALIGN);
  CHECK(moe_combine(&d0, &r, ys, y, nullptr) == MOE_OK);
  CHECK(moe_w4_ffn_combine(&d, x, &r, &bank, &bank, h, ys, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_w4_ffn_combine(&d, x, &r, &bank, &bank, h, ys, y + 1, nullptr) == MOE_EALIGN);
  CHECK(moe_w4_ffn_combine(&d0, x, &r, &bank, &bank, h, ys, y, nullptr) == MOE_OK);

  const uint8_t* q = g_mem + 36864;
  const uint16_t* s = reinterpret_cast<const uint16_t*>(g_mem + 40960);
  uint8_t* packed = g_mem + 45056;
  CHECK(moe_w4_pack(1, 15, 64, 0, q, s, s, packed, nullptr) == MOE_EINVAL);
  CHECK(moe_w4_pack(1, 16, 64, 2, q, s, s, packed, nullptr) == MOE_EINVAL);
  CHECK(moe_w4_pack(-1, 16, 64, 0, q, s, s, packed, nullptr) == MOE_EINVAL);
  CHECK(moe_w4_pack(1, 16, 64, 0, q + 1, s, s, packed, nullptr) == MOE_EALIGN);
  CHECK(moe_w4_pack(0, 16, 64, 0, q, s, s, packed, nullptr) == MOE_OK);
  CHECK(moe_w4_dequant(4, 63, q, s, s, h, nullptr) == MOE_EINVAL);
  CHECK(moe_w4_dequant(4, 64, q, s, s, h + 1, nullptr) == MOE_EALIGN);
  CHECK(moe_w4_dequant(0, 64, q, s, s, h, nullptr) == MOE_OK);
  CHECK(moe_w4_dequant_packed(1, 16, 64, 1, packed + 8, h, nullptr) == MOE_EALIGN);
  CHECK(moe_w4_dequant_packed(0, 16, 64, 1, packed, h, nullptr) == MOE_OK);
  CHECK(moe_read_probe(packed, 100, reinterpret_cast<uint32_t*>(ys), 4, nullptr) == MOE_EALIGN);
  CHECK(moe_read_probe(packed, 0, reinterpret_cast<uint32_t*>(ys), 4, nullptr) == MOE_OK);
  CHECK(moe_read_probe(packed, 64, reinterpret_cast<uint32_t*>(ys), 0, nullptr) == MOE_EINVAL);

  CHECK(moe_mfma_probe(0, 10, reinterpret_cast<float*>(ys), nullptr) == MOE_EINVAL);
  CHECK(moe_mfma_probe(4, 0, reinterpret_cast<float*>(ys), nullptr) == MOE_EINVAL);
  CHECK(moe_mfma_probe(4, 10, reinterpret_cast<float*>(g_mem + 2), nullptr) == MOE_EALIGN);
  CHECK(moe_mfma_probe(4, 10, nullptr, nullptr) == MOE_EINVAL);

  CHECK(moe::g_launches == 0);
  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("abi sanitizer driver ok\n");
  return 0;
}
