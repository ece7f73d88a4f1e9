// C ABI of the W4 MoE expert layer: argument validation, workspace layout and
// kernel launches.  Nothing here allocates, frees or synchronises.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "route.h"

using namespace moe;

// ---------------------------------------------------------------------------
// Library-owned routing scratch for moe_route_no_alloc.  The array lives in
// the code object, so every GPU the library runs on holds its own copy until
// the process ends.  Host code never uses the array's name as an address (on
// the host it only names the symbol): its device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept here.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = MOE_NO_ALLOC_WS_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
}  // namespace

namespace moe {
// 0 = unchecked, 1 = gfx950, 2 = other architecture
static std::atomic<int> g_arch_state[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EDEVICE;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_EDEVICE;
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? MOE_OK : MOE_EDEVICE;
}

}  // namespace moe

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int validate_dims(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->T < 0 || d->T > (1 << 20)) return MOE_EINVAL;
  if (d->H <= 0 || d->H % 64 || d->H > (1 << 16)) return MOE_EINVAL;
  if (d->I <= 0 || d->I % 64 || d->I > (1 << 16)) return MOE_EINVAL;
  if (d->E < 1 || d->E > kMaxE) return MOE_EINVAL;
  if (d->k < 1 || d->k > kMaxK || d->k > d->E) return MOE_EINVAL;
  if (d->n_shared != 0 && d->n_shared != 1) return MOE_EINVAL;
  if (d->tile_gran != 16 && d->tile_gran != 32) return MOE_EINVAL;
  if (d->tile_m_max < 16 || d->tile_m_max > 256 || d->tile_m_max % d->tile_gran) return MOE_EINVAL;
  return MOE_OK;
}

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
  size_t logits, bits, pref, part, total;
};

WsLayout ws_layout(const moe_dims& d, bool need_logits) {
  const size_t T = d.T, E = d.E;
  const size_t W = (T + 31) / 32;
  WsLayout L;
  size_t off = 0;
  L.logits = off;
  off += need_logits ? align256(T * E * 4) : 0;
  L.bits = off;
  off += align256(W * E * 4);
  L.pref = off;
  off += align256(W * E * 4);
  // Router class sums of the short-batch path (T <= 16, E <= 256).  The
  // region is sized for min(T, 16) tokens at every T, so that the total never
  // decreases with T: a workspace sized for a batch bound fits every smaller
  // batch, including the short ones that use this region.
  L.part = off;
  off += (E <= 256) ? align256(8 * std::min<size_t>(T, 16) * E * 4) : 0;
  L.total = off;
  return L;
}

int validate_route_out(const moe_route_out* r, bool for_route) {
  if (!r) return MOE_EINVAL;
  if (!r->topk_idx || !r->topk_w || !r->counts || !r->offsets || !r->sorted_slot || !r->slot_pos ||
      !r->blocks || !r->n_blocks || !r->status)
    return MOE_EINVAL;
  if (!aligned(r->topk_idx, 4) || !aligned(r->topk_w, 4) || !aligned(r->counts, 4) ||
      !aligned(r->offsets, 4) || !aligned(r->sorted_slot, 4) || !aligned(r->slot_pos, 4) ||
      !aligned(r->blocks, 16) || !aligned(r->n_blocks, 4) || !aligned(r->status, 4) ||
      (r->logits && !aligned(r->logits, 4)))
    return MOE_EALIGN;
  if (for_route) {
    if (!r->ws) return MOE_EINVAL;
    if (!aligned(r->ws, 16)) return MOE_EALIGN;
  }
  return MOE_OK;
}

int validate_bank(const moe_w4_bank* b) {
  if (!b || !b->gu || !b->dn) return MOE_EINVAL;
  if (!aligned(b->gu, 16) || !aligned(b->dn, 16)) return MOE_EALIGN;
  return MOE_OK;
}

BankView view(const moe_w4_bank* b) {
  BankView v{};
  if (b) v = BankView{b->gu, b->dn};
  return v;
}

bool pack_dims_ok(int32_t rows, int32_t K) {
  return rows > 0 && rows % 16 == 0 && rows <= (1 << 20) && K > 0 && K % 64 == 0 && K <= (1 << 16);
}

int32_t max_blocks_of(const moe_dims& d) {
  const long long S = static_cast<long long>(d.T) * d.k;
  long long nb = S / d.tile_m_max + (S < d.E ? S : d.E);
  if (d.n_shared) nb += (d.T + d.tile_m_max - 1) / d.tile_m_max;
  return static_cast<int32_t>(nb);
}

int validate_ffn_common(const moe_dims* d, const moe_route_out* r, const moe_w4_bank* routed,
                        const moe_w4_bank* shared) {
  int rc = validate_dims(d);
  if (rc) return rc;
  if ((rc = validate_route_out(r, false))) return rc;
  if ((rc = validate_bank(routed))) return rc;
  if (d->n_shared && (rc = validate_bank(shared))) return rc;
  return MOE_OK;
}

GemmArgs gemm_args(const moe_dims& d, const moe_route_out* r, const moe_w4_bank* routed,
                   const moe_w4_bank* shared) {
  GemmArgs a{};
  a.T = d.T;
  a.H = d.H;
  a.I = d.I;
  a.E = d.E;
  a.k = d.k;
  a.n_shared = d.n_shared;
  a.max_blocks = max_blocks_of(d);
  a.blocks = r->blocks;
  a.n_blocks = r->n_blocks;
  a.sorted_slot = r->sorted_slot;
  a.routed = view(routed);
  a.shared = view(d.n_shared ? shared : nullptr);
  a.status = r->status;
  a.n_shared_blocks = d.n_shared ? (d.T + d.tile_m_max - 1) / d.tile_m_max : 0;
  a.tile_gran = d.tile_gran;
  return a;
}

int launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

int validate_route_args(const moe_dims* d, const uint16_t* x, const float* w_router,
                        const float* logit_bias, const moe_route_out* out, bool need_ws) {
  int rc = validate_dims(d);
  if (rc) return rc;
  if ((rc = validate_route_out(out, need_ws))) return rc;
  if (!x || !w_router) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(w_router, 4) || (logit_bias && !aligned(logit_bias, 4)))
    return MOE_EALIGN;
  return MOE_OK;
}

// Routing with its scratch at ws (layout L): the kernels clear what they
// accumulate into (the token bitmask) themselves.
int enqueue_route(const moe_dims& d, const uint16_t* x, const float* w_router,
                  const float* logit_bias, const moe_route_out* out, char* ws, const WsLayout& L,
                  hipStream_t stream) {
  RouteBuffers rb{};
  rb.logits = out->logits ? out->logits : reinterpret_cast<float*>(ws + L.logits);
  rb.topk_idx = out->topk_idx;
  rb.topk_w = out->topk_w;
  rb.counts = out->counts;
  rb.offsets = out->offsets;
  rb.sorted_slot = out->sorted_slot;
  rb.slot_pos = out->slot_pos;
  rb.blocks = out->blocks;
  rb.n_blocks = out->n_blocks;
  rb.bits = reinterpret_cast<uint32_t*>(ws + L.bits);
  rb.pref = reinterpret_cast<int32_t*>(ws + L.pref);
  rb.part = reinterpret_cast<float*>(ws + L.part);
  rb.status = out->status;
  rb.max_blocks = max_blocks_of(d);
  (void)hipGetLastError();
  return launched(launch_route(d, x, w_router, logit_bias, rb, stream));
}

std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_ptr(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EDEVICE;
  char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return MOE_EDEVICE;
      p = static_cast<char*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_W4_ABI_VERSION; }

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer or dimension out of range)";
    case MOE_EALIGN: return "misaligned pointer";
    case MOE_EWS: return "workspace too small";
    case MOE_EDEVICE: return "current device is not gfx950 or a device query failed";
    case MOE_ELAUNCH: return "kernel launch failed";
    default: return "unknown error";
  }
}

int32_t moe_max_blocks(const moe_dims* d) {
  if (validate_dims(d)) return -1;
  return max_blocks_of(*d);
}

size_t moe_route_ws_bytes(const moe_dims* d) {
  if (validate_dims(d)) return 0;
  return ws_layout(*d, true).total;
}

int moe_route(const moe_dims* d, const uint16_t* x, const float* w_router, const float* logit_bias,
              const moe_route_out* out, void* stream) {
  int rc = validate_route_args(d, x, w_router, logit_bias, out, true);
  if (rc) return rc;
  const WsLayout L = ws_layout(*d, out->logits == nullptr);
  if (out->ws_bytes < L.total) return MOE_EWS;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  return enqueue_route(*d, x, w_router, logit_bias, out, static_cast<char*>(out->ws), L,
                       static_cast<hipStream_t>(stream));
}

int moe_route_no_alloc(const moe_dims* d, const uint16_t* x, const float* w_router,
                       const float* logit_bias, const moe_route_out* out, void* stream) {
  int rc = validate_route_args(d, x, w_router, logit_bias, out, false);
  if (rc) return rc;
  const WsLayout L = ws_layout(*d, out->logits == nullptr);
  if (L.total > kScratchBytes) return MOE_EWS;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  char* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  return enqueue_route(*d, x, w_router, logit_bias, out, ws, L, static_cast<hipStream_t>(stream));
}

int moe_w4_gate_up(const moe_dims* d, const uint16_t* x, const moe_route_out* r,
                   const moe_w4_bank* routed, const moe_w4_bank* shared, uint16_t* h,
                   void* stream) {
  int rc = validate_ffn_common(d, r, routed, shared);
  if (rc) return rc;
  if (!x || !h) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(h, 16)) return MOE_EALIGN;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  const GemmArgs a = gemm_args(*d, r, routed, shared);
  (void)hipGetLastError();
  return launched(launch_gate_up(a, gemm_m_max_for(d->tile_m_max), x, h,
                                 static_cast<hipStream_t>(stream)));
}

int moe_w4_down(const moe_dims* d, const moe_route_out* r, const moe_w4_bank* routed,
                const moe_w4_bank* shared, const uint16_t* h, uint16_t* y_slots, void* stream) {
  int rc = validate_ffn_common(d, r, routed, shared);
  if (rc) return rc;
  if (!h || !y_slots) return MOE_EINVAL;
  if (!aligned(h, 16) || !aligned(y_slots, 16)) return MOE_EALIGN;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  const GemmArgs a = gemm_args(*d, r, routed, shared);
  (void)hipGetLastError();
  return launched(launch_down(a, gemm_m_max_for(d->tile_m_max), h, y_slots,
                              static_cast<hipStream_t>(stream)));
}

int moe_grouped_w4_ffn(const moe_dims* d, const uint16_t* x, const moe_route_out* r,
                       const moe_w4_bank* routed, const moe_w4_bank* shared, uint16_t* h,
                       uint16_t* y_slots, void* stream) {
  int rc = validate_ffn_common(d, r, routed, shared);
  if (rc) return rc;
  if (!x || !h || !y_slots) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(h, 16) || !aligned(y_slots, 16)) return MOE_EALIGN;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  const GemmArgs a = gemm_args(*d, r, routed, shared);
  const int m_max = gemm_m_max_for(d->tile_m_max);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if ((rc = launched(launch_gate_up(a, m_max, x, h, s)))) return rc;
  return launched(launch_down(a, m_max, h, y_slots, s));
}

int moe_routed_w4_ffn(const moe_dims* d, const uint16_t* x, const moe_route_out* r,
                      const moe_w4_bank* routed, uint16_t* h, uint16_t* y_slots, void* stream) {
  int rc = validate_dims(d);
  if (rc) return rc;
  if ((rc = validate_route_out(r, false))) return rc;
  if ((rc = validate_bank(routed))) return rc;
  if (!x || !h || !y_slots) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(h, 16) || !aligned(y_slots, 16)) return MOE_EALIGN;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  GemmArgs a = gemm_args(*d, r, routed, nullptr);
  a.shared_mode = 1;
  const int m_max = gemm_m_max_for(d->tile_m_max);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if ((rc = launched(launch_gate_up(a, m_max, x, h, s)))) return rc;
  return launched(launch_down(a, m_max, h, y_slots, s));
}

int moe_shared_w4_ffn(const moe_dims* d, const uint16_t* x, const moe_w4_bank* shared, uint16_t* h,
                      uint16_t* y_slots, void* stream) {
  int rc = validate_dims(d);
  if (rc) return rc;
  if (d->n_shared != 1) return MOE_EINVAL;
  if ((rc = validate_bank(shared))) return rc;
  if (!x || !h || !y_slots) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(h, 16) || !aligned(y_slots, 16)) return MOE_EALIGN;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  // No routing tables: the shared group always holds all T rows.
  GemmArgs a{};
  a.T = d->T;
  a.H = d->H;
  a.I = d->I;
  a.E = d->E;
  a.k = d->k;
  a.n_shared = 1;
  a.max_blocks = max_blocks_of(*d);
  a.shared = view(shared);
  a.n_shared_blocks = (d->T + d->tile_m_max - 1) / d->tile_m_max;
  a.tile_gran = d->tile_gran;
  a.shared_mode = 2;
  const int m_max = gemm_m_max_for(d->tile_m_max);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if ((rc = launched(launch_gate_up(a, m_max, x, h, s)))) return rc;
  return launched(launch_down(a, m_max, h, y_slots, s));
}

int moe_w4_ffn_combine(const moe_dims* d, const uint16_t* x, const moe_route_out* r,
                       const moe_w4_bank* routed, const moe_w4_bank* shared, uint16_t* h,
                       uint16_t* y_slots, uint16_t* y, void* stream) {
  int rc = validate_ffn_common(d, r, routed, shared);
  if (rc) return rc;
  if (!x || !h || !y_slots || !y || !r->topk_w || !r->slot_pos || !r->status) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(h, 16) || !aligned(y_slots, 16) || !aligned(y, 16) ||
      !aligned(r->topk_w, 4) || !aligned(r->slot_pos, 4) || !aligned(r->status, 4))
    return MOE_EALIGN;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  const GemmArgs a = gemm_args(*d, r, routed, shared);
  const int m_max = gemm_m_max_for(d->tile_m_max);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if ((rc = launched(launch_gate_up(a, m_max, x, h, s)))) return rc;
  if (down_combine_fused(a))
    return launched(launch_down_combine_one(a, r->topk_w, r->slot_pos, h, y_slots, y, s));
  if ((rc = launched(launch_down(a, m_max, h, y_slots, s)))) return rc;
  return launched(launch_combine(d->T, d->H, d->k, d->n_shared, r->topk_w, r->slot_pos, y_slots, y,
                                 r->status, s));
}

int moe_combine(const moe_dims* d, const moe_route_out* r, const uint16_t* y_slots, uint16_t* y,
                void* stream) {
  int rc = validate_dims(d);
  if (rc) return rc;
  if (!r || !r->topk_w || !r->slot_pos || !r->status || !y_slots || !y) return MOE_EINVAL;
  if (!aligned(r->topk_w, 4) || !aligned(r->slot_pos, 4) || !aligned(r->status, 4) ||
      !aligned(y_slots, 16) || !aligned(y, 16))
    return MOE_EALIGN;
  if (d->T == 0) return MOE_OK;
  if ((rc = check_device())) return rc;
  (void)hipGetLastError();
  return launched(launch_combine(d->T, d->H, d->k, d->n_shared, r->topk_w, r->slot_pos, y_slots, y,
                                 r->status, static_cast<hipStream_t>(stream)));
}

size_t moe_w4_packed_bytes(int32_t rows, int32_t K) {
  return pack_dims_ok(rows, K) ? pack_bytes(rows, K) : 0;
}

int moe_w4_pack(int32_t n, int32_t rows, int32_t K, int32_t gate_up, const uint8_t* q,
                const uint16_t* s, const uint16_t* b, uint8_t* packed, void* stream) {
  if (n < 0 || !pack_dims_ok(rows, K) || (gate_up != 0 && gate_up != 1)) return MOE_EINVAL;
  if (!q || !s || !b || !packed) return MOE_EINVAL;
  if (!aligned(q, 16) || !aligned(s, 2) || !aligned(b, 2) || !aligned(packed, 16)) return MOE_EALIGN;
  if (n == 0) return MOE_OK;
  int rc = check_device();
  if (rc) return rc;
  (void)hipGetLastError();
  return launched(launch_pack(n, rows, K, gate_up, q, s, b, packed, static_cast<hipStream_t>(stream)));
}

int moe_w4_dequant(int32_t rows, int32_t K, const uint8_t* q, const uint16_t* s, const uint16_t* b,
                   uint16_t* out, void* stream) {
  if (rows < 0 || K <= 0 || K % 64 || K > (1 << 16)) return MOE_EINVAL;
  if (!q || !s || !b || !out) return MOE_EINVAL;
  if (!aligned(q, 4) || !aligned(s, 2) || !aligned(b, 2) || !aligned(out, 16)) return MOE_EALIGN;
  if (rows == 0) return MOE_OK;
  int rc = check_device();
  if (rc) return rc;
  (void)hipGetLastError();
  return launched(launch_dequant(rows, K, q, s, b, out, static_cast<hipStream_t>(stream)));
}

int moe_w4_dequant_packed(int32_t n, int32_t rows, int32_t K, int32_t gate_up, const uint8_t* packed,
                          uint16_t* out, void* stream) {
  if (n < 0 || !pack_dims_ok(rows, K) || (gate_up != 0 && gate_up != 1)) return MOE_EINVAL;
  if (!packed || !out) return MOE_EINVAL;
  if (!aligned(packed, 16) || !aligned(out, 16)) return MOE_EALIGN;
  if (n == 0) return MOE_OK;
  int rc = check_device();
  if (rc) return rc;
  (void)hipGetLastError();
  return launched(launch_dequant_packed(n, rows, K, gate_up, packed, out,
                                        static_cast<hipStream_t>(stream)));
}

int moe_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (!src || !sink || workgroups < 1 || workgroups > (1 << 20)) return MOE_EINVAL;
  if (!aligned(src, 16) || bytes % 16 || !aligned(sink, 4)) return MOE_EALIGN;
  if (bytes == 0) return MOE_OK;
  int rc = check_device();
  if (rc) return rc;
  (void)hipGetLastError();
  return launched(launch_read_probe(src, bytes, sink, workgroups, static_cast<hipStream_t>(stream)));
}

int moe_mfma_probe(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (!sink || workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24))
    return MOE_EINVAL;
  if (!aligned(sink, 4)) return MOE_EALIGN;
  int rc = check_device();
  if (rc) return rc;
  (void)hipGetLastError();
  return launched(launch_mfma_probe(workgroups, iters, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
