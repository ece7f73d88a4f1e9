// Host driver for the sanitizer build of the CPU oracle: every exported
// function on small inputs held in exactly sized heap buffers, so that an
// out-of-bounds access or undefined behaviour stops the run.  Test
// infrastructure only.
#include <stdint.h>
#include <stdio.h>

#include <vector>

extern "C" {
int orc_abi_version(void);
void orc_dequant(int rows, int K, const uint8_t* q, const uint16_t* s, const uint16_t* b, float* out);
uint16_t orc_f32_to_bf16(float f);
void orc_router_logits(int T, int H, int E, const uint16_t* x, const float* wr, const float* bias,
                       float* logits, int nthreads);
void orc_router_logits_f64(int T, int H, int E, const uint16_t* x, const float* wr,
                           const float* bias, double* logits, int nthreads);
void orc_topk(int T, int E, int k, const float* logits, int32_t* idx, double* w);
void orc_route_tables(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                      int32_t* sorted_slot, int32_t* slot_pos);
int32_t orc_max_blocks(int T, int E, int k, int n_shared, int tile_m_max);
int32_t orc_block_map(int T, int E, int k, int n_shared, int tile_m_max, int tile_gran,
                      const int32_t* counts, const int32_t* offsets, int32_t* blocks,
                      int32_t max_blocks);
void orc_expert_ffn(int H, int I, const uint16_t* x_row, const uint8_t* gu_q, const uint16_t* gu_s,
                    const uint16_t* gu_b, const uint8_t* dn_q, const uint16_t* dn_s,
                    const uint16_t* dn_b, double* h_out, double* y_out);
void orc_moe_layer(int T, int H, int I, int E, int k, int n_shared, const uint16_t* x,
                   const int32_t* idx, const double* w, const uint8_t* r_gu_q,
                   const uint16_t* r_gu_s, const uint16_t* r_gu_b, const uint8_t* r_dn_q,
                   const uint16_t* r_dn_s, const uint16_t* r_dn_b, const uint8_t* s_gu_q,
                   const uint16_t* s_gu_s, const uint16_t* s_gu_b, const uint8_t* s_dn_q,
                   const uint16_t* s_dn_s, const uint16_t* s_dn_b, int ntok, const int32_t* tok,
                   double* y_out, int nthreads);
}

namespace {

uint64_t g_state = 0x243F6A8885A308D3ull;
uint32_t next_u32() {  // xorshift64*: driver inputs only
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return static_cast<uint32_t>((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
float uniform(float lo, float hi) { return lo + (hi - lo) * (next_u32() >> 8) * (1.0f / 16777216.0f); }

template <class T>
std::vector<T> bytes_of(size_t n) {
  std::vector<T> v(n);
  for (auto& e : v) e = static_cast<T>(next_u32());
  return v;
}
std::vector<uint16_t> bf16_of(size_t n, float lo, float hi) {
  std::vector<uint16_t> v(n);
  for (auto& e : v) e = orc_f32_to_bf16(uniform(lo, hi));
  return v;
}

struct Bank {
  std::vector<uint8_t> gu_q, dn_q;
  std::vector<uint16_t> gu_s, gu_b, dn_s, dn_b;
  Bank(int n, int H, int I)
      : gu_q(bytes_of<uint8_t>(size_t(n) * 2 * I * H / 2)),
        dn_q(bytes_of<uint8_t>(size_t(n) * H * I / 2)),
        gu_s(bf16_of(size_t(n) * 2 * I * H / 64, 0.002f, 0.02f)),
        gu_b(bf16_of(size_t(n) * 2 * I * H / 64, -0.16f, 0.0f)),
        dn_s(bf16_of(size_t(n) * H * I / 64, 0.002f, 0.02f)),
        dn_b(bf16_of(size_t(n) * H * I / 64, -0.16f, 0.0f)) {}
};

// One layer call through every oracle stage at (T, H, I, E, k, shared).
void run_layer(int T, int H, int I, int E, int k, int n_shared, int tile_m_max, int tile_gran,
               int nthreads) {
  std::vector<uint16_t> x = bf16_of(size_t(T) * H, -2.f, 2.f);
  std::vector<float> wr(size_t(H) * E), bias(E);
  for (auto& v : wr) v = uniform(-0.05f, 0.05f);
  for (auto& v : bias) v = uniform(-1.f, 0.f);
  std::vector<float> logits(size_t(T) * E);
  std::vector<double> logits64(size_t(T) * E);
  orc_router_logits(T, H, E, x.data(), wr.data(), bias.data(), logits.data(), nthreads);
  orc_router_logits(T, H, E, x.data(), wr.data(), nullptr, logits.data(), nthreads);
  orc_router_logits_f64(T, H, E, x.data(), wr.data(), bias.data(), logits64.data(), nthreads);
  std::vector<int32_t> idx(size_t(T) * k);
  std::vector<double> w(size_t(T) * k);
  orc_topk(T, E, k, logits.data(), idx.data(), w.data());
  std::vector<int32_t> counts(E), offsets(E + 1), sorted(size_t(T) * k), pos(size_t(T) * k);
  orc_route_tables(T, E, k, idx.data(), counts.data(), offsets.data(), sorted.data(), pos.data());
  const int32_t mb = orc_max_blocks(T, E, k, n_shared, tile_m_max);
  std::vector<int32_t> blocks(size_t(mb) * 4);
  orc_block_map(T, E, k, n_shared, tile_m_max, tile_gran, counts.data(), offsets.data(),
                blocks.data(), mb);
  Bank routed(E, H, I), shared(1, H, I);
  std::vector<double> y(size_t(T) * H);
  orc_moe_layer(T, H, I, E, k, n_shared, x.data(), idx.data(), w.data(), routed.gu_q.data(),
                routed.gu_s.data(), routed.gu_b.data(), routed.dn_q.data(), routed.dn_s.data(),
                routed.dn_b.data(), shared.gu_q.data(), shared.gu_s.data(), shared.gu_b.data(),
                shared.dn_q.data(), shared.dn_s.data(), shared.dn_b.data(), 0, nullptr, y.data(),
                nthreads);
  if (T > 0) {  // a token list: the last token, then the first
    const int32_t tok[2] = {T - 1, 0};
    std::vector<double> y2(size_t(2) * H);
    orc_moe_layer(T, H, I, E, k, n_shared, x.data(), idx.data(), w.data(), routed.gu_q.data(),
                  routed.gu_s.data(), routed.gu_b.data(), routed.dn_q.data(), routed.dn_s.data(),
                  routed.dn_b.data(), shared.gu_q.data(), shared.gu_s.data(), shared.gu_b.data(),
                  shared.dn_q.data(), shared.dn_s.data(), shared.dn_b.data(), 2, tok, y2.data(),
                  nthreads);
  }
  if (T > 0) {
    std::vector<double> h(I), yr(H);
    orc_expert_ffn(H, I, x.data(), routed.gu_q.data(), routed.gu_s.data(), routed.gu_b.data(),
                   routed.dn_q.data(), routed.dn_s.data(), routed.dn_b.data(), h.data(), yr.data());
  }
}

}  // namespace

int main() {
  if (orc_abi_version() != 1) return 2;
  {
    const int rows = 16, K = 192;
    auto q = bytes_of<uint8_t>(size_t(rows) * K / 2);
    auto s = bf16_of(size_t(rows) * K / 64, 0.002f, 0.02f);
    auto b = bf16_of(size_t(rows) * K / 64, -0.16f, 0.f);
    std::vector<float> out(size_t(rows) * K);
    orc_dequant(rows, K, q.data(), s.data(), b.data(), out.data());
  }
  // special values through the bf16 rounding
  const float specials[] = {0.f, -0.f, 1e-40f, -1e-40f, 3.4e38f, 1.0f / 0.0f, -1.0f / 0.0f};
  for (float f : specials) (void)orc_f32_to_bf16(f);
  // shapes: empty, single token, ragged, more experts than slots, 1024 experts + shared
  run_layer(0, 64, 64, 8, 2, 1, 128, 16, 2);
  run_layer(1, 64, 64, 8, 2, 1, 128, 16, 1);
  run_layer(5, 128, 64, 8, 3, 1, 32, 16, 2);
  run_layer(37, 64, 128, 6, 2, 0, 16, 16, 3);
  run_layer(19, 64, 64, 300, 8, 1, 256, 32, 2);
  run_layer(3, 64, 64, 1024, 8, 1, 16, 16, 2);
  // block map at the tile-height bounds over many uneven groups
  for (int tm : {16, 32, 48, 128, 256}) {
    const int T = 700, E = 33, k = 4;
    std::vector<int32_t> counts(E), offsets(E + 1);
    int total = 0;
    for (int e = 0; e < E; ++e) {
      counts[e] = (e % 5 == 0) ? 0 : static_cast<int32_t>(next_u32() % 200);
      offsets[e] = total;
      total += counts[e];
    }
    offsets[E] = total;
    const int Tk = total / k + 1;
    const int32_t mb = orc_max_blocks(Tk, E, k, 1, tm);
    std::vector<int32_t> blocks(size_t(mb) * 4);
    orc_block_map(Tk, E, k, 1, tm, 16, counts.data(), offsets.data(), blocks.data(), mb);
    (void)T;
  }
  printf("oracle sanitizer driver ok\n");
  return 0;
}
