// CPU oracle for the sparse MoE expert layer with groupwise-affine 4-bit weights.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
// HIP path is checked against.  Only the tests, the smoke check and the
// benchmark's CPU-baseline leg may load it; the product path never does.  It
// shares no code, header, table or helper with the HIP library.
//
// Build: g++ -O2 -ffp-contract=off -fPIC -shared -pthread (no fast-math), so
// that every floating-point operation below is performed exactly as written.
//
// Sources (web pages on the Lily engine for Qwen3.6-35B-A3B):
//   [LB] "Lily Beats MLX-LM 1.35x on Decode: Perplexity's Rust+Metal Engine for
//        Apple Silicon", sections "Model structure and three workload shapes"
//        and "Prefill: fusing dequantisation and keeping routing GPU-resident".
//   [RL] "Introduction: Revolutionizing Local AI Inference on Apple Silicon",
//        sections "Understanding the Qwen3.6-35B-A3B Model" and "Optimizing
//        Prefill Operations".
// Where the pages are silent (router precision, tie-breaks, SwiGLU, the
// combine, nibble order, block-map rule) each function states the reading it
// implements.
//
// Parity pins: every function here is pinned by CPU tests against brute force,
// closed forms or invariants.  The one result with no external pin is the
// pages' own teacher-forced accuracy figure, which needs trained weights: it is
// not reproduced here (parity unpinned for that figure only).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---- bfloat16 <-> float32 ---------------------------------------------------

float bf16_to_float(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Round a float32 to the nearest bfloat16, ties to even (finite inputs; NaN is
// returned as a quiet NaN).
uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) {
    return static_cast<uint16_t>((u >> 16) | 0x0040u);
  }
  uint32_t kept = u >> 16;          // sign, exponent and top 7 mantissa bits
  uint32_t dropped = u & 0xFFFFu;   // the 16 bits that are rounded away
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
  return static_cast<uint16_t>(kept);
}

// ---- groupwise-affine 4-bit weights ------------------------------------------
//
// [LB, "Model structure and three workload shapes"]: every group of 64 weights
// shares one bfloat16 scale and one bfloat16 bias, and tensor operations take
// bfloat16, so each weight is reconstructed as a bfloat16 value before use.
// Readings: groups run along the input (reduction) dimension of each output
// row; byte b of a row holds element 2b in its low nibble and 2b+1 in its high
// nibble; codes are unsigned 0..15; the reconstruction is w = q*scale + bias
// evaluated as one fused float32 multiply-add, rounded once to bfloat16.

unsigned code_at(const uint8_t* row_codes, int kk) {
  uint8_t byte = row_codes[kk / 2];
  return (kk % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
}

float dequant_one(const uint8_t* row_codes, const uint16_t* row_scale, const uint16_t* row_bias,
                  int kk) {
  float q = static_cast<float>(code_at(row_codes, kk));
  float s = bf16_to_float(row_scale[kk / 64]);
  float b = bf16_to_float(row_bias[kk / 64]);
  return bf16_to_float(float_to_bf16_rne(std::fmaf(q, s, b)));
}

// Reconstructed weight (row n, input kk) of a [rows][K] matrix in the packed layout.
double weight(const uint8_t* q, const uint16_t* s, const uint16_t* b, int K, int n, int kk) {
  return static_cast<double>(dequant_one(q + static_cast<size_t>(n) * (K / 2),
                                         s + static_cast<size_t>(n) * (K / 64),
                                         b + static_cast<size_t>(n) * (K / 64), kk));
}

template <class F>
void parallel_for(int n, int nthreads, F&& body) {
  if (nthreads <= 1 || n <= 1) {
    for (int i = 0; i < n; ++i) body(i);
    return;
  }
  nthreads = std::min(nthreads, n);
  std::vector<std::thread> pool;
  for (int w = 0; w < nthreads; ++w) {
    pool.emplace_back([&, w]() {
      for (int i = w; i < n; i += nthreads) body(i);
    });
  }
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

int orc_abi_version(void) { return 1; }

void orc_dequant(int rows, int K, const uint8_t* q, const uint16_t* s, const uint16_t* b,
                 float* out) {
  for (int n = 0; n < rows; ++n)
    for (int kk = 0; kk < K; ++kk)
      out[static_cast<size_t>(n) * K + kk] = static_cast<float>(weight(q, s, b, K, n, kk));
}

uint16_t orc_f32_to_bf16(float f) { return float_to_bf16_rne(f); }

// ---- a1: router logits ---------------------------------------------------------
//
// [RL, "Understanding the Qwen3.6-35B-A3B Model"], [LB, "Model structure ..."]:
// a router scores the 256 experts of every token.  Reading: the score is the
// float32 dot product of the token's bfloat16 activations with the expert's
// float32 router column, plus an optional per-expert float32 bias.  Because the
// top-k decision must come out identical on the GPU, both sides evaluate it in
// one fixed float32 order:
//   partial m (m = 0..63) is a chain of fused multiply-adds, starting at +0,
//     over the inputs h = m, m+64, m+128, ... (increasing h);
//   the 64 partials are then added pairwise as a tree: for s = 32,16,8,4,2,1,
//     p[i] = p[i] + p[i+s] for every i < s;
//   logit = p[0] + bias[e] (no addition when there is no bias).
// Requires H % 64 == 0.
void orc_router_logits(int T, int H, int E, const uint16_t* x, const float* wr, const float* bias,
                       float* logits, int nthreads) {
  parallel_for(T, nthreads, [&](int t) {
    const uint16_t* xt = x + static_cast<size_t>(t) * H;
    for (int e = 0; e < E; ++e) {
      float p[64];
      for (int m = 0; m < 64; ++m) {
        float acc = 0.0f;
        for (int h = m; h < H; h += 64)
          acc = std::fmaf(bf16_to_float(xt[h]), wr[static_cast<size_t>(h) * E + e], acc);
        p[m] = acc;
      }
      for (int s = 32; s >= 1; s /= 2)
        for (int i = 0; i < s; ++i) p[i] = p[i] + p[i + s];
      float l = p[0];
      if (bias) l = l + bias[e];
      logits[static_cast<size_t>(t) * E + e] = l;
    }
  });
}

// The same scores in float64 with a plain left-to-right sum (diagnostic and pin).
void orc_router_logits_f64(int T, int H, int E, const uint16_t* x, const float* wr,
                           const float* bias, double* logits, int nthreads) {
  parallel_for(T, nthreads, [&](int t) {
    const uint16_t* xt = x + static_cast<size_t>(t) * H;
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += static_cast<double>(bf16_to_float(xt[h])) *
               static_cast<double>(wr[static_cast<size_t>(h) * E + e]);
      if (bias) acc += static_cast<double>(bias[e]);
      logits[static_cast<size_t>(t) * E + e] = acc;
    }
  });
}

// ---- a2: top-k selection and routing weights -------------------------------------
//
// [LB, "Model structure ..."]: the router selects eight of the 256 experts.
// Readings: selection compares the float32 logits; a higher logit comes first
// and equal logits are ordered by lower expert index; the k experts are stored
// in that order.  The weights are a softmax over all E logits, restricted to
// the selected experts and renormalised to sum to one (computed in float64
// from the float32 logits).
void orc_topk(int T, int E, int k, const float* logits, int32_t* idx, double* w) {
  std::vector<int> order(E);
  std::vector<double> p(E);
  for (int t = 0; t < T; ++t) {
    const float* lt = logits + static_cast<size_t>(t) * E;
    for (int e = 0; e < E; ++e) order[e] = e;
    std::sort(order.begin(), order.end(), [&](int a, int b) {
      if (lt[a] != lt[b]) return lt[a] > lt[b];
      return a < b;
    });
    double mx = static_cast<double>(lt[order[0]]);
    double z = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = std::exp(static_cast<double>(lt[e]) - mx);
      z += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= z;   // softmax over every expert
    double sel = 0.0;
    for (int j = 0; j < k; ++j) sel += p[order[j]];
    for (int j = 0; j < k; ++j) {
      idx[static_cast<size_t>(t) * k + j] = order[j];
      w[static_cast<size_t>(t) * k + j] = p[order[j]] / sel;   // renormalised
    }
  }
}

// ---- a3..a5: histogram, exclusive prefix scan, stable scatter ------------------------
//
// [RL, "Optimizing Prefill Operations"], [LB, "Prefill: ..."]: routing is a
// histogram of tokens per expert, a prefix scan of it, a scatter of the tokens
// into expert order and a block map.  A slot is (token t, rank j) with id
// t*k + j.  Reading: the scatter is stable in slot-id order.
void orc_route_tables(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                      int32_t* sorted_slot, int32_t* slot_pos) {
  const int S = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int s = 0; s < S; ++s) counts[idx[s]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> ids(S);
  for (int s = 0; s < S; ++s) ids[s] = s;
  std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return idx[a] < idx[b]; });
  for (int r = 0; r < S; ++r) {
    sorted_slot[r] = ids[r];
    slot_pos[ids[r]] = r;
  }
}

// ---- a6: block map -----------------------------------------------------------------
//
// [LB, "Prefill: ..."]: GEMM tiles of up to 32 rows over uneven expert groups.
// Reading (tile rows chosen per group): rows of the grouped GEMM are the T*k
// routed slots in expert order followed by T shared-expert rows (token order).
// Groups are the routed experts 0..E-1 and then the shared expert (group E).
// A group with c > 0 rows is cut into nb = ceil(c / tile_m_max) blocks whose
// row counts differ by at most one (the first c mod nb blocks get one more),
// each with tile height roundup(ceil(c / nb), tile_gran).  Entry = {group,
// first row, rows, tile height}, in group order then block order.
int32_t orc_max_blocks(int T, int E, int k, int n_shared, int tile_m_max) {
  long long S = static_cast<long long>(T) * k;
  long long nb = S / tile_m_max + std::min<long long>(E, S);
  if (n_shared) nb += (T + tile_m_max - 1) / tile_m_max;
  return static_cast<int32_t>(nb);
}

int32_t orc_block_map(int T, int E, int k, int n_shared, int tile_m_max, int tile_gran,
                      const int32_t* counts, const int32_t* offsets, int32_t* blocks,
                      int32_t max_blocks) {
  int32_t nb_total = 0;
  const int groups = E + (n_shared ? 1 : 0);
  for (int g = 0; g < groups; ++g) {
    int c = (g < E) ? counts[g] : T;
    int first = (g < E) ? offsets[g] : T * k;
    if (c == 0) continue;
    int nb = (c + tile_m_max - 1) / tile_m_max;
    int base = c / nb, rem = c % nb;
    int tallest = base + (rem > 0 ? 1 : 0);
    int tile_m = (tallest + tile_gran - 1) / tile_gran * tile_gran;
    int row = first;
    for (int i = 0; i < nb; ++i) {
      int rows = base + (i < rem ? 1 : 0);
      if (nb_total >= max_blocks) return -1;
      int32_t* ent = blocks + 4 * static_cast<size_t>(nb_total);
      ent[0] = g;
      ent[1] = row;
      ent[2] = rows;
      ent[3] = tile_m;
      row += rows;
      ++nb_total;
    }
  }
  return nb_total;
}

// ---- a7..a8: one expert's feed-forward network on one token --------------------------
//
// [LB, "Prefill: ..."]: the expert GEMMs use reconstructed weights with float32
// (here float64) accumulation.  Reading: the expert FFN is gate/up projection,
// SwiGLU, down projection: g = W_gate x, u = W_up x, a = silu(g) * u with
// silu(z) = z / (1 + exp(-z)), y = W_down a.  Gate rows are 0..I-1 and up rows
// I..2I-1 of the gate/up matrix.  Everything after the weight reconstruction
// is float64.
void orc_expert_ffn(int H, int I, const uint16_t* x_row, const uint8_t* gu_q, const uint16_t* gu_s,
                    const uint16_t* gu_b, const uint8_t* dn_q, const uint16_t* dn_s,
                    const uint16_t* dn_b, double* h_out, double* y_out) {
  std::vector<double> xv(H), a(I);
  for (int h = 0; h < H; ++h) xv[h] = static_cast<double>(bf16_to_float(x_row[h]));
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      g += xv[h] * weight(gu_q, gu_s, gu_b, H, i, h);
      u += xv[h] * weight(gu_q, gu_s, gu_b, H, I + i, h);
    }
    a[i] = g / (1.0 + std::exp(-g)) * u;
    if (h_out) h_out[i] = a[i];
  }
  for (int o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += a[i] * weight(dn_q, dn_s, dn_b, I, o, i);
    y_out[o] = acc;
  }
}

// ---- a9 (with a7..a8): the layer output for a list of tokens --------------------------
//
// [RL, "Understanding the Qwen3.6-35B-A3B Model"], [LB, "Model structure ..."]:
// each token goes through its selected experts alongside one shared expert
// that processes every token.  Reading: y = sum_j w_j * FFN_{e_j}(x) +
// FFN_shared(x), shared weight 1 and no gate, summed in float64.
// Banks are [n][...] arrays in the packed layout; the shared bank may be null
// when n_shared == 0.  tok lists the tokens to evaluate (null = all T);
// y_out has one row of H doubles per listed token.
void orc_moe_layer(int T, int H, int I, int E, int k, int n_shared, const uint16_t* x,
                   const int32_t* idx, const double* w, const uint8_t* r_gu_q,
                   const uint16_t* r_gu_s, const uint16_t* r_gu_b, const uint8_t* r_dn_q,
                   const uint16_t* r_dn_s, const uint16_t* r_dn_b, const uint8_t* s_gu_q,
                   const uint16_t* s_gu_s, const uint16_t* s_gu_b, const uint8_t* s_dn_q,
                   const uint16_t* s_dn_s, const uint16_t* s_dn_b, int ntok, const int32_t* tok,
                   double* y_out, int nthreads) {
  (void)E;
  const size_t gu_q_n = static_cast<size_t>(2 * I) * (H / 2);
  const size_t gu_s_n = static_cast<size_t>(2 * I) * (H / 64);
  const size_t dn_q_n = static_cast<size_t>(H) * (I / 2);
  const size_t dn_s_n = static_cast<size_t>(H) * (I / 64);
  const int n = tok ? ntok : T;
  parallel_for(n, nthreads, [&](int r) {
    const int t = tok ? tok[r] : r;
    const uint16_t* xt = x + static_cast<size_t>(t) * H;
    std::vector<double> ye(H);
    double* yo = y_out + static_cast<size_t>(r) * H;
    for (int o = 0; o < H; ++o) yo[o] = 0.0;
    for (int j = 0; j < k; ++j) {
      const size_t e = static_cast<size_t>(idx[static_cast<size_t>(t) * k + j]);
      orc_expert_ffn(H, I, xt, r_gu_q + e * gu_q_n, r_gu_s + e * gu_s_n, r_gu_b + e * gu_s_n,
                     r_dn_q + e * dn_q_n, r_dn_s + e * dn_s_n, r_dn_b + e * dn_s_n, nullptr,
                     ye.data());
      const double wj = w[static_cast<size_t>(t) * k + j];
      for (int o = 0; o < H; ++o) yo[o] += wj * ye[o];
    }
    if (n_shared) {
      orc_expert_ffn(H, I, xt, s_gu_q, s_gu_s, s_gu_b, s_dn_q, s_dn_s, s_dn_b, nullptr, ye.data());
      for (int o = 0; o < H; ++o) yo[o] += ye[o];
    }
  });
}

}  // extern "C"
