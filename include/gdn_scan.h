/*
 * gdn_scan.h - C ABI of the MI355X (gfx950) Gated DeltaNet recurrent scan
 * with the state held in registers for the whole sequence.
 *
 * Source (web pages on the Lily engine for Qwen3.6-35B-A3B):
 *   [LB] "Lily Beats MLX-LM 1.35x on Decode: Perplexity's Rust+Metal Engine for
 *        Apple Silicon": "Model structure and three workload shapes" (the
 *        model interleaves Gated DeltaNet layers, a fixed-size recurrence,
 *        with its attention layers) and "Prefill: fusing dequantisation and
 *        keeping routing GPU-resident" (a register-resident Gated DeltaNet
 *        scan: each simdgroup carries one column of recurrent state through
 *        the whole scan instead of moving an intermediate of 256 MiB per
 *        layer).
 * The pages do not write the recurrence out; it is the gated delta rule as
 * published (Yang, Kautz, Hatamizadeh, "Gated Delta Networks: Improving
 * Mamba2 with Delta Rule", ICLR 2025).  Per value head h, state
 * S in R^{dv x dk}, for t = 0 .. T-1:
 *     S_t = S_{t-1} * alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t,          alpha_t = exp(g_t)
 * Value head h reads key head h / (n_v_heads / n_k_heads).
 *
 * Conventions (as for moe_w4.h): array arguments are DEVICE pointers the
 * caller allocated and owns; the library never allocates, frees or
 * synchronises; `stream` is a hipStream_t passed as void*; bfloat16 values
 * are uint16_t bit patterns; every argument is validated before anything is
 * enqueued, and the return codes are moe_w4.h's MOE_* codes.
 */
#ifndef GDN_SCAN_H
#define GDN_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of one scan.  dk and dv must both be 128 (the head width of the
 * model's linear-attention layers); 1 <= n_k_heads <= n_v_heads <= 1024 with
 * n_v_heads a multiple of n_k_heads; 0 <= T <= 2^24. */
typedef struct gdn_dims {
  int32_t T, n_k_heads, n_v_heads, dk, dv;
} gdn_dims;

/*
 * One sequence of T tokens through the gated delta rule.
 *   q, k      [T][n_k_heads][dk] bfloat16, 16-byte aligned (used as given:
 *             any normalisation or scaling belongs to the caller)
 *   v         [T][n_v_heads][dv] bfloat16, 16-byte aligned
 *   g         [T][n_v_heads] float32 log-decay (alpha = exp(g)), 4-byte aligned
 *   beta      [T][n_v_heads] float32 write strength, 4-byte aligned
 *   state_in  [n_v_heads][dv][dk] float32 initial state (row j = value
 *             dimension j), 16-byte aligned, or NULL for zeros
 *   state_out [n_v_heads][dv][dk] float32 final state, or NULL; may equal
 *             state_in (updated in place)
 *   o         [T][n_v_heads][dv] bfloat16 outputs, 16-byte aligned (may be
 *             NULL only when T = 0)
 * Arithmetic: float32 state and products, each output rounded once to
 * bfloat16.  With T = 0 the call copies state_in (or zeros) to state_out.
 * Returns MOE_OK, MOE_EINVAL (null pointer, shape out of range), MOE_EALIGN,
 * MOE_EDEVICE or MOE_ELAUNCH.
 */
int gdn_scan(const gdn_dims *d, const uint16_t *q, const uint16_t *k, const uint16_t *v,
             const float *g, const float *beta, const float *state_in, float *state_out,
             uint16_t *o, void *stream);

/*
 * gdn_scan_chunked - the same scan regrouped over chunks of 32 tokens, on the
 * matrix cores: per chunk, the part that does not depend on the state (the
 * chunk's k.k and q.k products, the triangular solve of the delta rule's
 * writes, the decays) is computed for every chunk in parallel into `ws`;
 * then one pass over the chunks carries the state on chip and applies each
 * chunk with four matrix products (the chunkwise form of the Gated DeltaNet
 * paper, Yang, Kautz, Hatamizadeh, ICLR 2025).  The state never goes through
 * memory between chunks.  Same arguments, layouts and results as gdn_scan (to
 * rounding: float32 throughout, outputs rounded once to bfloat16), plus
 *   ws        device scratch of at least gdn_scan_chunked_ws_bytes(d) bytes,
 *             256-byte aligned, owned by the caller (may be NULL when that
 *             size is 0); its contents are overwritten
 * Returns as gdn_scan, and MOE_EWS when ws_bytes is too small.
 */
size_t gdn_scan_chunked_ws_bytes(const gdn_dims *d);  /* 0 for invalid dims */
int gdn_scan_chunked(const gdn_dims *d, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const float *g, const float *beta, const float *state_in, float *state_out,
                     uint16_t *o, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_SCAN_H */
