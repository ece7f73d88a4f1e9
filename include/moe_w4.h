/*
 * moe_w4.h - C ABI of the MI355X (gfx950) sparse MoE expert layer with fused
 * groupwise-affine 4-bit weight reconstruction.
 *
 * Sources (web pages on the Lily engine for Qwen3.6-35B-A3B):
 *   [LB] "Lily Beats MLX-LM 1.35x on Decode: Perplexity's Rust+Metal Engine for
 *        Apple Silicon": "Model structure and three workload shapes" (router
 *        over 256 experts, eight selected, one shared expert for every token;
 *        4-bit codes, a bfloat16 scale and bias per group of 64 weights,
 *        weights reconstructed to bfloat16 for the tensor operations) and
 *        "Prefill: fusing dequantisation and keeping routing GPU-resident"
 *        (reconstruction one tile at a time inside the grouped GEMM with float32
 *        accumulation, the expanded array never written to memory; histogram,
 *        prefix scan, scatter and block map on the GPU with no CPU
 *        synchronisation; 32-row tiles; bounded chunks for long prompts).
 *   [RL] "Introduction: Revolutionizing Local AI Inference on Apple Silicon":
 *        "Understanding the Qwen3.6-35B-A3B Model", "Optimizing Prefill
 *        Operations" (the same routing stages and the fused dequantisation).
 *
 * Conventions shared by every call:
 *   - All array arguments are DEVICE pointers to memory the caller allocated and
 *     owns; the library never allocates, frees or synchronises, and keeps no
 *     state between calls apart from a per-device architecture check.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously in call order; the caller synchronises.
 *   - bfloat16 values are passed as uint16_t bit patterns.
 *   - Every argument is validated before anything is enqueued, so an error
 *     return leaves nothing half-launched.  T = 0 is valid and enqueues nothing.
 *   - Faults found on the device (a NaN router score, an out-of-range index in
 *     the routing tables) set bits in out->status, which the caller reads after
 *     its own synchronisation.  No C++ exception crosses this interface.
 */
#ifndef MOE_W4_H
#define MOE_W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_W4_ABI_VERSION 4

/* Return codes. */
#define MOE_OK 0
#define MOE_EINVAL (-1)  /* null required pointer or a dimension out of range   */
#define MOE_EALIGN (-2)  /* a pointer is not aligned as documented              */
#define MOE_EWS (-3)     /* workspace smaller than moe_route_ws_bytes()        */
#define MOE_EDEVICE (-4) /* current device is not gfx950, or a HIP query failed */
#define MOE_ELAUNCH (-5) /* a kernel launch reported an error                   */

/* Bits of the device status word. */
#define MOE_STATUS_NAN_LOGIT 1u   /* a router score was NaN (treated as -inf)           */
#define MOE_STATUS_BAD_INDEX 2u   /* a routing table entry was out of range (skipped)   */
#define MOE_STATUS_BLOCK_OVERFLOW 4u /* block map longer than moe_max_blocks (truncated) */

/*
 * Layer dimensions.
 *   T          tokens in this call (one chunk of a long prompt), 0 <= T <= 2^20
 *   H          hidden size, a positive multiple of 64
 *   I          expert intermediate size, a positive multiple of 64
 *   E          routed experts, 1..1024
 *   k          experts selected per token, 1..min(E, 32)
 *   n_shared   always-on shared experts, 0 or 1 (same shape as a routed expert)
 *   tile_m_max largest GEMM tile height, a multiple of tile_gran in 16..256
 *   tile_gran  tile height granularity, 16 or 32
 * A slot is (token t, rank j < k) with id t*k + j.  The grouped GEMMs work on
 * Rows = T*k + n_shared*T rows: the routed slots in expert order, then one
 * shared-expert row per token in token order.
 */
typedef struct moe_dims {
  int32_t T, H, I, E, k, n_shared;
  int32_t tile_m_max, tile_gran;
} moe_dims;

/*
 * Weights.  The checkpoint format [LB, "Model structure ..."] of one matrix of
 * N output rows and K inputs is groupwise-affine 4-bit ("canonical layout"):
 *   q [N][K/2] uint8: byte b of a row holds input 2b in its low nibble and
 *                     2b+1 in its high nibble; codes are unsigned 0..15
 *   s, b [N][K/64] bfloat16: scale and bias of each group of 64 consecutive
 *                     inputs of a row
 * and a weight is w = bf16(fma(q, s, b)) (float32 fused multiply-add, rounded
 * once to nearest-even bfloat16).  Gate/up matrices have N = 2I rows (gate
 * rows 0..I-1, up rows I..2I-1) and K = H; down matrices N = H, K = I.
 *
 * How each GEMM kernel forms the weights (the same affine map, two roundings):
 *   - tiles of more than 32 rows (the tall-tile kernels): w = bf16(fma(q, s, b))
 *     as above, each weight rebuilt in registers;
 *   - tiles of at most 32 rows, and every call with at most 16 tokens: the
 *     scale is applied after the product, per group of 64 inputs,
 *     sum_i a_i (q_i s + b) = s sum_i a_i (128 + q_i) + (b - 128 s) sum_i a_i,
 *     with bf16(128 + q) exact, so the weight q s + b is used exactly (never
 *     rounded to bfloat16) and only the float32 sums round.
 * Which kernel serves a row depends on its block's tile height, so a token's
 * output bits can depend on the batch it is in; both forms are held to the
 * same tolerance against the float64 oracle.
 *
 * The GEMMs read the same bytes permuted into a streaming layout, written
 * once by moe_w4_pack: for every 16-row slice and every 128-input step, one
 * 1152-byte block holding the slice's codes in the order the GPU lanes load
 * them (eight inputs per 32-bit word, nibbles regrouped in pairs) followed by
 * the (scale, bias) pairs, with inputs past K padded as code 0, scale 0, bias
 * 0; gate/up slices pair 8 gate rows with their 8 up rows.
 * The packed matrix has moe_w4_packed_bytes(N, K) bytes (4.5 bits per weight
 * when K is a multiple of 128).
 *
 * One bank of n experts, packed (both pointers 16-byte aligned):
 *   gu  n consecutive packed gate/up matrices, moe_w4_packed_bytes(2I, H) each
 *   dn  n consecutive packed down matrices, moe_w4_packed_bytes(H, I) each
 */
typedef struct moe_w4_bank {
  const uint8_t *gu;
  const uint8_t *dn;
} moe_w4_bank;

/*
 * Routing tables written by moe_route and read by the later calls.  All are
 * device arrays owned by the caller (4-byte aligned unless stated).
 *   topk_idx [T][k] int32   selected experts, best first (higher score first,
 *                           equal scores by lower expert index)
 *   topk_w   [T][k] float   softmax over all E scores, restricted to the
 *                           selected experts and renormalised to sum to one
 *   counts   [E]    int32   slots routed to each expert (the histogram)
 *   offsets  [E+1]  int32   exclusive prefix sum of counts; offsets[E] = T*k
 *   sorted_slot [T*k] int32 slot ids in expert order, stable in slot-id order
 *   slot_pos [T*k]  int32   inverse permutation: row of each slot
 *   blocks [moe_max_blocks][4] int32  {group, first row, rows, tile height}:
 *                           groups are experts 0..E-1 then the shared expert
 *                           E; a group of c rows is cut into ceil(c/tile_m_max)
 *                           blocks whose sizes differ by at most one, tile
 *                           height = ceil(c/nb) rounded up to tile_gran
 *   n_blocks [1] int32      entries written to blocks
 *   logits [T][E] float or NULL: exported router scores (diagnostic)
 *   status [1] uint32       device error word (MOE_STATUS_*); moe_route clears
 *                           it, later calls on the stream only set bits
 *   ws, ws_bytes            scratch of at least moe_route_ws_bytes() bytes,
 *                           16-byte aligned, used by moe_route only
 */
typedef struct moe_route_out {
  int32_t *topk_idx;
  float *topk_w;
  int32_t *counts, *offsets;
  int32_t *sorted_slot, *slot_pos;
  int32_t *blocks, *n_blocks;
  float *logits;
  uint32_t *status;
  void *ws;
  size_t ws_bytes;
} moe_route_out;

/* Bytes of one packed matrix of `rows` output rows (a multiple of 16) and K
 * inputs (a multiple of 64); 0 if the sizes are invalid. */
size_t moe_w4_packed_bytes(int32_t rows, int32_t K);

/*
 * moe_w4_pack - one-time repack of n canonical-layout matrices (consecutive in
 * q, s, b) into the streaming layout, n * moe_w4_packed_bytes(rows, K) bytes at
 * `packed`.  gate_up = 1 pairs gate row i with up row rows/2 + i (use it for
 * gate/up matrices), 0 keeps rows in order (down matrices).
 *   q (16-byte aligned), s, b (2-byte aligned), packed (16-byte aligned): device.
 *   rows a positive multiple of 16, K a positive multiple of 64, n >= 0.
 */
int moe_w4_pack(int32_t n, int32_t rows, int32_t K, int32_t gate_up, const uint8_t *q,
                const uint16_t *s, const uint16_t *b, uint8_t *packed, void *stream);

/* MOE_W4_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* Static text for a return code. */
const char *moe_strerror(int code);

/* Upper bound on the block map length for d:
 * floor(T*k / tile_m_max) + min(E, T*k) + n_shared * ceil(T / tile_m_max).
 * Returns -1 if d is invalid. */
int32_t moe_max_blocks(const moe_dims *d);

/* Scratch bytes moe_route needs for d (0 if d is invalid). */
size_t moe_route_ws_bytes(const moe_dims *d);

/*
 * moe_route - router scores, top-k, weights, histogram, prefix scan, scatter and
 * block map, all on the GPU and enqueued with no host synchronisation
 * [LB, "Prefill: ..."], [RL, "Optimizing Prefill Operations"].
 *   x          [T][H] bfloat16 token activations (16-byte aligned)
 *   w_router   [H][E] float32 router weights (row h = weights of input h)
 *   logit_bias [E] float32 added to every token's scores, or NULL
 * Scores are float32 in a fixed order: partial m (0..63) is a fused
 * multiply-add chain from +0 over inputs h = m, m+64, ... in increasing h;
 * the partials are added as a tree (for s = 32..1: p[i] += p[i+s], i < s);
 * then the bias is added.  This makes the selection reproducible bit for bit.
 */
int moe_route(const moe_dims *d, const uint16_t *x, const float *w_router, const float *logit_bias,
              const moe_route_out *out, void *stream);

/*
 * moe_route_no_alloc - moe_route for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same outputs, with the routing
 * scratch taken from an array of MOE_NO_ALLOC_WS_BYTES the library owns on
 * each device instead of out->ws (out->ws and out->ws_bytes are ignored and
 * may be NULL / 0).  It calls no allocator.
 *   - Returns MOE_EWS when the call needs more scratch than the array holds
 *     (moe_route_ws_bytes without the exported-score region: 4 MiB covers up
 *     to 2048 tokens at 256 experts with scores not exported).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one
 *     device (two streams, two threads) race and must be serialised by the
 *     caller.  The kernels clear what they accumulate into, so the contents
 *     left by an earlier call do not matter.
 *   - The array is held for the life of the process on every device the
 *     library is used on.  The first call on a device looks up the array's
 *     device address (a runtime query, not an allocation).
 */
#define MOE_NO_ALLOC_WS_BYTES (4u << 20)
int moe_route_no_alloc(const moe_dims *d, const uint16_t *x, const float *w_router,
                       const float *logit_bias, const moe_route_out *out, void *stream);

/*
 * moe_w4_gate_up - grouped gate/up GEMM with the 4-bit weights reconstructed
 * tile by tile inside the kernel (never written out), float32 accumulation and
 * SwiGLU in the epilogue [LB, "Prefill: ..."].  For every block of the map:
 * h[row] = silu(g) * u, g = W_gate x_t, u = W_up x_t, rounded to bfloat16,
 * where t is the row's token (sorted_slot[row] / k for routed rows,
 * row - T*k for shared rows).
 *   x        [T][H] bfloat16, the same activations given to moe_route
 *   r        tables from moe_route (blocks, n_blocks, sorted_slot, status)
 *   routed   packed bank of E experts;  shared  packed bank of 1 expert, or NULL
 *            if n_shared = 0
 *   h        [Rows][I] bfloat16 output (16-byte aligned)
 */
int moe_w4_gate_up(const moe_dims *d, const uint16_t *x, const moe_route_out *r,
                   const moe_w4_bank *routed, const moe_w4_bank *shared, uint16_t *h,
                   void *stream);

/*
 * moe_w4_down - grouped down GEMM with fused reconstruction:
 * y_slots[row] = W_down h[row], float32 accumulation, rounded to bfloat16.
 *   h        [Rows][I] bfloat16 from moe_w4_gate_up (16-byte aligned)
 *   y_slots  [Rows][H] bfloat16 output (16-byte aligned)
 */
int moe_w4_down(const moe_dims *d, const moe_route_out *r, const moe_w4_bank *routed,
                const moe_w4_bank *shared, const uint16_t *h, uint16_t *y_slots, void *stream);

/* moe_grouped_w4_ffn - moe_w4_gate_up followed by moe_w4_down on one stream. */
int moe_grouped_w4_ffn(const moe_dims *d, const uint16_t *x, const moe_route_out *r,
                       const moe_w4_bank *routed, const moe_w4_bank *shared, uint16_t *h,
                       uint16_t *y_slots, void *stream);

/*
 * Shared-expert overlap.  The shared expert processes every token regardless
 * of routing [RL, "Understanding the Qwen3.6-35B-A3B Model"], so its FFN needs
 * no routing tables and can run on a second stream while moe_route runs on
 * the first.  The pair moe_shared_w4_ffn + moe_routed_w4_ffn writes exactly
 * what moe_grouped_w4_ffn writes (bit for bit: the same kernels compute the
 * same blocks); moe_combine then needs both done (an event from the second
 * stream).
 *
 * moe_shared_w4_ffn - the shared expert's rows of h and y_slots (rows T*k ..
 * T*k+T-1), from x and the shared bank alone.  Requires n_shared = 1
 * (else MOE_EINVAL).  h, y_slots and x as for moe_grouped_w4_ffn.
 */
int moe_shared_w4_ffn(const moe_dims *d, const uint16_t *x, const moe_w4_bank *shared, uint16_t *h,
                      uint16_t *y_slots, void *stream);

/*
 * moe_routed_w4_ffn - moe_grouped_w4_ffn without the shared expert's blocks:
 * the routed rows 0 .. T*k-1 of h and y_slots.  The routing tables must come
 * from moe_route on the same stream.
 */
int moe_routed_w4_ffn(const moe_dims *d, const uint16_t *x, const moe_route_out *r,
                      const moe_w4_bank *routed, uint16_t *h, uint16_t *y_slots, void *stream);

/*
 * moe_combine - weighted top-k combine [RL, "Understanding the Qwen3.6-35B-A3B
 * Model"]: y[t] = sum_j topk_w[t][j] * y_slots[slot_pos[t*k+j]]
 * (+ y_slots[T*k + t] when n_shared = 1), float32, j ascending, shared last,
 * rounded to bfloat16.
 *   y_slots [Rows][H] bfloat16;  y [T][H] bfloat16 output (both 16-byte aligned)
 */
int moe_combine(const moe_dims *d, const moe_route_out *r, const uint16_t *y_slots, uint16_t *y,
                void *stream);

/*
 * moe_w4_ffn_combine - moe_grouped_w4_ffn followed by moe_combine on one
 * stream, with the same outputs bit for bit (h, y_slots and y).  For a single
 * token (T = 1, k + n_shared <= 16, I < 1024) the down GEMM and the combine
 * run as one kernel, which keeps the token's expert outputs on chip between
 * the two [LB, "Decode: eliminating per-token CPU round trips": chains of
 * kernels fused so that intermediates stay in registers].  Arguments, layout
 * and errors as for the two calls together.
 */
int moe_w4_ffn_combine(const moe_dims *d, const uint16_t *x, const moe_route_out *r,
                       const moe_w4_bank *routed, const moe_w4_bank *shared, uint16_t *h,
                       uint16_t *y_slots, uint16_t *y, void *stream);

/*
 * moe_w4_dequant - expand a canonical-layout [rows][K] matrix to bfloat16 in memory,
 * w = bf16(fma(q, s, b)).  Diagnostic: it materialises exactly the array the
 * fused GEMMs avoid, for bit-exactness checks and for the unfused comparison
 * [LB, "Prefill: ..."].
 *   q [rows][K/2] (16-byte aligned), s, b [rows][K/64], out [rows][K] (16-byte aligned)
 *   K a positive multiple of 64, rows >= 0.
 */
int moe_w4_dequant(int32_t rows, int32_t K, const uint8_t *q, const uint16_t *s, const uint16_t *b,
                   uint16_t *out, void *stream);

/*
 * moe_w4_dequant_packed - expand n packed matrices (moe_w4_pack's output for
 * `rows` x K matrices, `gate_up` as given to moe_w4_pack) back to bfloat16 in
 * the canonical [n][rows][K] order, through the packed addressing and the
 * reconstruction w = bf16(fma(q, s, b)) of the tall-tile GEMM kernel.
 * Diagnostic: it checks that kernel's reconstruction bit for bit and gives the
 * unfused comparison its bfloat16 weights.
 *   packed (16-byte aligned) n * moe_w4_packed_bytes(rows, K) bytes;
 *   out [n][rows][K] bfloat16 (16-byte aligned).  Same size rules as
 *   moe_w4_pack.
 */
int moe_w4_dequant_packed(int32_t n, int32_t rows, int32_t K, int32_t gate_up, const uint8_t *packed,
                          uint16_t *out, void *stream);

/*
 * moe_read_probe - measurement aid, not part of the layer: one kernel that
 * reads `bytes` (a multiple of 16) at `src` once, in 16-byte loads spread over
 * `workgroups` workgroups of 256 threads, and writes one folded word per
 * workgroup to sink[workgroups].  Timing it gives the streaming-read ceiling
 * for a weight stream of the same size through the same launch path.
 */
int moe_read_probe(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups, void *stream);

/*
 * moe_mfma_probe - measurement aid, not part of the layer: `workgroups`
 * workgroups of four waves (two per SIMD at two workgroups per CU, as the
 * tall-tile GEMM runs) each issue `iters` rounds of eight independent
 * v_mfma_f32_32x32x16_bf16 on register operands, and lane 0 of each wave
 * writes a folded value to sink[4 * workgroups].  Work:
 * workgroups * 4 * iters * 8 * 32768 flops.  Timing it gives the matrix-core
 * throughput this launch shape reaches with no memory traffic at all.
 * 1 <= workgroups <= 2^20, 1 <= iters <= 2^24; MOE_EINVAL otherwise.
 */
int moe_mfma_probe(int32_t workgroups, int32_t iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_H */
