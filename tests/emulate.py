"""A CPU model of the HIP layer's rounding pipeline (test infrastructure only).

The oracle computes the layer as the pages define it: bfloat16-reconstructed
weights and float64 arithmetic after them.  The GPU path rounds in a few more
places, by design:
  - h, the SwiGLU output, is stored as bfloat16: it is the A operand of the
    down GEMM's bfloat16 matrix instructions;
  - y_slots, the per-slot expert outputs, are stored as bfloat16 (a bandwidth
    choice: they are written once and read once by the combine);
  - the combine runs in float32 (fused multiply-adds, slots in rank order,
    shared expert last) and rounds y once to bfloat16;
  - kernels that apply the group scale after the product (tiles of at most 32
    rows, and every batch of at most 16 tokens) use the affine weight
    q*s + b exactly, never rounded to bfloat16; the tall-tile kernel rounds
    each reconstructed weight to bfloat16 as the pages describe.
This module reproduces those roundings on the CPU (float64 sums stand in for
the float32 accumulators), so that a test can tell how far from the oracle a
correct kernel is expected to land on the same tokens.  It shares nothing with
the HIP code: weights are unpacked here from the checkpoint layout, and the
kernel that serves a block follows the documented dispatch rule below.
"""

from __future__ import annotations

import numpy as np

from synth import bf16_bits_to_f32

SMALL_TILE = 32     # blocks with tile height <= this use the scale-after kernels
SHORT_BATCH = 16    # batches of at most this many tokens use the short-batch kernel


def bf16_round(v) -> np.ndarray:
    """Round to float32, then to nearest-even bfloat16 (returned as float64)."""
    u = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_round(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def weights(q, s, b, exact: bool) -> np.ndarray:
    """[rows][K] weights of a checkpoint-layout matrix: q*s + b exactly, or its
    float32 fused multiply-add rounded once to bfloat16."""
    rows, half = q.shape
    codes = np.empty((rows, 2 * half), dtype=np.float64)
    codes[:, 0::2] = q & 0x0F
    codes[:, 1::2] = q >> 4
    sf = np.repeat(bf16_bits_to_f32(s).astype(np.float64), 64, axis=1)
    bf = np.repeat(bf16_bits_to_f32(b).astype(np.float64), 64, axis=1)
    w = codes * sf + bf        # exact in float64 (a 4-bit code times a bfloat16)
    return w if exact else bf16_round(w)


def exact_weights_per_block(T, k, E, tile_m_max, blocks) -> np.ndarray:
    """For each block of the map: True where its kernel applies the scale after
    the product (exact weights), False for the tall-tile rebuild."""
    blocks = np.asarray(blocks).reshape(-1, 4)
    if T <= SHORT_BATCH:
        return np.ones(len(blocks), dtype=bool)
    # blocks of at most 32 rows take the scale-after product in whichever
    # kernel serves them (the tall-tile kernel too, when it takes every block)
    return blocks[:, 3] <= SMALL_TILE


def _keep(v):
    return np.asarray(v, dtype=np.float64)


def row_weight_forms(T, k, E, n_rows, tile_m_max, blocks) -> np.ndarray:
    """Per grouped-GEMM row: True where its block's kernel uses exact weights."""
    blocks = np.asarray(blocks).reshape(-1, 4)
    ex_blk = exact_weights_per_block(T, k, E, tile_m_max, blocks)
    row_exact = np.zeros(n_rows, dtype=bool)
    for (g, r0, rows, tm), e in zip(blocks.tolist(), ex_blk):
        row_exact[r0:r0 + rows] = e
    return row_exact


def expert_rows(xf, want, row_exact, routed, shared, y_slots_bf16=True, rounded=True):
    """Emulated h and y_slots of grouped-GEMM rows.  want: (row, token, expert)
    triples, expert E = the shared expert; xf: the tokens as float64."""
    rnd_bf16 = bf16_round if rounded else _keep
    rnd_f32 = f32_round if rounded else _keep
    E = routed["gu_q"].shape[0]
    I = routed["gu_q"].shape[1] // 2
    groups = {}
    for r, t, e in want:
        groups.setdefault((e, bool(row_exact[r])), []).append((r, t))
    h_rows, ys_rows = {}, {}
    for (e, ex), members in groups.items():
        bank, ee = (routed, e) if e < E else (shared, 0)
        gu = weights(bank["gu_q"][ee], bank["gu_s"][ee], bank["gu_b"][ee], ex)
        dn = weights(bank["dn_q"][ee], bank["dn_s"][ee], bank["dn_b"][ee], ex)
        a = xf[[t for _, t in members]]
        g = a @ gu[:I].T
        u = a @ gu[I:].T
        h = rnd_bf16(g / (1.0 + np.exp(-g)) * u)
        ys = h @ dn.T
        ys = rnd_bf16(ys) if y_slots_bf16 else rnd_f32(ys)
        for i, (r, _) in enumerate(members):
            h_rows[r] = h[i]
            ys_rows[r] = ys[i]
    return h_rows, ys_rows


def layer(x, route, routed, shared, tile_m_max, tokens=None, y_slots_bf16=True,
          exact=None, rounded=True):
    """Emulated bfloat16 output y (float64 values) for the listed tokens.

    route: the oracle's routing dict (topk_idx, topk_w, sorted_slot,
    slot_pos, blocks).  exact: None follows the dispatch rule; True/False
    forces one weight form for every row.  y_slots_bf16=False keeps y_slots
    in float32.  rounded=False drops every rounding after the weights (h,
    y_slots, the combine and y stay float64).  Returns (y, h_rows, ys_rows)
    where h_rows / ys_rows map a grouped-GEMM row to its emulated h / y_slots.
    """
    rnd_bf16 = bf16_round if rounded else _keep
    rnd_f32 = f32_round if rounded else _keep
    x = np.asarray(x)
    T, H = x.shape
    idx, w = route["topk_idx"], route["topk_w"]
    k = idx.shape[1]
    E = routed["gu_q"].shape[0]
    I = routed["gu_q"].shape[1] // 2
    Sk = T * k
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    n_rows = Sk + (T if shared is not None else 0)
    row_exact = row_weight_forms(T, k, E, n_rows, tile_m_max, route["blocks"])
    if exact is not None:
        row_exact[:] = bool(exact)
    xf = bf16_bits_to_f32(x).astype(np.float64)

    # the grouped-GEMM rows of the listed tokens
    want = []
    for t in tokens:
        for j in range(k):
            want.append((int(route["slot_pos"][t * k + j]), int(t), int(idx[t, j])))
        if shared is not None:
            want.append((Sk + int(t), int(t), E))
    h_rows, ys_rows = expert_rows(xf, want, row_exact, routed, shared, y_slots_bf16, rounded)
    y = np.empty((len(tokens), H))
    for n, t in enumerate(tokens):
        acc = np.zeros(H)
        for j in range(k):
            wj = float(np.float32(w[t, j])) if rounded else float(w[t, j])
            acc = rnd_f32(wj * ys_rows[int(route["slot_pos"][t * k + j])] + acc)
        if shared is not None:
            acc = rnd_f32(acc + ys_rows[Sk + int(t)])
        y[n] = rnd_bf16(acc)
    return y, h_rows, ys_rows
