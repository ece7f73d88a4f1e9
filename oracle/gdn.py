"""Oracle of the Gated DeltaNet recurrent scan (test infrastructure only).

The pages name the operation and its structure but do not write it out: the
model interleaves Gated DeltaNet layers, a fixed-size recurrence, and the
engine keeps the recurrent state on the GPU, each simdgroup carrying one
column of state through the whole scan instead of moving an intermediate of
256 MiB per layer (["Lily Beats MLX-LM 1.35x on Decode", "Model structure and
three workload shapes" and "Prefill: fusing dequantisation and keeping
routing GPU-resident"]).  The recurrence itself is the gated delta rule as
published (S. Yang, J. Kautz, A. Hatamizadeh, "Gated Delta Networks:
Improving Mamba2 with Delta Rule", ICLR 2025), per value head h with state
S in R^{dv x dk}:

    S_t = S_{t-1} * alpha_t * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t,            alpha_t = exp(g_t)

Value head h reads key head h // (Hv / Hk) (consecutive value heads share a
key head).  Everything here is float64 after widening the bfloat16 inputs; the
transition matrix (I - beta k k^T) is formed explicitly and applied as a
matrix product, exactly as the definition reads, with no reordering.  This
module never imports or calls the HIP library.
"""

from __future__ import annotations

import numpy as np


def gated_delta_scan(q, k, v, g, beta, state0=None):
    """q, k [T][Hk][dk], v [T][Hv][dv], g, beta [T][Hv] (any float dtype, widened
    to float64); state0 [Hv][dv][dk] or None for zeros.
    Returns (o [T][Hv][dv], S_T [Hv][dv][dk]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, Hk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    assert q.shape == k.shape and v.shape[0] == T and Hv % Hk == 0
    assert g.shape == (T, Hv) and beta.shape == (T, Hv)
    rep = Hv // Hk
    S = np.zeros((Hv, dv, dk)) if state0 is None else np.array(state0, dtype=np.float64)
    assert S.shape == (Hv, dv, dk)
    eye = np.eye(dk)
    o = np.zeros((T, Hv, dv))
    for t in range(T):
        kt = np.repeat(k[t], rep, axis=0)          # [Hv][dk]: head h reads key head h // rep
        qt = np.repeat(q[t], rep, axis=0)
        alpha = np.exp(g[t])                        # [Hv]
        # transition alpha_t (I - beta_t k_t k_t^T), one dk x dk matrix per head
        trans = alpha[:, None, None] * (eye[None] - beta[t][:, None, None] * kt[:, :, None] * kt[:, None, :])
        write = beta[t][:, None, None] * v[t][:, :, None] * kt[:, None, :]   # beta v k^T
        S = S @ trans + write
        o[t] = np.einsum("hij,hj->hi", S, qt)
    return o, S
