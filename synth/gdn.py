"""Seeded inputs of the Gated DeltaNet recurrent scan (numbers only).

Shapes follow the linear-attention layers of the model family the pages
describe: 16 key heads and 32 value heads of width 128 (two value heads read
each key head), one sequence.  Recipe, per token:
  k  N(0, 1) per element, scaled to unit L2 norm per head, then bfloat16;
  q  the same, then times 128^-1/2, then bfloat16;
  v  N(0, 1), bfloat16;
  beta  logistic of N(0, 1), float32 (strictly inside (0, 1));
  g  -softplus(N(0, 1) - 3), float32: the log of the per-token decay, so the
     decay exp(g) mostly sits near 0.95 with a tail down to about 0.5.
The normalisation and the two squashing functions shape the input
distribution the way the layer's projections feed the scan; none of the
scan's own arithmetic is here.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import gen


@dataclass(frozen=True)
class GdnShape:
    T: int
    n_k_heads: int
    n_v_heads: int
    dk: int = 128
    dv: int = 128


GDN_CONFIGS = {
    "gdn_tiny": dict(shape=GdnShape(T=37, n_k_heads=2, n_v_heads=4), seed=11),
    "gdn_prefill2048": dict(shape=GdnShape(T=2048, n_k_heads=16, n_v_heads=32), seed=12),
}


def _unit_rows(seed: int, name: str, rows: int, width: int, scale: float) -> np.ndarray:
    a = gen.normal(seed, name, rows * width).reshape(rows, width)
    a = a / np.sqrt(np.sum(a * a, axis=1, keepdims=True)) * scale
    return gen.f64_to_bf16_bits(a)


def make_gdn_inputs(shape: GdnShape, seed: int, t0: int = 0, with_state: bool = False) -> dict:
    """bfloat16 bits for q, k [T][Hk][dk] and v [T][Hv][dv]; float32 g and beta
    [T][Hv]; tokens t0 .. t0+T-1 of the seeded streams.  with_state adds a
    float32 initial state [Hv][dv][dk] drawn from N(0, 0.1^2)."""
    T, Hk, Hv, dk, dv = shape.T, shape.n_k_heads, shape.n_v_heads, shape.dk, shape.dv
    out = {}
    for name, scale in (("k", 1.0), ("q", dk ** -0.5)):
        rows = _unit_rows(seed, f"gdn.{name}", (t0 + T) * Hk, dk, scale)[t0 * Hk:]
        out[name] = rows.reshape(T, Hk, dk)
    out["v"] = gen.f64_to_bf16_bits(gen.normal(seed, "gdn.v", T * Hv * dv, t0 * Hv * dv)).reshape(T, Hv, dv)
    z = gen.normal(seed, "gdn.beta", T * Hv, t0 * Hv)
    out["beta"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32).reshape(T, Hv)
    z = gen.normal(seed, "gdn.g", T * Hv, t0 * Hv) - 3.0
    out["g"] = (-np.logaddexp(0.0, z)).astype(np.float32).reshape(T, Hv)
    if with_state:
        out["state"] = (0.1 * gen.normal(seed, "gdn.state", Hv * dv * dk)).astype(np.float32).reshape(Hv, dv, dk)
    return out


def build_gdn_config(name: str, T: int | None = None, t0: int = 0, with_state: bool = False) -> dict:
    c = GDN_CONFIGS[name]
    sh = c["shape"]
    if T is not None:
        sh = GdnShape(T=T, n_k_heads=sh.n_k_heads, n_v_heads=sh.n_v_heads, dk=sh.dk, dv=sh.dv)
    d = make_gdn_inputs(sh, c["seed"], t0=t0, with_state=with_state)
    d["shape"] = sh
    return d
