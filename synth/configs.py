"""The five workloads of the MoE expert layer, as seeded recipes.

Shapes: the full layer has hidden size 2048, 256 routed experts (top-8) plus one
always-on shared expert of the same shape, expert intermediate size 512; the
tiny layer has hidden 256, 8 experts (top-2) plus one shared expert, intermediate
128.  Weights are groupwise-affine 4-bit (group 64 along the input dimension)
with bfloat16 scale U(0.002, 0.02) and bias -8*scale.  All full-shape workloads
share one weight set, drawn from seed 1.
"""

from __future__ import annotations

import functools
import math
from dataclasses import dataclass

import numpy as np

from . import gen


@dataclass(frozen=True)
class LayerShape:
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # routed experts
    k: int          # experts selected per token
    n_shared: int   # always-on shared experts (0 or 1)


FULL_SHAPE = LayerShape(H=2048, I=512, E=256, k=8, n_shared=1)
TINY_SHAPE = LayerShape(H=256, I=128, E=8, k=2, n_shared=1)

# name -> recipe.  "T" is tokens per layer call; "chunk" splits a long prompt into
# independent calls; "repeats" draws fresh tokens for repeated batch-1 calls.
CONFIGS = {
    "tiny16": dict(shape=TINY_SHAPE, T=16, weight_seed=0, x_seed=0,
                   router_std=0.05, router_seed=0, zipf=None),
    "prefill512": dict(shape=FULL_SHAPE, T=512, weight_seed=1, x_seed=1,
                       router_std=0.02, router_seed=1, zipf=None),
    "prefill2048_zipf": dict(shape=FULL_SHAPE, T=2048, weight_seed=1, x_seed=2,
                             router_std=0.02, router_seed=1, zipf=(1.1, 2)),
    "chunked16384": dict(shape=FULL_SHAPE, T=16384, chunk=2048, weight_seed=1, x_seed=3,
                         router_std=1.0 / math.sqrt(2048), router_seed=3, zipf=None),
    "decode1": dict(shape=FULL_SHAPE, T=1, repeats=1000, weight_seed=1, x_seed=4,
                    router_std=0.02, router_seed=1, zipf=None),
}


@functools.lru_cache(maxsize=4)
def _banks(shape: LayerShape, seed: int):
    routed = gen.make_bank(shape.E, shape.H, shape.I, seed, "routed")
    shared = gen.make_bank(shape.n_shared, shape.H, shape.I, seed, "shared") if shape.n_shared else None
    return routed, shared


def build_config(name: str, T: int | None = None, t0: int = 0, with_weights: bool = True) -> dict:
    """Materialise a workload as numpy arrays.

    T overrides the token count (rows t0..t0+T-1 of the token stream are drawn),
    which is how chunks, repeated decode tokens and reduced-size parity cases
    are produced from the same streams.
    """
    c = CONFIGS[name]
    sh: LayerShape = c["shape"]
    T = c["T"] if T is None else T
    out = dict(name=name, shape=sh, T=T,
               x=gen.make_tokens(T, sh.H, c["x_seed"], "x", t0=t0),
               wr=gen.make_router(sh.H, sh.E, c["router_std"], c["router_seed"]),
               bias=None)
    if c["zipf"] is not None:
        s, seed = c["zipf"]
        out["bias"] = gen.make_zipf_bias(sh.E, s, seed)
    if with_weights:
        out["routed"], out["shared"] = _banks(sh, c["weight_seed"])
    return out


def bank_nbytes(shape: LayerShape) -> int:
    """Bytes of one expert's packed codes plus scales and biases."""
    w = 3 * shape.H * shape.I
    return w // 2 + (w // 64) * 4


__all__ = ["LayerShape", "FULL_SHAPE", "TINY_SHAPE", "CONFIGS", "build_config", "bank_nbytes",
           "np"]
