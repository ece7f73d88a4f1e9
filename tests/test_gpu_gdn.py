"""Gated DeltaNet scan on the GPU against the float64 oracle.

Parity bar, from the arithmetic: the kernel keeps the state in float32 and
rounds each output once to bfloat16 (round to nearest even).  That rounding
moves an output by at most half a bfloat16 ulp, which is 2^-8 of the largest
power of two below it.  So, per element, a correct output is within one
bfloat16 ulp of the float64 reference (the rounding plus float32 arithmetic
far below half an ulp), up to float32 noise of 1e-5 of the head's largest
output; per (token, head), the worst error over the head's 128 outputs is
within 2^-8 of the largest reference output there, plus 1e-4 for the float32
arithmetic.  The float32 final state is held to 1e-4 of its largest value per
head.  A wrong index, sign or term moves all three by orders of magnitude
more.  Outputs are written into buffers with guard bytes on both sides,
checked after each call.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import w4_dequant_expert_amd as moe  # noqa: E402
from synth import bf16_bits_to_f32, build_gdn_config  # noqa: E402
from synth.gdn import GdnShape, make_gdn_inputs  # noqa: E402

GUARD, GUARD_BYTE = 256, 0xA5
O_TOL = 2.0 ** -8 + 1e-4
S_TOL = 1e-4


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


class Guarded:
    def __init__(self):
        self.bufs = []

    def __call__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        raw = torch.full((n + 2 * GUARD,), GUARD_BYTE, dtype=torch.uint8, device="cuda")
        self.bufs.append((raw, n))
        t = raw[GUARD:GUARD + n].view(dtype).view(shape)
        if fill is not None:
            t.copy_(fill)
        return t

    def check(self, label):
        torch.cuda.synchronize()
        for raw, n in self.bufs:
            assert bool((raw[:GUARD] == GUARD_BYTE).all()) and bool((raw[GUARD + n:] == GUARD_BYTE).all()), \
                f"{label}: a kernel wrote outside an output buffer"


def f64(bits):
    return bf16_bits_to_f32(np.asarray(bits).view(np.uint16)).astype(np.float64)


METHODS = ("direct", "chunked")


def run_gpu(c, state=None, in_place=False, method="direct"):
    """One gdn_scan (register-resident) or gdn_scan_chunked call; returns
    (o bits [T][Hv][dv], final state)."""
    sh = c["shape"]
    g = Guarded()
    o = g((sh.T, sh.n_v_heads, sh.dv), torch.int16)
    s_in = dev(state) if state is not None else None
    if in_place:
        s_out = g((sh.n_v_heads, sh.dv, sh.dk), torch.float32, fill=s_in)
        s_in = s_out
    else:
        s_out = g((sh.n_v_heads, sh.dv, sh.dk), torch.float32)
    d = moe.GdnDims(sh.T, sh.n_k_heads, sh.n_v_heads, sh.dk, sh.dv)
    args = (d, dev(c["q"]), dev(c["k"]), dev(c["v"]), dev(c["g"]), dev(c["beta"]), s_in, s_out,
            o if sh.T > 0 else None)
    if method == "chunked":
        nbytes = moe.gdn_scan_chunked_ws_bytes(d)
        ws = g((max(nbytes, 1),), torch.uint8)
        moe.gdn_scan_chunked(*args, ws if nbytes else None, nbytes)
    else:
        moe.gdn_scan(*args)
    g.check(f"gdn {method} T={sh.T}")
    return o.cpu().numpy().view(np.uint16), s_out.cpu().numpy()


def reference(c, state=None):
    return oracle.gated_delta_scan(f64(c["q"]), f64(c["k"]), f64(c["v"]), c["g"], c["beta"], state)


def check(label, o_bits, s_gpu, o_ref, s_ref):
    o = f64(o_bits)
    nw = el = 0.0
    if o.size:
        head_max = np.abs(o_ref).max(axis=2, keepdims=True)
        nw = (np.abs(o - o_ref).max(axis=2) / np.maximum(head_max[..., 0], 1e-30)).max()
        # per element, in units of the allowance: one bfloat16 ulp + float32 noise
        el = (np.abs(o - o_ref) / (bf16_ulp(o_ref) + 1e-5 * head_max)).max()
    sden = np.maximum(np.abs(s_ref).max(axis=(1, 2)), 1e-30)
    snw = (np.abs(s_gpu - s_ref).max(axis=(1, 2)) / sden).max()
    note(f"{label}: output error {nw:.3e} (bar {O_TOL:.3e}), per element {el:.3f} of one "
         f"bf16 ulp, state error {snw:.3e} (bar {S_TOL:.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s_gpu))
    assert nw <= O_TOL, nw
    assert el <= 1.0, el
    assert snw <= S_TOL, snw


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("T", [1, 5, 16, 37, 64, 100])
def test_tiny_shapes_against_oracle(T, method):
    """Two key heads, four value heads (heads not a multiple of eight), T
    covering one token, a ragged run of 16, whole chunks of 32 and a tail."""
    note(f"case gdn_tiny T={T} {method}")
    c = build_gdn_config("gdn_tiny", T=T)
    o, s = run_gpu(c, method=method)
    o_ref, s_ref = reference(c)
    check(f"gdn_tiny T={T} {method}", o, s, o_ref, s_ref)


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("Hk,Hv,T", [(8, 8, 70), (4, 16, 33), (1, 8, 48)])
def test_head_groupings(Hk, Hv, T, method):
    """Value heads per key head 1, 4 and 8, with head counts that take the
    XCD-grouped workgroup order."""
    note(f"case gdn heads Hk={Hk} Hv={Hv} T={T} {method}")
    c = make_gdn_inputs(GdnShape(T=T, n_k_heads=Hk, n_v_heads=Hv), seed=21)
    c["shape"] = GdnShape(T=T, n_k_heads=Hk, n_v_heads=Hv)
    o, s = run_gpu(c, method=method)
    o_ref, s_ref = reference(c)
    check(f"gdn Hk={Hk} Hv={Hv} T={T} {method}", o, s, o_ref, s_ref)


@pytest.mark.parametrize("method", METHODS)
def test_initial_state_in_place_and_empty(method):
    note(f"case gdn initial state, in place, T=0 {method}")
    c = build_gdn_config("gdn_tiny", T=45, with_state=True)
    o_ref, s_ref = reference(c, c["state"])
    o, s = run_gpu(c, state=c["state"], method=method)
    check(f"gdn_tiny T=45 with state {method}", o, s, o_ref, s_ref)
    o2, s2 = run_gpu(c, state=c["state"], in_place=True, method=method)
    assert np.array_equal(o2, o) and np.array_equal(s2, s)
    e = build_gdn_config("gdn_tiny", T=0, with_state=True)
    _, s0 = run_gpu(e, state=c["state"], method=method)
    assert np.array_equal(s0, c["state"])
    _, z = run_gpu(e, method=method)
    assert not np.any(z)


def test_split_sequence_matches_one_call():
    """Tokens go through the state in pairs counted from the start of a call.
    Scanning 38 tokens and then 62 more from the returned state pairs the
    tokens exactly as one call over 100 does, so the bits are the same (the
    state is carried exactly in float32).  A split after an odd count (37 +
    63) pairs them differently: both results then stay within the bar."""
    note("case gdn split sequence")
    c = build_gdn_config("gdn_tiny", T=100)
    o, s = run_gpu(c)
    a = build_gdn_config("gdn_tiny", T=38)
    b = build_gdn_config("gdn_tiny", T=62, t0=38)
    oa, sa = run_gpu(a)
    ob, sb = run_gpu(b, state=sa)
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(sb, s)
    a = build_gdn_config("gdn_tiny", T=37)
    b = build_gdn_config("gdn_tiny", T=63, t0=37)
    oa, sa = run_gpu(a)
    ob, sb = run_gpu(b, state=sa)
    o_ref, s_ref = reference(c)
    check("gdn_tiny 37 + 63", np.concatenate([oa, ob]), sb, o_ref, s_ref)


def test_chunked_split_at_chunk_boundary_matches_one_call():
    """The chunked scan splits a sequence at multiples of 32 tokens into the
    same chunks as one call, so 64 + 36 tokens give the bits of one call over
    100."""
    note("case gdn chunked split sequence")
    c = build_gdn_config("gdn_tiny", T=100)
    o, s = run_gpu(c, method="chunked")
    a = build_gdn_config("gdn_tiny", T=64)
    b = build_gdn_config("gdn_tiny", T=36, t0=64)
    oa, sa = run_gpu(a, method="chunked")
    ob, sb = run_gpu(b, state=sa, method="chunked")
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(sb, s)


@pytest.fixture(scope="module")
def prefill2048_ref():
    c = build_gdn_config("gdn_prefill2048")
    return c, reference(c)


@pytest.mark.parametrize("method", METHODS)
def test_prefill2048_full_against_oracle(prefill2048_ref, method):
    """The 2048-token sequence at 16 key and 32 value heads, every output and
    the final state against the oracle."""
    note(f"case gdn_prefill2048 full {method}")
    c, (o_ref, s_ref) = prefill2048_ref
    o, s = run_gpu(c, method=method)
    check(f"gdn_prefill2048 {method}", o, s, o_ref, s_ref)
