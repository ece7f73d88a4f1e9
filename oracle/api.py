"""ctypes wrapper around the C++ oracle (test infrastructure only).

Every function takes and returns numpy arrays.  Shapes follow the packed
layout of the weights: gu_q [n][2I][H/2] uint8, gu_s/gu_b [n][2I][H/64] bf16
bits, dn_q [n][H][I/2], dn_s/dn_b [n][H][I/64].
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-pthread", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _threads(n):
    if n is not None:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


def router_logits(x, wr, bias=None, nthreads=None):
    """float32 logits [T][E] in the fixed evaluation order (64 strided partials, then a tree)."""
    lib = load()
    x = _c(x, np.uint16)
    wr = _c(wr, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = wr.shape[1]
    out = np.empty((T, E), dtype=np.float32)
    lib.orc_router_logits(T, H, E, _p(x), _p(wr), _p(bias), _p(out), _threads(nthreads))
    return out


def router_logits_f64(x, wr, bias=None, nthreads=None):
    lib = load()
    x = _c(x, np.uint16)
    wr = _c(wr, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = wr.shape[1]
    out = np.empty((T, E), dtype=np.float64)
    lib.orc_router_logits_f64(T, H, E, _p(x), _p(wr), _p(bias), _p(out), _threads(nthreads))
    return out


def topk(logits, k):
    """(idx int32 [T][k], w float64 [T][k]) from float32 logits."""
    lib = load()
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib.orc_topk(T, E, k, _p(logits), _p(idx), _p(w))
    return idx, w


def route_tables(idx, E):
    """(counts [E], offsets [E+1], sorted_slot [T*k], slot_pos [T*k])."""
    lib = load()
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    ss = np.empty(T * k, dtype=np.int32)
    sp = np.empty(T * k, dtype=np.int32)
    lib.orc_route_tables(T, E, k, _p(idx), _p(counts), _p(offsets), _p(ss), _p(sp))
    return counts, offsets, ss, sp


def max_blocks(T, E, k, n_shared, tile_m_max):
    lib = load()
    lib.orc_max_blocks.restype = ctypes.c_int32
    return int(lib.orc_max_blocks(T, E, k, n_shared, tile_m_max))


def block_map(T, E, k, n_shared, tile_m_max, tile_gran, counts, offsets):
    """blocks int32 [n_blocks][4] = {group, first row, rows, tile height}."""
    lib = load()
    lib.orc_block_map.restype = ctypes.c_int32
    mb = max_blocks(T, E, k, n_shared, tile_m_max)
    blocks = np.zeros((max(mb, 1), 4), dtype=np.int32)
    counts = _c(counts, np.int32)
    offsets = _c(offsets, np.int32)
    n = lib.orc_block_map(T, E, k, n_shared, tile_m_max, tile_gran, _p(counts), _p(offsets),
                          _p(blocks), mb)
    if n < 0:
        raise RuntimeError("block map exceeded its bound")
    return blocks[:n].copy()


def dequant(q, s, b):
    """Reconstructed weights (float32 holding bfloat16 values) of a [rows][K] packed matrix."""
    lib = load()
    q = _c(q, np.uint8)
    s = _c(s, np.uint16)
    b = _c(b, np.uint16)
    rows, half = q.shape
    K = 2 * half
    out = np.empty((rows, K), dtype=np.float32)
    lib.orc_dequant(rows, K, _p(q), _p(s), _p(b), _p(out))
    return out


def f32_to_bf16(v):
    lib = load()
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    v = np.asarray(v, dtype=np.float32).ravel()
    return np.array([lib.orc_f32_to_bf16(float(a)) for a in v], dtype=np.uint16)


def expert_ffn(x_row, bank, e):
    """(h float64 [I], y float64 [H]) of expert e of a bank on one bf16 token row."""
    lib = load()
    x_row = _c(x_row, np.uint16)
    H = x_row.shape[0]
    I = bank["gu_q"].shape[1] // 2
    parts = [np.ascontiguousarray(bank[n][e]) for n in ("gu_q", "gu_s", "gu_b", "dn_q", "dn_s", "dn_b")]
    h = np.empty(I, dtype=np.float64)
    y = np.empty(H, dtype=np.float64)
    lib.orc_expert_ffn(H, I, _p(x_row), *[_p(a) for a in parts], _p(h), _p(y))
    return h, y


def moe_layer(x, idx, w, routed, shared, tokens=None, nthreads=None):
    """float64 layer output for the listed tokens (all tokens if None)."""
    lib = load()
    x = _c(x, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    T, H = x.shape
    k = idx.shape[1]
    E = routed["gu_q"].shape[0]
    I = routed["gu_q"].shape[1] // 2
    r = [_c(routed[n], None) for n in ("gu_q", "gu_s", "gu_b", "dn_q", "dn_s", "dn_b")]
    n_shared = 0 if shared is None else 1
    if shared is None:
        s = [None] * 6
    else:
        s = [_c(shared[n][0], None) for n in ("gu_q", "gu_s", "gu_b", "dn_q", "dn_s", "dn_b")]
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if tok is None else tok.shape[0]
    y = np.empty((n, H), dtype=np.float64)
    lib.orc_moe_layer(T, H, I, E, k, n_shared, _p(x), _p(idx), _p(w), *[_p(a) for a in r],
                      *[_p(a) for a in s], n, _p(tok), _p(y), _threads(nthreads))
    return y


def route(x, wr, bias, k, n_shared, tile_m_max, tile_gran, nthreads=None):
    """Every routing output of one layer call, as a dict of numpy arrays."""
    logits = router_logits(x, wr, bias, nthreads)
    idx, w = topk(logits, k)
    E = wr.shape[1]
    T = x.shape[0]
    counts, offsets, ss, sp = route_tables(idx, E)
    blocks = block_map(T, E, k, n_shared, tile_m_max, tile_gran, counts, offsets)
    return dict(logits=logits, topk_idx=idx, topk_w=w, counts=counts, offsets=offsets,
                sorted_slot=ss, slot_pos=sp, blocks=blocks)


def relative_error(y, y_ref):
    """Normwise relative error, worst token: max_t max_i |y - y_ref| / max_i |y_ref[t, i]|.

    This is the layer-output metric the parity tests gate at 1e-2.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.size == 0:
        return 0.0
    y = y.reshape(-1, y.shape[-1])
    y_ref = y_ref.reshape(-1, y_ref.shape[-1])
    num = np.max(np.abs(y - y_ref), axis=1)
    den = np.max(np.abs(y_ref), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def relative_error_elementwise(y, y_ref):
    """Diagnostic: max over (t, i) of |y - y_ref| / max(|y_ref[t,i]|, rms(y_ref[t,:]))."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.size == 0:
        return 0.0
    y = y.reshape(-1, y.shape[-1])
    y_ref = y_ref.reshape(-1, y_ref.shape[-1])
    rms = np.sqrt(np.mean(y_ref * y_ref, axis=1, keepdims=True))
    den = np.maximum(np.abs(y_ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y - y_ref) / den))
