"""Counter-based random streams and tensor recipes.

Generator: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014).  A stream is named by
(seed, name); its i-th 64-bit output is mix64(key + (i + 1) * GAMMA), i.e. the
SplitMix64 sequence started from state ``key``.  Every element of every tensor
is therefore a pure function of (seed, name, index) and any slice can be drawn
without drawing what comes before it.

Uniform doubles take the top 53 bits.  Normals use the Box-Muller transform
(Box & Muller, 1958) on the pair of uniforms at stream indices 2i and 2i+1.
Values are rounded once, to nearest-even, straight from float64 to the target
type (bfloat16 or float32), never through an intermediate format.
"""

from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64_mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _fnv1a64(name: str) -> int:
    h = 0xCBF29CE484222325
    for byte in name.encode("utf-8"):
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def stream_key(seed: int, name: str) -> np.uint64:
    """Starting state of the stream (seed, name)."""
    h = splitmix64_mix(np.array([_fnv1a64(name)], dtype=np.uint64))[0]
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    return splitmix64_mix(np.array([s ^ h], dtype=np.uint64))[0]


def stream_u64(seed: int, name: str, n: int, offset: int = 0) -> np.ndarray:
    """Outputs offset .. offset+n-1 of stream (seed, name) as uint64."""
    key = stream_key(seed, name)
    idx = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = key + idx * GAMMA
    return splitmix64_mix(state)


def uniform(seed: int, name: str, n: int, offset: int = 0) -> np.ndarray:
    """Uniform doubles in [0, 1) from the top 53 bits of each output."""
    u = stream_u64(seed, name, n, offset)
    return (u >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(seed: int, name: str, n: int, offset: int = 0) -> np.ndarray:
    """Standard normals; element i uses uniforms 2i and 2i+1 (Box-Muller, cosine branch)."""
    u = uniform(seed, name, 2 * n, 2 * offset)
    u1 = u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))  # 1 - u1 lies in (0, 1]
    return r * np.cos(2.0 * np.pi * u2)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to nearest-even bfloat16, returned as uint16 bit patterns.

    Only finite values inside the normal float32 range (or zero) are accepted;
    every recipe here stays far inside it.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value")
    a = np.abs(v)
    if np.any((a != 0) & ((a < 2.0 ** -126) | (a >= 2.0 ** 127))):
        raise ValueError("value outside the normal bfloat16 range")
    m, e = np.frexp(v)                      # v = m * 2**e, 0.5 <= |m| < 1
    r = np.round(m * 256.0) / 256.0         # 8 significant bits, ties to even
    q = np.ldexp(r, e).astype(np.float32)   # exact: q is representable in bf16
    return (q.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def random_bytes(seed: int, name: str, nbytes: int) -> np.ndarray:
    """nbytes uniform random bytes: the stream's 64-bit outputs, little-endian."""
    n64 = (nbytes + 7) // 8
    u = stream_u64(seed, name, n64).astype("<u8")
    return u.view(np.uint8)[:nbytes].copy()


def make_bank(n: int, H: int, I: int, seed: int, prefix: str,
              s_lo: float = 0.002, s_hi: float = 0.02) -> dict:
    """Groupwise-affine 4-bit expert weights for n experts.

    Layout (row-major, every row split into groups of 64 consecutive
    input-dimension elements):
      gu_q [n][2I][H/2]  uint8: rows 0..I-1 gate, I..2I-1 up; byte b of a row
                               holds element 2b in its low nibble, 2b+1 high
      gu_s, gu_b [n][2I][H/64] bfloat16 bits
      dn_q [n][H][I/2], dn_s, dn_b [n][H][I/64]
    Codes are uniform on 0..15 (uniform random bytes), scales are
    U(s_lo, s_hi) rounded to bfloat16, and bias = -8 * scale (exact).
    """
    assert H % 64 == 0 and I % 64 == 0
    out = {}
    for part, rows, K in (("gu", 2 * I, H), ("dn", H, I)):
        q = np.empty((n, rows, K // 2), dtype=np.uint8)
        s = np.empty((n, rows, K // 64), dtype=np.uint16)
        for e in range(n):
            q[e] = random_bytes(seed, f"{prefix}.{e}.{part}_q", rows * K // 2).reshape(rows, K // 2)
            u = uniform(seed, f"{prefix}.{e}.{part}_s", rows * (K // 64))
            s[e] = f64_to_bf16_bits(s_lo + (s_hi - s_lo) * u).reshape(rows, K // 64)
        sf = bf16_bits_to_f32(s).astype(np.float64)
        b = f64_to_bf16_bits(-8.0 * sf)
        out[f"{part}_q"] = q
        out[f"{part}_s"] = s
        out[f"{part}_b"] = b
    return out


def make_router(H: int, E: int, std: float, seed: int, name: str = "router") -> np.ndarray:
    """Router weights, float32 [H][E] (row h holds the weights of input h), N(0, std^2)."""
    return (std * normal(seed, name, H * E)).astype(np.float32).reshape(H, E)


def make_zipf_bias(E: int, s: float, seed: int, name: str = "zipf_perm") -> np.ndarray:
    """Per-expert logit bias -s*ln(rank), rank a seeded Fisher-Yates permutation of 1..E.

    exp(bias) is proportional to the Zipf(s) mass of the expert's rank; the
    normaliser is a common additive constant on every logit and is dropped.
    """
    a = np.arange(1, E + 1, dtype=np.int64)
    u = uniform(seed, name, max(E - 1, 0))
    for n_step in range(E - 1):
        i = E - 1 - n_step
        j = min(int(u[n_step] * (i + 1)), i)
        a[i], a[j] = a[j], a[i]
    return (-s * np.log(a.astype(np.float64))).astype(np.float32)


def make_tokens(T: int, H: int, seed: int, name: str = "x", t0: int = 0) -> np.ndarray:
    """Token activations rows t0..t0+T-1 of stream (seed, name): N(0,1) -> bfloat16 bits [T][H]."""
    v = normal(seed, name, T * H, offset=t0 * H)
    return f64_to_bf16_bits(v).reshape(T, H)
