"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments with the documented codes before any launch."""

import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import pytest

import w4_dequant_expert_amd as moe
from w4_dequant_expert_amd.moe import Bank, Dims, RouteOut

INCLUDE = os.path.join(ROOT, "include")


def declared_functions():
    """Every function declared in include/*.h (comments stripped)."""
    names = set()
    for fn in sorted(os.listdir(INCLUDE)):
        if fn.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, fn)).read(), flags=re.S)
            names.update(re.findall(r"\b((?:moe|gdn)_\w+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "moe_route" in names and "moe_combine" in names and "moe_grouped_w4_ffn" in names
    assert "gdn_scan" in names
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(moe.EXPORTED) == names


def test_version_and_strerror():
    header = open(os.path.join(ROOT, "include", "moe_w4.h")).read()
    m = re.search(r"#define MOE_W4_ABI_VERSION (\d+)", header)
    assert m and moe.moe_abi_version() == int(m.group(1))
    for code in (0, -1, -2, -3, -4, -5):
        assert moe.strerror(code) and moe.strerror(code) != "unknown error"


def full(T=512):
    return moe.make_dims(T, 2048, 512, 256, 8, 1, 128, 16)


def test_max_blocks_and_workspace():
    import oracle
    for T in (0, 1, 16, 512, 2048):
        d = full(T)
        assert moe.moe_max_blocks(d) == oracle.max_blocks(T, 256, 8, 1, 128)
    d = full(2048)
    assert moe.moe_route_ws_bytes(d) >= 2048 * 256 * 4 + 2 * 64 * 256 * 4
    assert moe.moe_max_blocks(moe.make_dims(4, 64, 64, 8, 9, 0)) == -1      # k > E
    assert moe.moe_route_ws_bytes(moe.make_dims(4, 100, 64, 8, 2, 0)) == 0  # H % 64


@pytest.mark.parametrize("field,value", [("H", 96), ("I", 0), ("E", 0), ("E", 2000), ("k", 0),
                                         ("k", 33), ("n_shared", 2), ("tile_m_max", 24),
                                         ("tile_m_max", 272), ("tile_gran", 8), ("T", -1)])
def test_invalid_dims_rejected(field, value):
    d = full(4)
    setattr(d, field, value)
    assert moe.moe_max_blocks(d) == -1
    out = RouteOut(*([0x1000] * 11), 1 << 30)
    rc = moe.lib().moe_route(ctypes.byref(d), 0x1000, 0x1000, None, ctypes.byref(out), None)
    assert rc == moe.moe.MOE_EINVAL


def _route_out(ws_bytes=1 << 30, base=0x10000):
    return RouteOut(*[base + 256 * i for i in range(11)], ws_bytes)


def test_route_validation_codes():
    L = moe.lib()
    d = full(4)
    out = _route_out()
    assert L.moe_route(ctypes.byref(d), None, 0x1000, None, ctypes.byref(out), None) == -1
    assert L.moe_route(ctypes.byref(d), 0x1008, 0x1000, None, ctypes.byref(out), None) == -2
    assert L.moe_route(ctypes.byref(d), 0x1000, 0x1002, None, ctypes.byref(out), None) == -2
    small = _route_out(ws_bytes=16)
    assert L.moe_route(ctypes.byref(d), 0x1000, 0x1000, None, ctypes.byref(small), None) == -3
    bad = _route_out()
    bad.blocks = 0x10004                     # block map needs 16-byte alignment
    assert L.moe_route(ctypes.byref(d), 0x1000, 0x1000, None, ctypes.byref(bad), None) == -2
    nul = _route_out()
    nul.status = None
    assert L.moe_route(ctypes.byref(d), 0x1000, 0x1000, None, ctypes.byref(nul), None) == -1
    # T = 0 is a valid no-op and touches nothing
    d0 = full(0)
    assert L.moe_route(ctypes.byref(d0), 0x1000, 0x1000, None, ctypes.byref(out), None) == 0


def test_ffn_and_combine_validation_codes():
    L = moe.lib()
    d = full(4)
    out = _route_out()
    bank = Bank(0x2000, 0x3000)
    assert L.moe_w4_gate_up(ctypes.byref(d), 0x1000, ctypes.byref(out), ctypes.byref(bank),
                            None, 0x8000, None) == -1          # shared bank missing
    mis = Bank(0x2008, 0x3000)
    assert L.moe_w4_gate_up(ctypes.byref(d), 0x1000, ctypes.byref(out), ctypes.byref(mis),
                            ctypes.byref(bank), 0x8000, None) == -2
    assert L.moe_w4_down(ctypes.byref(d), ctypes.byref(out), ctypes.byref(bank),
                         ctypes.byref(bank), 0x8000, 0x9004, None) == -2
    assert L.moe_grouped_w4_ffn(ctypes.byref(d), 0x1000, ctypes.byref(out), ctypes.byref(bank),
                                ctypes.byref(bank), 0x8000, None, None) == -1
    assert L.moe_combine(ctypes.byref(d), ctypes.byref(out), 0x1000, 0x1001, None) == -2
    assert L.moe_w4_ffn_combine(ctypes.byref(d), 0x1000, ctypes.byref(out), ctypes.byref(bank),
                                ctypes.byref(bank), 0x8000, 0x9000, None, None) == -1   # y missing
    assert L.moe_w4_ffn_combine(ctypes.byref(d), 0x1000, ctypes.byref(out), ctypes.byref(bank),
                                ctypes.byref(bank), 0x8000, 0x9000, 0xA008, None) == -2
    d0 = full(0)
    assert L.moe_w4_ffn_combine(ctypes.byref(d0), 0x1000, ctypes.byref(out), ctypes.byref(bank),
                                ctypes.byref(bank), 0x8000, 0x9000, 0xA000, None) == 0
    assert L.moe_grouped_w4_ffn(ctypes.byref(d0), 0x1000, ctypes.byref(out), ctypes.byref(bank),
                                ctypes.byref(bank), 0x8000, 0x9000, None) == 0
    assert L.moe_w4_dequant(4, 100, 0x1000, 0x2000, 0x3000, 0x4000, None) == -1
    assert L.moe_w4_dequant(0, 64, 0x1000, 0x2000, 0x3000, 0x4000, None) == 0


def test_split_ffn_validation_codes():
    L = moe.lib()
    d = full(4)
    out = _route_out()
    bank = Bank(0x2000, 0x3000)
    mis = Bank(0x2008, 0x3000)
    # the shared-expert half: needs n_shared = 1, a bank and aligned buffers
    d_noshared = moe.make_dims(4, 2048, 512, 256, 8, 0, 128, 16)
    assert L.moe_shared_w4_ffn(ctypes.byref(d_noshared), 0x1000, ctypes.byref(bank), 0x8000,
                               0x9000, None) == -1
    assert L.moe_shared_w4_ffn(ctypes.byref(d), 0x1000, None, 0x8000, 0x9000, None) == -1
    assert L.moe_shared_w4_ffn(ctypes.byref(d), 0x1000, ctypes.byref(mis), 0x8000, 0x9000, None) == -2
    assert L.moe_shared_w4_ffn(ctypes.byref(d), 0x1000, ctypes.byref(bank), None, 0x9000, None) == -1
    assert L.moe_shared_w4_ffn(ctypes.byref(d), 0x1008, ctypes.byref(bank), 0x8000, 0x9000, None) == -2
    # the routed half: routing tables and the routed bank, no shared bank
    assert L.moe_routed_w4_ffn(ctypes.byref(d), 0x1000, ctypes.byref(out), None, 0x8000, 0x9000,
                               None) == -1
    assert L.moe_routed_w4_ffn(ctypes.byref(d), 0x1000, None, ctypes.byref(bank), 0x8000, 0x9000,
                               None) == -1
    assert L.moe_routed_w4_ffn(ctypes.byref(d), 0x1000, ctypes.byref(out), ctypes.byref(bank),
                               0x8000, 0x9004, None) == -2
    d0 = full(0)
    assert L.moe_shared_w4_ffn(ctypes.byref(d0), 0x1000, ctypes.byref(bank), 0x8000, 0x9000, None) == 0
    assert L.moe_routed_w4_ffn(ctypes.byref(d0), 0x1000, ctypes.byref(out), ctypes.byref(bank),
                               0x8000, 0x9000, None) == 0


def test_pack_sizes_and_validation():
    L = moe.lib()
    # one 1152-byte block per (16-row slice, 128-input step)
    assert moe.moe_w4_packed_bytes(1024, 2048) == 64 * 16 * 1152
    assert moe.moe_w4_packed_bytes(1024, 2048) * 8 == 1024 * 2048 * 4.5
    assert moe.moe_w4_packed_bytes(2048, 512) == 128 * 4 * 1152
    assert moe.moe_w4_packed_bytes(16, 64) == 1152          # K tail padded to a full step
    assert moe.moe_w4_packed_bytes(24, 64) == 0             # rows not a multiple of 16
    assert moe.moe_w4_packed_bytes(16, 96) == 0             # K not a multiple of 64
    assert L.moe_w4_pack(1, 16, 64, 2, 0x1000, 0x2000, 0x3000, 0x4000, None) == -1
    assert L.moe_w4_pack(1, 16, 64, 0, 0x1008, 0x2000, 0x3000, 0x4000, None) == -2
    assert L.moe_w4_pack(1, 16, 64, 0, 0x1000, 0x2000, 0x3000, 0x4008, None) == -2
    assert L.moe_w4_pack(0, 16, 64, 0, 0x1000, 0x2000, 0x3000, 0x4000, None) == 0


def test_route_workspace_never_shrinks_with_T():
    """A workspace sized for a batch bound fits every smaller batch: the bytes
    needed are non-decreasing in T (the short-batch path's class sums included)."""
    for E, k in ((8, 2), (256, 8), (300, 8), (1024, 4)):
        prev = 0
        for T in list(range(0, 70)) + [100, 511, 512, 513, 2048, 4096]:
            n = moe.moe_route_ws_bytes(moe.make_dims(T, 256, 128, E, k, 1, 32, 16))
            assert n >= prev, (E, T, n, prev)
            prev = n


def test_block_bound_covers_1024_experts_with_shared():
    """moe_max_blocks at the largest expert count with a shared expert
    matches the oracle's bound (1025 groups)."""
    import oracle
    for T in (1, 5, 64, 300):
        d = moe.make_dims(T, 128, 64, 1024, 4, 1, 16, 16)
        assert moe.moe_max_blocks(d) == oracle.max_blocks(T, 1024, 4, 1, 16)


def test_gdn_scan_validation_codes():
    """gdn_scan rejects bad shapes, null and misaligned pointers before any
    launch; T = 0 with no output state enqueues nothing."""
    from w4_dequant_expert_amd.moe import GdnDims
    L = moe.lib()
    q, k, v, g, b, si, so, o = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000, 0x70000, 0x80000

    def call(d, **kw):
        a = dict(q=q, k=k, v=v, g=g, b=b, si=si, so=so, o=o)
        a.update(kw)
        return L.gdn_scan(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["b"], a["si"], a["so"],
                          a["o"], None)

    good = GdnDims(16, 2, 4, 128, 128)
    for bad in (GdnDims(16, 2, 4, 64, 128), GdnDims(16, 2, 4, 128, 64), GdnDims(-1, 2, 4, 128, 128),
                GdnDims((1 << 24) + 1, 2, 4, 128, 128), GdnDims(16, 0, 4, 128, 128),
                GdnDims(16, 3, 4, 128, 128), GdnDims(16, 4, 2, 128, 128), GdnDims(16, 1, 1025, 128, 128)):
        assert call(bad) == -1
    assert L.gdn_scan(None, q, k, v, g, b, si, so, o, None) == -1
    for name in ("q", "k", "v", "g", "b", "o"):
        assert call(good, **{name: None}) == -1, name
    for name in ("q", "k", "v", "o", "si", "so"):
        assert call(good, **{name: 0x10008}) == -2, name
    assert call(good, g=0x40002) == -2
    assert call(GdnDims(0, 2, 4, 128, 128), q=None, k=None, v=None, g=None, b=None, o=None,
                so=None) == 0


def test_gdn_scan_chunked_validation_codes():
    """The chunked scan: workspace size from the dimensions, and a workspace
    too small, missing or misaligned is rejected before any launch."""
    from w4_dequant_expert_amd.moe import GdnDims
    L = moe.lib()
    d = GdnDims(100, 2, 4, 128, 128)
    need = moe.gdn_scan_chunked_ws_bytes(d)
    # four chunks of 32 tokens for each of four value heads, one 256-byte
    # aligned record each, holding at least a 32 x 128 and two 32 x 32 float
    # matrices
    rec = need // 16
    assert need % 16 == 0 and rec % 256 == 0 and rec >= (32 * 128 + 2 * 32 * 32) * 4
    assert moe.gdn_scan_chunked_ws_bytes(GdnDims(64, 2, 4, 128, 128)) == need // 4 * 2
    assert moe.gdn_scan_chunked_ws_bytes(GdnDims(0, 2, 4, 128, 128)) == 0
    assert moe.gdn_scan_chunked_ws_bytes(GdnDims(10, 3, 4, 128, 128)) == 0
    assert L.gdn_scan_chunked_ws_bytes(None) == 0
    q, k, v, g, b, so, o, ws = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x70000, 0x80000, 0x100000

    def call(dd, ws_=ws, nb=need):
        return L.gdn_scan_chunked(ctypes.byref(dd), q, k, v, g, b, None, so, o, ws_, nb, None)

    assert call(d, nb=need - 1) == -3
    assert call(d, ws_=None) == -1
    assert call(d, ws_=ws + 16) == -2
    assert call(GdnDims(16, 2, 4, 64, 128)) == -1
    assert L.gdn_scan_chunked(ctypes.byref(GdnDims(0, 2, 4, 128, 128)), None, None, None, None, None,
                              None, None, None, None, 0, None) == 0
