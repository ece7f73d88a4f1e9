"""moe_route_no_alloc (routing scratch in a library-owned device array)
against moe_route (caller workspace), through the C ABI: identical tables on
two calls in a row, the second with a smaller batch, and a clear error for a
batch whose scratch exceeds the array."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import w4_dequant_expert_amd as moe  # noqa: E402
from synth import build_config  # noqa: E402

TABLES = ("topk_idx", "topk_w", "counts", "offsets", "sorted_slot", "slot_pos", "blocks",
          "n_blocks", "status")


def _tables(d, device="cuda"):
    rt = moe.RouteTables(d, device, export_logits=False)
    return rt


def _no_ws(rt):
    """The same output tables with no workspace at all."""
    c = rt.c
    return moe.RouteOut(c.topk_idx, c.topk_w, c.counts, c.offsets, c.sorted_slot, c.slot_pos,
                        c.blocks, c.n_blocks, None, c.status, None, 0)


@pytest.mark.parametrize("cfg,T1,T2", [("prefill2048_zipf", 2048, 300), ("decode1", 16, 1)])
def test_no_alloc_route_matches_route(cfg, T1, T2):
    print(f"case no-alloc route {cfg} T={T1} then T={T2}", flush=True)
    c = build_config(cfg, T=T1, with_weights=False)
    sh = c["shape"]
    wr = torch.from_numpy(c["wr"]).to("cuda")
    bias = None if c["bias"] is None else torch.from_numpy(c["bias"]).to("cuda")
    x_all = torch.from_numpy(c["x"].view(np.int16)).to("cuda")
    for T in (T1, T2):
        d = moe.make_dims(T, sh.H, sh.I, sh.E, sh.k, sh.n_shared, 128, 16)
        ref, got = _tables(d), _tables(d)
        for t in (ref, got):        # stale contents must not matter
            for name in TABLES:
                getattr(t, name).fill_(-7)
        x = x_all[:T]
        moe.moe_route(d, x, wr, bias, ref.c)
        moe.moe_route_no_alloc(d, x, wr, bias, _no_ws(got))
        torch.cuda.synchronize()
        a, b = ref.host(), got.host()
        assert a["status"] == 0 and b["status"] == 0
        assert a["n_blocks"] == b["n_blocks"]
        for name in ("topk_idx", "counts", "offsets", "sorted_slot", "slot_pos", "blocks"):
            assert np.array_equal(a[name], b[name]), (T, name)
        assert np.array_equal(a["topk_w"].view(np.uint32), b["topk_w"].view(np.uint32)), T


def test_no_alloc_route_rejects_oversized_batch():
    d = moe.make_dims(8192, 2048, 512, 256, 8, 1, 128, 16)
    assert moe.moe_route_ws_bytes(d) > moe.moe.NO_ALLOC_WS_BYTES
    rt = _tables(moe.make_dims(16, 2048, 512, 256, 8, 1, 128, 16))
    rc = moe.lib().moe_route_no_alloc(ctypes.byref(d), rt.topk_idx.data_ptr(),
                                      rt.topk_w.data_ptr(), None, ctypes.byref(_no_ws(rt)), None)
    assert rc == moe.moe.MOE_EWS
