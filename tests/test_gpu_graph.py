"""HIP graph capture of the layer: replays against eager calls.

The layer's four calls launch kernels only (no allocation, no memset, no
host synchronisation), so a decode step can be captured once and replayed.
Each replay is checked bit for bit against the eager result of the same
token, with eager work and synchronisations between the replays.
"""

from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import w4_dequant_expert_amd as moe  # noqa: E402
from synth import FULL_SHAPE, build_config, make_tokens  # noqa: E402
from synth.configs import _banks  # noqa: E402


def _layer(T, tile_m_max):
    c = build_config("decode1", with_weights=False)
    sh = c["shape"]
    routed, shared = _banks(FULL_SHAPE, 1)
    rd, sd = moe.DeviceBank(routed), moe.DeviceBank(shared)
    layer = moe.MoeLayer(sh.H, sh.I, sh.E, sh.k, sh.n_shared, rd, sd, c["wr"], c["bias"],
                         T_max=T, tile_m_max=tile_m_max)
    return layer, sh


# (256, 128): the shared expert's 256 rows make tall blocks, so both GEMM
# kernels are in the captured graph.
@pytest.mark.parametrize("T,tile_m_max", [(1, 32), (48, 32), (256, 128)])
def test_graph_replays_match_eager(T, tile_m_max):
    print(f"case graph replay T={T}", flush=True)
    layer, sh = _layer(T, tile_m_max)
    xs = [torch.from_numpy(make_tokens(T, sh.H, 4, t0=1000 + T * i).view(np.int16)).to("cuda")
          for i in range(3)]
    x_buf = torch.empty_like(xs[0])
    y_buf = torch.empty((T, sh.H), dtype=torch.int16, device="cuda")
    ref = []
    for xi in xs:
        x_buf.copy_(xi)
        layer.forward(x_buf, y_buf)
        ref.append(y_buf.clone())
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x_buf, y_buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.forward(x_buf, y_buf)
    torch.cuda.synchronize()

    y_eager = torch.empty_like(y_buf)
    for rep in range(3):
        for i, xi in enumerate(xs):
            x_buf.copy_(xi)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_buf, ref[i]), (rep, i)
            # eager work between replays, on the same tables
            layer.forward(xs[(i + 1) % len(xs)], y_eager)
            torch.cuda.synchronize()
            assert torch.equal(y_eager, ref[(i + 1) % len(xs)]), (rep, i, "eager")
