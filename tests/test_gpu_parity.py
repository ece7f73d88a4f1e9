"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing tables (top-k indices, histogram, offsets, scatter, block map) must
match bit for bit, the exported float32 scores too; routing weights within
1e-6; the layer output within a relative error of 1e-2, measured per token as
max_i |y - y_ref| / max_i |y_ref| (the worst token counts); sampled rows of the
two GEMM outputs (h and y_slots) are held to the same bound against the
oracle's single-expert FFN.
"""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import w4_dequant_expert_amd as moe  # noqa: E402
from synth import FULL_SHAPE, bf16_bits_to_f32, build_config, make_bank, make_router, make_tokens  # noqa: E402
from synth.configs import _banks  # noqa: E402

TOL_Y = 1e-2
TOL_W = 1e-6
NTHREADS = 16


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def y_to_f64(y_bits):
    return bf16_bits_to_f32(np.asarray(y_bits).view(np.uint16)).astype(np.float64)


@pytest.fixture(scope="module")
def full_banks():
    routed, shared = _banks(FULL_SHAPE, 1)
    return routed, shared, moe.DeviceBank(routed), moe.DeviceBank(shared)


def run_layer(x, wr, bias, routed_np, shared_np, routed_dev, shared_dev, k, tile_m_max=128,
              tile_gran=16, n_shared=1):
    T, H = x.shape
    E = wr.shape[1]
    I = routed_np["gu_q"].shape[1] // 2
    layer = moe.MoeLayer(H, I, E, k, n_shared, routed_dev, shared_dev if n_shared else None, wr,
                         bias, T_max=max(T, 1), tile_m_max=tile_m_max, tile_gran=tile_gran,
                         export_logits=True)
    xd = dev(x)
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    layer.forward(xd, y)
    torch.cuda.synchronize()
    return layer, layer.rt.host(), y.cpu().numpy()


def check_routing(g, r, label=""):
    assert g["status"] == 0, f"{label} status {g['status']}"
    assert np.array_equal(g["logits"].view(np.uint32), r["logits"].view(np.uint32)), label
    assert np.array_equal(g["topk_idx"], r["topk_idx"]), label
    assert np.array_equal(g["counts"], r["counts"]), label
    assert np.array_equal(g["offsets"], r["offsets"]), label
    assert np.array_equal(g["sorted_slot"], r["sorted_slot"]), label
    assert np.array_equal(g["slot_pos"], r["slot_pos"]), label
    assert g["n_blocks"] == len(r["blocks"]), label
    assert np.array_equal(g["blocks"], r["blocks"]), label
    assert np.max(np.abs(g["topk_w"] - r["topk_w"])) <= TOL_W, label


def check_intermediates(layer, g, x, routed_np, shared_np, k, nrows=6, seed=0):
    """Sampled rows of h (gate/up output) and y_slots (down output) against the
    oracle's single-expert FFN: each GEMM is checked on its own."""
    T = x.shape[0]
    Sk = T * k
    rows_total = Sk + (T if shared_np is not None else 0)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, rows_total - 1], rng.choice(rows_total, min(nrows, rows_total), replace=False)]))
    h = layer.h.cpu().numpy().view(np.uint16)
    ys = layer.y_slots.cpu().numpy().view(np.uint16)
    for r in rows:
        if r < Sk:
            slot = int(g["sorted_slot"][r])
            t, e, bank = slot // k, int(g["topk_idx"][slot // k, slot % k]), routed_np
        else:
            t, e, bank = int(r - Sk), 0, shared_np
        h_ref, y_ref = oracle.expert_ffn(x[t], bank, e)
        eh = oracle.relative_error(bf16_bits_to_f32(h[r]).astype(np.float64), h_ref)
        ey = oracle.relative_error(bf16_bits_to_f32(ys[r]).astype(np.float64), y_ref)
        assert eh <= TOL_Y and ey <= TOL_Y, (r, eh, ey)


def check_layer(cfg, T=None, t0=0, tile_m_max=128, sample=None, banks=None, label=""):
    c = build_config(cfg, T=T, t0=t0, with_weights=False)
    sh = c["shape"]
    routed_np, shared_np, routed_dev, shared_dev = banks
    note(f"case {label or cfg}: T={c['T']} t0={t0} tile_m_max={tile_m_max}")
    layer, g, y = run_layer(c["x"], c["wr"], c["bias"], routed_np, shared_np, routed_dev,
                            shared_dev, sh.k, tile_m_max)
    r = oracle.route(c["x"], c["wr"], c["bias"], sh.k, sh.n_shared, tile_m_max, 16, NTHREADS)
    check_routing(g, r, label or cfg)
    Tn = c["T"]
    if sample is None or sample >= Tn:
        toks = np.arange(Tn)
    else:
        rng = np.random.default_rng(Tn + t0)
        toks = np.unique(np.concatenate([[0, Tn - 1], rng.choice(Tn, sample - 2, replace=False)]))
    yref = oracle.moe_layer(c["x"], r["topk_idx"], r["topk_w"], routed_np, shared_np,
                            tokens=toks, nthreads=NTHREADS)
    err = oracle.relative_error(y_to_f64(y[toks]), yref)
    err_el = oracle.relative_error_elementwise(y_to_f64(y[toks]), yref)
    note(f"  rel err {err:.3e} (elementwise/rms-floor {err_el:.3e}) over {len(toks)} tokens, "
         f"blocks {g['n_blocks']}")
    assert err <= TOL_Y
    check_intermediates(layer, g, c["x"], routed_np, shared_np, sh.k, seed=Tn + t0)
    return layer, g, y


# ----------------------------------------------------------------------------- dequant

def test_dequant_bit_exact(full_banks):
    routed_np = full_banks[0]
    note("case dequant expert 3 gate/up and down")
    for part, rows, K in (("gu", 1024, 2048), ("dn", 2048, 512)):
        q, s_, b = (dev(routed_np[f"{part}_{n}"][3]) for n in ("q", "s", "b"))
        out = torch.empty((rows, K), dtype=torch.int16, device="cuda")
        moe.moe_w4_dequant(rows, K, q, s_, b, out)
        torch.cuda.synchronize()
        got = bf16_bits_to_f32(out.cpu().numpy().view(np.uint16))
        ref = oracle.dequant(routed_np[f"{part}_q"][3], routed_np[f"{part}_s"][3],
                             routed_np[f"{part}_b"][3])
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def unpack_host(packed, N, K, gate_up):
    """Decode the streaming layout (as documented in include/moe_w4.h) back to
    canonical q, s, b arrays, independently of the device code."""
    nk = -(-K // 128)
    blocks = packed.reshape(N // 16, nk, 1152)
    q = np.zeros((N, K // 2), dtype=np.uint8)
    s = np.zeros((N, K // 64), dtype=np.uint16)
    b = np.zeros((N, K // 64), dtype=np.uint16)
    for c in range(N // 16):
        rows = [(c * 8 + r if r < 8 else N // 2 + c * 8 + r - 8) if gate_up else c * 16 + r
                for r in range(16)]
        for st in range(nk):
            blk = blocks[c, st]
            codes = blk[:1024].reshape(64, 16)
            sb = blk[1024:].view(np.uint32).reshape(16, 2).T
            words = codes.view("<u4").reshape(64, 4)
            for lane in range(64):
                r, g = lane % 16, lane // 16
                for j in range(4):
                    k0 = st * 128 + 32 * j + 8 * g
                    w = int(words[lane, j])
                    if k0 >= K:
                        assert w == 0
                        continue
                    # pair order: nibble t holds element 2t, nibble t+4 element 2t+1
                    elems = [(w >> (4 * (e // 2 if e % 2 == 0 else 4 + e // 2))) & 0xF for e in range(8)]
                    for e in range(0, 8, 2):
                        q[rows[r], (k0 + e) // 2] = elems[e] | (elems[e + 1] << 4)
            for gg in range(2):
                grp = st * 2 + gg
                for r in range(16):
                    if grp * 64 < K:
                        s[rows[r], grp] = sb[gg, r] & 0xFFFF
                        b[rows[r], grp] = sb[gg, r] >> 16
                    else:
                        assert sb[gg, r] == 0
    return q, s, b


@pytest.mark.parametrize("N,K,gate_up", [(64, 256, True), (32, 192, False), (48, 64, False)])
def test_pack_layout(N, K, gate_up):
    note(f"case pack layout N={N} K={K} gate_up={gate_up}")
    rng = np.random.default_rng(N + K)
    q = rng.integers(0, 256, (2, N, K // 2), dtype=np.uint8)
    s_ = rng.integers(0, 65536, (2, N, K // 64), dtype=np.uint16)
    b = rng.integers(0, 65536, (2, N, K // 64), dtype=np.uint16)
    nbytes = moe.moe_w4_packed_bytes(N, K)
    out = torch.zeros((2, nbytes), dtype=torch.uint8, device="cuda")
    moe.moe_w4_pack(2, N, K, gate_up, dev(q), dev(s_), dev(b), out)
    torch.cuda.synchronize()
    packed = out.cpu().numpy()
    for e in range(2):
        uq, us, ub = unpack_host(packed[e], N, K, gate_up)
        assert np.array_equal(uq, q[e]) and np.array_equal(us, s_[e]) and np.array_equal(ub, b[e])


def test_dequant_general_bias():
    note("case dequant general scale/bias")
    rng = np.random.default_rng(11)
    rows, K = 64, 256
    q = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    from synth import f64_to_bf16_bits
    s = f64_to_bf16_bits(rng.uniform(-3, 3, (rows, K // 64)) * np.exp(rng.uniform(-30, 30, (rows, K // 64))))
    b = f64_to_bf16_bits(rng.uniform(-3, 3, (rows, K // 64)) * np.exp(rng.uniform(-30, 30, (rows, K // 64))))
    out = torch.empty((rows, K), dtype=torch.int16, device="cuda")
    moe.moe_w4_dequant(rows, K, dev(q), dev(s), dev(b), out)
    torch.cuda.synchronize()
    got = bf16_bits_to_f32(out.cpu().numpy().view(np.uint16))
    ref = oracle.dequant(q, s, b)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ----------------------------------------------------------------------------- tiny layer

def test_tiny_layer_full_parity():
    c = build_config("tiny16")
    rd, sd = moe.DeviceBank(c["routed"]), moe.DeviceBank(c["shared"])
    check_layer("tiny16", banks=(c["routed"], c["shared"], rd, sd))


@pytest.mark.parametrize("tile_m_max", [16, 32, 64])
def test_tiny_layer_tiles(tile_m_max):
    c = build_config("tiny16", T=150)
    rd, sd = moe.DeviceBank(c["routed"]), moe.DeviceBank(c["shared"])
    check_layer("tiny16", T=150, tile_m_max=tile_m_max, banks=(c["routed"], c["shared"], rd, sd),
                label=f"tiny16 T=150 M={tile_m_max}")


# ----------------------------------------------------------------------------- full shape

@pytest.mark.parametrize("T", [1, 37, 300])
def test_full_shape_reduced_T_all_tokens(full_banks, T):
    sample = None if T <= 64 else 48
    check_layer("prefill512", T=T, banks=full_banks, sample=sample, label=f"full T={T}")


def test_prefill512(full_banks):
    check_layer("prefill512", banks=full_banks, sample=24)


def test_prefill2048_zipf(full_banks):
    _, g, _ = check_layer("prefill2048_zipf", banks=full_banks, sample=24)
    counts = g["counts"]
    assert (counts == 0).sum() >= 1 and (counts > 200).sum() >= 1


@pytest.mark.parametrize("tile_m_max", [32, 64])
def test_prefill2048_zipf_tiles(full_banks, tile_m_max):
    check_layer("prefill2048_zipf", tile_m_max=tile_m_max, banks=full_banks, sample=12,
                label=f"zipf M={tile_m_max}")


@pytest.mark.parametrize("chunk", [0, 7])
def test_chunked16384_chunks(full_banks, chunk):
    check_layer("chunked16384", T=2048, t0=2048 * chunk, banks=full_banks, sample=12,
                label=f"chunk {chunk}")


@pytest.mark.parametrize("T", [1, 5, 16, 48])
def test_grouped_ffn_matches_separate_calls(full_banks, T):
    """moe_grouped_w4_ffn (the layer's path) against moe_w4_gate_up followed
    by moe_w4_down: h and y_slots equal bit for bit, on several calls in a
    row and after a fresh route, with the status word clear."""
    note(f"case grouped FFN T={T}")
    c = build_config("decode1", T=T, t0=500, with_weights=False)
    sh = c["shape"]
    routed_np, shared_np, routed_dev, shared_dev = full_banks
    layer = moe.MoeLayer(sh.H, sh.I, sh.E, sh.k, sh.n_shared, routed_dev, shared_dev, c["wr"],
                         c["bias"], T_max=T, tile_m_max=32)
    x = dev(c["x"])
    d = layer.route(x)
    layer.gate_up(d, x)
    layer.down(d)
    torch.cuda.synchronize()
    h_ref, ys_ref = layer.h.clone(), layer.y_slots.clone()
    for rep in range(3):
        layer.h.zero_()
        layer.y_slots.zero_()
        layer.ffn(d, x)
        torch.cuda.synchronize()
        assert int(layer.rt.status.item()) == 0, rep
        assert torch.equal(layer.h, h_ref), rep
        assert torch.equal(layer.y_slots, ys_ref), rep
    # a fresh route call between fused calls also leaves everything consistent
    d = layer.route(x)
    layer.ffn(d, x)
    torch.cuda.synchronize()
    assert int(layer.rt.status.item()) == 0
    assert torch.equal(layer.y_slots, ys_ref)


@pytest.mark.parametrize("cfg,T,tile_m_max", [("decode1", 1, 32), ("decode1", 5, 32),
                                               ("decode1", 48, 32), ("prefill512", 512, 32),
                                               ("decode1", 300, 128), ("prefill2048_zipf", 2048, 128)])
def test_split_ffn_matches_grouped(full_banks, cfg, T, tile_m_max):
    """The shared expert on a second stream, concurrent with routing, then the
    routed experts (moe_shared_w4_ffn + moe_routed_w4_ffn): h and y_slots equal
    moe_grouped_w4_ffn's bit for bit, on three calls in a row, status clear."""
    note(f"case split FFN {cfg} T={T} tile {tile_m_max}")
    c = build_config(cfg, T=T, t0=100 if cfg == "decode1" else 0, with_weights=False)
    sh = c["shape"]
    routed_np, shared_np, routed_dev, shared_dev = full_banks
    layer = moe.MoeLayer(sh.H, sh.I, sh.E, sh.k, sh.n_shared, routed_dev, shared_dev, c["wr"],
                         c["bias"], T_max=T, tile_m_max=tile_m_max)
    x = dev(c["x"])
    d = layer.route(x)
    layer.ffn(d, x)
    torch.cuda.synchronize()
    h_ref, ys_ref = layer.h.clone(), layer.y_slots.clone()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for rep in range(3):
        layer.h.zero_()
        layer.y_slots.zero_()
        ready = torch.cuda.Event()
        ready.record(main)
        side.wait_event(ready)
        layer.shared_ffn(d, x, stream=side)
        d = layer.route(x, stream=main)
        layer.routed_ffn(d, x, stream=main)
        done = torch.cuda.Event()
        done.record(side)
        main.wait_event(done)
        torch.cuda.synchronize()
        assert int(layer.rt.status.item()) == 0, rep
        assert torch.equal(layer.h, h_ref), rep
        assert torch.equal(layer.y_slots, ys_ref), rep


@pytest.mark.parametrize("tok", [0, 1, 999])
def test_decode1_tokens(full_banks, tok):
    check_layer("decode1", T=1, t0=tok, banks=full_banks, label=f"decode token {tok}")


def test_deterministic_and_chunk_independent(full_banks):
    routed_np, shared_np, rd, sd = full_banks
    c = build_config("chunked16384", T=4096, with_weights=False)
    note("case chunk independence T=4096 vs 2x2048")
    _, g_all, y_all = run_layer(c["x"], c["wr"], None, routed_np, shared_np, rd, sd, 8)
    _, _, y_all2 = run_layer(c["x"], c["wr"], None, routed_np, shared_np, rd, sd, 8)
    assert np.array_equal(y_all, y_all2)
    ys = []
    for ch in range(2):
        _, g, y = run_layer(c["x"][2048 * ch:2048 * (ch + 1)], c["wr"], None, routed_np, shared_np,
                            rd, sd, 8)
        assert np.array_equal(g["topk_idx"], g_all["topk_idx"][2048 * ch:2048 * (ch + 1)])
        ys.append(y)
    assert np.array_equal(np.concatenate(ys), y_all)


# ----------------------------------------------------------------------------- routing

@pytest.mark.parametrize("T", [2, 5, 16, 17, 64, 1024])
def test_routing_batch_sizes(full_banks, T):
    """Each router-score kernel variant (short batches up to 16 tokens, 16- and
    32-token tiles) and the scan against the oracle, with a logit bias."""
    note(f"case routing T={T}")
    c = build_config("prefill2048_zipf", T=T, with_weights=False)
    sh = c["shape"]
    _, _, routed_dev, shared_dev = full_banks
    layer = moe.MoeLayer(sh.H, sh.I, sh.E, sh.k, sh.n_shared, routed_dev, shared_dev, c["wr"],
                         c["bias"], T_max=T, tile_m_max=128, export_logits=True)
    layer.route(dev(c["x"]))
    torch.cuda.synchronize()
    r = oracle.route(c["x"], c["wr"], c["bias"], sh.k, sh.n_shared, 128, 16, NTHREADS)
    check_routing(layer.rt.host(), r, f"T={T}")


# ----------------------------------------------------------------------------- odd shapes

@pytest.mark.parametrize("H,I,E,k,n_shared,T,tile_m_max", [
    (192, 64, 5, 5, 1, 33, 32),     # K tails (H % 128 = 64, I = 64), E < 32, k = E
    (128, 128, 40, 1, 0, 70, 32),   # no shared expert, k = 1
    (256, 192, 33, 3, 1, 9, 32),    # E not a multiple of 32, I % 128 = 64
    (1088, 320, 24, 4, 1, 5, 32),   # short batch: inputs split over two waves, K tails in both GEMMs
    (2112, 64, 16, 2, 1, 3, 32),    # short batch: a wave with more steps than one load chunk
    (192, 64, 5, 5, 1, 200, 128),   # tall tiles (every expert 200 rows: blocks of 100) with K tails
    (1088, 320, 24, 4, 1, 300, 128),  # tall and small tiles, K tails in both GEMMs
])
def test_odd_shapes(H, I, E, k, n_shared, T, tile_m_max):
    note(f"case odd shape H={H} I={I} E={E} k={k} shared={n_shared} T={T} tile {tile_m_max}")
    routed = make_bank(E, H, I, seed=21, prefix="odd")
    shared = make_bank(1, H, I, seed=21, prefix="odd_shared") if n_shared else None
    wr = make_router(H, E, 0.1, seed=21)
    x = make_tokens(T, H, seed=21)
    rd = moe.DeviceBank(routed)
    sd = moe.DeviceBank(shared) if n_shared else None
    _, g, y = run_layer(x, wr, None, routed, shared, rd, sd, k, tile_m_max=tile_m_max,
                        n_shared=n_shared)
    r = oracle.route(x, wr, None, k, n_shared, tile_m_max, 16, NTHREADS)
    check_routing(g, r)
    yref = oracle.moe_layer(x, r["topk_idx"], r["topk_w"], routed, shared, nthreads=NTHREADS)
    assert oracle.relative_error(y_to_f64(y), yref) <= TOL_Y


def test_nan_input_sets_status_and_keeps_indices_in_range():
    note("case NaN token")
    c = build_config("tiny16")
    x = c["x"].copy()
    x[3, 5] = 0x7FC0  # NaN
    rd, sd = moe.DeviceBank(c["routed"]), moe.DeviceBank(c["shared"])
    _, g, _ = run_layer(x, c["wr"], None, c["routed"], c["shared"], rd, sd, 2)
    assert g["status"] & moe.STATUS_NAN_LOGIT
    assert g["topk_idx"].min() >= 0 and g["topk_idx"].max() < 8
    assert np.array_equal(np.sort(g["sorted_slot"]), np.arange(32))
