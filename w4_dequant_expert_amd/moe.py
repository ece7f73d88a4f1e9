"""Python binding of libmoe_w4.so: argument marshalling only.

Every call goes straight to the C ABI declared in include/moe_w4.h; all of the
layer's arithmetic runs in the HIP kernels.  PyTorch is used only to allocate
device memory and to name the stream the kernels are enqueued on.  If the
library is missing the import fails: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_w4.so")

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EWS, MOE_EDEVICE, MOE_ELAUNCH = 0, -1, -2, -3, -4, -5
NO_ALLOC_WS_BYTES = 4 << 20   # MOE_NO_ALLOC_WS_BYTES
STATUS_NAN_LOGIT, STATUS_BAD_INDEX, STATUS_BLOCK_OVERFLOW = 1, 2, 4

EXPORTED = ("moe_abi_version", "moe_strerror", "moe_max_blocks", "moe_route_ws_bytes", "moe_route",
            "moe_route_no_alloc",
            "moe_w4_gate_up", "moe_w4_down", "moe_grouped_w4_ffn", "moe_shared_w4_ffn",
            "moe_routed_w4_ffn", "moe_combine", "moe_w4_ffn_combine", "moe_w4_dequant",
            "moe_w4_dequant_packed", "moe_w4_packed_bytes",
            "moe_w4_pack", "moe_read_probe", "moe_mfma_probe", "gdn_scan",
            "gdn_scan_chunked", "gdn_scan_chunked_ws_bytes")


class GdnDims(ctypes.Structure):
    """gdn_dims of include/gdn_scan.h."""
    _fields_ = [("T", ctypes.c_int32), ("n_k_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32)]


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "I", "E", "k", "n_shared", "tile_m_max",
                                              "tile_gran")]


class Bank(ctypes.Structure):
    """Packed bank: gate/up and down matrices of n experts."""
    _fields_ = [("gu", ctypes.c_void_p), ("dn", ctypes.c_void_p)]


class RouteOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_w", "counts", "offsets",
                                               "sorted_slot", "slot_pos", "blocks", "n_blocks",
                                               "logits", "status", "ws")] + [("ws_bytes", ctypes.c_size_t)]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} (code {code})")
        self.code = code


_lib = None


def lib():
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime.  Import it first so that loading the
        # library resolves libamdhip64.so.7 to that same runtime; loading the
        # library first would bring a second HIP runtime into the process, and
        # torch's streams and memory would then be foreign to our kernels.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python __graft_entry__.py, or python w4_dequant_expert_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        L.moe_abi_version.restype = ctypes.c_int
        L.moe_abi_version.argtypes = []
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_max_blocks.restype = ctypes.c_int32
        L.moe_max_blocks.argtypes = [P(Dims)]
        L.moe_route_ws_bytes.restype = ctypes.c_size_t
        L.moe_route_ws_bytes.argtypes = [P(Dims)]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [P(Dims), vp, vp, vp, P(RouteOut), vp]
        L.moe_route_no_alloc.restype = ctypes.c_int
        L.moe_route_no_alloc.argtypes = [P(Dims), vp, vp, vp, P(RouteOut), vp]
        L.moe_w4_gate_up.restype = ctypes.c_int
        L.moe_w4_gate_up.argtypes = [P(Dims), vp, P(RouteOut), P(Bank), P(Bank), vp, vp]
        L.moe_w4_down.restype = ctypes.c_int
        L.moe_w4_down.argtypes = [P(Dims), P(RouteOut), P(Bank), P(Bank), vp, vp, vp]
        L.moe_grouped_w4_ffn.restype = ctypes.c_int
        L.moe_grouped_w4_ffn.argtypes = [P(Dims), vp, P(RouteOut), P(Bank), P(Bank), vp, vp, vp]
        L.moe_shared_w4_ffn.restype = ctypes.c_int
        L.moe_shared_w4_ffn.argtypes = [P(Dims), vp, P(Bank), vp, vp, vp]
        L.moe_routed_w4_ffn.restype = ctypes.c_int
        L.moe_routed_w4_ffn.argtypes = [P(Dims), vp, P(RouteOut), P(Bank), vp, vp, vp]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [P(Dims), P(RouteOut), vp, vp, vp]
        L.moe_w4_ffn_combine.restype = ctypes.c_int
        L.moe_w4_ffn_combine.argtypes = [P(Dims), vp, P(RouteOut), P(Bank), P(Bank), vp, vp, vp, vp]
        L.moe_w4_dequant.restype = ctypes.c_int
        L.moe_w4_dequant.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp]
        L.moe_w4_dequant_packed.restype = ctypes.c_int
        L.moe_w4_dequant_packed.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, vp, vp, vp]
        L.moe_read_probe.restype = ctypes.c_int
        L.moe_read_probe.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int32, vp]
        L.moe_w4_packed_bytes.restype = ctypes.c_size_t
        L.moe_w4_packed_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.moe_w4_pack.restype = ctypes.c_int
        L.moe_w4_pack.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  vp, vp, vp, vp, vp]
        L.moe_mfma_probe.restype = ctypes.c_int
        L.moe_mfma_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp]
        L.gdn_scan_chunked.restype = ctypes.c_int
        L.gdn_scan_chunked.argtypes = [P(GdnDims), vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.gdn_scan_chunked_ws_bytes.restype = ctypes.c_size_t
        L.gdn_scan_chunked_ws_bytes.argtypes = [P(GdnDims)]
        L.gdn_scan.restype = ctypes.c_int
        L.gdn_scan.argtypes = [P(GdnDims), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def _ptr(t):
    """Device address of a torch tensor (None -> NULL); ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------- the C ABI

def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_max_blocks(d: Dims) -> int:
    return lib().moe_max_blocks(ctypes.byref(d))


def moe_route_ws_bytes(d: Dims) -> int:
    return lib().moe_route_ws_bytes(ctypes.byref(d))


def moe_route(d: Dims, x, w_router, logit_bias, out: RouteOut, stream=None):
    _check(lib().moe_route(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                           ctypes.byref(out), _stream(stream)), "moe_route")


def moe_route_no_alloc(d: Dims, x, w_router, logit_bias, out: RouteOut, stream=None):
    _check(lib().moe_route_no_alloc(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                    ctypes.byref(out), _stream(stream)), "moe_route_no_alloc")


def moe_w4_gate_up(d: Dims, x, out: RouteOut, routed: Bank, shared, h, stream=None):
    _check(lib().moe_w4_gate_up(ctypes.byref(d), _ptr(x), ctypes.byref(out), ctypes.byref(routed),
                                ctypes.byref(shared) if shared is not None else None, _ptr(h),
                                _stream(stream)), "moe_w4_gate_up")


def moe_w4_down(d: Dims, out: RouteOut, routed: Bank, shared, h, y_slots, stream=None):
    _check(lib().moe_w4_down(ctypes.byref(d), ctypes.byref(out), ctypes.byref(routed),
                             ctypes.byref(shared) if shared is not None else None, _ptr(h),
                             _ptr(y_slots), _stream(stream)), "moe_w4_down")


def moe_grouped_w4_ffn(d: Dims, x, out: RouteOut, routed: Bank, shared, h, y_slots, stream=None):
    _check(lib().moe_grouped_w4_ffn(ctypes.byref(d), _ptr(x), ctypes.byref(out),
                                    ctypes.byref(routed),
                                    ctypes.byref(shared) if shared is not None else None,
                                    _ptr(h), _ptr(y_slots), _stream(stream)), "moe_grouped_w4_ffn")


def moe_shared_w4_ffn(d: Dims, x, shared: Bank, h, y_slots, stream=None):
    _check(lib().moe_shared_w4_ffn(ctypes.byref(d), _ptr(x), ctypes.byref(shared), _ptr(h),
                                   _ptr(y_slots), _stream(stream)), "moe_shared_w4_ffn")


def moe_routed_w4_ffn(d: Dims, x, out: RouteOut, routed: Bank, h, y_slots, stream=None):
    _check(lib().moe_routed_w4_ffn(ctypes.byref(d), _ptr(x), ctypes.byref(out), ctypes.byref(routed),
                                   _ptr(h), _ptr(y_slots), _stream(stream)), "moe_routed_w4_ffn")


def moe_combine(d: Dims, out: RouteOut, y_slots, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(d), ctypes.byref(out), _ptr(y_slots), _ptr(y),
                             _stream(stream)), "moe_combine")


def moe_w4_ffn_combine(d: Dims, x, out: RouteOut, routed: Bank, shared, h, y_slots, y, stream=None):
    _check(lib().moe_w4_ffn_combine(ctypes.byref(d), _ptr(x), ctypes.byref(out), ctypes.byref(routed),
                                    ctypes.byref(shared) if shared is not None else None,
                                    _ptr(h), _ptr(y_slots), _ptr(y), _stream(stream)),
           "moe_w4_ffn_combine")


def moe_w4_dequant(rows: int, K: int, q, s, b, out, stream=None):
    _check(lib().moe_w4_dequant(rows, K, _ptr(q), _ptr(s), _ptr(b), _ptr(out), _stream(stream)),
           "moe_w4_dequant")


def moe_w4_dequant_packed(n: int, rows: int, K: int, gate_up: bool, packed, out, stream=None):
    _check(lib().moe_w4_dequant_packed(n, rows, K, 1 if gate_up else 0, _ptr(packed), _ptr(out),
                                       _stream(stream)), "moe_w4_dequant_packed")


def moe_read_probe(src, nbytes: int, sink, workgroups: int, stream=None):
    _check(lib().moe_read_probe(_ptr(src), nbytes, _ptr(sink), workgroups, _stream(stream)),
           "moe_read_probe")


def moe_mfma_probe(workgroups: int, iters: int, sink, stream=None):
    _check(lib().moe_mfma_probe(workgroups, iters, _ptr(sink), _stream(stream)), "moe_mfma_probe")


def moe_w4_packed_bytes(rows: int, K: int) -> int:
    return lib().moe_w4_packed_bytes(rows, K)


def moe_w4_pack(n: int, rows: int, K: int, gate_up: bool, q, s, b, packed, stream=None):
    _check(lib().moe_w4_pack(n, rows, K, 1 if gate_up else 0, _ptr(q), _ptr(s), _ptr(b),
                             _ptr(packed), _stream(stream)), "moe_w4_pack")


def gdn_scan(d: GdnDims, q, k, v, g, beta, state_in, state_out, o, stream=None):
    """Gated DeltaNet scan of include/gdn_scan.h (device tensors or raw addresses)."""
    _check(lib().gdn_scan(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                          _ptr(state_in), _ptr(state_out), _ptr(o), _stream(stream)), "gdn_scan")


def gdn_scan_chunked_ws_bytes(d: GdnDims) -> int:
    return lib().gdn_scan_chunked_ws_bytes(ctypes.byref(d))


def gdn_scan_chunked(d: GdnDims, q, k, v, g, beta, state_in, state_out, o, ws, ws_bytes: int,
                     stream=None):
    """Chunked Gated DeltaNet scan of include/gdn_scan.h."""
    _check(lib().gdn_scan_chunked(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(state_in), _ptr(state_out), _ptr(o), _ptr(ws), ws_bytes,
                                  _stream(stream)), "gdn_scan_chunked")


# --------------------------------------------------------------------- device buffers

def make_dims(T, H, I, E, k, n_shared, tile_m_max=128, tile_gran=16) -> Dims:
    return Dims(T, H, I, E, k, n_shared, tile_m_max, tile_gran)


def _dev(a: np.ndarray, device):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceBank:
    """An expert bank resident in device memory in the packed streaming layout.

    The canonical-layout arrays (numpy, as in a checkpoint) are uploaded once,
    repacked on the device by moe_w4_pack, and released.
    """

    CANON = ("gu_q", "gu_s", "gu_b", "dn_q", "dn_s", "dn_b")

    def __init__(self, bank: dict, device="cuda"):
        import torch
        n, two_i, half_h = bank["gu_q"].shape
        H = 2 * half_h
        I = two_i // 2
        self.n, self.H, self.I = n, H, I
        canon = {k: _dev(bank[k], device) for k in self.CANON}
        gu = torch.empty((n, moe_w4_packed_bytes(2 * I, H)), dtype=torch.uint8, device=device)
        dn = torch.empty((n, moe_w4_packed_bytes(H, I)), dtype=torch.uint8, device=device)
        moe_w4_pack(n, 2 * I, H, True, canon["gu_q"], canon["gu_s"], canon["gu_b"], gu)
        moe_w4_pack(n, H, I, False, canon["dn_q"], canon["dn_s"], canon["dn_b"], dn)
        torch.cuda.current_stream().synchronize()
        del canon
        self.t = {"gu": gu, "dn": dn}
        self.c = Bank(gu.data_ptr(), dn.data_ptr())

    @classmethod
    def from_tensors(cls, tensors: dict, n, H, I):
        self = cls.__new__(cls)
        self.t = tensors
        self.n, self.H, self.I = n, H, I
        self.c = Bank(tensors["gu"].data_ptr(), tensors["dn"].data_ptr())
        return self

    def clone(self):
        return DeviceBank.from_tensors({k: v.clone() for k, v in self.t.items()}, self.n, self.H,
                                       self.I)

    def nbytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in self.t.values())


class RouteTables:
    """Device arrays for every routing output of one layer call of up to T tokens."""

    def __init__(self, d: Dims, device="cuda", export_logits=True):
        import torch
        T, E, k = d.T, d.E, d.k
        i32 = dict(dtype=torch.int32, device=device)
        self.d = d
        self.topk_idx = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.counts = torch.empty((E,), **i32)
        self.offsets = torch.empty((E + 1,), **i32)
        self.sorted_slot = torch.empty((T * k,), **i32)
        self.slot_pos = torch.empty((T * k,), **i32)
        self.max_blocks = moe_max_blocks(d)
        if self.max_blocks < 0:
            raise MoeError(MOE_EINVAL, "moe_max_blocks")
        self.blocks = torch.empty((max(self.max_blocks, 1), 4), **i32)
        self.n_blocks = torch.empty((1,), **i32)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device) if export_logits else None
        self.status = torch.zeros((1,), **i32)
        self.ws_bytes = moe_route_ws_bytes(d)
        self.ws = torch.empty((max(self.ws_bytes, 16),), dtype=torch.uint8, device=device)
        self.c = RouteOut(self.topk_idx.data_ptr(), self.topk_w.data_ptr(), self.counts.data_ptr(),
                          self.offsets.data_ptr(), self.sorted_slot.data_ptr(),
                          self.slot_pos.data_ptr(), self.blocks.data_ptr(),
                          self.n_blocks.data_ptr(),
                          self.logits.data_ptr() if self.logits is not None else None,
                          self.status.data_ptr(), self.ws.data_ptr(), self.ws_bytes)

    def host(self) -> dict:
        """Copy every table to host numpy arrays (synchronising)."""
        nb = int(self.n_blocks.item())
        out = dict(topk_idx=self.topk_idx.cpu().numpy(), topk_w=self.topk_w.cpu().numpy(),
                   counts=self.counts.cpu().numpy(), offsets=self.offsets.cpu().numpy(),
                   sorted_slot=self.sorted_slot.cpu().numpy(), slot_pos=self.slot_pos.cpu().numpy(),
                   blocks=self.blocks[:nb].cpu().numpy(), n_blocks=nb,
                   status=int(self.status.item()) & 0xFFFFFFFF)
        if self.logits is not None:
            out["logits"] = self.logits.cpu().numpy()
        return out


class MoeLayer:
    """One MoE layer resident on the device: weights, router and work buffers.

    forward(x) enqueues moe_route, moe_w4_gate_up, moe_w4_down and moe_combine
    on the current stream; nothing synchronises.
    """

    def __init__(self, H, I, E, k, n_shared, routed: DeviceBank, shared, w_router, logit_bias=None,
                 T_max=2048, tile_m_max=128, tile_gran=16, device="cuda", export_logits=False):
        import torch
        self.H, self.I, self.E, self.k, self.n_shared = H, I, E, k, n_shared
        self.routed, self.shared = routed, shared
        self.w_router = w_router if not isinstance(w_router, np.ndarray) else _dev(w_router, device)
        self.bias = (None if logit_bias is None else
                     logit_bias if not isinstance(logit_bias, np.ndarray) else _dev(logit_bias, device))
        self.tile_m_max, self.tile_gran = tile_m_max, tile_gran
        self.T_max = T_max
        self.dmax = make_dims(T_max, H, I, E, k, n_shared, tile_m_max, tile_gran)
        self.rt = RouteTables(self.dmax, device, export_logits)
        rows = T_max * k + (T_max if n_shared else 0)
        self.h = torch.empty((rows, I), dtype=torch.int16, device=device)
        self.y_slots = torch.empty((rows, H), dtype=torch.int16, device=device)

    def dims(self, T):
        if T > self.T_max:
            raise ValueError(f"T={T} exceeds the layer's T_max={self.T_max}")
        return make_dims(T, self.H, self.I, self.E, self.k, self.n_shared, self.tile_m_max,
                         self.tile_gran)

    def route(self, x, T=None, stream=None):
        d = self.dims(x.shape[0] if T is None else T)
        moe_route(d, x, self.w_router, self.bias, self.rt.c, stream)
        return d

    def gate_up(self, d, x, routed=None, shared=None, stream=None):
        r = routed or self.routed
        s = shared or self.shared
        moe_w4_gate_up(d, x, self.rt.c, r.c, s.c if s is not None else None, self.h, stream)

    def down(self, d, routed=None, shared=None, stream=None):
        r = routed or self.routed
        s = shared or self.shared
        moe_w4_down(d, self.rt.c, r.c, s.c if s is not None else None, self.h, self.y_slots, stream)

    def ffn(self, d, x, routed=None, shared=None, stream=None):
        """gate/up then down through the library's grouped call."""
        r = routed or self.routed
        s = shared or self.shared
        moe_grouped_w4_ffn(d, x, self.rt.c, r.c, s.c if s is not None else None, self.h,
                           self.y_slots, stream)

    def shared_ffn(self, d, x, shared=None, stream=None):
        """The shared expert's rows of h and y_slots; needs no routing."""
        s = shared or self.shared
        moe_shared_w4_ffn(d, x, s.c, self.h, self.y_slots, stream)

    def routed_ffn(self, d, x, routed=None, stream=None):
        """The routed rows of h and y_slots (after route on the same stream)."""
        r = routed or self.routed
        moe_routed_w4_ffn(d, x, self.rt.c, r.c, self.h, self.y_slots, stream)

    def combine(self, d, y, stream=None):
        moe_combine(d, self.rt.c, self.y_slots, y, stream)

    def ffn_combine(self, d, x, y, routed=None, shared=None, stream=None):
        """gate/up, down and combine in one library call (down and combine
        fused for a single token)."""
        r = routed or self.routed
        s = shared or self.shared
        moe_w4_ffn_combine(d, x, self.rt.c, r.c, s.c if s is not None else None, self.h,
                           self.y_slots, y, stream)

    def forward(self, x, y, routed=None, shared=None, stream=None):
        d = self.route(x, stream=stream)
        self.ffn_combine(d, x, y, routed, shared, stream)
        return y
