"""Routed-MoE expert layer with 2-bit routed experts on one MI355X (gfx950).

Thin ctypes binding over the C-ABI library ``libmoe.so`` (``include/moe.h``).
Every step of the layer runs in the library's HIP kernels; this module only
marshals arguments (device pointers from PyTorch tensors, the caller's HIP
stream) and raises on a non-zero status.  There is no CPU fallback: if the
library is missing, loading fails loudly.

Names follow the C ABI: ``moe_route``, ``moe_expert_ffn_decode``,
``moe_expert_ffn_prefill``, ``q2_pack``, ``q2_unpack``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmoe.so")

FMT_CB2, FMT_Q2K, FMT_Q4K, FMT_BF16, FMT_Q5K, FMT_Q6K, FMT_CB2S = 1, 2, 3, 4, 5, 6, 7
ACT_F32, ACT_BF16 = 0, 1
PATH_ROUTE, PATH_DECODE, PATH_PREFILL, PATH_LAYER_DECODE = 0, 1, 2, 3
LAYER_TOKENWISE_DECODE = 1
LAYER_ONE_STREAM = 2
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP"}
BLOCK_BYTES = {FMT_CB2: 38, FMT_Q2K: 84, FMT_Q4K: 144, FMT_Q5K: 176, FMT_Q6K: 210, FMT_CB2S: 66}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status), detail))
        self.status = status


class Layer(ctypes.Structure):
    """struct moe_layer (host struct of device pointers)."""
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("fmt_gate_up", ctypes.c_int32), ("fmt_down", ctypes.c_int32),
                ("sh_inter", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("codebook", ctypes.c_void_p),
                ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
                ("w_router", ctypes.c_void_p), ("expert_slot", ctypes.c_void_p)]


class ExpertCacheC(ctypes.Structure):
    """struct moe_expert_cache (host struct of device pointers)."""
    _fields_ = [("n_layers", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("fmt_gate_up", ctypes.c_int32),
                ("fmt_down", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("gate_bytes", ctypes.c_int64), ("down_bytes", ctypes.c_int64),
                ("slots_gate", ctypes.c_void_p), ("slots_up", ctypes.c_void_p), ("slots_down", ctypes.c_void_p),
                ("slot_of", ctypes.c_void_p), ("key_of", ctypes.c_void_p), ("stamp", ctypes.c_void_p),
                ("ctl", ctypes.c_void_p), ("stats", ctypes.c_void_p)]


class Profile(ctypes.Structure):
    """struct moe_profile: bracket launch number `kernel` with two hipEvents."""
    _fields_ = [("kernel", ctypes.c_int32), ("n_launches", ctypes.c_int32),
                ("ev_start", ctypes.c_void_p), ("ev_stop", ctypes.c_void_p),
                ("name", ctypes.c_char_p)]


_lib = None
# the C ABI declared in include/moe.h
EXPORTS = ["moe_route", "moe_expert_ffn_decode", "moe_expert_ffn_prefill", "q2_pack", "q2_unpack",
           "q2_packed_bytes", "moe_workspace_bytes", "moe_status_str", "moe_last_error",
           "moe_expert_ffn_decode_noalloc", "moe_layer_decode", "moe_expert_cache_bytes", "moe_expert_cache_init",
           "moe_expert_cache_map", "moe_expert_cache_prefetch"]
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
# measurement kernels the benchmark uses (csrc/moe_probe.h; not part of the layer's ABI)
PROBE_EXPORTS = ["moe_probe_stream_read", "moe_probe_mfma_loop"]


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmoe.so not built at %s; run `python -m bit_quantized_routed_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lp, pp = ctypes.POINTER(Layer), ctypes.POINTER(Profile)
    L.moe_route.argtypes = [lp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, pp]
    L.moe_route.restype = i32
    for f in (L.moe_expert_ffn_decode, L.moe_expert_ffn_prefill):
        f.argtypes = [lp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, pp]
        f.restype = i32
    L.moe_layer_decode.argtypes = [lp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, pp]
    L.moe_layer_decode.restype = i32
    L.moe_expert_ffn_decode_noalloc.argtypes = [lp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, pp]
    L.moe_expert_ffn_decode_noalloc.restype = i32
    L.q2_pack.argtypes = [i32, vp, i64, i32, vp, vp]
    L.q2_pack.restype = i32
    L.q2_unpack.argtypes = [i32, vp, i64, i32, vp, vp, vp]
    L.q2_unpack.restype = i32
    L.q2_packed_bytes.argtypes = [i32, i64, i32]
    L.q2_packed_bytes.restype = sz
    L.moe_workspace_bytes.argtypes = [lp, i32, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_status_str.argtypes = [i32]
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    cp = ctypes.POINTER(ExpertCacheC)
    L.moe_expert_cache_bytes.argtypes = [lp, i32, i32]
    L.moe_expert_cache_bytes.restype = sz
    L.moe_expert_cache_init.argtypes = [cp, lp, i32, i32, vp, sz, vp]
    L.moe_expert_cache_init.restype = i32
    L.moe_expert_cache_map.argtypes = [cp, i32, lp, vp, i32, lp, vp]
    L.moe_expert_cache_map.restype = i32
    L.moe_expert_cache_prefetch.argtypes = [cp, i32, lp, vp, i32, vp]
    L.moe_expert_cache_prefetch.restype = i32
    L.moe_probe_stream_read.argtypes = [vp, sz, i32, i32, vp, vp]
    L.moe_probe_stream_read.restype = i32
    L.moe_probe_mfma_loop.argtypes = [i32, i32, i32, vp, vp]
    L.moe_probe_mfma_loop.restype = i32
    _lib = L
    return L


def _check(rc: int, where: str):
    if rc != 0:
        raise MoeError(rc, where, lib().moe_last_error().decode())


def _ptr(t):
    """Device (or host numpy) pointer of a tensor/array, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ helpers
def q2_packed_bytes(fmt: int, rows: int, K: int) -> int:
    return int(lib().q2_packed_bytes(fmt, rows, K))


def workspace_bytes(layer: Layer, T: int, path: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(layer), T, path))


# ------------------------------------------------------------------ entry points
def q2_pack(fmt: int, w: np.ndarray, codebook: np.ndarray | None = None) -> np.ndarray:
    """Host quantizer: fp32 [rows, K] -> packed uint8 bytes."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    out = np.empty(q2_packed_bytes(fmt, rows, K), np.uint8)
    cb = None
    if codebook is not None:                       # CB2: int8 codebook; CB2S: uint8 grid (same bytes)
        cb = np.ascontiguousarray(codebook)
        cb = cb.view(np.int8) if cb.dtype == np.uint8 else cb.astype(np.int8)
    _check(lib().q2_pack(fmt, w.ctypes.data, rows, K, _ptr(cb), out.ctypes.data), "q2_pack")
    return out


def q2_unpack(fmt: int, packed, rows: int, K: int, codebook, out, stream=None):
    """Device dequantizer: packed (uint8 device) -> out (fp32 device [rows, K])."""
    _check(lib().q2_unpack(fmt, _ptr(packed), rows, K, _ptr(codebook), _ptr(out), _stream(stream)), "q2_unpack")


def probe_stream_read(buf, grid: int, sink, nontemporal: bool = False, stream=None):
    """Machine-ceiling probe: read every byte of buf (uint8 device) once."""
    _check(lib().moe_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), grid, int(nontemporal),
                                       _ptr(sink), _stream(stream)), "moe_probe_stream_read")


def probe_mfma_loop(shape: int, grid: int, iters: int, sink, stream=None):
    """Machine-ceiling probe: grid*4*iters*8*(16384 or 32768) flop of bf16 MFMA
    (shape 0: 16x16x32, shape 1: 32x32x16)."""
    _check(lib().moe_probe_mfma_loop(shape, grid, iters, _ptr(sink), _stream(stream)), "moe_probe_mfma_loop")


def moe_route(layer: Layer, x, act: int, T: int, bias, topk_idx, topk_w, offsets, perm, inv, ws,
              stream=None, prof: Profile | None = None):
    _check(lib().moe_route(ctypes.byref(layer), _ptr(x), act, T, _ptr(bias), _ptr(topk_idx), _ptr(topk_w),
                           _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream), None if prof is None else ctypes.byref(prof)), "moe_route")


def _ffn(fn, name, layer, x, act, T, topk_idx, topk_w, offsets, perm, inv, y, ws, stream, prof):
    _check(fn(ctypes.byref(layer), _ptr(x), act, T, _ptr(topk_idx), _ptr(topk_w), _ptr(offsets), _ptr(perm),
              _ptr(inv), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream),
              None if prof is None else ctypes.byref(prof)), name)


def moe_expert_ffn_decode(layer, x, act, T, topk_idx, topk_w, offsets, perm, inv, y, ws, stream=None, prof=None):
    _ffn(lib().moe_expert_ffn_decode, "moe_expert_ffn_decode", layer, x, act, T, topk_idx, topk_w, offsets,
         perm, inv, y, ws, stream, prof)


def moe_expert_ffn_decode_noalloc(layer, x, act, T, topk_idx, topk_w, offsets, perm, inv, y, stream=None,
                                  prof=None):
    """moe_expert_ffn_decode on the library's fixed per-device scratch (no workspace argument)."""
    _check(lib().moe_expert_ffn_decode_noalloc(ctypes.byref(layer), _ptr(x), act, T, _ptr(topk_idx), _ptr(topk_w),
                                               _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(y), _stream(stream),
                                               None if prof is None else ctypes.byref(prof)),
           "moe_expert_ffn_decode_noalloc")


def moe_layer_decode(layer: Layer, x, act: int, T: int, bias, topk_idx, topk_w, offsets, perm, inv, y, ws,
                     stream=None, prof: Profile | None = None):
    """Router + decode FFN in one call (the single-token layer runs the router
    inside the FFN's launches)."""
    _check(lib().moe_layer_decode(ctypes.byref(layer), _ptr(x), act, T, _ptr(bias), _ptr(topk_idx), _ptr(topk_w),
                                  _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(y), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream),
                                  None if prof is None else ctypes.byref(prof)), "moe_layer_decode")


def moe_expert_ffn_prefill(layer, x, act, T, topk_idx, topk_w, offsets, perm, inv, y, ws, stream=None, prof=None):
    _ffn(lib().moe_expert_ffn_prefill, "moe_expert_ffn_prefill", layer, x, act, T, topk_idx, topk_w, offsets,
         perm, inv, y, ws, stream, prof)


# ------------------------------------------------------------------ device layer
class DeviceLayer:
    """Device-resident weights of one layer plus the moe_layer struct over them.

    Holds torch tensors (device memory) so the pointers stay valid; all
    arithmetic happens in the library.
    """

    def __init__(self, hidden, inter, n_experts, top_k, fmt_gate_up, fmt_down, w_gate, w_up, w_down,
                 codebook, w_router, sh_gate=None, sh_up=None, sh_down=None, sh_inter=0, flags=0):
        self.tensors = [w_gate, w_up, w_down, codebook, w_router, sh_gate, sh_up, sh_down]
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.sh_inter = sh_inter
        self.c = Layer(hidden, inter, n_experts, top_k, fmt_gate_up, fmt_down, sh_inter, flags,
                       _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(codebook),
                       _ptr(sh_gate), _ptr(sh_up), _ptr(sh_down), _ptr(w_router), None)

    def workspace(self, T: int, path: int, device="cuda"):
        """A workspace for `path` at T tokens (the library needs no particular
        initial contents; zeroed so that nothing reads stale data from earlier
        tests)."""
        import torch
        n = max(workspace_bytes(self.c, T, path), 256)
        return torch.zeros(n, dtype=torch.uint8, device=device)


class Routing:
    """Device routing buffers for T tokens."""

    def __init__(self, T, k, E, device="cuda"):
        import torch
        self.T = T
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.perm = torch.empty(T * k, dtype=torch.int32, device=device)
        self.inv = torch.empty(T * k, dtype=torch.int32, device=device)


def route(dl: DeviceLayer, x, act, T, bias, r: Routing, ws, stream=None, prof=None):
    moe_route(dl.c, x, act, T, bias, r.topk_idx, r.topk_w, r.offsets, r.perm, r.inv, ws, stream, prof)


def ffn_decode(dl: DeviceLayer, x, act, T, r: Routing, y, ws, stream=None, prof=None):
    moe_expert_ffn_decode(dl.c, x, act, T, r.topk_idx, r.topk_w, r.offsets, r.perm, r.inv, y, ws, stream, prof)


def layer_decode(dl: DeviceLayer, x, act, T, bias, r: Routing, y, ws, stream=None, prof=None):
    moe_layer_decode(dl.c, x, act, T, bias, r.topk_idx, r.topk_w, r.offsets, r.perm, r.inv, y, ws, stream, prof)


def ffn_prefill(dl: DeviceLayer, x, act, T, r: Routing, y, ws, stream=None, prof=None):
    moe_expert_ffn_prefill(dl.c, x, act, T, r.topk_idx, r.topk_w, r.offsets, r.perm, r.inv, y, ws, stream, prof)


# ------------------------------------------------------------------ expert streaming
class HostLayer(DeviceLayer):
    """A layer whose routed weights (gate, up, down) live in pinned host
    memory while the codebook, router and shared expert stay on the device:
    the backing store of an expert cache."""

    def __init__(self, dl: DeviceLayer):
        import torch
        w_gate, w_up, w_down = (t.cpu().pin_memory() for t in dl.tensors[:3])
        codebook, w_router, sh_gate, sh_up, sh_down = dl.tensors[3:]
        c = dl.c
        super().__init__(c.hidden, c.inter, c.n_experts, c.top_k, c.fmt_gate_up, c.fmt_down, w_gate, w_up, w_down,
                         codebook, w_router, sh_gate, sh_up, sh_down, c.sh_inter, c.flags)
        assert all(t.is_pinned() for t in (w_gate, w_up, w_down)), torch.cuda.is_available()


class LayerView:
    """The layer view an expert cache hands out (struct moe_layer with the slot
    arrays and the slot map); FFN calls take it like a device layer."""

    def __init__(self, c: Layer, keep):
        self.c, self._keep = c, keep

    def workspace(self, T: int, path: int, device="cuda"):
        import torch
        return torch.zeros(max(workspace_bytes(self.c, T, path), 256), dtype=torch.uint8, device=device)


def expert_cache_bytes(layer: Layer, n_layers: int, n_slots: int) -> int:
    return int(lib().moe_expert_cache_bytes(ctypes.byref(layer), n_layers, n_slots))


class ExpertCache:
    """An HBM cache of n_slots routed-expert slots for n_layers layers of one
    geometry (device memory held by a torch tensor)."""

    def __init__(self, layer: Layer, n_layers: int, n_slots: int, stream=None, device="cuda"):
        import torch
        n = expert_cache_bytes(layer, n_layers, n_slots)
        if n == 0:
            raise ValueError("invalid cache geometry (n_layers=%d, n_slots=%d)" % (n_layers, n_slots))
        self.mem = torch.empty(n, dtype=torch.uint8, device=device)
        self.c = ExpertCacheC()
        _check(lib().moe_expert_cache_init(ctypes.byref(self.c), ctypes.byref(layer), n_layers, n_slots,
                                           _ptr(self.mem), n, _stream(stream)), "moe_expert_cache_init")

    def _field(self, ptr, count, dtype):
        off = ptr - self.mem.data_ptr()
        return self.mem[off:off + count * dtype.itemsize].view(dtype)

    def map(self, layer_id: int, host: DeviceLayer, topk_idx, T: int, stream=None) -> LayerView:
        v = Layer()
        _check(lib().moe_expert_cache_map(ctypes.byref(self.c), layer_id, ctypes.byref(host.c), _ptr(topk_idx), T,
                                          ctypes.byref(v), _stream(stream)), "moe_expert_cache_map")
        return LayerView(v, (self, host))

    def prefetch(self, layer_id: int, host: DeviceLayer, experts, n: int, stream=None):
        _check(lib().moe_expert_cache_prefetch(ctypes.byref(self.c), layer_id, ctypes.byref(host.c), _ptr(experts),
                                               n, _stream(stream)), "moe_expert_cache_prefetch")

    def stats(self):
        """(hits, misses, bytes copied, calls) since init (synchronises)."""
        import torch
        return [int(v) for v in self._field(self.c.stats, 4, torch.int64).cpu()]

    def slot_of(self, layer_id: int):
        import torch
        E = self.c.n_experts
        return self._field(self.c.slot_of + 4 * E * layer_id, E, torch.int32)

    def key_of(self):
        import torch
        return self._field(self.c.key_of, self.c.n_slots, torch.int32)
