"""Host-side checks of the C-ABI library (no GPU needed).

The library must load and export every function include/moe.h declares;
argument validation must return the documented status before any HIP call;
q2_pack must write exactly the oracle's bytes.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_quantized_routed_amd as M
import synthetic as S
from oracle import formats as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CB = S.codebook()
GRID = S.grid_cb2s()


def _cb(fmt):
    return GRID if fmt == F.CB2S else CB
FAKE = 0x1000            # never dereferenced: every call below fails validation first


def test_exports_every_declared_function():
    src = "".join(open(os.path.join(ROOT, "include", h)).read() for h in sorted(os.listdir(os.path.join(ROOT, "include"))))
    declared = set(re.findall(r"^(?:int|size_t|const char \*)\s*(\w+)\s*\(", src, flags=re.M))
    assert {"moe_route", "moe_expert_ffn_decode", "moe_expert_ffn_prefill", "q2_pack", "q2_unpack"} <= declared
    L = M.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert declared == set(M.EXPORTS)
    # the benchmark's measurement kernels live in a header of their own, outside the public ABI
    probe = open(os.path.join(ROOT, "bit_quantized_routed_amd", "csrc", "moe_probe.h")).read()
    declared_probe = set(re.findall(r"^(?:int|size_t|const char \*)\s*(\w+)\s*\(", probe, flags=re.M))
    assert declared_probe == set(M.PROBE_EXPORTS)
    for name in declared_probe:
        assert hasattr(L, name), name


def _layer(**kw):
    base = dict(hidden=256, inter=128, n_experts=8, top_k=2, fmt_gate_up=1, fmt_down=2, sh_inter=0, flags=0,
                w_gate=FAKE, w_up=FAKE, w_down=FAKE, codebook=FAKE, sh_gate=None, sh_up=None, sh_down=None,
                w_router=FAKE)
    base.update(kw)
    return M.Layer(**base)


def _route(L, T=4, act=1, ws_bytes=1 << 30, ws=FAKE, out=FAKE):
    return M.lib().moe_route(ctypes.byref(L) if L is not None else None, FAKE, act, T, None, out, out, out, out,
                             out, ws, ws_bytes, None, None)


def _ffn(fn, L, T=4, act=1, ws_bytes=1 << 30, ws=FAKE, out=FAKE):
    return fn(ctypes.byref(L) if L is not None else None, FAKE, act, T, out, out, out, out, out, out, ws,
              ws_bytes, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=0), -1), (dict(top_k=9), -1), (dict(n_experts=2000, top_k=2), -1), (dict(hidden=100), -1),
    (dict(w_router=None), -1)])
def test_route_validation(kw, code):
    assert _route(_layer(**kw)) == code
    assert M.lib().moe_last_error()


def test_route_validation_misc():
    L = _layer()
    assert _route(None) == -1
    assert _route(L, T=-1) == -1
    assert _route(L, act=7) == -1
    assert _route(L, out=None) == -1
    assert _route(L, ws=None) == -1
    assert _route(L, ws_bytes=10) == -3
    assert _route(L, T=0, ws=None, out=None) == 0          # T == 0: no launch, OK


@pytest.mark.parametrize("kw,code", [
    (dict(fmt_gate_up=6), -1), (dict(fmt_gate_up=4), -1), (dict(fmt_gate_up=8), -1), (dict(fmt_down=1), -1),
    (dict(fmt_down=7), -1), (dict(fmt_gate_up=7, codebook=None), -1),
    (dict(inter=100), -1), (dict(w_down=None), -1),
    (dict(codebook=None), -1), (dict(sh_inter=128, sh_gate=FAKE, sh_up=FAKE, sh_down=FAKE), -1),
    (dict(sh_inter=256), -1), (dict(sh_inter=-1), -1)])
def test_ffn_validation(kw, code):
    for fn in (M.lib().moe_expert_ffn_decode, M.lib().moe_expert_ffn_prefill):
        assert _ffn(fn, _layer(**kw)) == code


def test_tokenwise_flag_validation():
    dec, pre = M.lib().moe_expert_ffn_decode, M.lib().moe_expert_ffn_prefill
    for fn in (dec, pre):
        assert _ffn(fn, _layer(flags=4)) == -1                 # unknown bits
        assert b"flags" in M.lib().moe_last_error()
        # the one-stream flag (alone or with the token-wise one) passes validation
        assert _ffn(fn, _layer(flags=M.LAYER_ONE_STREAM), ws_bytes=10) == -3
    assert _ffn(pre, _layer(flags=M.LAYER_ONE_STREAM | M.LAYER_TOKENWISE_DECODE), ws_bytes=10) == -3
    assert _route(_layer(flags=4, w_router=FAKE), ws_bytes=10) == -3   # the router does not read the flags
    # token by token needs the single-token kernels; H = 256 is not a multiple of 512
    assert _ffn(dec, _layer(flags=M.LAYER_TOKENWISE_DECODE)) == -2
    assert b"token-by-token" in M.lib().moe_last_error()
    assert _ffn(dec, _layer(flags=M.LAYER_TOKENWISE_DECODE, fmt_gate_up=3, fmt_down=3)) == -2


def test_ffn_validation_misc():
    dec, pre = M.lib().moe_expert_ffn_decode, M.lib().moe_expert_ffn_prefill
    L = _layer()
    assert _ffn(pre, L, act=0) == -1                           # prefill needs bf16 activations
    assert _ffn(dec, _layer(fmt_gate_up=3, fmt_down=3)) == -2  # decode: Q4K needs K multiples of 512
    for fg, fd in ((2, 2), (5, 6), (1, 6), (3, 5), (7, 2), (7, 3)):   # pairs that run on the 512-multiple GEMMs only
        assert _ffn(pre, _layer(fmt_gate_up=fg, fmt_down=fd)) == -2
        assert _ffn(dec, _layer(fmt_gate_up=fg, fmt_down=fd)) == -2
    assert _ffn(dec, L, ws_bytes=100) == -3
    assert _ffn(pre, L, ws_bytes=100) == -3
    assert _ffn(dec, L, T=-2) == -1
    assert _ffn(dec, L, T=0, ws=None, out=None) == 0
    assert _ffn(pre, L, out=None) == -1


def test_route_alignment():
    """moe_route reads x and W_r in 8- and 16-byte pieces: misaligned pointers are refused."""
    L = M.lib()
    out = FAKE
    args = lambda lay, x, ws: (ctypes.byref(lay), x, 1, 4, None, out, out, out, out, out, ws, 1 << 30, None, None)
    assert L.moe_route(*args(_layer(), FAKE + 8, FAKE)) == -1
    assert b"aligned" in L.moe_last_error()
    assert L.moe_route(*args(_layer(w_router=FAKE + 4), FAKE, FAKE)) == -1
    assert L.moe_route(*args(_layer(), FAKE, FAKE + 2)) == -1


def test_ffn_activation_offset_guard():
    """Calls whose activation rows would pass 2^31 elements are refused (the
    grouped-GEMM kernels use 32-bit element offsets) before any launch."""
    dec, pre = M.lib().moe_expert_ffn_decode, M.lib().moe_expert_ffn_prefill
    L = _layer()                                   # H 256, I 128, k 2, no shared: 2 T * 128 >= 2^31 from T = 8.4 M
    for fn in (dec, pre):
        assert _ffn(fn, L, T=9_000_000) == -2
        assert b"2^31" in M.lib().moe_last_error()
    assert _ffn(dec, _layer(hidden=7168 * 2, inter=256), T=160_000) == -2    # T * H >= 2^31


def test_pack_sets_last_error():
    P = M.lib().q2_pack
    w = np.zeros((2, 256), np.float32)
    o = np.zeros(1024, np.uint8)
    assert P(9, w.ctypes.data, 2, 256, None, o.ctypes.data) == -1
    assert b"q2_pack" in M.lib().moe_last_error()
    assert P(1, w.ctypes.data, 2, 256, None, o.ctypes.data) == -1          # CB2 needs a codebook
    assert b"codebook" in M.lib().moe_last_error()
    assert P(7, w.ctypes.data, 2, 256, None, o.ctypes.data) == -1          # CB2S needs its grid
    assert b"grid" in M.lib().moe_last_error()
    assert P(2, w.ctypes.data, -1, 256, None, o.ctypes.data) == -1
    assert P(2, None, 2, 256, None, o.ctypes.data) == -1


def test_layer_decode_validation():
    F_ = M.lib().moe_layer_decode
    call = lambda L, T=4, act=1, ws_bytes=1 << 30, ws=FAKE, out=FAKE, x=FAKE: F_(
        ctypes.byref(L) if L is not None else None, x, act, T, None, out, out, out, out, out, out, ws, ws_bytes, None,
        None)
    L = _layer()
    assert call(None) == -1
    assert call(_layer(top_k=0)) == -1
    assert call(L, T=-1) == -1
    assert call(L, act=5) == -1
    assert call(L, out=None) == -1
    assert call(L, ws=None) == -1
    assert call(L, x=FAKE + 4) == -1
    assert call(L, ws_bytes=64) == -3
    assert call(L, T=0, ws=None, out=None) == 0
    need = M.workspace_bytes(L, 4, M.PATH_LAYER_DECODE)
    assert need >= M.workspace_bytes(L, 4, M.PATH_ROUTE) + M.workspace_bytes(L, 4, M.PATH_DECODE)


def test_unpack_validation():
    U = M.lib().q2_unpack
    assert U(9, FAKE, 4, 256, FAKE, FAKE, None) == -1
    assert U(1, FAKE, 4, 256, None, FAKE, None) == -1          # CB2 needs a codebook
    assert U(7, FAKE, 4, 256, None, FAKE, None) == -1          # CB2S needs its grid
    assert U(2, None, 4, 256, None, FAKE, None) == -1
    assert U(2, FAKE, -1, 256, None, FAKE, None) == -1
    assert U(2, FAKE, 0, 256, None, None, None) == 0


def test_sizes():
    assert M.q2_packed_bytes(1, 2048, 7168) == F.packed_bytes(F.CB2, 2048, 7168)
    assert M.q2_packed_bytes(2, 7168, 2048) == F.packed_bytes(F.Q2K, 7168, 2048)
    assert M.q2_packed_bytes(3, 7, 300) == F.packed_bytes(F.Q4K, 7, 300)
    assert M.q2_packed_bytes(5, 7168, 2048) == F.packed_bytes(F.Q5K, 7168, 2048)
    assert M.q2_packed_bytes(6, 33, 700) == F.packed_bytes(F.Q6K, 33, 700)
    assert M.q2_packed_bytes(7, 2048, 7168) == F.packed_bytes(F.CB2S, 2048, 7168) == 2048 * 28 * 66
    assert M.q2_packed_bytes(4, 7, 300) == 0
    assert M.q2_packed_bytes(8, 7, 300) == 0
    L = _layer()
    for path in (0, 1, 2):
        a, b = M.workspace_bytes(L, 4, path), M.workspace_bytes(L, 400, path)
        assert 0 < a < b
    assert M.workspace_bytes(_layer(top_k=0), 4, 1) == 0
    assert [M.lib().moe_status_str(c).decode() for c in (0, -1, -2, -3, -4)] == [
        "ok", "invalid argument", "unsupported", "workspace too small", "HIP error"]


@pytest.mark.parametrize("fmt", [F.CB2, F.Q2K, F.Q4K, F.Q5K, F.Q6K, F.CB2S])
@pytest.mark.parametrize("shape", [(1, 256), (7, 100), (33, 384), (5, 1000)])
def test_pack_matches_oracle_bytes(fmt, shape):
    rng = np.random.default_rng(hash((fmt, shape)) % 2**32)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    assert np.array_equal(M.q2_pack(fmt, w, _cb(fmt)), F.pack(fmt, w, _cb(fmt)))


def test_pack_matches_oracle_on_workload_rows():
    cfg = S.config("decode1")
    for which, fmt in (("gate", F.CB2), ("down", F.Q2K), ("down", F.Q4K), ("up", F.Q4K), ("up", F.Q5K),
                       ("down", F.Q6K), ("gate", F.Q2K), ("gate", F.CB2S), ("up", F.CB2S)):
        w = S.expert_weight(cfg, which, 17)[:96]
        assert np.array_equal(M.q2_pack(fmt, w, _cb(fmt)), F.pack(fmt, w, _cb(fmt))), which


def test_pack_edge_values():
    # zeros, a constant row, all-negative and all-positive sub-blocks, a huge outlier
    rows = np.zeros((6, 256), np.float32)
    rows[1] = 0.5
    rows[2] = -np.abs(np.linspace(0.01, 0.3, 256, dtype=np.float32))
    rows[3] = np.abs(np.linspace(0.01, 0.3, 256, dtype=np.float32))
    rows[4, 7] = 30.0
    rows[5] = np.tile(np.array([1e-6, -2e-6], np.float32), 128)
    for fmt in (F.CB2, F.Q2K, F.Q4K, F.Q5K, F.Q6K, F.CB2S):
        assert np.array_equal(M.q2_pack(fmt, rows, _cb(fmt)), F.pack(fmt, rows, _cb(fmt))), fmt


def test_probe_argument_checks():
    L = M.lib()
    assert L.moe_probe_stream_read(None, 16, 1, 0, FAKE, None) == -1
    assert L.moe_probe_stream_read(FAKE, 15, 1, 0, FAKE, None) == -1
    assert L.moe_probe_stream_read(FAKE, 16, 0, 1, FAKE, None) == -1
    assert L.moe_probe_mfma_loop(0, 0, 1, FAKE, None) == -1
    assert L.moe_probe_mfma_loop(0, 1, 0, FAKE, None) == -1
    assert L.moe_probe_mfma_loop(0, 1, 1, None, None) == -1
    assert L.moe_probe_mfma_loop(2, 1, 1, FAKE, None) == -1


# ------------------------------------------------------------------ expert cache (host checks only)
def _cache_struct(layer, n_layers=2, n_slots=4):
    c = M.ExpertCacheC()
    c.n_layers, c.n_experts, c.n_slots = n_layers, layer.n_experts, n_slots
    c.hidden, c.inter, c.fmt_gate_up, c.fmt_down = layer.hidden, layer.inter, layer.fmt_gate_up, layer.fmt_down
    return c


def test_expert_cache_sizes():
    L = _layer()
    per = 2 * M.q2_packed_bytes(1, 128, 256) + M.q2_packed_bytes(2, 256, 128)
    b = M.expert_cache_bytes(L, 3, 5)
    assert b >= 5 * per + 3 * 8 * 4
    assert M.expert_cache_bytes(L, 3, 6) > b
    for nl, ns in ((0, 4), (1, 0), (1, 8193), (1 << 22, 4)):
        assert M.expert_cache_bytes(L, nl, ns) == 0
    assert M.expert_cache_bytes(_layer(top_k=0), 1, 4) == 0


def test_expert_cache_init_validation():
    I = M.lib().moe_expert_cache_init
    L = _layer()
    c = M.ExpertCacheC()
    need = M.expert_cache_bytes(L, 1, 4)
    assert I(None, ctypes.byref(L), 1, 4, FAKE, need, None) == -1
    assert I(ctypes.byref(c), ctypes.byref(L), 1, 0, FAKE, need, None) == -1
    assert I(ctypes.byref(c), ctypes.byref(L), 1, 4, FAKE + 16, need, None) == -1      # 256-byte alignment
    assert I(ctypes.byref(c), ctypes.byref(L), 1, 4, FAKE, need - 1, None) == -3


def test_expert_cache_map_validation():
    Mp, Pf = M.lib().moe_expert_cache_map, M.lib().moe_expert_cache_prefetch
    L = _layer()
    c = _cache_struct(L, n_layers=2, n_slots=4)
    v = M.Layer()
    call = lambda lid=0, lay=L, T=2, view=v, cache=c: Mp(ctypes.byref(cache) if cache is not None else None, lid,
                                                         ctypes.byref(lay), FAKE, T, ctypes.byref(view) if view is not None else None, None)
    assert call(view=None) == -1
    assert call(cache=None) == -1
    assert call(lid=2) == -1 and b"layer_id" in M.lib().moe_last_error()
    assert call(lid=-1) == -1
    assert call(lay=_layer(inter=256)) == -1 and b"differ" in M.lib().moe_last_error()
    assert call(lay=_layer(fmt_down=3)) == -1
    assert call(T=-1) == -1
    # T * k = 6 experts may be needed, only 4 slots: refused before any launch
    assert call(T=3) == -2 and b"slots" in M.lib().moe_last_error()
    assert Pf(ctypes.byref(c), 0, ctypes.byref(L), FAKE, 5, None) == -2
    assert Pf(ctypes.byref(c), 0, ctypes.byref(L), None, 3, None) == -1


def test_layer_decode_refuses_a_cache_view():
    F_ = M.lib().moe_layer_decode
    L = _layer(expert_slot=FAKE)
    assert F_(ctypes.byref(L), FAKE, 1, 1, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None, None) == -2
    assert b"moe_expert_cache_map" in M.lib().moe_last_error()
    assert _ffn(M.lib().moe_expert_ffn_decode, _layer(expert_slot=FAKE + 2)) == -1      # alignment
