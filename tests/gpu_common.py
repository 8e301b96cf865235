"""Shared pieces of the GPU parity tests: oracle-side references and metrics.

The GPU side always runs the library (q2_pack on the host, everything else
in HIP kernels); the oracle side packs its own weights from the same fp32
draws and checks that the bytes agree before using them.
"""
import os

import numpy as np
import pytest

import synthetic as S
from oracle import formats as F
from oracle import moe_ref as R

CACHE = os.environ.get("MOE_CACHE_DIR", "/tmp/moe_layer_cache")


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def x_as_f32(cfg, T=None):
    x, kind = S.tokens(cfg, T)
    return S.bf16_to_f32(x) if kind == "bf16" else x


def oracle_routing(cfg, T=None):
    x = x_as_f32(cfg, T)
    idx, w, l = R.route(x, S.router_weight(cfg), cfg["top_k"], S.logit_bias(cfg))
    off, perm, inv = R.group(idx, cfg["n_experts"])
    return x, idx, w, l, off, perm, inv


def oracle_experts(cfg, experts, lib_packed=None):
    """Dequantized (oracle-packed) weights of the given experts.  When the
    library's packed bytes are given, they must equal the oracle's."""
    cb = S.codebook_for(cfg["fmt_gate_up"])
    H, I = cfg["hidden"], cfg["inter"]
    out = {}
    for e in experts:
        ws = []
        for j, (which, fmt, rows, K) in enumerate((("gate", cfg["fmt_gate_up"], I, H), ("up", cfg["fmt_gate_up"], I, H),
                                                   ("down", cfg["fmt_down"], H, I))):
            p = F.pack(fmt, S.expert_weight(cfg, which, int(e)), cb)
            if lib_packed is not None:
                assert np.array_equal(p, np.asarray(lib_packed[j][int(e)])), ("packed bytes differ", which, e)
            ws.append(F.unpack(fmt, p, rows, K, cb))
        out[int(e)] = tuple(ws)
    return out


def expert_loader(cfg, lib_packed=None):
    """e -> dequantized (oracle-packed) weights of routed expert e, one expert at
    a time (for R.moe_layer's loader form).  When the library's packed bytes are
    given, they must equal the oracle's."""
    def load(e):
        return oracle_experts(cfg, [e], lib_packed)[int(e)]
    return load


ORACLE_THREADS = min(16, os.cpu_count() or 1)


def oracle_shared(cfg):
    if not cfg["sh_inter"]:
        return None
    return tuple(S.bf16_to_f32(S.shared_weight_bf16(cfg, w)) for w in ("gate", "up", "down"))
