"""Device-resident layers and inputs for the benchmark and test workloads.

Draws the fp32 weights from ``synthetic`` (seeded), quantizes them with the
library's host packer ``q2_pack`` and uploads them with PyTorch.  The packed
bytes can be cached on disk (``cache_dir``) so that several processes of one
run (tests, then the benchmark) quantize the 11.3 G-weight layer only once.
Never imports the oracle.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time
import warnings
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import bit_quantized_routed_amd as M
import synthetic as S


def _log(msg):
    print("[workload] " + msg, file=sys.__stderr__, flush=True)


def layer_key(cfg: dict) -> str:
    keys = ("hidden", "inter", "n_experts", "top_k", "sh_inter", "fmt_gate_up", "fmt_down")
    d = {k: cfg[k] for k in keys}
    d["seed"] = cfg.get("seed", S.LAYER_SEED)
    return hashlib.sha1(json.dumps(d, sort_keys=True).encode()).hexdigest()[:16]


def pack_layer(cfg: dict, threads: int = 8, cache_dir: str | None = None, progress: bool = False):
    """Packed routed experts as three uint8 arrays [E, bytes_per_matrix] (gate, up, down)."""
    H, I, E = cfg["hidden"], cfg["inter"], cfg["n_experts"]
    fg, fd = cfg["fmt_gate_up"], cfg["fmt_down"]
    seed = cfg.get("seed", S.LAYER_SEED)
    paths = None
    if cache_dir:
        os.makedirs(cache_dir, exist_ok=True)
        key = layer_key(cfg)
        paths = [os.path.join(cache_dir, "%s_%s.npy" % (key, n)) for n in ("gate", "up", "down")]
        if all(os.path.exists(p) for p in paths):
            return [np.load(p, mmap_mode="r") for p in paths]
    cb = S.codebook_for(fg, seed)
    gate = np.empty((E, M.q2_packed_bytes(fg, I, H)), np.uint8)
    up = np.empty_like(gate)
    down = np.empty((E, M.q2_packed_bytes(fd, H, I)), np.uint8)
    t0 = time.time()
    done = [0]

    def job(e):
        gate[e] = M.q2_pack(fg, S.expert_weight(cfg, "gate", e, seed), cb)
        up[e] = M.q2_pack(fg, S.expert_weight(cfg, "up", e, seed), cb)
        down[e] = M.q2_pack(fd, S.expert_weight(cfg, "down", e, seed), cb)
        done[0] += 1
        if progress and done[0] % 32 == 0:
            _log("packed %d/%d experts (%.0f s)" % (done[0], E, time.time() - t0))

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, range(E)))
    if paths:
        for p, a in zip(paths, (gate, up, down)):
            tmp = p + ".tmp%d.npy" % os.getpid()
            np.save(tmp, a)
            os.replace(tmp, p)
    return [gate, up, down]


class Workload:
    """One layer on the device plus the token batch of a workload."""

    def __init__(self, cfg: dict, device: str = "cuda", cache_dir: str | None = None, progress: bool = False,
                 replicas: int = 1):
        import torch
        self.cfg = cfg
        H, I, E, k = cfg["hidden"], cfg["inter"], cfg["n_experts"], cfg["top_k"]
        seed = cfg.get("seed", S.LAYER_SEED)
        self.packed = pack_layer(cfg, cache_dir=cache_dir, progress=progress)
        self.codebook = torch.from_numpy(S.codebook_for(cfg["fmt_gate_up"], seed)).to(device)
        self.w_router = torch.from_numpy(S.router_weight(cfg, seed)).to(device)
        sh = cfg["sh_inter"]
        self.shared = None
        if sh:
            self.shared = [torch.from_numpy(S.shared_weight_bf16(cfg, w, seed).view(np.int16)).to(device)
                           for w in ("gate", "up", "down")]
        # `replicas` copies of the routed weights at distinct addresses (a model
        # cycles through its layers, so the benchmark rotates over copies to keep
        # the weights out of the on-chip caches)
        self.layers = []
        self.routed = []
        for _ in range(replicas):
            with warnings.catch_warnings():
                # the cached packed bytes are memory-mapped read-only; the host
                # tensor is only read, to copy it to the device
                warnings.filterwarnings("ignore", message="The given NumPy array is not writable")
                dev = [torch.from_numpy(np.ascontiguousarray(a)).to(device) for a in self.packed]
            wr = self.w_router.clone() if replicas > 1 else self.w_router
            shd = [s.clone() for s in self.shared] if (self.shared and replicas > 1) else self.shared
            self.routed.append((dev, wr, shd))
            self.layers.append(M.DeviceLayer(
                H, I, E, k, cfg["fmt_gate_up"], cfg["fmt_down"], dev[0], dev[1], dev[2], self.codebook, wr,
                shd[0] if shd else None, shd[1] if shd else None, shd[2] if shd else None, sh))
        self.layer = self.layers[0]
        self.device = device

    def tokens(self, cfg: dict | None = None, T: int | None = None):
        """x of workload cfg (default: this layer's) on the device and its kind (M.ACT_F32 / M.ACT_BF16)."""
        import torch
        x, kind = S.tokens(cfg or self.cfg, T)
        if kind == "bf16":
            return torch.from_numpy(x.view(np.int16)).to(self.device), M.ACT_BF16
        return torch.from_numpy(x).to(self.device), M.ACT_F32

    def bias(self, cfg: dict | None = None):
        import torch
        b = S.logit_bias(cfg or self.cfg)
        return None if b is None else torch.from_numpy(b).to(self.device)
