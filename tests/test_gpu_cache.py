"""Expert streaming through the C ABI: an HBM cache of routed-expert slots
backed by pinned host memory.

The FFN on a cache view must give bit for bit the resident layer's output
(same routing, tiles and sums; only the weight addresses differ), and the
cache's slot state after every call must be the one its documented policy
gives: hits keep their slots, misses take the least recently used slots the
call does not need (empty ones first, the lower slot on ties), in expert
order.  `LruModel` below restates that policy on the host.
"""
import numpy as np
import pytest
import torch

import bit_quantized_routed_amd as M
import synthetic as S
import workload as W
from oracle import moe_ref as R
from gpu_common import CACHE, expert_loader, need_gpu, oracle_routing, oracle_shared, rel_l2

pytestmark = pytest.mark.gpu

GEMM = dict(hidden=1024, inter=512, sh_inter=512, n_experts=16, top_k=4, x_dtype="bf16", skew=True,
            fmt_gate_up=S.FMT_CB2, fmt_down=S.FMT_Q2K, name="mid")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    print("[gpu] libmoe:", M.LIB_PATH, flush=True)


class LruModel:
    """The cache policy on the host: slot_of[layer][expert], key_of[slot]."""

    def __init__(self, n_layers, E, S_):
        self.E, self.S = E, S_
        self.slot_of = -np.ones((n_layers, E), np.int64)
        self.key_of = -np.ones(S_, np.int64)
        self.stamp = np.zeros(S_, np.int64)
        self.clock = 0
        self.hits = self.misses = 0

    def call(self, layer, ids):
        E = self.E
        needed = sorted({int(i) for i in np.asarray(ids).reshape(-1) if 0 <= i < E})
        self.clock += 1
        miss = []
        for e in needed:
            s = self.slot_of[layer, e]
            if s >= 0:
                self.stamp[s] = self.clock
                self.hits += 1
            else:
                miss.append(e)
        cand = sorted((self.stamp[s], s) for s in range(self.S) if self.stamp[s] != self.clock)
        for r, e in enumerate(miss):
            s = cand[r][1]
            old = self.key_of[s]
            if old >= 0:
                self.slot_of[old // E, old % E] = -1
            self.key_of[s] = layer * E + e
            self.slot_of[layer, e] = s
            self.stamp[s] = self.clock
        self.misses += len(miss)
        return len(miss)


def check_state(cache, model, n_layers):
    for l in range(n_layers):
        assert np.array_equal(cache.slot_of(l).cpu().numpy(), model.slot_of[l]), l
    assert np.array_equal(cache.key_of().cpu().numpy(), model.key_of)
    hits, misses, nbytes, calls = cache.stats()
    assert (hits, misses, calls) == (model.hits, model.misses, model.clock)
    c = cache.c
    assert nbytes == misses * (2 * c.gate_bytes + c.down_bytes)


def route(wl, x, act, T, cfg):
    r = M.Routing(T, wl.cfg["top_k"], wl.cfg["n_experts"])
    M.route(wl.layer, x, act, T, wl.bias(cfg), r, wl.layer.workspace(T, M.PATH_ROUTE))
    return r


def ffn(layer, x, act, T, r, decode):
    y = torch.full((T, x.shape[1]), float("nan"), device="cuda")
    (M.ffn_decode if decode else M.ffn_prefill)(layer, x, act, T, r, y,
                                                layer.workspace(T, M.PATH_DECODE if decode else M.PATH_PREFILL))
    return y


def same_bits(a, b):
    torch.cuda.synchronize()
    return np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_single_token_decode_through_a_small_cache():
    """Twelve single-token decode steps (the staged single-token kernels) on a
    cache of 6 slots for a layer of 16 experts, top-4: hits, misses and
    evictions, each step's y bit-identical to the resident layer's, the slot
    state as the policy says, and one step against the oracle."""
    cfg = dict(GEMM, T=1, index=90)
    wl = W.Workload(cfg)
    host = M.HostLayer(wl.layer)
    cache = M.ExpertCache(wl.layer.c, 1, 6)
    model = LruModel(1, 16, 6)
    for i in range(12):
        c = dict(cfg, index=100 + i % 7)                    # some tokens repeat: their experts hit
        x, act = wl.tokens(c)
        r = route(wl, x, act, 1, c)
        view = cache.map(0, host, r.topk_idx, 1)
        y = ffn(view, x, act, 1, r, True)
        y_res = ffn(wl.layer, x, act, 1, r, True)
        assert same_bits(y, y_res), i
        model.call(0, r.topk_idx.cpu().numpy())
        check_state(cache, model, 1)
    assert model.hits > 0 and model.misses > 6               # both kinds happened, with evictions
    xf, idx, w, l, off, perm, inv = oracle_routing(c)
    yref = R.moe_layer(xf, idx, w, expert_loader(c, wl.packed), oracle_shared(c))
    assert rel_l2(y.cpu().numpy(), yref) <= 1e-4


def test_two_layers_share_one_cache_prefill_and_batched_decode():
    """Two layers of one geometry take turns in one cache of 16 slots (= the
    experts of one layer): prefill (T = 64, every expert needed), batched
    decode (T = 3, the grouped GEMMs), each call bit-identical to its resident
    layer, the slot state as the policy says."""
    wls = [W.Workload(dict(GEMM, T=64, index=91, seed=2000 + l)) for l in range(2)]
    hosts = [M.HostLayer(w.layer) for w in wls]
    cache = M.ExpertCache(wls[0].layer.c, 2, 16)
    model = LruModel(2, 16, 16)
    steps = [(0, 64, False), (1, 64, False), (0, 3, True), (1, 3, True), (1, 3, True), (0, 64, False)]
    for n, (l, T, decode) in enumerate(steps):
        wl = wls[l]
        c = dict(wl.cfg, T=T, index=92 + n)
        x, act = wl.tokens(c)
        r = route(wl, x, act, T, c)
        view = cache.map(l, hosts[l], r.topk_idx, T)
        y = ffn(view, x, act, T, r, decode)
        assert same_bits(y, ffn(wl.layer, x, act, T, r, decode)), n
        model.call(l, r.topk_idx.cpu().numpy())
        check_state(cache, model, 2)


def test_prefetch_on_a_second_stream_overlaps_the_previous_layer():
    """Layer 1's experts are prefetched into its own cache on a second stream
    while layer 0 computes on the first; layer 1's map then finds every expert
    resident (no misses) and its output is the resident layer's."""
    wls = [W.Workload(dict(GEMM, T=64, index=93, seed=2100 + l)) for l in range(2)]
    hosts = [M.HostLayer(w.layer) for w in wls]
    caches = [M.ExpertCache(w.layer.c, 1, 16) for w in wls]
    s_main, s_copy = torch.cuda.current_stream(), torch.cuda.Stream()
    experts = torch.arange(16, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    c0 = dict(wls[0].cfg, index=94)
    x0, act = wls[0].tokens(c0)
    r0 = route(wls[0], x0, act, 64, c0)
    with torch.cuda.stream(s_copy):
        caches[1].prefetch(0, hosts[1], experts, 16, stream=s_copy)
        done = torch.cuda.Event()
        done.record(s_copy)
    view0 = caches[0].map(0, hosts[0], r0.topk_idx, 64)
    y0 = ffn(view0, x0, act, 64, r0, False)
    s_main.wait_event(done)
    c1 = dict(wls[1].cfg, index=95)
    x1, act1 = wls[1].tokens(c1)
    r1 = route(wls[1], x1, act1, 64, c1)
    view1 = caches[1].map(0, hosts[1], r1.topk_idx, 64)
    y1 = ffn(view1, x1, act1, 64, r1, False)
    assert same_bits(y0, ffn(wls[0].layer, x0, act, 64, r0, False))
    assert same_bits(y1, ffn(wls[1].layer, x1, act1, 64, r1, False))
    h1, m1, _, calls1 = caches[1].stats()
    assert (m1, calls1) == (16, 2) and h1 == len(np.unique(r1.topk_idx.cpu().numpy()))


@pytest.fixture(scope="module")
def big():
    return W.Workload(S.config("decode1"), cache_dir=CACHE, progress=True)


def test_full_size_decode_through_a_cache(big):
    """The full layer (H=7168, I=2048, 256 experts, top-8) with its routed
    experts in pinned host memory and 32 HBM slots: eight single-token decode
    steps cycling over three tokens (their 24 experts fit, so the second round
    hits), each bit-identical to the resident layer, slot state as the policy
    says."""
    host = M.HostLayer(big.layer)
    cache = M.ExpertCache(big.layer.c, 1, 32)
    model = LruModel(1, 256, 32)
    cfg = S.config("decode32")
    for i in range(8):
        x, act = big.tokens(cfg)
        x = x[i % 3:i % 3 + 1].contiguous()
        r = route(big, x, act, 1, S.config("decode1"))
        view = cache.map(0, host, r.topk_idx, 1)
        y = ffn(view, x, act, 1, r, True)
        assert same_bits(y, ffn(big.layer, x, act, 1, r, True)), i
        model.call(0, r.topk_idx.cpu().numpy())
        check_state(cache, model, 1)
    assert model.hits > 0
