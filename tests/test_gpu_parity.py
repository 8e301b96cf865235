"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: routing indices, offsets, perm, inv and dequantized weights bit-exact;
routing weights within 2 fp32 ulps (fp64 sums in a different order);
layer output relative L2 <= 1e-4 on the decode path and <= 5e-3 on the
prefill path.  Small and mid-size cases compare every element; the full-size
workloads (the benchmark's launch configuration) compare routing in full and
the output on sampled tokens, which the oracle evaluates one by one.
"""
import numpy as np
import pytest
import torch

import bit_quantized_routed_amd as M
import synthetic as S
import workload as W
from oracle import formats as F
from oracle import moe_ref as R
from gpu_common import (CACHE, ORACLE_THREADS, expert_loader, need_gpu, oracle_experts, oracle_routing,
                        oracle_shared, rel_l2)

pytestmark = pytest.mark.gpu

DEC_TOL, PRE_TOL = 1e-4, 5e-3

MID = dict(hidden=512, inter=384, n_experts=16, top_k=4, sh_inter=256, x_dtype="bf16", skew=False,
           fmt_gate_up=S.FMT_CB2, fmt_down=S.FMT_Q2K, name="mid")


def mid(T, index, **kw):
    c = dict(MID, T=T, index=index)
    c.update(kw)
    return c


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    print("[gpu] libmoe:", M.LIB_PATH, flush=True)


# ------------------------------------------------------------------ unpack
@pytest.mark.parametrize("fmt", [F.CB2, F.Q2K, F.Q4K, F.Q5K, F.Q6K, F.CB2S])
@pytest.mark.parametrize("rows,K", [(1, 256), (5, 100), (19, 640), (64, 7168), (64, 2048)])
def test_unpack_bit_exact(fmt, rows, K):
    rng = np.random.default_rng(rows * 1000 + K + fmt)
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    cb = S.codebook_for(fmt)
    p = F.pack(fmt, w, cb)
    ref = F.unpack(fmt, p, rows, K, cb)
    out = torch.full((rows, K), float("nan"), device="cuda")
    M.q2_unpack(fmt, torch.from_numpy(p).cuda(), rows, K, torch.from_numpy(cb).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ helpers
def run_route(wl, cfg, T=None):
    x, act = wl.tokens(cfg, T)
    T = x.shape[0]
    c = wl.cfg
    r = M.Routing(T, c["top_k"], c["n_experts"])
    ws = wl.layer.workspace(T, M.PATH_ROUTE)
    M.route(wl.layer, x, act, T, wl.bias(cfg), r, ws)
    torch.cuda.synchronize()
    return x, act, r


def check_route(r, idx, w, off, perm, inv):
    assert np.array_equal(r.topk_idx.cpu().numpy(), idx)
    assert np.array_equal(r.offsets.cpu().numpy(), off)
    assert np.array_equal(r.perm.cpu().numpy(), perm)
    assert np.array_equal(r.inv.cpu().numpy(), inv)
    gw = r.topk_w.cpu().numpy()
    assert np.allclose(gw, w, rtol=2.4e-7, atol=0), np.abs(gw - w).max()


def run_ffn(wl, x, act, r, decode, T=None):
    T = x.shape[0] if T is None else T
    y = torch.full((x.shape[0], wl.cfg["hidden"]), float("nan"), device="cuda")
    ws = wl.layer.workspace(T, M.PATH_DECODE if decode else M.PATH_PREFILL)
    (M.ffn_decode if decode else M.ffn_prefill)(wl.layer, x, act, T, r, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def full_reference(cfg, T=None):
    x, idx, w, l, off, perm, inv = oracle_routing(cfg, T)
    ex = oracle_experts(cfg, np.unique(idx))
    y = R.moe_layer(x, idx, w, ex, oracle_shared(cfg))
    return y, (idx, w, off, perm, inv)


# ------------------------------------------------------------------ small / mid, every element
SMALL = [
    ("tiny", S.config("tiny")),
    ("mid_T37", mid(37, 11)),
    ("mid_T1", mid(1, 12)),
    ("mid_T64_skew", mid(64, 13, skew=True)),
    ("mid_T300", mid(300, 14)),
    ("mid_allexperts", mid(9, 15, top_k=16, n_experts=16)),
    ("mid_f32x", mid(20, 16, x_dtype="f32")),
    # single-token decode path: H % 512 == 0, I % 256 == 0, shared I % 512 == 0
    ("one_T1", mid(1, 22, hidden=1024, inter=512, sh_inter=512)),
    ("one_T1_f32x", mid(1, 23, hidden=1024, inter=512, sh_inter=512, x_dtype="f32")),
    ("one_T1_noshared", mid(1, 24, hidden=1024, inter=768, sh_inter=0)),
    ("one_T1_k16", mid(1, 25, hidden=512, inter=256, sh_inter=512, n_experts=32, top_k=16)),
    # batched decode through the grouped GEMMs (every K a multiple of 512)
    ("gemm_T37", mid(37, 26, hidden=1024, inter=512, sh_inter=512)),
    ("gemm_T20_f32x", mid(20, 27, hidden=1024, inter=512, sh_inter=512, x_dtype="f32")),
    ("gemm_T9_noshared", mid(9, 28, hidden=1024, inter=512, sh_inter=0)),
]


@pytest.fixture(scope="module")
def small_cases():
    return {}


def _case(small_cases, name, cfg):
    if name not in small_cases:
        wl = W.Workload(cfg)
        y, routing = full_reference(cfg)
        small_cases[name] = (wl, y, routing)
    return small_cases[name]


@pytest.mark.parametrize("name,cfg", SMALL, ids=[n for n, _ in SMALL])
def test_route_small(small_cases, name, cfg):
    wl, _, routing = _case(small_cases, name, cfg)
    _, _, r = run_route(wl, cfg)
    check_route(r, *routing)


@pytest.mark.parametrize("name,cfg", SMALL, ids=[n for n, _ in SMALL])
def test_decode_small(small_cases, name, cfg):
    wl, yref, _ = _case(small_cases, name, cfg)
    x, act, r = run_route(wl, cfg)
    y = run_ffn(wl, x, act, r, decode=True)
    err = rel_l2(y, yref)
    print("[decode] %s rel_l2=%.3e" % (name, err))
    assert err <= DEC_TOL


@pytest.mark.parametrize("name,cfg", [c for c in SMALL if c[1]["x_dtype"] == "bf16"] +
                         [("tiny_bf16", S.config("tiny", x_dtype="bf16")),
                          ("mid_q4k", mid(150, 17, fmt_gate_up=S.FMT_Q4K, fmt_down=S.FMT_Q4K)),
                          ("mid_q4k_T1", mid(1, 18, fmt_gate_up=S.FMT_Q4K, fmt_down=S.FMT_Q4K))],
                         ids=lambda v: v if isinstance(v, str) else "")
def test_prefill_small(small_cases, name, cfg):
    wl, yref, routing = _case(small_cases, name, cfg)
    x, act, r = run_route(wl, cfg)
    check_route(r, *routing)
    y = run_ffn(wl, x, act, r, decode=False)
    err = rel_l2(y, yref)
    print("[prefill] %s rel_l2=%.3e" % (name, err))
    assert err <= PRE_TOL


Q4D = dict(hidden=1024, inter=512, sh_inter=512, fmt_gate_up=S.FMT_Q4K, fmt_down=S.FMT_Q4K)

# Shapes where every K is a multiple of 512, so the in-register-dequant grouped
# GEMMs run (prefill: 96-row routed tiles, 80-row shared tiles; batched decode:
# 32-row tiles), with enough rows per expert that hot experts span several
# tiles and end in a partial one, and the shared expert spans several tiles.
GEMM = dict(hidden=1024, inter=512, sh_inter=512, n_experts=8, top_k=2)
MULTI_PRE = [
    ("np_T600_skew", mid(600, 40, skew=True, **GEMM)),
    ("np_T480_k4", mid(480, 41, **dict(GEMM, top_k=4))),
    ("np_T600_skew_q4k", mid(600, 42, skew=True, fmt_gate_up=S.FMT_Q4K, fmt_down=S.FMT_Q4K, **GEMM)),
    ("np_T400_k4_q4k", mid(400, 43, fmt_gate_up=S.FMT_Q4K, fmt_down=S.FMT_Q4K, **dict(GEMM, top_k=4))),
]
MULTI_DEC = [
    ("npd_T100_skew", mid(100, 44, skew=True, **GEMM)),
    ("npd_T90_skew_f32x", mid(90, 45, x_dtype="f32", skew=True, **GEMM)),
    ("npd_T128_skew_q4k", mid(128, 46, skew=True, fmt_gate_up=S.FMT_Q4K, fmt_down=S.FMT_Q4K, **GEMM)),
]


def _tile_structure(off, bm, T, bm_sh):
    """The routing puts several tiles on one expert, a partial last tile on
    some expert, and several tiles on the shared expert."""
    counts = np.diff(off)
    assert counts.max() > 2 * bm, counts
    assert np.any((counts % bm != 0) & (counts > bm)), counts
    assert T > 2 * bm_sh


@pytest.mark.parametrize("name,cfg", MULTI_PRE, ids=[n for n, _ in MULTI_PRE])
def test_prefill_multitile(small_cases, name, cfg):
    """Every output element of the prefill grouped GEMMs on multi-tile experts
    (routed tiles of 96 rows, shared tiles of 80, the 32x32x16 down body on
    1..3 row fragments)."""
    wl, yref, routing = _case(small_cases, name, cfg)
    _tile_structure(routing[2], 96, cfg["T"], 80)
    x, act, r = run_route(wl, cfg)
    check_route(r, *routing)
    y = run_ffn(wl, x, act, r, decode=False)
    err = rel_l2(y, yref)
    print("[prefill] %s rel_l2=%.3e" % (name, err))
    assert np.all(np.isfinite(y))
    assert err <= PRE_TOL


@pytest.mark.parametrize("name,cfg", MULTI_DEC, ids=[n for n, _ in MULTI_DEC])
def test_decode_multitile(small_cases, name, cfg):
    """Every output element of the batched decode GEMMs (32-row tiles, the
    shared expert split over K parts) on multi-tile experts."""
    wl, yref, routing = _case(small_cases, name, cfg)
    _tile_structure(routing[2], 32, cfg["T"], 32)
    x, act, r = run_route(wl, cfg)
    check_route(r, *routing)
    y = run_ffn(wl, x, act, r, decode=True)
    err = rel_l2(y, yref)
    print("[decode] %s rel_l2=%.3e" % (name, err))
    assert np.all(np.isfinite(y))
    assert err <= DEC_TOL


@pytest.mark.parametrize("name,cfg", [("q4k_dec_T1", mid(1, 31, **Q4D)),
                                      ("q4k_dec_T5", mid(5, 32, **Q4D)),
                                      ("q4k_dec_T40_f32", mid(40, 33, x_dtype="f32", **Q4D)),
                                      ("q4k_dec_T70_skew", mid(70, 34, skew=True, **Q4D))],
                         ids=lambda v: v if isinstance(v, str) else "")
def test_decode_q4k(small_cases, name, cfg):
    """Decode precision with Q4_K gate/up and down (exact sc*q in two bf16 terms,
    the min term apart, d and dmin per block)."""
    wl, yref, routing = _case(small_cases, name, cfg)
    x, act, r = run_route(wl, cfg)
    check_route(r, *routing)
    y = run_ffn(wl, x, act, r, decode=True)
    err = rel_l2(y, yref)
    print("[decode] %s rel_l2=%.3e" % (name, err))
    assert err <= DEC_TOL


def test_decode_q4k_needs_512_multiples(small_cases):
    """Q4_K decode on a shape whose K is not a multiple of 512 is refused."""
    cfg = mid(8, 35, fmt_gate_up=S.FMT_Q4K, fmt_down=S.FMT_Q4K)     # inter 384
    wl = W.Workload(cfg)
    x, act, r = run_route(wl, cfg)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        run_ffn(wl, x, act, r, decode=True)


def test_route_ties_go_to_lower_index():
    cfg = mid(40, 19)
    wl = W.Workload(cfg)
    wr = S.router_weight(cfg)
    wr[9] = wr[3]
    wr[12] = wr[3]
    wl.layer.tensors[4].copy_(torch.from_numpy(wr))
    x, act = wl.tokens(cfg)
    r = M.Routing(40, cfg["top_k"], cfg["n_experts"])
    M.route(wl.layer, x, act, 40, None, r, wl.layer.workspace(40, M.PATH_ROUTE))
    torch.cuda.synchronize()
    xf = S.bf16_to_f32(S.tokens(cfg)[0])
    idx, w, _ = R.route(xf, wr, cfg["top_k"])
    assert np.array_equal(r.topk_idx.cpu().numpy(), idx)
    got = r.topk_idx.cpu().numpy()
    for t in range(40):
        row = got[t].tolist()
        if 3 in row and 9 in row:
            assert row.index(3) < row.index(9)


def test_T0_is_a_noop():
    cfg = mid(4, 20)
    wl = W.Workload(cfg)
    x, act = wl.tokens(cfg)
    r = M.Routing(4, cfg["top_k"], cfg["n_experts"])
    y = torch.full((4, cfg["hidden"]), 7.0, device="cuda")
    ws = wl.layer.workspace(4, M.PATH_PREFILL)
    M.route(wl.layer, x, act, 0, None, r, wl.layer.workspace(4, M.PATH_ROUTE))
    M.ffn_decode(wl.layer, x, act, 0, r, y, ws)
    M.ffn_prefill(wl.layer, x, act, 0, r, y, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("name,cfg", [c for c in SMALL if c[1]["T"] == 1], ids=lambda v: v if isinstance(v, str) else "")
def test_repeated_calls_reuse_workspace(small_cases, name, cfg):
    """Three calls on one workspace give bit-identical results (no state is
    carried between calls)."""
    wl, _, _ = _case(small_cases, name, cfg)
    x, act = wl.tokens(cfg)
    T = x.shape[0]
    r = M.Routing(T, cfg["top_k"], cfg["n_experts"])
    ws_r = wl.layer.workspace(T, M.PATH_ROUTE)
    ws_f = wl.layer.workspace(T, M.PATH_DECODE)
    outs = []
    for _ in range(3):
        y = torch.full((T, cfg["hidden"]), float("nan"), device="cuda")
        M.route(wl.layer, x, act, T, wl.bias(cfg), r, ws_r)
        M.ffn_decode(wl.layer, x, act, T, r, y, ws_f)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_decode_batch_invariance():
    """Each token's decode output is the same whether it is computed alone or
    in a batch of 24 (the pages require batched decode rows to return exactly
    the logits of running each session alone -- "Part 5: serving layer",
    section 6)."""
    cfg = mid(24, 21, skew=True)
    wl = W.Workload(cfg)
    x, act, r = run_route(wl, cfg)
    yb = run_ffn(wl, x, act, r, decode=True)
    for t in (0, 5, 23):
        xt = x[t:t + 1].contiguous()
        r1 = M.Routing(1, cfg["top_k"], cfg["n_experts"])
        M.route(wl.layer, xt, act, 1, wl.bias(cfg), r1, wl.layer.workspace(1, M.PATH_ROUTE))
        y1 = run_ffn(wl, xt, act, r1, decode=True)
        assert np.array_equal(y1[0].view(np.uint32), yb[t].view(np.uint32)), t


def test_decode_batch_invariance_gemm():
    """The same for the grouped-GEMM decode path (T >= 2): a token's output
    does not depend on which other tokens share its call or its row tiles."""
    cfg = mid(24, 29, hidden=1024, inter=512, sh_inter=512, skew=True)
    wl = W.Workload(cfg)
    x, act, r = run_route(wl, cfg)
    yb = run_ffn(wl, x, act, r, decode=True)
    # sub-batches of 6 tokens: above the size that runs token by token
    for t in (0, 5, 18):
        xt = x[t:t + 6].contiguous()
        r6 = M.Routing(6, cfg["top_k"], cfg["n_experts"])
        M.route(wl.layer, xt, act, 6, wl.bias(cfg), r6, wl.layer.workspace(6, M.PATH_ROUTE))
        y6 = run_ffn(wl, xt, act, r6, decode=True)
        assert np.array_equal(y6.view(np.uint32), yb[t:t + 6].view(np.uint32)), t


# ------------------------------------------------------------------ full-size workloads
@pytest.fixture(scope="module")
def big():
    return W.Workload(S.config("decode1"), cache_dir=CACHE, progress=True)


@pytest.fixture(scope="module")
def big_q4k():
    return W.Workload(S.config("prefill8192_q4k"), cache_dir=CACHE, progress=True)


def sampled_check(wl, cfg, decode, n_sample, hot=0):
    """Routing in full; y on sampled tokens: the first, the last, n_sample drawn
    ones and, with hot > 0, the tokens in the first and last rows of the `hot`
    most-assigned experts (their last row tile is the partial one).  n_sample
    >= T compares every token."""
    x, act, r = run_route(wl, cfg)
    xf, idx, w, l, off, perm, inv = oracle_routing(cfg)
    check_route(r, idx, w, off, perm, inv)
    y = run_ffn(wl, x, act, r, decode=decode)
    T, k = x.shape[0], cfg["top_k"]
    rng = np.random.default_rng(T)
    picks = [[0, T - 1], rng.choice(T, size=min(n_sample, T), replace=False)]
    if hot:
        counts = np.diff(off)
        for e in np.argsort(-counts, kind="stable")[:hot]:
            picks.append([perm[off[e]] // k, perm[off[e + 1] - 1] // k])
    toks = np.unique(np.concatenate(picks))
    yref = R.moe_layer(xf[toks], idx[toks], w[toks], expert_loader(cfg, wl.packed), oracle_shared(cfg),
                       threads=ORACLE_THREADS)
    err = rel_l2(y[toks], yref)
    print("[%s] %s tokens=%s rel_l2=%.3e" % ("decode" if decode else "prefill", cfg["name"], toks.tolist(), err))
    assert np.all(np.isfinite(y))
    return err


def test_full_decode1(big):
    assert sampled_check(big, S.config("decode1"), True, 1) <= DEC_TOL


def test_full_decode32(big):
    """Every one of the 32 tokens at the full layer shape."""
    assert sampled_check(big, S.config("decode32"), True, 32) <= DEC_TOL


@pytest.mark.parametrize("T", [2, 3, 4, 6])
def test_full_decode_small_batches(big, T):
    """Batched decode at the full layer shape for the smallest batches (one or
    two rows per selected expert, the shared expert in one row tile)."""
    assert sampled_check(big, S.config("decode32", T=T), True, 1) <= DEC_TOL


def test_full_decode_tokenwise_bit_identical(big):
    """Decode batches of up to four tokens run the single-token kernels token by
    token, so each token's y is bit-identical to decoding it alone."""
    cfg = S.config("decode32", T=4)
    x, act, r = run_route(big, cfg)
    yb = run_ffn(big, x, act, r, decode=True)
    for t in (0, 3):
        xt = x[t:t + 1].contiguous()
        r1 = M.Routing(1, cfg["top_k"], cfg["n_experts"])
        M.route(big.layer, xt, act, 1, big.bias(cfg), r1, big.layer.workspace(1, M.PATH_ROUTE))
        y1 = run_ffn(big, xt, act, r1, decode=True)
        assert np.array_equal(y1[0].view(np.uint32), yb[t].view(np.uint32)), t


def test_full_decode_tokenwise_flag(big):
    """With the layer's token-by-token flag every decode batch runs the
    single-token kernels, so all 32 tokens of the full-size decode batch come
    out bit-identical to the same tokens in batches of 1, 3 and 8 (the pages
    require batched decode to return exactly what each session alone would --
    "Part 5: serving layer", section 6), and still match the oracle."""
    cfg = S.config("decode32")
    x, act, r = run_route(big, cfg)
    T, k, E = x.shape[0], cfg["top_k"], cfg["n_experts"]
    big.layer.c.flags = M.LAYER_TOKENWISE_DECODE
    try:
        y = run_ffn(big, x, act, r, decode=True)
        for B in (1, 3, 8):
            for t0 in range(0, T - B + 1, max(B, 5)):
                xt = x[t0:t0 + B].contiguous()
                rb = M.Routing(B, k, E)
                M.route(big.layer, xt, act, B, big.bias(cfg), rb, big.layer.workspace(B, M.PATH_ROUTE))
                yb = run_ffn(big, xt, act, rb, decode=True)
                assert np.array_equal(yb.view(np.uint32), y[t0:t0 + B].view(np.uint32)), (B, t0)
    finally:
        big.layer.c.flags = 0
    xf, idx, w, l, off, perm, inv = oracle_routing(cfg)
    toks = np.array([0, 7, 19, 31])
    yref = R.moe_layer(xf[toks], idx[toks], w[toks], expert_loader(cfg, big.packed), oracle_shared(cfg),
                       threads=ORACLE_THREADS)
    assert rel_l2(y[toks], yref) <= DEC_TOL


def test_full_decode32_one_stream_flag(big):
    """Batched decode of the full layer runs the shared expert's chain on a
    second stream beside the routed kernels; with the one-stream flag every
    launch stays on the caller's stream, and y is the same bit for bit.  Three
    calls enqueued back to back on one stream without a host wait between
    them (each forks and joins on its own) give each call's result too."""
    cfg = S.config("decode32")
    x, act, r = run_route(big, cfg)
    T, k, E, H = x.shape[0], cfg["top_k"], cfg["n_experts"], cfg["hidden"]
    y2 = run_ffn(big, x, act, r, decode=True)
    big.layer.c.flags = M.LAYER_ONE_STREAM
    try:
        y1 = run_ffn(big, x, act, r, decode=True)
    finally:
        big.layer.c.flags = 0
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    parts = [(0, 32), (3, 20), (11, 27)]
    alone, queued = [], []
    for a, b in parts:
        xt = x[a:b].contiguous()
        rb = M.Routing(b - a, k, E)
        M.route(big.layer, xt, act, b - a, big.bias(cfg), rb, big.layer.workspace(b - a, M.PATH_ROUTE))
        alone.append(run_ffn(big, xt, act, rb, decode=True))
        queued.append((xt, rb, torch.full((b - a, H), float("nan"), device="cuda"),
                       big.layer.workspace(b - a, M.PATH_DECODE)))
    torch.cuda.synchronize()
    for xt, rb, yq, ws in queued:
        M.ffn_decode(big.layer, xt, act, xt.shape[0], rb, yq, ws)
    torch.cuda.synchronize()
    for (xt, rb, yq, ws), ya in zip(queued, alone):
        assert np.array_equal(yq.cpu().numpy().view(np.uint32), ya.view(np.uint32))


def test_full_decode32_graph_replay(big):
    """The batched decode call -- routed kernels on the caller's stream, the
    shared expert's chain forked onto the library's second stream and joined
    back -- captured into a HIP graph (after an eager call, which creates the
    second stream): every replay, with eager calls and synchronisations
    between the replays, gives the eager y bit for bit."""
    cfg = S.config("decode32")
    x, act, r = run_route(big, cfg)
    T, H = x.shape[0], cfg["hidden"]
    y_eager = run_ffn(big, x, act, r, decode=True)
    ws = big.layer.workspace(T, M.PATH_DECODE)
    y = torch.full((T, H), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.ffn_decode(big.layer, x, act, T, r, y, ws, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        M.ffn_decode(big.layer, x, act, T, r, y, ws, s)
    torch.cuda.synchronize()
    for i in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_eager.view(np.uint32)), i
        assert np.array_equal(run_ffn(big, x, act, r, decode=True).view(np.uint32), y_eager.view(np.uint32)), i


def test_full_decode32_two_threads(big):
    """Two host threads each enqueue four batched decode calls on a stream and a
    workspace of their own; every call forks the shared expert's chain onto
    the device's one second stream and joins it back (the library serialises
    those enqueues).  Every output equals the single-threaded one bit for
    bit."""
    import threading
    cfg = S.config("decode32")
    x, act, r = run_route(big, cfg)
    T, H = x.shape[0], cfg["hidden"]
    y_ref = run_ffn(big, x, act, r, decode=True)
    jobs = []
    for _ in range(2):
        st = torch.cuda.Stream()
        ws = big.layer.workspace(T, M.PATH_DECODE)
        ys = [torch.full((T, H), float("nan"), device="cuda") for _ in range(4)]
        jobs.append((st, ws, ys))
    torch.cuda.synchronize()
    errs = []

    def worker(st, ws, ys):
        try:
            for y in ys:
                M.ffn_decode(big.layer, x, act, T, r, y, ws, st)
        except Exception as e:          # reported below, on the main thread
            errs.append(e)

    th = [threading.Thread(target=worker, args=j) for j in jobs]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for st, ws, ys in jobs:
        for y in ys:
            assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


def test_full_decode32_q4k(big_q4k):
    assert sampled_check(big_q4k, S.config("decode32_q4k"), True, 8) <= DEC_TOL


def test_full_prefill2048(big):
    assert sampled_check(big, S.config("prefill2048"), False, 2, hot=8) <= PRE_TOL


def test_full_prefill8192(big):
    assert sampled_check(big, S.config("prefill8192"), False, 2, hot=8) <= PRE_TOL


def test_full_prefill8192_q4k(big_q4k):
    assert sampled_check(big_q4k, S.config("prefill8192_q4k"), False, 2, hot=8) <= PRE_TOL


@pytest.fixture(scope="module")
def big_cb2s():
    return W.Workload(S.config("prefill2048_cb2s"), cache_dir=CACHE, progress=True)


def test_full_prefill2048_cb2s(big_cb2s):
    """The signed codebook format at the full layer shape: the in-register
    dequant grouped GEMM, sampled tokens including the first and last rows of
    the two most-assigned experts (the oracle packs every expert it reads and
    checks the library's bytes against its own)."""
    assert sampled_check(big_cb2s, S.config("prefill2048_cb2s"), False, 1, hot=2) <= PRE_TOL


def test_full_decode32_cb2s(big_cb2s):
    assert sampled_check(big_cb2s, S.config("decode32_cb2s"), True, 2) <= DEC_TOL


# ------------------------------------------------------------------ router shapes
# Router alone (the expert weights are never read by moe_route): every
# selection-kernel specialisation at T = 1 (experts per lane 1, 2, 4, 8, 16),
# the fp64 MFMA logits with token and expert tails and a bias, and the plain
# tiled logits when H is not a multiple of 64.
@pytest.mark.parametrize("T,E,k,H,bias", [(1, 100, 6, 512, False), (1, 500, 8, 768, True), (1, 1000, 12, 256, False),
                                          (1, 64, 64, 512, False), (130, 300, 8, 640, True), (100, 40, 5, 352, False),
                                          (70, 1024, 3, 128, True)],
                         ids=["T1_E100", "T1_E500_bias", "T1_E1000", "T1_k_eq_E", "T130_E300_bias", "T100_H352",
                              "T70_E1024_bias"])
def test_route_shapes(T, E, k, H, bias):
    rng = np.random.default_rng(T * 7919 + E * 31 + k)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    xb = S.bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    b = (rng.standard_normal(E) * 0.01).astype(np.float32) if bias else None
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    cb = torch.from_numpy(S.codebook()).cuda()
    dl = M.DeviceLayer(H, 256, E, k, S.FMT_CB2, S.FMT_Q2K, dummy, dummy, dummy, cb, torch.from_numpy(wr).cuda())
    r = M.Routing(T, k, E)
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    bt = torch.from_numpy(b).cuda() if bias else None
    M.route(dl, x, M.ACT_BF16, T, bt, r, dl.workspace(T, M.PATH_ROUTE))
    torch.cuda.synchronize()
    idx, w, _ = R.route(S.bf16_to_f32(xb), wr, k, b)
    off, perm, inv = R.group(idx, E)
    check_route(r, idx, w, off, perm, inv)


# ------------------------------------------------------------------ non-finite router input
@pytest.mark.parametrize("T", [1, 20, 100])
def test_route_nan_token_stays_a_permutation(T):
    """A token whose activations are NaN has NaN logits, which rank below every
    number: its k experts are still distinct, perm stays a permutation, and the
    other tokens route exactly as the oracle routes them (one T per router
    path: single token, small batch, large batch)."""
    cfg = mid(T, 47, n_experts=16, top_k=4)
    wl = W.Workload(cfg)
    x, act = wl.tokens(cfg)
    bad = T // 2
    x[bad] = 0x7fc0                                      # bf16 quiet NaN
    r = M.Routing(T, cfg["top_k"], cfg["n_experts"])
    M.route(wl.layer, x, act, T, None, r, wl.layer.workspace(T, M.PATH_ROUTE))
    torch.cuda.synchronize()
    idx, off, perm, inv = (a.cpu().numpy() for a in (r.topk_idx, r.offsets, r.perm, r.inv))
    k, E = cfg["top_k"], cfg["n_experts"]
    assert all(len(set(row.tolist())) == k for row in idx)
    assert idx.min() >= 0 and idx.max() < E
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    assert np.array_equal(inv[perm], np.arange(T * k))
    assert np.array_equal(np.diff(off), np.bincount(idx.reshape(-1), minlength=E))
    xf = S.bf16_to_f32(S.tokens(cfg)[0])
    ref, _, _ = R.route(xf, S.router_weight(cfg), k)
    keep = np.arange(T) != bad
    assert np.array_equal(idx[keep], ref[keep])


# ------------------------------------------------------------------ format breadth
# The wider routed layouts (Q5_K gate/up, Q5_K / Q6_K down, Q2_K gate/up) on
# the in-register-dequant grouped GEMMs: every output element, prefill with
# multi-tile experts, decode batched and single-token, fp32 and bf16 x.
FMT_PAIRS = [(S.FMT_Q5K, S.FMT_Q6K), (S.FMT_Q2K, S.FMT_Q5K), (S.FMT_Q4K, S.FMT_Q6K), (S.FMT_CB2, S.FMT_Q6K),
             (S.FMT_Q5K, S.FMT_Q5K), (S.FMT_CB2S, S.FMT_Q2K), (S.FMT_CB2S, S.FMT_Q4K)]
PAIR_IDS = ["%s_%s" % ({1: "cb2", 2: "q2k", 3: "q4k", 5: "q5k", 7: "cb2s"}[a],
                       {2: "q2k", 3: "q4k", 5: "q5k", 6: "q6k"}[b]) for a, b in FMT_PAIRS]


@pytest.mark.parametrize("fg,fd", FMT_PAIRS, ids=PAIR_IDS)
def test_prefill_formats(small_cases, fg, fd):
    name = "fmt_pre_%d_%d" % (fg, fd)
    cfg = mid(400, 60 + 2 * fg + fd, skew=True, fmt_gate_up=fg, fmt_down=fd, **dict(GEMM, top_k=4))
    wl, yref, routing = _case(small_cases, name, cfg)
    x, act, r = run_route(wl, cfg)
    check_route(r, *routing)
    y = run_ffn(wl, x, act, r, decode=False)
    err = rel_l2(y, yref)
    print("[prefill] %s rel_l2=%.3e" % (name, err))
    assert err <= PRE_TOL


@pytest.mark.parametrize("T,xdt", [(1, "bf16"), (3, "f32"), (45, "bf16"), (70, "f32")])
@pytest.mark.parametrize("fg,fd", FMT_PAIRS, ids=PAIR_IDS)
def test_decode_formats(small_cases, fg, fd, T, xdt):
    name = "fmt_dec_%d_%d_%d_%s" % (fg, fd, T, xdt)
    cfg = mid(T, 70 + 2 * fg + fd, skew=True, x_dtype=xdt, fmt_gate_up=fg, fmt_down=fd, **GEMM)
    wl, yref, routing = _case(small_cases, name, cfg)
    x, act, r = run_route(wl, cfg)
    check_route(r, *routing)
    y = run_ffn(wl, x, act, r, decode=True)
    err = rel_l2(y, yref)
    print("[decode] %s rel_l2=%.3e" % (name, err))
    assert err <= DEC_TOL


@pytest.mark.parametrize("recipe", ["q2-q4", "q5-q6", "q2s"])
def test_layer_recipe_stack(recipe):
    """A stack of four layers quantized by a per-layer recipe, each layer's fp32
    output the next layer's input (decode path), every layer's output compared
    with the oracle's own chain.  Each layer is its own seeded layer."""
    n, T = 4, 12
    base = mid(T, 80, x_dtype="bf16", **GEMM)
    x_dev, act = None, None
    x_ref = S.bf16_to_f32(S.tokens(base)[0])
    for l in range(n):
        fg, fd = S.layer_formats(recipe, l, n)
        cfg = dict(base, seed=1000 + l, fmt_gate_up=fg, fmt_down=fd, x_dtype="bf16" if l == 0 else "f32")
        wl = W.Workload(cfg)
        if l == 0:
            x_dev, act = wl.tokens(cfg)
        r = M.Routing(T, cfg["top_k"], cfg["n_experts"])
        M.route(wl.layer, x_dev, act, T, None, r, wl.layer.workspace(T, M.PATH_ROUTE))
        y = torch.empty((T, cfg["hidden"]), device="cuda")
        M.ffn_decode(wl.layer, x_dev, act, T, r, y, wl.layer.workspace(T, M.PATH_DECODE))
        torch.cuda.synchronize()
        seed = cfg["seed"]
        idx, w, _ = R.route(x_ref, S.router_weight(cfg, seed), cfg["top_k"])
        ex = {}
        cb = S.codebook_for(fg, seed)
        for e in np.unique(idx):
            mats = []
            for which, fmt, rows, K in (("gate", fg, cfg["inter"], cfg["hidden"]), ("up", fg, cfg["inter"], cfg["hidden"]),
                                        ("down", fd, cfg["hidden"], cfg["inter"])):
                mats.append(F.unpack(fmt, F.pack(fmt, S.expert_weight(cfg, which, int(e), seed), cb), rows, K, cb))
            ex[int(e)] = tuple(mats)
        sh = tuple(S.bf16_to_f32(S.shared_weight_bf16(cfg, nm, seed)) for nm in ("gate", "up", "down"))
        yref = R.moe_layer(x_ref, idx, w, ex, sh)
        got = y.cpu().numpy()
        err = rel_l2(got, yref)
        print("[recipe %s] layer %d formats %d/%d rel_l2=%.3e" % (recipe, l, fg, fd, err))
        assert err <= DEC_TOL
        x_dev, act = y, M.ACT_F32
        x_ref = yref.astype(np.float32)


# ------------------------------------------------------------------ fused layer decode
def run_layer_decode(wl, cfg, T=None):
    x, act = wl.tokens(cfg, T)
    T = x.shape[0]
    r = M.Routing(T, wl.cfg["top_k"], wl.cfg["n_experts"])
    y = torch.full((T, wl.cfg["hidden"]), float("nan"), device="cuda")
    M.layer_decode(wl.layer, x, act, T, wl.bias(cfg), r, y, wl.layer.workspace(T, M.PATH_LAYER_DECODE))
    torch.cuda.synchronize()
    return r, y.cpu().numpy()


LAYER = [c for c in SMALL if c[0].startswith("one_T1") or c[0] in ("mid_T1", "gemm_T37", "tiny")] + [
    ("one_T1_skew", mid(1, 48, hidden=1024, inter=512, sh_inter=512, skew=True)),
    ("one_T1_E300", mid(1, 49, hidden=1024, inter=512, sh_inter=512, n_experts=300, top_k=8)),
]


@pytest.mark.parametrize("name,cfg", LAYER, ids=[n for n, _ in LAYER])
def test_layer_decode(small_cases, name, cfg):
    """moe_layer_decode: the routing outputs equal the oracle's, y is within the
    decode bar, and both are bit-identical to moe_route + moe_expert_ffn_decode
    (single tokens run the router inside the FFN's launches; other cases the
    two calls)."""
    wl, yref, routing = _case(small_cases, name, cfg)
    r, y = run_layer_decode(wl, cfg)
    check_route(r, *routing)
    err = rel_l2(y, yref)
    print("[layer] %s rel_l2=%.3e" % (name, err))
    assert err <= DEC_TOL
    x2, act2, r2 = run_route(wl, cfg)
    y2 = run_ffn(wl, x2, act2, r2, decode=True)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    for a, b in ((r.topk_idx, r2.topk_idx), (r.topk_w, r2.topk_w), (r.offsets, r2.offsets), (r.perm, r2.perm),
                 (r.inv, r2.inv)):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("wname", ["decode1", "decode32_T1"])
def test_full_layer_decode(big, wname):
    """The fused single-token layer at the full layer shape (with the Zipf bias
    for decode32's first token): routing in full and y against the oracle, and
    bit-identical to the two separate calls, also on a reused workspace."""
    cfg = S.config("decode1") if wname == "decode1" else S.config("decode32", T=1)
    r, y = run_layer_decode(big, cfg)
    xf, idx, w, l, off, perm, inv = oracle_routing(cfg)
    check_route(r, idx, w, off, perm, inv)
    yref = R.moe_layer(xf, idx, w, expert_loader(cfg, big.packed), oracle_shared(cfg), threads=ORACLE_THREADS)
    err = rel_l2(y, yref)
    print("[layer] %s rel_l2=%.3e" % (wname, err))
    assert err <= DEC_TOL
    x2, act2, r2 = run_route(big, cfg)
    y2 = run_ffn(big, x2, act2, r2, decode=True)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    r3, y3 = run_layer_decode(big, cfg)
    assert np.array_equal(y.view(np.uint32), y3.view(np.uint32))
