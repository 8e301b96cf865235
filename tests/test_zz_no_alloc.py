"""The no-allocation decode entry point (moe_expert_ffn_decode_noalloc, for
callers that cannot allocate device memory) against moe_expert_ffn_decode.

Both run the same kernels, so the outputs must agree bit for bit.  Two calls in
a row on the shared scratch array, the second with a smaller batch, so the
second runs over what the first left behind; the reference calls get a
workspace filled with 0xff bytes, so neither side may read workspace it did
not write.  Called through the C ABI (ctypes), as a caller would.
"""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_routed_amd as M
import synthetic as S
import workload as W
from gpu_common import need_gpu

pytestmark = pytest.mark.gpu

GEMM = dict(hidden=1024, inter=512, sh_inter=512, n_experts=16, top_k=4, x_dtype="bf16", skew=True,
            fmt_gate_up=S.FMT_CB2, fmt_down=S.FMT_Q2K, name="noalloc")


def _route(wl, cfg, T):
    x, act = wl.tokens(cfg, T)
    r = M.Routing(T, cfg["top_k"], cfg["n_experts"])
    M.route(wl.layer, x, act, T, wl.bias(cfg), r, wl.layer.workspace(T, M.PATH_ROUTE))
    return x, act, r


def _ref(wl, cfg, x, act, r, T):
    ws = wl.layer.workspace(T, M.PATH_DECODE)
    ws.fill_(0xFF)
    y = torch.full((T, cfg["hidden"]), float("nan"), device="cuda")
    M.ffn_decode(wl.layer, x, act, T, r, y, ws)
    return y


def _noalloc(wl, cfg, x, act, r, T):
    y = torch.full((T, cfg["hidden"]), float("nan"), device="cuda")
    rc = M.lib().moe_expert_ffn_decode_noalloc(
        ctypes.byref(wl.layer.c), x.data_ptr(), act, T, r.topk_idx.data_ptr(), r.topk_w.data_ptr(),
        r.offsets.data_ptr(), r.perm.data_ptr(), r.inv.data_ptr(), y.data_ptr(),
        torch.cuda.current_stream().cuda_stream, None)
    assert rc == 0, M.lib().moe_last_error()
    return y


@pytest.mark.parametrize("cfg,T1,T2", [
    (dict(GEMM, index=50), 40, 7),                       # grouped-GEMM decode, twice
    (dict(GEMM, index=51, x_dtype="f32"), 24, 1),        # grouped GEMM, then the single-token kernels
    (dict(GEMM, index=52, fmt_gate_up=S.FMT_Q4K, fmt_down=S.FMT_Q4K), 33, 5),
])
def test_noalloc_matches_decode(cfg, T1, T2):
    need_gpu()
    print("[noalloc] %s T=%d then T=%d" % (cfg["index"], T1, T2), flush=True)
    cfg = dict(cfg, T=T1)
    wl = W.Workload(cfg)
    for T in (T1, T2):
        x, act, r = _route(wl, cfg, T)
        ref = _ref(wl, cfg, x, act, r, T)
        got = _noalloc(wl, cfg, x, act, r, T)
        torch.cuda.synchronize()
        a, b = ref.cpu().numpy(), got.cpu().numpy()
        assert np.all(np.isfinite(a))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), T


def test_noalloc_refuses_oversized_batch():
    need_gpu()
    cfg = dict(GEMM, index=53, T=4)
    wl = W.Workload(cfg)
    T = 1
    while M.workspace_bytes(wl.layer.c, T, M.PATH_DECODE) <= M.NOALLOC_SCRATCH_BYTES:
        T *= 2
    x = torch.zeros((T, cfg["hidden"]), dtype=torch.int16, device="cuda")
    r = M.Routing(T, cfg["top_k"], cfg["n_experts"])
    y = torch.empty((T, cfg["hidden"]), device="cuda")
    rc = M.lib().moe_expert_ffn_decode_noalloc(
        ctypes.byref(wl.layer.c), x.data_ptr(), M.ACT_BF16, T, r.topk_idx.data_ptr(), r.topk_w.data_ptr(),
        r.offsets.data_ptr(), r.perm.data_ptr(), r.inv.data_ptr(), y.data_ptr(),
        torch.cuda.current_stream().cuda_stream, None)
    assert rc == -3 and b"scratch" in M.lib().moe_last_error()
