"""Reference routed-MoE layer: router, grouping, expert FFN, combine (fp64).

TEST INFRASTRUCTURE ONLY (oracle).

The layer computes, for each token t,

    y[t] = FFN_sh(x_t) + sum_{j<k} w[t,j] * FFN_{e(t,j)}(x_t)
    FFN_e(x) = W_down,e . ( silu(W_gate,e . x) * (W_up,e . x) ),  silu(g) = g / (1 + exp(-g))

with the routed W the exact dequantized weights and the shared expert in
bf16.  The pages fix which parts are quantized and that the router stays at
full precision ("DwarfStar" README, section on model weights; deep-dive
article, section 3.4.3, which keeps the router high precision so routing
decisions stay reliable).  The router function itself (sigmoid scores over
x.W_r, top-k, scores renormalised to sum 1) and the SwiGLU form are the
workload's definition; the pages do not print them.

Readings taken where the definition leaves a step open:
  * logits accumulate in fp64 (x and W_r widened exactly);
  * top-k orders by logit, descending; equal logits go to the lower expert
    index (sigmoid is monotone, so this is the order of the scores too);
  * the weights are the selected sigmoid scores divided by their sum,
    computed in fp64 and rounded to fp32;
  * grouping sorts assignments a = t*k + j by (expert, token); perm lists
    them in that order, inv is its inverse, offsets[e] is the first position
    of expert e (exclusive prefix sum of the per-expert counts);
  * the combine adds the k routed outputs in top-k order (j = 0..k-1) after
    the shared-expert output, in fp64, and rounds y to fp32 at the end.
"""
from __future__ import annotations

import numpy as np


def router_logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """l[t, e] = sum_h x[t,h] * W_r[e,h] + b[e], in fp64."""
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def topk(logits: np.ndarray, k: int):
    """Indices of the k largest logits per row, descending, ties to the lower index."""
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def route_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w = s_sel / sum(s_sel) with s = 1 / (1 + exp(-l)); fp64 -> fp32."""
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    s = 1.0 / (1.0 + np.exp(-sel))
    return (s / s.sum(axis=1, keepdims=True)).astype(np.float32)


def route(x, w_router, k, bias=None):
    """Full router: returns (topk_idx int32 [T,k], topk_w fp32 [T,k], logits fp64 [T,E])."""
    l = router_logits(x, w_router, bias)
    idx = topk(l, k)
    return idx, route_weights(l, idx), l


def group(topk_idx: np.ndarray, n_experts: int):
    """Counting sort of the assignments by (expert, token).

    Returns offsets int32 [E+1], perm int32 [T*k] (assignment ids a = t*k+j in
    sorted order) and inv int32 [T*k] (inv[a] = position of a in perm).
    """
    T, k = topk_idx.shape
    e = topk_idx.reshape(-1).astype(np.int64)
    a = np.arange(T * k, dtype=np.int64)
    t = a // k
    perm = np.lexsort((t, e)).astype(np.int32)          # primary key e, then t
    inv = np.empty(T * k, np.int32)
    inv[perm] = np.arange(T * k, dtype=np.int32)
    counts = np.bincount(e, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return offsets, perm, inv


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def swiglu_ffn(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """FFN(x) = W_down (silu(W_gate x) * (W_up x)) for the rows of x, fp64.

    w_gate, w_up: [I, H]; w_down: [H, I]; x: [n, H].  Returns [n, H] fp64.
    """
    x = np.asarray(x, np.float64)
    g = x @ np.asarray(w_gate, np.float64).T
    u = x @ np.asarray(w_up, np.float64).T
    h = silu(g) * u
    return h @ np.asarray(w_down, np.float64).T


def moe_layer(x, topk_idx, topk_w, expert_weights, shared=None, threads: int = 1) -> np.ndarray:
    """y [T, H] fp64 for the given routing.

    expert_weights: mapping e -> (W_gate, W_up, W_down) of dequantized fp32
    weights, or a callable e -> the same (called once per selected expert, so
    a full-size layer never has to be held at once); only the experts the
    routing selects are looked up.
    shared: (W_gate, W_up, W_down) of the shared expert (bf16 values as fp32)
    or None.
    threads > 1 evaluates the selected experts concurrently; each expert's
    outputs depend on that expert alone, so the result is the same.
    """
    x = np.asarray(x, np.float64)
    T, k = topk_idx.shape
    H = x.shape[1]
    routed = np.zeros((T, k, H), np.float64)
    get = expert_weights if callable(expert_weights) else expert_weights.__getitem__

    def one(e):
        rows, cols = np.nonzero(topk_idx == e)
        wg, wu, wd = get(int(e))
        routed[rows, cols] = swiglu_ffn(x[rows], wg, wu, wd)

    experts = np.unique(topk_idx)
    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, experts))
    else:
        for e in experts:
            one(e)
    y = swiglu_ffn(x, *shared) if shared is not None else np.zeros((T, H), np.float64)
    w = np.asarray(topk_w, np.float64)
    for j in range(k):
        y = y + w[:, j:j + 1] * routed[:, j]
    return y
