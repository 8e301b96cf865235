"""Pins for the oracle expert FFN and combine (CPU only).

Checked against: a hand-evaluated SwiGLU, an independent dense evaluation
(einsum over all experts with a dense [T, E] routing matrix, no grouping),
the k = 1 reduction to one dense FFN, x = 0 -> y = 0, invariance under
relabelling the experts, linearity in the routing weights and row
independence of the tokens.
"""
import json
import os

import numpy as np

from oracle import moe_ref as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")))


def _layer(rng, E=6, H=24, I=10, sh=True):
    ex = {e: ((rng.standard_normal((I, H)) * 0.2), (rng.standard_normal((I, H)) * 0.2),
              (rng.standard_normal((H, I)) * 0.2)) for e in range(E)}
    shared = ((rng.standard_normal((I, H)) * 0.2), (rng.standard_normal((I, H)) * 0.2),
              (rng.standard_normal((H, I)) * 0.2)) if sh else None
    Wr = rng.standard_normal((E, H)) * 0.3
    return ex, shared, Wr


def test_hand_swiglu():
    g = GOLD["swiglu"]
    y = R.swiglu_ffn(np.array(g["x"]), np.array(g["w_gate"]), np.array(g["w_up"]), np.array(g["w_down"]))
    assert np.allclose(y, g["expect_y"], rtol=0, atol=1e-15)


def test_matches_dense_einsum():
    rng = np.random.default_rng(31)
    E, H, I, T, k = 6, 24, 10, 9, 3
    ex, shared, Wr = _layer(rng, E, H, I)
    x = rng.standard_normal((T, H))
    idx, w, _ = R.route(x, Wr, k)
    y = R.moe_layer(x, idx, w, ex, shared)
    # dense: every expert on every token, weighted by a dense routing matrix
    Rm = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            Rm[t, idx[t, j]] = w[t, j]
    G = np.stack([ex[e][0] for e in range(E)])
    U = np.stack([ex[e][1] for e in range(E)])
    D = np.stack([ex[e][2] for e in range(E)])
    g = np.einsum("th,eih->tei", x, G)
    u = np.einsum("th,eih->tei", x, U)
    h = g / (1 + np.exp(-g)) * u
    routed = np.einsum("tei,ehi->teh", h, D)
    gs, us = x @ shared[0].T, x @ shared[1].T
    dense = np.einsum("te,teh->th", Rm, routed) + (gs / (1 + np.exp(-gs)) * us) @ shared[2].T
    assert np.allclose(y, dense, rtol=0, atol=1e-12)


def test_k1_is_one_dense_ffn():
    rng = np.random.default_rng(32)
    ex, _, Wr = _layer(rng, sh=False)
    x = rng.standard_normal((5, 24))
    idx = np.full((5, 1), 3, np.int32)
    w = np.ones((5, 1), np.float32)
    y = R.moe_layer(x, idx, w, ex, None)
    wg, wu, wd = ex[3]
    g, u = x @ wg.T, x @ wu.T
    assert np.allclose(y, (g / (1 + np.exp(-g)) * u) @ wd.T, rtol=0, atol=1e-13)


def test_zero_input_gives_zero():
    rng = np.random.default_rng(33)
    ex, shared, Wr = _layer(rng)
    x = np.zeros((4, 24))
    idx, w, _ = R.route(x, Wr, 2)
    assert np.all(R.moe_layer(x, idx, w, ex, shared) == 0)


def test_relabelling_invariance():
    rng = np.random.default_rng(34)
    E = 6
    ex, shared, Wr = _layer(rng, E)
    x = rng.standard_normal((7, 24))
    idx, w, _ = R.route(x, Wr, 2)
    y = R.moe_layer(x, idx, w, ex, shared)
    p = rng.permutation(E)                      # new label of old expert e is p[e]
    ex2 = {int(p[e]): ex[e] for e in range(E)}
    Wr2 = np.empty_like(Wr)
    Wr2[p] = Wr
    idx2, w2, _ = R.route(x, Wr2, 2)
    assert np.array_equal(idx2, p[idx])
    assert np.allclose(R.moe_layer(x, idx2, w2, ex2, shared), y, rtol=0, atol=1e-13)


def test_linear_in_routing_weights():
    rng = np.random.default_rng(35)
    ex, shared, Wr = _layer(rng)
    x = rng.standard_normal((5, 24))
    idx, w, _ = R.route(x, Wr, 3)
    w = w.astype(np.float64)
    base = R.moe_layer(x, idx, np.zeros_like(w), ex, shared)
    r1 = R.moe_layer(x, idx, w, ex, shared) - base
    r2 = R.moe_layer(x, idx, 2.5 * w, ex, shared) - base
    assert np.allclose(r2, 2.5 * r1, rtol=1e-12, atol=1e-13)


def test_tokens_are_independent():
    rng = np.random.default_rng(36)
    ex, shared, Wr = _layer(rng)
    x = rng.standard_normal((6, 24))
    idx, w, _ = R.route(x, Wr, 2)
    y = R.moe_layer(x, idx, w, ex, shared)
    for t in range(6):
        yt = R.moe_layer(x[t:t + 1], idx[t:t + 1], w[t:t + 1], ex, shared)
        assert np.allclose(yt[0], y[t], rtol=0, atol=1e-14)


def test_expert_loader_and_threads_give_the_same_layer():
    """Passing the experts as a loader (one at a time) and evaluating them in
    threads changes nothing: same bits as the mapping form."""
    rng = np.random.default_rng(5)
    T, H, I, E, k = 9, 32, 16, 6, 3
    x = rng.standard_normal((T, H))
    ex = {e: tuple(rng.standard_normal(s) * 0.1 for s in ((I, H), (I, H), (H, I))) for e in range(E)}
    idx = np.argsort(rng.standard_normal((T, E)), axis=1)[:, :k].astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    calls = []
    load = lambda e: (calls.append(e), ex[e])[1]
    a = R.moe_layer(x, idx, w, ex)
    b = R.moe_layer(x, idx, w, load, threads=4)
    assert np.array_equal(a, b)
    assert sorted(calls) == sorted(set(idx.reshape(-1).tolist()))
