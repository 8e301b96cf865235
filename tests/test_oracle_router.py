"""Pins for the oracle router and grouping (CPU only).

Checked against: a hand-evaluated example, correctly rounded sums
(math.fsum) with a brute-force sort, constructed ties, k = E, the sum-to-one
and positivity invariants, and a brute-force (expert, token) ordering.
"""
import json
import math
import os

import numpy as np

from oracle import moe_ref as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")))


def test_hand_example():
    g = GOLD["router"]
    idx, w, _ = R.route(np.array(g["x"]), np.array(g["w_router"], np.float32), g["k"])
    assert idx.tolist() == g["expect_idx"]
    assert np.allclose(w, g["expect_w"], rtol=0, atol=1e-7)


def test_bruteforce_topk_and_weights():
    rng = np.random.default_rng(21)
    T, E, H, k = 6, 12, 40, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    Wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    idx, w, l = R.route(x, Wr, k, b)
    for t in range(T):
        exact = [math.fsum([float(x[t, h]) * float(Wr[e, h]) for h in range(H)] + [float(b[e])])
                 for e in range(E)]
        assert np.allclose(l[t], exact, rtol=0, atol=1e-15)
        order = sorted(range(E), key=lambda e: (-exact[e], e))[:k]
        assert idx[t].tolist() == order
        s = [1.0 / (1.0 + math.exp(-exact[e])) for e in order]
        assert np.allclose(w[t], [v / sum(s) for v in s], rtol=1e-7, atol=0)


def test_ties_go_to_lower_index():
    rng = np.random.default_rng(22)
    E, H = 8, 16
    Wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    Wr[5] = Wr[2]          # experts 2 and 5 always tie
    Wr[7] = Wr[2]
    x = rng.standard_normal((20, H)).astype(np.float32)
    idx, _, l = R.route(x, Wr, 8)
    for t in range(20):
        row = idx[t].tolist()
        assert row.index(2) < row.index(5) < row.index(7)
        assert l[t, 2] == l[t, 5] == l[t, 7]


def test_k_equals_E_selects_all():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((3, 10)).astype(np.float32)
    Wr = rng.standard_normal((5, 10)).astype(np.float32)
    idx, w, l = R.route(x, Wr, 5)
    for t in range(3):
        assert sorted(idx[t].tolist()) == list(range(5))
        assert np.all(np.diff(l[t, idx[t]]) <= 0)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_weights_positive_and_normalised():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((50, 64)).astype(np.float32)
    Wr = (rng.standard_normal((32, 64)) * 0.02).astype(np.float32)
    _, w, _ = R.route(x, Wr, 8)
    assert np.all(w > 0)
    assert np.allclose(w.sum(axis=1), 1.0, atol=4e-7)


def test_large_bias_forces_expert():
    rng = np.random.default_rng(25)
    x = rng.standard_normal((10, 32)).astype(np.float32)
    Wr = (rng.standard_normal((16, 32)) * 0.02).astype(np.float32)
    b = np.zeros(16, np.float32)
    b[9] = 100.0
    idx, _, _ = R.route(x, Wr, 2, b)
    assert np.all(idx[:, 0] == 9)


def test_group_matches_bruteforce_sort():
    rng = np.random.default_rng(26)
    T, E, k = 37, 11, 3
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    off, perm, inv = R.group(idx, E)
    pairs = sorted((int(idx[a // k, a % k]), a // k, a) for a in range(T * k))
    assert perm.tolist() == [p[2] for p in pairs]
    assert all(inv[perm[p]] == p for p in range(T * k))
    for e in range(E):
        n = sum(1 for t in range(T) for j in range(k) if idx[t, j] == e)
        assert off[e + 1] - off[e] == n
        seg = perm[off[e]:off[e + 1]]
        assert all(idx[a // k, a % k] == e for a in seg)
    assert off[0] == 0 and off[E] == T * k
