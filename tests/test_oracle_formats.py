"""Pins for the oracle's block formats and reference quantizers (CPU only).

Each check is fixed independently of the oracle's own code: a library
routine (numpy's fp16 conversion), hand-written blocks, the quantizer
inverting the dequantizer on its own image, nearest-level / nearest-codeword
optimality by brute force on small inputs, and the zero-padding closed form.
"""
import json
import os

import numpy as np
import pytest

from oracle import formats as F
import synthetic as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")))
CB = S.codebook()
GRID = S.grid_cb2s()


def _cb(fmt):
    return GRID if fmt == F.CB2S else CB


# ------------------------------------------------------------------ fp16 RNE
def test_f16_conversion_matches_numpy():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(20000).astype(np.float32) * np.float32(0.01))
    vals += list((rng.standard_normal(5000) * 1e4).astype(np.float32))
    # ties at several binades, subnormal boundary, overflow boundary
    for e in range(-24, 16):
        for m in range(0, 1024, 37):
            base = np.float32(np.ldexp(1024 + m, e - 10))
            vals += [base, np.nextafter(base, np.float32(np.inf))]
    vals += [np.float32(x) for x in (0.0, -0.0, 6.1035156e-05, 5.9604645e-08, 2.9802322e-08,
                                     65504.0, 65519.99, 65520.0, 1e-9, -1e-9, 3.0517578e-05)]
    for v in vals:
        with np.errstate(over="ignore"):
            want = int(np.array(v, np.float32).astype(np.float16).view(np.uint16))
        assert F.f32_to_f16_bits(float(v)) == want, v


# --------------------------------------------------------------- hand blocks
def _block(fmt, set_bytes):
    b = np.zeros(F.BLOCK_BYTES[fmt], np.uint8)
    for k, v in set_bytes.items():
        b[int(k)] = v
    return b


def test_q2k_hand_block():
    g = GOLD["q2k"]
    w = F.unpack(F.Q2K, _block(F.Q2K, g["set_bytes"]), 1, 256)[0]
    assert w[:16].tolist() == g["expect_first16"]
    assert np.all(w[16:] == 0)


def test_cb2_hand_block():
    g = GOLD["cb2"]
    w = F.unpack(F.CB2, _block(F.CB2, g["set_bytes"]), 1, 256, CB)[0]
    assert np.array_equal(w[:8], CB[g["codeword"]].astype(np.float32))
    assert np.array_equal(w[8:32], np.tile(CB[0], 3).astype(np.float32))
    assert np.all(w[32:] == 0)


def test_cb2s_hand_block():
    g = GOLD["cb2s"]
    w = F.unpack(F.CB2S, _block(F.CB2S, g["set_bytes"]), 1, 256, GRID)[0]
    G = GRID.astype(np.float32)
    assert np.array_equal(w[0:8], np.array(g["signs_group0"], np.float32) * G[g["idx_group0"]])
    assert np.array_equal(w[8:16], np.array(g["signs_group1"], np.float32) * G[0])
    assert np.array_equal(w[16:32], np.tile(G[0], 2))
    assert np.all(w[32:] == 0)


def test_q4k_hand_scales_and_block():
    g = GOLD["q4k"]
    blk = _block(F.Q4K, g["set_bytes"])
    blk[4:16] = np.frombuffer(bytes.fromhex(g["scale_bytes_hex"]), np.uint8)
    fl = F.fields(F.Q4K, blk, 1, 256)
    assert fl["sc"][0, 0].tolist() == g["sc"]
    assert fl["m"][0, 0].tolist() == g["m"]
    w = F.unpack(F.Q4K, blk, 1, 256)[0]
    assert w[:3].tolist() == g["expect_first3"]
    assert np.all(w[2:32] == 0)
    for j in range(1, 8):
        assert np.all(w[32 * j:32 * (j + 1)] == g["expect_subblock_value"][j])


def test_q5k_hand_block():
    g = GOLD["q5k"]
    blk = _block(F.Q5K, g["set_bytes"])
    blk[4:16] = np.frombuffer(bytes.fromhex(g["scale_bytes_hex"]), np.uint8)
    w = F.unpack(F.Q5K, blk, 1, 256)[0]
    assert w[:10].tolist() == g["expect_first10"]
    assert np.all(w[10:32] == 0)
    for j in range(1, 8):
        assert np.all(w[32 * j:32 * (j + 1)] == g["expect_subblock_value"][j])


def test_q6k_hand_block():
    g = GOLD["q6k"]
    w = F.unpack(F.Q6K, _block(F.Q6K, g["set_bytes"]), 1, 256)[0]
    assert w[:3].tolist() == g["expect_first3"]
    assert np.all(w[2:16] == -32)
    assert np.all(w[16:32] == g["expect_subblock_value"][1])
    assert np.all(w[32:] == g["expect_subblock_value"][2])


def test_q4k_pack_scale_stream_agrees_with_parser():
    # the writer (C) and the parser (numpy) are separate code; read the 12
    # scale bytes of freshly packed blocks as one little-endian 96-bit stream
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((4, 512)) * 0.02).astype(np.float32)
    p = F.pack(F.Q4K, w).reshape(4, 2, 144)
    fl = F.fields(F.Q4K, p, 4, 512)
    for r in range(4):
        for b in range(2):
            stream = int.from_bytes(bytes(p[r, b, 4:16]), "little")
            got = [(stream >> (6 * n)) & 63 for n in range(16)]
            assert got[:8] == fl["sc"][r, b].tolist() and got[8:] == fl["m"][r, b].tolist()


# ------------------------------------------------- reconstruction (exact)
def _random_affine_codes(rng, nsub, n, L, S_, rows, nb):
    """Codes on the quantizer's image: each sub-block has sc>=1, a q=0 and a
    q=L, and each block has max sc = max m = S_."""
    sc = rng.integers(1, S_ + 1, size=(rows, nb, nsub))
    m = rng.integers(0, S_ + 1, size=(rows, nb, nsub))
    sc[..., 0] = S_
    m[..., 1] = S_
    q = rng.integers(0, L + 1, size=(rows, nb, nsub, n))
    q[..., 0] = 0
    q[..., 1] = L
    d = np.float16(2.0 ** rng.uniform(-12, -6, size=(rows, nb))).astype(np.float32)
    dmin = np.float16(2.0 ** rng.uniform(-12, -6, size=(rows, nb))).astype(np.float32)
    w = ((d[..., None] * sc)[..., None] * q - (dmin[..., None] * m)[..., None]).astype(np.float32)
    return w.reshape(rows, nb * nsub * n), d, dmin, sc, m, q


@pytest.mark.parametrize("fmt,nsub,n,L,S_", [(F.Q2K, 16, 16, 3, 15), (F.Q4K, 8, 32, 15, 63),
                                            (F.Q5K, 8, 32, 31, 63)])
def test_affine_quantizer_inverts_dequant(fmt, nsub, n, L, S_):
    rng = np.random.default_rng(7)
    rows, nb = 24, 3
    w, d, dmin, sc, m, q = _random_affine_codes(rng, nsub, n, L, S_, rows, nb)
    p = F.pack(fmt, w)
    fl = F.fields(fmt, p, rows, nb * 256)
    assert np.array_equal(fl["d"], d) and np.array_equal(fl["dmin"], dmin)
    assert np.array_equal(fl["sc"], sc) and np.array_equal(fl["m"], m)
    assert np.array_equal(fl["q"], q.reshape(rows, nb, 256))
    assert np.array_equal(F.unpack(fmt, p, rows, nb * 256), w)


def test_q6k_quantizer_inverts_dequant():
    """Codes on the symmetric quantizer's image: every sub-block holds a code of
    magnitude 31 (so its max |w| is 31 d sc_j) and every block a scale of 127."""
    rng = np.random.default_rng(9)
    rows, nb = 20, 3
    sc = rng.integers(1, 128, size=(rows, nb, 16))
    sc[..., 3] = 127
    q = rng.integers(-31, 32, size=(rows, nb, 16, 16))
    q[..., 5] = rng.choice([-31, 31], size=(rows, nb, 16))
    d = np.float16(2.0 ** rng.uniform(-14, -8, size=(rows, nb))).astype(np.float32)
    w = ((d[..., None] * sc)[..., None] * q).astype(np.float32).reshape(rows, nb * 256)
    p = F.pack(F.Q6K, w)
    fl = F.fields(F.Q6K, p, rows, nb * 256)
    assert np.array_equal(fl["d"], d)
    assert np.array_equal(fl["sc"], sc)
    assert np.array_equal(fl["q"], q.reshape(rows, nb, 256))
    assert np.array_equal(F.unpack(F.Q6K, p, rows, nb * 256), w)


def test_cb2_quantizer_inverts_dequant():
    rng = np.random.default_rng(8)
    rows, nb = 16, 3
    # codewords that contain a +-3 so that max|w| = 3*d*s in every sub-block
    has3 = np.nonzero(np.abs(CB).max(axis=1) == 3)[0]
    idx = rng.choice(has3, size=(rows, nb, 32))
    s = rng.integers(1, 16, size=(rows, nb, 8))
    s[..., 0] = 15
    d = np.float16(2.0 ** rng.uniform(-12, -6, size=(rows, nb))).astype(np.float32)
    step = np.repeat(d[..., None] * s, 4, axis=-1)
    w = (step[..., None] * CB[idx].astype(np.float32)).reshape(rows, nb * 256).astype(np.float32)
    p = F.pack(F.CB2, w, CB)
    fl = F.fields(F.CB2, p, rows, nb * 256)
    assert np.array_equal(fl["d"], d)
    assert np.array_equal(fl["s"], s)
    assert np.array_equal(fl["idx"], idx)


def _even_sign_patterns():
    """All 128 sign vectors of 8 entries with an even number of -1 (brute force)."""
    pats = np.array([[1 - 2 * ((m >> i) & 1) for i in range(8)] for m in range(256)], np.float64)
    return pats[(pats < 0).sum(axis=1) % 2 == 0]


def test_cb2s_quantizer_inverts_dequant():
    """Weights on the format's own image (magnitudes from the grid, an even
    number of negatives per group, a 5 in every sub-block so that max|w| =
    5*d*s) come back as exactly the codes that made them."""
    rng = np.random.default_rng(18)
    rows, nb = 16, 3
    has5 = np.nonzero(GRID.max(axis=1) == 5)[0]
    idx = rng.choice(has5, size=(rows, nb, 32))
    pats = _even_sign_patterns()
    sg = pats[rng.integers(0, len(pats), size=(rows, nb, 32))]          # [r, nb, 32, 8]
    s = rng.integers(1, 16, size=(rows, nb, 8))
    s[..., 0] = 15
    d = np.float16(2.0 ** rng.uniform(-12, -6, size=(rows, nb))).astype(np.float32)
    step = np.repeat(d[..., None] * s, 4, axis=-1)
    w = (step[..., None] * (sg * GRID[idx])).reshape(rows, nb * 256).astype(np.float32)
    p = F.pack(F.CB2S, w, GRID)
    fl = F.fields(F.CB2S, p, rows, nb * 256)
    assert np.array_equal(fl["d"], d)
    assert np.array_equal(fl["s"], s)
    assert np.array_equal(fl["idx"], idx)
    assert np.array_equal(fl["neg"], (sg < 0).astype(np.int32))
    assert np.array_equal(F.unpack(F.CB2S, p, rows, nb * 256, GRID), w)


# ---------------------------------------------------- optimality (brute force)
@pytest.mark.parametrize("fmt,n,L", [(F.Q2K, 16, 3), (F.Q4K, 32, 15), (F.Q5K, 32, 31)])
def test_affine_codes_are_nearest_levels(fmt, n, L):
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((8, 512)) * 0.02).astype(np.float32)
    p = F.pack(fmt, w)
    fl = F.fields(fmt, p, 8, 512)
    step = (fl["d"][..., None] * fl["sc"]).astype(np.float64)          # [r, nb, nsub]
    off = (fl["dmin"][..., None] * fl["m"]).astype(np.float64)
    levels = step[..., None] * np.arange(L + 1) - off[..., None]        # [r, nb, nsub, L+1]
    wv = w.astype(np.float64).reshape(8, 2, -1, n)                       # [r, nb, nsub, n]
    err = np.abs(wv[..., None] - levels[..., None, :])                   # [..., n, L+1]
    chosen = np.take_along_axis(err, fl["q"].reshape(8, 2, -1, n)[..., None], axis=-1)[..., 0]
    best = err.min(axis=-1)
    slack = 1e-6 * np.maximum(step, 1e-30)[..., None]
    live = (step > 0)[..., None] & np.ones_like(chosen, bool)
    assert np.all(chosen[live] <= best[live] + np.broadcast_to(slack, chosen.shape)[live])
    # the quantization error stays within half a step plus the range slack
    # left by rounding sc and m to integers
    recon = F.unpack(fmt, p, 8, 512).astype(np.float64).reshape(wv.shape)
    bound = 0.5 * step[..., None] + 0.5 * fl["dmin"].astype(np.float64)[..., None, None] \
        + 0.5 * L * fl["d"].astype(np.float64)[..., None, None]
    assert np.all(np.abs(recon - wv) <= bound + 1e-12)


def test_q6k_codes_are_nearest_levels():
    rng = np.random.default_rng(16)
    w = (rng.standard_normal((8, 512)) * 0.02).astype(np.float32)
    p = F.pack(F.Q6K, w)
    fl = F.fields(F.Q6K, p, 8, 512)
    step = (fl["d"][..., None] * fl["sc"]).astype(np.float64)          # [r, nb, 16]
    levels = step[..., None] * np.arange(-32, 32)                       # [r, nb, 16, 64]
    wv = w.astype(np.float64).reshape(8, 2, 16, 16)
    err = np.abs(wv[..., None] - levels[..., None, :])                   # [r, nb, 16, 16, 64]
    chosen = np.take_along_axis(err, (fl["q"].reshape(8, 2, 16, 16) + 32)[..., None], axis=-1)[..., 0]
    assert np.all(chosen <= err.min(axis=-1) + 1e-6 * step[..., None])
    # |w| <= 31.5 steps of the rounded scale: the error is at most half a step
    # plus the part of the range lost to rounding sc_j
    recon = F.unpack(F.Q6K, p, 8, 512).astype(np.float64).reshape(wv.shape)
    bound = 0.5 * step[..., None] + 31.5 * 0.5 * fl["d"].astype(np.float64)[..., None, None]
    assert np.all(np.abs(recon - wv) <= bound + 1e-12)


def test_cb2_codes_are_nearest_codewords():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    p = F.pack(F.CB2, w, CB)
    fl = F.fields(F.CB2, p, 4, 256)
    step = fl["d"][..., None].astype(np.float64) * fl["s"]                # [4,1,8]
    Cf = CB.astype(np.float64)
    for r in range(4):
        for g in range(32):
            st = step[r, 0, g // 4]
            if st == 0:
                assert fl["idx"][r, 0, g] == 0
                continue
            target = w[r, 8 * g:8 * g + 8].astype(np.float64) / st
            dist = ((target[None, :] - Cf) ** 2).sum(axis=1)
            chosen = dist[fl["idx"][r, 0, g]]
            # fixed-point targets (1/4096) may flip only near-ties
            assert chosen <= dist.min() + 8 * (2.0 / 4096) * 4 + 1e-9


def test_cb2s_codes_are_optimal_over_every_signed_codeword():
    """For the block's step, the chosen (grid entry, signs) minimises the
    squared error over all 256 x 128 codewords with an even number of negative
    signs, by brute force."""
    rng = np.random.default_rng(19)
    w = (rng.standard_normal((3, 256)) * 0.02).astype(np.float32)
    w[0, :8] = [0.01, -0.02, 0.0, 0.03, -0.001, 0.002, -0.04, 0.005]     # odd number of negatives
    p = F.pack(F.CB2S, w, GRID)
    fl = F.fields(F.CB2S, p, 3, 256)
    step = fl["d"][..., None].astype(np.float64) * fl["s"]              # [3, 1, 8]
    cand = (_even_sign_patterns()[None, :, :] * GRID.astype(np.float64)[:, None, :]).reshape(-1, 8)
    for r in range(3):
        for g in range(32):
            st = step[r, 0, g // 4]
            if st == 0:
                assert fl["idx"][r, 0, g] == 0 and not fl["neg"][r, 0, g].any()
                continue
            t = w[r, 8 * g:8 * g + 8].astype(np.float64) / st
            err = ((t[None, :] - cand) ** 2).sum(axis=1)
            code = (1 - 2 * fl["neg"][r, 0, g]) * GRID[fl["idx"][r, 0, g]].astype(np.float64)
            chosen = ((t - code) ** 2).sum()
            # targets are fixed point (1/4096): each term may move by at most
            # 2 (|t| + 5) (0.6 / 4096), so only near-ties can flip
            slack = 2.0 * (np.abs(t) + 5.0).sum() * 0.6 / 4096
            assert chosen <= err.min() + slack


def test_cb2s_error_beats_cb2():
    """The sign field is what the signed format adds: on bell-shaped weights it
    fits much closer than the sign-less codebook of the same grid size."""
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    rel = {}
    for fmt in (F.CB2, F.CB2S):
        r = F.unpack(fmt, F.pack(fmt, w, _cb(fmt)), 64, 1024, _cb(fmt))
        rel[fmt] = np.linalg.norm(r - w) / np.linalg.norm(w)
    assert rel[F.CB2S] < 0.75 * rel[F.CB2]
    assert rel[F.CB2S] < 0.6


def test_cb2_error_is_bounded():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    p = F.pack(F.CB2, w, CB)
    r = F.unpack(F.CB2, p, 64, 1024, CB)
    rel = np.linalg.norm(r - w) / np.linalg.norm(w)
    # a seeded 256-entry codebook with no separate sign bits covers few of the
    # 2^8 sign patterns of a group, so the fit is coarse; it must still beat
    # the zero vector (relative error 1) and the best single scale of the
    # dequantized block must be positive (the fit points the right way)
    assert rel < 0.97
    assert float((r * w).sum()) > 0


# -------------------------------------------------------------- zero padding
@pytest.mark.parametrize("fmt", [F.CB2, F.Q2K, F.Q4K, F.Q5K, F.Q6K, F.CB2S])
def test_padding_is_zero_extension(fmt):
    rng = np.random.default_rng(14)
    K = 128 + 64
    w = (rng.standard_normal((5, K)) * 0.02).astype(np.float32)
    wp = np.zeros((5, 256), np.float32)
    wp[:, :K] = w
    a = F.pack(fmt, w, _cb(fmt))
    b = F.pack(fmt, wp, _cb(fmt))
    assert np.array_equal(a, b)
    full = F.unpack(fmt, b, 5, 256, _cb(fmt))
    assert np.array_equal(F.unpack(fmt, a, 5, K, _cb(fmt)), full[:, :K])


def test_fully_padded_subblocks_dequantize_to_zero():
    rng = np.random.default_rng(15)
    w = (rng.standard_normal((3, 128)) * 0.02).astype(np.float32)
    for fmt, sub in ((F.Q2K, 16), (F.Q4K, 32), (F.CB2, 32), (F.Q5K, 32), (F.Q6K, 16), (F.CB2S, 32)):
        p = F.pack(fmt, w, _cb(fmt))
        full = F.unpack(fmt, p, 3, 256, _cb(fmt))
        assert np.all(full[:, 128:] == 0)


def test_packed_sizes():
    assert F.packed_bytes(F.CB2, 2048, 7168) == 2048 * 28 * 38
    assert F.packed_bytes(F.Q2K, 7168, 2048) == 7168 * 8 * 84
    assert F.packed_bytes(F.Q4K, 7168, 2048) == 7168 * 8 * 144
    assert F.packed_bytes(F.Q5K, 7168, 2048) == 7168 * 8 * 176
    assert F.packed_bytes(F.Q6K, 7168, 2048) == 7168 * 8 * 210
    assert F.packed_bytes(F.CB2S, 2048, 7168) == 2048 * 28 * 66
    assert 66 * 8 / 256 == 2.0625                                        # bits per weight


def test_codebook_is_distinct_and_on_levels():
    assert CB.shape == (256, 8)
    assert set(np.unique(CB).tolist()) <= {-3, -1, 1, 3}
    assert len({r.tobytes() for r in CB}) == 256


def test_cb2s_grid_is_distinct_and_on_levels():
    assert GRID.shape == (256, 8) and GRID.dtype == np.uint8
    assert set(np.unique(GRID).tolist()) <= {1, 3, 5}
    assert len({r.tobytes() for r in GRID}) == 256
