"""Block formats of the quantized routed experts: pack (reference quantizer) and unpack.

TEST INFRASTRUCTURE ONLY (oracle).

Which tensors are quantized, and to what, follows the pages: routed-expert
up/gate in a 2-bit codebook format, routed down in Q2_K, Q4_K as the wider
variant; shared expert, router and other projections unquantized ("DwarfStar"
README and the "ds4" README mirror, sections on model weights; deep-dive
article, section 3.4.3).  The pages print no bit layout; the layouts here are
this project's own (see quant_ref.c for the byte map).  Blocks hold 256
consecutive weights of one row; a row of K weights occupies ceil(K/256)
blocks (zero padded).

CB2S is the signed variant of the 2-bit codebook format, sized like the
pages' IQ2_XXS (66 bytes per 256 weights): per group of 8 weights an index
into a grid of non-negative magnitudes plus seven sign flags, the eighth sign
being fixed by even parity (the pages name IQ2_XXS but print neither its
grid nor its layout; grid, layout and quantizer here are this project's own).

Dequantization is exact in fp32: every product d*s*C, d*sc*q, dmin*m needs at
most 24 significant bits (Q6_K: 11 + 7 + 6), so the only rounding is the
single subtraction of the min term (round-to-nearest-even, as numpy float32
arithmetic does).  Q5_K and Q6_K are the wider layouts the pages list for
other models' routed experts ("ds4" README mirror, section on model weights).
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import lib

CB2, Q2K, Q4K, BF16, Q5K, Q6K, CB2S = 1, 2, 3, 4, 5, 6, 7
QK = 256
BLOCK_BYTES = {CB2: 38, Q2K: 84, Q4K: 144, Q5K: 176, Q6K: 210, CB2S: 66}


def n_blocks(K: int) -> int:
    return (K + QK - 1) // QK


def packed_bytes(fmt: int, rows: int, K: int) -> int:
    return rows * n_blocks(K) * BLOCK_BYTES[fmt]


def f32_to_f16_bits(x: float) -> int:
    """The oracle's own fp32 -> fp16 (RNE) conversion, exposed for pinning."""
    return int(lib().ref_f32_to_f16_bits(float(x)))


# -------------------------------------------------------------------- pack
def pack(fmt: int, w: np.ndarray, codebook: np.ndarray | None = None,
         threads: int | None = None) -> np.ndarray:
    """Quantize a row-major fp32 matrix [rows, K] into packed blocks (uint8).

    Rows are independent; they are split over threads (ctypes releases the
    GIL), each thread running the plain per-row C quantizer.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    out = np.zeros(packed_bytes(fmt, rows, K), dtype=np.uint8)
    if fmt in (CB2, CB2S):
        if codebook is None:
            raise ValueError("CB2 and CB2S need a codebook (CB2S: the magnitude grid)")
        cb = np.ascontiguousarray(codebook, dtype=np.int8 if fmt == CB2 else np.uint8)
        cb_ptr = cb.ctypes.data
    else:
        cb = None
        cb_ptr = None
    L = lib()
    threads = threads or min(16, os.cpu_count() or 1)
    chunk = max(1, (rows + threads - 1) // threads)

    def job(r0):
        r1 = min(rows, r0 + chunk)
        rc = L.ref_quant_rows(fmt, w.ctypes.data, r0, r1, K, cb_ptr, out.ctypes.data)
        if rc != 0:
            raise ValueError("bad format %d" % fmt)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, range(0, rows, chunk)))
    del cb
    return out


# ------------------------------------------------------------------ fields
def _f16(b: np.ndarray) -> np.ndarray:
    """Two little-endian bytes -> fp16 -> fp32 (exact widening)."""
    return np.ascontiguousarray(b).view(np.float16)[..., 0].astype(np.float32)


def fields(fmt: int, packed: np.ndarray, rows: int, K: int) -> dict:
    """Parse packed blocks into their integer/fp16 fields.

    CB2 : d [r,nb], s [r,nb,8], idx [r,nb,32]
    CB2S: d [r,nb], s [r,nb,8], idx [r,nb,32], neg [r,nb,32,8] (0/1, parity filled in)
    Q2_K: d, dmin [r,nb], sc, m [r,nb,16], q [r,nb,256]
    Q4_K, Q5_K: d, dmin [r,nb], sc, m [r,nb,8],  q [r,nb,256]
    Q6_K: d [r,nb], sc [r,nb,16] (signed), q [r,nb,256] (-32..31)
    """
    nb = n_blocks(K)
    blk = np.asarray(packed, dtype=np.uint8).reshape(rows, nb, BLOCK_BYTES[fmt])
    if fmt == Q6K:
        lo = blk[..., 18:146].astype(np.int32)
        hi = blk[..., 146:210].astype(np.int32)
        u = np.stack([(lo >> (4 * t)) & 0xF for t in range(2)], axis=-1).reshape(rows, nb, QK)
        u = u | (np.stack([(hi >> (2 * t)) & 3 for t in range(4)], axis=-1).reshape(rows, nb, QK) << 4)
        return dict(d=_f16(blk[..., 0:2]), sc=blk[..., 2:18].view(np.int8).astype(np.int32), q=u - 32)
    if fmt == CB2S:
        rec = blk[..., 2:66].reshape(rows, nb, 8, 8)                     # eight 8-byte sub-block records
        word = rec[..., 4:8].astype(np.int64)
        word = word[..., 0] | (word[..., 1] << 8) | (word[..., 2] << 16) | (word[..., 3] << 24)
        neg = np.zeros((rows, nb, 8, 4, 8), np.int32)
        for u in range(4):
            for i in range(7):
                neg[..., u, i] = (word >> (7 * u + i)) & 1
        neg[..., 7] = neg[..., :7].sum(axis=-1) & 1                      # even count of negatives
        return dict(d=_f16(blk[..., 0:2]), s=(word >> 28).astype(np.int32),
                    idx=rec[..., 0:4].reshape(rows, nb, 32).astype(np.int32), neg=neg.reshape(rows, nb, 32, 8))
    if fmt == CB2:
        sb = blk[..., 2:6].astype(np.int32)
        s = np.empty((rows, nb, 8), np.int32)
        s[..., 0::2] = sb & 0xF
        s[..., 1::2] = sb >> 4
        return dict(d=_f16(blk[..., 0:2]), s=s, idx=blk[..., 6:38].astype(np.int32))
    d = _f16(blk[..., 0:2])
    dmin = _f16(blk[..., 2:4])
    if fmt == Q2K:
        sm = blk[..., 4:20].astype(np.int32)
        qb = blk[..., 20:84].astype(np.int32)
        q = np.stack([(qb >> (2 * t)) & 3 for t in range(4)], axis=-1).reshape(rows, nb, QK)
        return dict(d=d, dmin=dmin, sc=sm & 0xF, m=sm >> 4, q=q)
    if fmt in (Q4K, Q5K):
        sb = blk[..., 4:16].astype(np.int64)
        f = np.zeros((rows, nb, 16), np.int32)
        for n in range(16):
            for t in range(6):
                bit = 6 * n + t
                f[..., n] |= (((sb[..., bit // 8] >> (bit % 8)) & 1) << t).astype(np.int32)
        qb = blk[..., 16:144].astype(np.int32)
        q = np.stack([(qb >> (4 * t)) & 0xF for t in range(2)], axis=-1).reshape(rows, nb, QK)
        if fmt == Q5K:
            hb = blk[..., 144:176].astype(np.int32)
            q = q | (np.stack([(hb >> t) & 1 for t in range(8)], axis=-1).reshape(rows, nb, QK) << 4)
        return dict(d=d, dmin=dmin, sc=f[..., :8], m=f[..., 8:], q=q)
    raise ValueError("bad format %d" % fmt)


# ------------------------------------------------------------------ unpack
def unpack(fmt: int, packed: np.ndarray, rows: int, K: int,
           codebook: np.ndarray | None = None) -> np.ndarray:
    """Dequantize packed blocks to fp32 [rows, K] (padding dropped)."""
    F = fields(fmt, packed, rows, K)
    nb = n_blocks(K)
    if fmt == CB2:
        C = np.asarray(codebook, dtype=np.int8).astype(np.float32)       # [256, 8]
        step = F["d"][..., None] * F["s"].astype(np.float32)             # [r,nb,8]
        step_g = np.repeat(step, 4, axis=-1)                             # group g -> sub-block g//4
        w = step_g[..., None] * C[F["idx"]]                              # [r,nb,32,8]
    elif fmt == CB2S:
        G = np.asarray(codebook, dtype=np.uint8).astype(np.float32)      # [256, 8] magnitudes
        step = F["d"][..., None] * F["s"].astype(np.float32)             # [r,nb,8], exact
        step_g = np.repeat(step, 4, axis=-1)
        sgn = 1.0 - 2.0 * F["neg"].astype(np.float32)                    # [r,nb,32,8]
        w = step_g[..., None] * (sgn * G[F["idx"]])                      # exact (<= 18 bits)
    elif fmt == Q6K:
        mul = F["d"][..., None] * F["sc"].astype(np.float32)             # [r,nb,16], exact
        w = np.repeat(mul, 16, axis=-1) * F["q"].astype(np.float32)      # exact (<= 24 bits)
    else:
        sub = 16 if fmt == Q2K else 32
        mul = (F["d"][..., None] * F["sc"].astype(np.float32))           # [r,nb,nsub]
        off = (F["dmin"][..., None] * F["m"].astype(np.float32))
        mul_i = np.repeat(mul, sub, axis=-1)                             # per weight
        off_i = np.repeat(off, sub, axis=-1)
        w = mul_i * F["q"].astype(np.float32) - off_i
    return np.ascontiguousarray(w.reshape(rows, nb * QK)[:, :K], dtype=np.float32)
