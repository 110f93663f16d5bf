"""Test-side packer: dense quantised matrices -> packed expert record bytes.

Written as the inverse of the record layout with array reshapes, independently
of the oracle's scalar indexing, so that a decoding mistake in either one shows
up as a mismatch against the dense source matrices.

Layout (hidden H, intermediate I): G, U are [I][H], D is [H][I].  The record
is a sequence of segments, one per 64-row x 64-input tile: the tile's codes,
then its 64 (scale fp16, bias fp16) pairs in row order.
  gate/up tiles first, [block b of 32 rows of I][input group g of H]: the
  tile's rows are the 32 G rows of the block, then the same 32 U rows.
  down tiles next, [64-row tile t of H][input group g of I].
  Codes of a tile: [runs of 16 bytes][64 rows][16 bytes]: 4-bit records have
  two runs of 32 inputs (byte m holds input 2m in the low nibble, 2m+1 in the
  high nibble), 2-bit records one run of 64 inputs (input 4m+j in bits
  [2j, 2j+2) of byte m).
"""
from __future__ import annotations

import numpy as np


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    q = q.astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def pack_crumbs(q: np.ndarray) -> np.ndarray:
    """2-bit codes: input 4m+j in bits [2j, 2j+2) of byte m."""
    q = q.astype(np.uint8)
    return (q[..., 0::4] | (q[..., 1::4] << 2) | (q[..., 2::4] << 4) | (q[..., 3::4] << 6)).astype(np.uint8)


def _segments(q: np.ndarray, s_bits: np.ndarray, b_bits: np.ndarray, bits: int) -> np.ndarray:
    """q [n][64][K] codes of n tile rows-sets (64 rows each), s/b [n][64][K/64]
    fp16 bits -> [n][K/64][segment bytes] (codes of each 64-input tile, then its
    pairs)."""
    n, _, K = q.shape
    per_run = 128 // bits                                        # inputs per 16-byte run
    pack = pack_nibbles if bits == 4 else pack_crumbs
    t = q.reshape(n, 64, K // 64, 64 // per_run, per_run)        # [n][row][group][run][input]
    t = t.transpose(0, 2, 3, 1, 4)                               # [n][group][run][row][input]
    codes = pack(t).reshape(n, K // 64, -1)                      # [n][group][runs*64*16]
    pairs = np.stack([s_bits.transpose(0, 2, 1), b_bits.transpose(0, 2, 1)], axis=-1)  # [n][group][row][2]
    pairs = np.ascontiguousarray(pairs, dtype=np.uint16).view(np.uint8).reshape(n, K // 64, 256)
    return np.concatenate([codes, pairs], axis=-1)


def pack_record(qG, qU, qD, sG, bG, sU, bU, sD, bD, bits: int = 4) -> np.ndarray:
    """q*: int arrays 0..2^bits-1 (G, U [I][H]; D [H][I]); s*, b*: fp16 bit
    arrays (G, U [I][H/64]; D [H][I/64]).  Returns the record as uint8."""
    I, H = qG.shape
    assert qU.shape == (I, H) and qD.shape == (H, I)
    assert H % 64 == 0 and I % 64 == 0 and bits in (2, 4)
    nb = I // 32
    gu_q = np.concatenate([qG.reshape(nb, 32, H), qU.reshape(nb, 32, H)], axis=1)          # [b][row][H]
    gu_s = np.concatenate([sG.reshape(nb, 32, H // 64), sU.reshape(nb, 32, H // 64)], axis=1)
    gu_b = np.concatenate([bG.reshape(nb, 32, H // 64), bU.reshape(nb, 32, H // 64)], axis=1)
    nt = H // 64
    d_q = qD.reshape(nt, 64, I)                                                              # [t][row][I]
    d_s, d_b = sD.reshape(nt, 64, I // 64), bD.reshape(nt, 64, I // 64)
    return np.concatenate([_segments(gu_q, gu_s, gu_b, bits).reshape(-1),
                           _segments(d_q, d_s, d_b, bits).reshape(-1)])


def dense(q: np.ndarray, s_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """W = s * q + b with s, b repeated over each 64-wide input group (float64)."""
    s = np.repeat(s_bits.view(np.float16).astype(np.float64), 64, axis=1)
    b = np.repeat(b_bits.view(np.float16).astype(np.float64), 64, axis=1)
    return s * q.astype(np.float64) + b


class DenseExpert:
    """Random (or given) dense quantised expert and its packed record."""

    def __init__(self, H: int, I: int, rng: np.random.Generator, qG=None, qU=None, qD=None,
                 s_range=(1e-3, 1e-2), b_range=(-8e-3, 0.0), sb=None, bits: int = 4):
        self.H, self.I, self.bits = H, I, bits
        r = rng
        nq = 1 << bits
        self.qG = r.integers(0, nq, (I, H)) if qG is None else qG
        self.qU = r.integers(0, nq, (I, H)) if qU is None else qU
        self.qD = r.integers(0, nq, (H, I)) if qD is None else qD

        def f16(shape, lo, hi):
            return r.uniform(lo, hi, shape).astype(np.float16).view(np.uint16)

        if sb is None:
            self.sG, self.sU = f16((I, H // 64), *s_range), f16((I, H // 64), *s_range)
            self.bG, self.bU = f16((I, H // 64), *b_range), f16((I, H // 64), *b_range)
            self.sD, self.bD = f16((H, I // 64), *s_range), f16((H, I // 64), *b_range)
        else:
            (self.sG, self.bG, self.sU, self.bU, self.sD, self.bD) = sb
        self.rec = pack_record(self.qG, self.qU, self.qD, self.sG, self.bG, self.sU, self.bU,
                               self.sD, self.bD, bits)
        self.G = dense(self.qG, self.sG, self.bG)
        self.U = dense(self.qU, self.sU, self.bU)
        self.D = dense(self.qD, self.sD, self.bD)

    def ffn(self, x: np.ndarray) -> np.ndarray:
        from scipy.special import expit
        g = self.G @ x
        u = self.U @ x
        return self.D @ (g * expit(g) * u)
