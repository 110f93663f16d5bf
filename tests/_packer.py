"""Test-side packer: dense quantised matrices -> packed expert record bytes.

Written as the inverse of the record layout with array reshapes, independently
of the oracle's scalar indexing, so that a decoding mistake in either one shows
up as a mismatch against the dense source matrices.

Layout (hidden H, intermediate I): G, U are [I][H], D is [H][I].
  nibble region: for each block b of 32 rows i: the GU tile [H/32 chunks][64
  tile rows (32 G rows, then the same 32 U rows)][16 bytes], then the D block
  [H output rows][16 bytes of D[o][32b:32b+32]].  Byte m of a 16-byte run holds
  input 2m in the low nibble and 2m+1 in the high nibble.
  The 2-bit variant packs 64 inputs per 16-byte run (input 4m+j in bits
  [2j, 2j+2) of byte m): GU tiles [H/64 chunks][64 rows][16 bytes], D blocks
  [H rows][8 bytes].
  scale/bias region: for each slab g of 64 rows i: GU tile 2g pairs
  [H/64 groups][64 tile rows], GU tile 2g+1 pairs, then D pairs [H] for input
  group g.  Each pair is (scale fp16, bias fp16).
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


def pack_record(qG, qU, qD, sG, bG, sU, bU, sD, bD, bits: int = 4) -> np.ndarray:
    """q*: int arrays 0..2^bits-1 (G, U [I][H]; D [H][I]); s*, b*: fp16 bit
    arrays (G, U [I][H/64]; D [H][I/64]).  bits 4: 32 inputs per 16-byte run;
    bits 2: 64.  Returns the record as uint8."""
    I, H = qG.shape
    assert qU.shape == (I, H) and qD.shape == (H, I)
    assert H % 64 == 0 and I % 64 == 0 and bits in (2, 4)
    per_run = 128 // bits           # inputs per 16-byte run
    pack = pack_nibbles if bits == 4 else pack_crumbs
    parts = []
    for b in range(I // 32):
        rows = np.concatenate([qG[32 * b:32 * b + 32], qU[32 * b:32 * b + 32]], axis=0)
        tile = rows.reshape(64, H // per_run, per_run).transpose(1, 0, 2)   # [chunk][row][run]
        parts.append(pack(tile).reshape(-1))
        parts.append(pack(qD[:, 32 * b:32 * b + 32]).reshape(-1))           # [o][32 inputs]
    for g in range(I // 64):
        for t in (2 * g, 2 * g + 1):
            s_rows = np.concatenate([sG[32 * t:32 * t + 32], sU[32 * t:32 * t + 32]], axis=0)
            b_rows = np.concatenate([bG[32 * t:32 * t + 32], bU[32 * t:32 * t + 32]], axis=0)
            pairs = np.stack([s_rows.T, b_rows.T], axis=-1)               # [group][row][2]
            parts.append(np.ascontiguousarray(pairs, dtype=np.uint16).reshape(-1).view(np.uint8))
        pairs = np.stack([sD[:, g], bD[:, g]], axis=-1)                    # [o][2]
        parts.append(np.ascontiguousarray(pairs, dtype=np.uint16).reshape(-1).view(np.uint8))
    return np.concatenate(parts)


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
