"""Build Q4_K blocks from their fields (test-side input construction).

This is the encoder direction of the GGUF Q4_K super-block layout: given d, dmin,
eight 6-bit scales, eight 6-bit mins and 256 four-bit quants, produce the 144
bytes. Tests use it to craft inputs whose expected results are known from the
fields alone, so the oracle's decoder is checked against something other than
itself. It contains no dot products or activations.
"""
from __future__ import annotations

import numpy as np


def f16_bits(v: float) -> int:
    return int(np.array(v, dtype=np.float16).view(np.uint16))


def pack_scales(sc, mn) -> np.ndarray:
    """Twelve bytes: bytes 0-3 = low 6 bits of scales 0-3 plus the top 2 bits of
    scales 4-7; bytes 4-7 = low 6 bits of mins 0-3 plus the top 2 bits of mins
    4-7; bytes 8-11 = low nibble from scale 4+j, high nibble from min 4+j."""
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    assert len(sc) == 8 and len(mn) == 8
    assert all(0 <= v < 64 for v in sc + mn)
    s = np.zeros(12, np.uint8)
    for j in range(4):
        s[j] = (sc[j] & 0x3F) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (mn[j] & 0x3F) | ((mn[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 0x0F) | ((mn[j + 4] & 0x0F) << 4)
    return s


def pack_quants(q) -> np.ndarray:
    """128 bytes: byte 32g + r carries element 64g + r (low nibble) and element
    64g + 32 + r (high nibble), g = 0..3, r = 0..31."""
    q = np.asarray(q, dtype=np.int64).reshape(256)
    assert q.min() >= 0 and q.max() < 16
    out = np.zeros(128, np.uint8)
    for g in range(4):
        for r in range(32):
            out[32 * g + r] = q[64 * g + r] | (q[64 * g + 32 + r] << 4)
    return out


def pack_block(d, dmin, sc, mn, q) -> np.ndarray:
    """144 bytes of one block. d, dmin are floats (rounded to binary16) or, when
    given as numpy uint16, raw binary16 bit patterns."""
    blk = np.zeros(144, np.uint8)
    db = int(d) if isinstance(d, np.uint16) else f16_bits(d)
    mb = int(dmin) if isinstance(dmin, np.uint16) else f16_bits(dmin)
    blk[0], blk[1] = db & 0xFF, db >> 8
    blk[2], blk[3] = mb & 0xFF, mb >> 8
    blk[4:16] = pack_scales(sc, mn)
    blk[16:144] = pack_quants(q)
    return blk


class Fields:
    """Random field values for a rows x cols matrix, kept alongside its bytes."""

    def __init__(self, rng: np.random.Generator, rows: int, cols: int,
                 d=None, dmin=None, sc=None, mn=None, q=None):
        nb = cols // 256
        self.rows, self.cols, self.nb = rows, cols, nb
        self.d = (rng.uniform(1e-4, 2e-3, (rows, nb)) if d is None else
                  np.broadcast_to(d, (rows, nb))).astype(np.float16)
        self.dmin = (rng.uniform(1e-4, 2e-3, (rows, nb)) if dmin is None else
                     np.broadcast_to(dmin, (rows, nb))).astype(np.float16)
        self.sc = (rng.integers(0, 64, (rows, nb, 8)) if sc is None else
                   np.broadcast_to(sc, (rows, nb, 8))).astype(np.int64)
        self.mn = (rng.integers(0, 64, (rows, nb, 8)) if mn is None else
                   np.broadcast_to(mn, (rows, nb, 8))).astype(np.int64)
        self.q = (rng.integers(0, 16, (rows, nb, 256)) if q is None else
                  np.broadcast_to(q, (rows, nb, 256))).astype(np.int64)

    def to_bytes(self) -> np.ndarray:
        out = np.zeros((self.rows, self.nb, 144), np.uint8)
        for i in range(self.rows):
            for b in range(self.nb):
                out[i, b] = pack_block(self.d[i, b].view(np.uint16), self.dmin[i, b].view(np.uint16),
                                       self.sc[i, b], self.mn[i, b], self.q[i, b])
        return out.reshape(self.rows, self.nb * 144)

    def dense(self) -> np.ndarray:
        """w = d * sc[s] * q - dmin * m[s] per element (s = element // 32), f64."""
        d = self.d.astype(np.float64)[:, :, None]
        dmin = self.dmin.astype(np.float64)[:, :, None]
        s = np.arange(256) // 32
        w = d * self.sc[:, :, s] * self.q - dmin * self.mn[:, :, s]
        return w.reshape(self.rows, self.cols)


# ------------------------------------------------------------------ Q6_K ---

def pack_q6k_block(d, scales, q) -> np.ndarray:
    """210 bytes of one GGUF Q6_K block from its fields: 256 six-bit quants q
    (0..63), 16 signed 8-bit scales (one per 16 consecutive weights) and d.
    Quant e = 128n + 32j + l puts its low 4 bits in nibble j//2 of byte
    64n + 32(j%2) + l and its high 2 bits in bits 2j..2j+1 of byte
    128 + 32n + l; the scales fill bytes 192..207 and d bytes 208..209.
    d is a float (rounded to binary16) or a numpy uint16 bit pattern."""
    q = np.asarray(q, dtype=np.int64).reshape(256)
    scales = np.asarray(scales, dtype=np.int64).reshape(16)
    assert q.min() >= 0 and q.max() < 64
    assert scales.min() >= -128 and scales.max() < 128
    blk = np.zeros(210, np.uint8)
    for e in range(256):
        n, j, l = e // 128, (e % 128) // 32, e % 32
        lo_byte = 64 * n + 32 * (j % 2) + l
        blk[lo_byte] |= (q[e] & 0x0F) << (4 * (j // 2))
        blk[128 + 32 * n + l] |= (q[e] >> 4) << (2 * j)
    blk[192:208] = (scales & 0xFF).astype(np.uint8)
    db = int(d) if isinstance(d, np.uint16) else f16_bits(d)
    blk[208], blk[209] = db & 0xFF, db >> 8
    return blk
