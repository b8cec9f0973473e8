"""The stored fixtures under tests/golden/ (written by tests/golden/make_golden.py
from the oracle) checked on the CPU:

* the seeded generator still produces the inputs the fixtures were taken on
  (SHA-256 of the input bytes);
* the values are pinned by a decoder independent of the oracle: the GGUF Q4_K
  bytes are decoded here field by field with numpy (binary16 through numpy's
  float16, the 6-bit fields from their bit positions, the nibble order of the
  format) and multiplied with numpy in f64;
* the oracle still reproduces them (a regression check of the oracle's
  arithmetic, not a pin).
"""
import hashlib
import importlib.util
import math
import os

import numpy as np
import pytest

from quantized_decode_q4_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load_maker():
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLDEN, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


mg = _load_maker()


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def decode_rows(W: np.ndarray, rows, cols: int) -> np.ndarray:
    """Dense f64 weights of the given rows, decoded without the oracle."""
    nb = cols // 256
    blk = W.reshape(-1, nb, 144)[np.asarray(rows)]                 # [r, nb, 144]
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = blk[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    # the 96 bits of bytes 4..15 as one little-endian bit string
    bits = np.unpackbits(blk[..., 4:16], axis=-1, bitorder="little").astype(np.int64)   # [r, nb, 96]

    def field(pos):
        """value of the bits at the listed positions (least significant first)"""
        return sum(bits[..., p] << i for i, p in enumerate(pos))

    sc = np.zeros(blk.shape[:2] + (8,), np.int64)
    mn = np.zeros_like(sc)
    for j in range(4):
        sc[..., j] = field([8 * j + i for i in range(6)])               # byte j, bits 0..5
        mn[..., j] = field([8 * (j + 4) + i for i in range(6)])         # byte j+4, bits 0..5
        # sub-block j+4: low 4 bits from byte j+8 (scale: low nibble, min: high
        # nibble), top 2 bits from bits 6..7 of byte j (scale) / byte j+4 (min)
        sc[..., j + 4] = field([8 * (j + 8) + i for i in range(4)] + [8 * j + 6, 8 * j + 7])
        mn[..., j + 4] = field([8 * (j + 8) + 4 + i for i in range(4)] + [8 * (j + 4) + 6, 8 * (j + 4) + 7])
    qs = blk[..., 16:144].astype(np.int64)                               # [r, nb, 128]
    q = np.zeros(blk.shape[:2] + (256,), np.int64)
    for e in range(256):
        g, r = divmod(e, 64)
        q[..., e] = (qs[..., 32 * g + r] & 15) if r < 32 else (qs[..., 32 * g + r - 32] >> 4)
    s = np.arange(256) // 32
    w = d[..., None] * sc[..., s] * q - dmin[..., None] * mn[..., s]   # [r, nb, 256]
    return w.reshape(len(rows), cols)


def test_tiny_fixture_inputs_and_values():
    fx = mg.read(mg.TINY)
    c = inputs.tiny_matvec()
    assert digest(c["W"], c["x"]) == fx["sha256"]
    rows = np.array([int(r[0]) for r in fx["rows"]])
    y = np.array([float(r[1]) for r in fx["rows"]])
    A = np.array([float(r[2]) for r in fx["rows"]])
    assert rows.tolist() == list(range(256))
    w = decode_rows(c["W"], rows, 512)
    x = c["x"].astype(np.float64)
    np.testing.assert_allclose(w @ x, y, rtol=0, atol=1e-12 * float(A.max()))
    np.testing.assert_allclose(np.abs(w) @ np.abs(x), A, rtol=1e-12)


def test_lmhead_fixture_inputs_and_values():
    fx = mg.read(mg.LMHEAD)
    c = inputs.lm_head(0)
    assert digest(c["W"], c["x"]) == fx["sha256"]
    rows = [int(r[1]) for r in fx["rows"]]
    logit = np.array([float(r[2]) for r in fx["rows"]])
    A = np.array([float(r[3]) for r in fx["rows"]])
    prob = np.array([float(r[4]) for r in fx["rows"]])
    w = decode_rows(c["W"], rows, inputs.HIDDEN)
    x = c["x"].astype(np.float64)
    np.testing.assert_allclose(w @ x, logit, rtol=0, atol=1e-12 * float(A.max()))
    np.testing.assert_allclose(np.abs(w) @ np.abs(x), A, rtol=1e-12)
    # ranks: value descending (ties: index ascending)
    assert all((logit[i], -rows[i]) > (logit[i + 1], -rows[i + 1]) for i in range(4))
    # probabilities are exp(logit - lse)
    lse = fx["logsumexp"]
    np.testing.assert_allclose(prob, np.exp(logit - lse), rtol=1e-12)
    # lse lies between the top logit and top logit + log(rows)
    assert logit[0] < lse < logit[0] + math.log(inputs.VOCAB)


def test_oracle_reproduces_fixtures(orc):
    fx = mg.read(mg.TINY)
    c = inputs.tiny_matvec()
    y, A = orc.matvec(c["W"], c["x"], 256, 512)
    assert [float(r[1]) for r in fx["rows"]] == y.tolist()
    assert [float(r[2]) for r in fx["rows"]] == A.tolist()
    fx = mg.read(mg.LMHEAD)
    c = inputs.lm_head(0)
    y, A = orc.matvec(c["W"], c["x"], inputs.VOCAB, inputs.HIDDEN)
    idx, val = orc.topk(y, 5)
    assert [int(r[1]) for r in fx["rows"]] == idx.tolist()
    assert [float(r[2]) for r in fx["rows"]] == val.tolist()
    assert fx["logsumexp"] == orc.logsumexp(y)
