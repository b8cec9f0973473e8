"""Write the stored expected values under tests/golden/ from the CPU oracle.

Every number in the fixtures comes from ``oracle/`` (the plain f64 C
implementation) applied to the seeded synthetic inputs of
``quantized_decode_q4_amd.inputs``; nothing here runs the HIP library. The
fixtures also record a SHA-256 digest of those input bytes, so a test can
check that the generator still produces the inputs the values were taken on.

What the values are (the pages print no Q4_K numbers, so none are quoted):
  * tiny_matvec.txt  -- the 256 x 512 matvec of the tiny workload (GGUF Q4_K
    rows, the format "Design Principles" item 8 of the infer-compute README
    names; the q4k_matvec call of its "Quick Start"): y_i and A_i = sum_j
    |w_ij x_j| for every row.
  * lmhead_top5.txt  -- the 262144 x 2560 lm_head of the vocabulary workload:
    the top-5 rows by (logit desc, index asc) with their logits, A and softmax
    probabilities over all rows, and the log-sum-exp (the top-5 predictions of
    the infer-inference README Overview example, computed on the GPU per the
    "Honest Path Breakdown" of its performance page).

Usage:  python tests/golden/make_golden.py      (about 10 s; needs gcc for the oracle)
"""
from __future__ import annotations

import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from quantized_decode_q4_amd import inputs  # noqa: E402

TINY = os.path.join(HERE, "tiny_matvec.txt")
LMHEAD = os.path.join(HERE, "lmhead_top5.txt")


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def write_tiny(path: str = TINY) -> None:
    c = inputs.tiny_matvec()
    y, A = oracle.matvec(c["W"], c["x"], 256, 512)
    with open(path, "w") as f:
        f.write("# tiny Q4_K matvec, W 256 x 512 (GGUF Q4_K rows), x f32[512] ~ N(0,1)\n")
        f.write("# inputs: quantized_decode_q4_amd.inputs.tiny_matvec() "
                "(PCG64 seeds [0x51344B, 0, 0, 0] for W, [0x51344B, 0, 3, 0] for x)\n")
        f.write(f"# sha256(W bytes, x bytes) = {digest(c['W'], c['x'])}\n")
        f.write("# values: oracle.matvec (f64): row y A\n")
        for i in range(256):
            f.write(f"{i} {float(y[i])!r} {float(A[i])!r}\n")


def write_lmhead(path: str = LMHEAD) -> None:
    rows, cols, k = inputs.VOCAB, inputs.HIDDEN, 5
    c = inputs.lm_head(0)
    y, A = oracle.matvec(c["W"], c["x"], rows, cols)
    idx, val = oracle.topk(y, k)
    p = oracle.softmax(y)
    lse = oracle.logsumexp(y)
    with open(path, "w") as f:
        f.write("# lm_head top-5, W 262144 x 2560 (GGUF Q4_K rows), x f32[2560] ~ N(0,1)/sqrt(2560)\n")
        f.write("# inputs: quantized_decode_q4_amd.inputs.lm_head(0) "
                "(PCG64 seeds [0x51344B, 3, 0, 0] for W, [0x51344B, 3, 3, 0] for x)\n")
        f.write(f"# sha256(W bytes, x bytes) = {digest(c['W'], c['x'])}\n")
        f.write(f"# logsumexp = {float(lse)!r}\n")
        f.write("# values: oracle.matvec / oracle.topk / oracle.softmax (f64): rank row logit A prob\n")
        for r in range(k):
            f.write(f"{r} {int(idx[r])} {float(val[r])!r} {float(A[idx[r]])!r} {float(p[idx[r]])!r}\n")


def read(path: str) -> dict:
    """Parsed fixture: 'sha256', optional 'logsumexp', and 'rows' (list of token lists)."""
    out = {"rows": []}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("# sha256"):
                out["sha256"] = line.split("=")[1].strip()
            elif line.startswith("# logsumexp"):
                out["logsumexp"] = float(line.split("=")[1])
            elif line and not line.startswith("#"):
                out["rows"].append(line.split())
    return out


if __name__ == "__main__":
    oracle.lib()
    write_tiny()
    write_lmhead()
    print("wrote", TINY, LMHEAD)
