"""Seeded synthetic inputs for the Q4_K decode path.

This module is the only code shared by the HIP path's tests/benchmarks and the
CPU oracle. It draws random numbers and lays them out as bytes; it performs none
of the method's arithmetic (no dequantisation, no dot products, no activation).

Workload shapes follow the Gemma-3-4B decode figures of the infer-inference
PERFORMANCE page (hidden 2560, 34 layers, vocabulary ~262K) and the head layout of
its RoPE comparison table (head_dim 256, 8 query heads); the value distributions
are the synthetic "random weights" regime of that page's GPU decode table.

Q4_K block bytes (GGUF layout, 144 B per 256 weights):
  bytes 0-1 : d    (IEEE binary16, little-endian)
  bytes 2-3 : dmin (IEEE binary16, little-endian)
  bytes 4-15: 96 bits of packed 6-bit scales and mins
  bytes 16-143: 256 four-bit quants
Random blocks use uniform bytes 4..143 (every 6-bit field and nibble is then an
independent uniform integer) and d, dmin drawn uniformly from [1e-4, 2e-3) and
rounded to binary16 by numpy (round-to-nearest-even).

Q6_K block bytes (GGUF layout, 210 B per 256 weights):
  bytes 0-127  : low 4 bits of the 256 quants
  bytes 128-191: high 2 bits of the 256 quants
  bytes 192-207: 16 signed 8-bit scales
  bytes 208-209: d (IEEE binary16, little-endian)
Random blocks use uniform bytes 0..207 (every quant and scale is then an
independent uniform integer) and d drawn uniformly from [1e-4, 2e-3) and
rounded to binary16.

Seeding: numpy PCG64 via ``default_rng([0x51344B, config, tensor_id, index])``.
Configs: 0 tiny matvec, 1 QKV, 2 FFN, 3 lm_head, 4 prefill activations, 5 the
attention output projection, 6 Q6_K matvec at the down-projection shape, 7 the
residual stream and norm weights of the fused RMSNorm.
Tensor ids: 0 = W / Wqkv / Wg, 1 = Wu, 2 = Wd, 3 = x / X. ``index`` is the layer
or copy number. Draw order inside ``q4k_random``: the 144-byte rows of raw bytes
first, then all d values, then all dmin values (row-major over blocks).
"""
from __future__ import annotations

import numpy as np

QK_K = 256            # weights per super-block
BLOCK_BYTES = 144     # bytes per Q4_K super-block
Q6K_BLOCK_BYTES = 210 # bytes per Q6_K super-block
SEED_ROOT = 0x51344B

# Shapes of the five workloads (rows, cols, ...)
HIDDEN = 2560
INTER = 10240
Q_ROWS = 2048          # 8 query heads x 256
KV_ROWS = 1024         # 4 kv heads x 256
VOCAB = 262144
N_LAYERS = 34
PREFILL_SEQ = 64

D_LO, D_HI = 1e-4, 2e-3


def rng_for(config: int, tensor_id: int, index: int = 0) -> np.random.Generator:
    """Counter-style seeding: one independent PCG64 stream per (config, tensor, index)."""
    return np.random.default_rng([SEED_ROOT, int(config), int(tensor_id), int(index)])


def row_bytes(cols: int) -> int:
    if cols <= 0 or cols % QK_K:
        raise ValueError(f"cols must be a positive multiple of {QK_K}, got {cols}")
    return cols // QK_K * BLOCK_BYTES


def q4k_random(rng: np.random.Generator, rows: int, cols: int,
               d_range=(D_LO, D_HI), dmin_range=(D_LO, D_HI)) -> np.ndarray:
    """Random Q4_K matrix as uint8[rows, cols/256*144] (row-major blocks)."""
    nb = cols // QK_K
    rb = row_bytes(cols)
    raw = rng.integers(0, 256, size=(rows, nb, BLOCK_BYTES), dtype=np.uint8)
    d = rng.uniform(d_range[0], d_range[1], size=(rows, nb)).astype(np.float16)
    dmin = rng.uniform(dmin_range[0], dmin_range[1], size=(rows, nb)).astype(np.float16)
    raw[:, :, 0:2] = d.astype("<f2").view(np.uint8).reshape(rows, nb, 2)
    raw[:, :, 2:4] = dmin.astype("<f2").view(np.uint8).reshape(rows, nb, 2)
    return raw.reshape(rows, rb)


def q6k_random(rng: np.random.Generator, rows: int, cols: int,
               d_range=(D_LO, D_HI)) -> np.ndarray:
    """Random Q6_K matrix as uint8[rows, cols/256*210] (row-major blocks)."""
    if cols <= 0 or cols % QK_K:
        raise ValueError(f"cols must be a positive multiple of {QK_K}, got {cols}")
    nb = cols // QK_K
    raw = rng.integers(0, 256, size=(rows, nb, Q6K_BLOCK_BYTES), dtype=np.uint8)
    d = rng.uniform(d_range[0], d_range[1], size=(rows, nb)).astype(np.float16)
    raw[:, :, 208:210] = d.astype("<f2").view(np.uint8).reshape(rows, nb, 2)
    return raw.reshape(rows, nb * Q6K_BLOCK_BYTES)


def normal_f32(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """N(0,1) drawn in f64, multiplied by ``scale`` in f64, then cast to f32."""
    v = rng.standard_normal(size=shape)
    if scale != 1.0:
        v = v * scale
    return v.astype(np.float32)


# ----------------------------------------------------------------------------
# The five named workloads. Each returns a dict of numpy arrays (host memory).
# ----------------------------------------------------------------------------

def tiny_matvec(rows: int = 256, cols: int = 512):
    """Tiny Q4_K matvec: W 256 x 512 (2 super-blocks per row), x ~ N(0,1)."""
    return {"W": q4k_random(rng_for(0, 0), rows, cols),
            "x": normal_f32(rng_for(0, 3), cols)}


def qkv(copy: int = 0, cols: int = HIDDEN, q_rows: int = Q_ROWS, kv_rows: int = KV_ROWS):
    """Fused QKV: concatenated [q; k; v] rows x hidden; x ~ N(0,1)."""
    rows = q_rows + 2 * kv_rows
    return {"W": q4k_random(rng_for(1, 0, copy), rows, cols),
            "x": normal_f32(rng_for(1, 3, copy), cols),
            "q_rows": q_rows, "kv_rows": kv_rows}


def ffn_layer(layer: int = 0, hidden: int = HIDDEN, inter: int = INTER):
    """One FFN layer: Wg, Wu (inter x hidden), Wd (hidden x inter), x ~ N(0,1)."""
    return {"Wg": q4k_random(rng_for(2, 0, layer), inter, hidden),
            "Wu": q4k_random(rng_for(2, 1, layer), inter, hidden),
            "Wd": q4k_random(rng_for(2, 2, layer), hidden, inter),
            "x": normal_f32(rng_for(2, 3, layer), hidden)}


def lm_head(copy: int = 0, rows: int = VOCAB, cols: int = HIDDEN):
    """lm_head: W vocab x hidden; x ~ N(0,1) / sqrt(hidden)."""
    return {"W": q4k_random(rng_for(3, 0, copy), rows, cols),
            "x": normal_f32(rng_for(3, 3, copy), cols, scale=1.0 / np.sqrt(cols))}


def o_proj(layer: int = 0, hidden: int = HIDDEN, q_dim: int = Q_ROWS):
    """Attention output projection: W_o hidden x (8 heads x 256), input ~ N(0,1)."""
    return {"W": q4k_random(rng_for(5, 0, layer), hidden, q_dim),
            "x": normal_f32(rng_for(5, 3, layer), q_dim)}


def q6k_down(layer: int = 0, hidden: int = HIDDEN, inter: int = INTER):
    """Q6_K matvec at the FFN down-projection shape: W hidden x inter, x ~ N(0,1)."""
    return {"W": q6k_random(rng_for(6, 0, layer), hidden, inter),
            "x": normal_f32(rng_for(6, 3, layer), inter)}


def norm_inputs(index: int = 0, n: int = HIDDEN):
    """Residual RMSNorm inputs: stream h ~ 4 N(0,1), delta ~ N(0,1), norm weight
    w = 1 + 0.1 N(0,1) (all f32), eps = 1e-6."""
    return {"h": normal_f32(rng_for(7, 0, index), n, scale=4.0),
            "delta": normal_f32(rng_for(7, 1, index), n),
            "w": (1.0 + 0.1 * rng_for(7, 2, index).standard_normal(n)).astype(np.float32),
            "eps": 1e-6}


def prefill_x(seq: int = PREFILL_SEQ, hidden: int = HIDDEN, index: int = 0):
    """Prefill activations X[seq, hidden] ~ N(0,1); weights are ffn_layer(...)'s."""
    return normal_f32(rng_for(4, 3, index), (seq, hidden))
