"""GPU parity of the Q6_K matvec (q6k_matvec) through the C ABI.

Pass rule, per output element: |gpu - oracle| <= 1e-4 * A, A = sum_j |w_ij x_j|
from the f64 oracle. Shapes with an odd number of blocks per row put blocks
at both alignments (0 and 2 mod 4 bytes) inside a row and across rows.
"""
import numpy as np
import pytest
import torch

from quantized_decode_q4_amd import inputs
from q4k_fields import pack_q6k_block

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def q4k():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_decode_q4_amd import q4k as mod
    return mod


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_q6k(q4k, W, x, rows, cols):
    y = torch.full((rows,), float("nan"), device="cuda")
    q4k.q6k_matvec(dev(W), dev(x), y, rows, cols)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(got, ref, A, what):
    err = np.abs(got.astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(A > 0, err / A, np.where(err == 0, 0.0, np.inf))
    worst = float(r.max()) if r.size else 0.0
    print(f"{what}: max |err|/A = {worst:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert worst <= TOL, f"{what}: {worst:.3e} > {TOL}"


# (rows, cols): one block; ragged row counts; odd blocks per row (both
# alignments); the decode shapes; the widest rows (one row per sweep,
# 1024-thread workgroups).
SHAPES = [(1, 256), (37, 256), (100, 768), (129, 1280), (1000, 2560), (5000, 512),
          (4096, 2560), (700, 10240), (3, 65536), (257, 33024)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_q6k_matvec_shapes(q4k, orc, rows, cols):
    print(f"q6k_matvec rows={rows} cols={cols}", flush=True)
    rng = np.random.default_rng(rows * 13 + cols)
    W = inputs.q6k_random(rng, rows, cols)
    x = inputs.normal_f32(rng, cols)
    y = gpu_q6k(q4k, W, x, rows, cols)
    ref, A = orc.q6k_matvec(W, x, rows, cols)
    check(y, ref, A, f"q6k {rows}x{cols}")


def test_q6k_matvec_down_shape_config(q4k, orc):
    """Gemma-3-4B down-projection shape, 2560 x 10240, Q6_K weights."""
    c = inputs.q6k_down(0)
    rows, cols = inputs.HIDDEN, inputs.INTER
    y = gpu_q6k(q4k, c["W"], c["x"], rows, cols)
    ref, A = orc.q6k_matvec(c["W"], c["x"], rows, cols)
    check(y, ref, A, "q6k down 2560x10240")


def test_q6k_one_hot_columns_are_exact(q4k, orc):
    """x = e_j reads column j: d * scale * (q - 32) is exact in f32."""
    rng = np.random.default_rng(61)
    rows, cols = 300, 1280
    W = inputs.q6k_random(rng, rows, cols)
    dense = orc.q6k_dequant(W, rows, cols)
    for j in list(rng.choice(cols, 6, replace=False)) + [0, cols - 1, 255, 256]:
        x = np.zeros(cols, np.float32)
        x[j] = 1.0
        y = gpu_q6k(q4k, W, x, rows, cols)
        assert np.array_equal(y.astype(np.float64), dense[:, j]), j


def test_q6k_fields_extremes(q4k, orc):
    """Saturated quants and scales (q = 0 / 63, scale -128 / 127) in every
    position, against the closed form."""
    rows, cols = 8, 512
    blocks = []
    vals = []
    for r in range(rows):
        q = np.full(256, 63 if r % 2 else 0)
        sc = np.full(16, 127 if r % 4 < 2 else -128)
        blocks.append(np.concatenate([pack_q6k_block(1.0 / 1024, sc, q)] * (cols // 256)))
        vals.append((1.0 / 1024) * sc[0] * (q[0] - 32))
    W = np.stack(blocks)
    x = np.ones(cols, np.float32)
    y = gpu_q6k(q4k, W, x, rows, cols)
    assert np.array_equal(y.astype(np.float64), np.array(vals) * cols)


def test_q6k_nan_scale_propagates_to_its_row_only(q4k, orc):
    rng = np.random.default_rng(62)
    rows, cols = 50, 768
    W = inputs.q6k_random(rng, rows, cols)
    W[7, 210 + 208:210 + 210] = np.array([0x00, 0x7E], np.uint8)   # block 1 of row 7: d = NaN
    x = inputs.normal_f32(rng, cols)
    y = gpu_q6k(q4k, W, x, rows, cols)
    assert np.isnan(y[7]) and np.all(np.isfinite(np.delete(y, 7)))
    ref, A = orc.q6k_matvec(W, x, rows, cols)
    ok = np.arange(rows) != 7
    check(y[ok], ref[ok], A[ok], "q6k rows around a NaN block")


def test_q6k_deterministic_and_zero_rows(q4k):
    rng = np.random.default_rng(63)
    rows, cols = 2000, 2560
    W, x = dev(inputs.q6k_random(rng, rows, cols)), dev(inputs.normal_f32(rng, cols))
    outs = []
    for _ in range(2):
        y = torch.full((rows,), float("nan"), device="cuda")
        q4k.q6k_matvec(W, x, y, rows, cols)
        torch.cuda.synchronize()
        outs.append(y.clone())
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    y = torch.full((4,), 5.0, device="cuda")
    q4k.q6k_matvec(W, x, y, 0, cols)     # rows = 0: nothing is written
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)
