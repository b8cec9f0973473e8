"""GPU parity of the matrix-core prefill (seq >= 64) through the C ABI.

Bound, per output element: |gpu - oracle| <= 1e-2 * A against the exact f64
oracle. For the matrix product and for the full-size FFN, A = sum_j |w_ij x_j|
of the last stage. For the smaller FFN shapes A is the FFN's propagated error
scale (the oracle's ffn_prefill_scale): there, bf16 rounding of X alone moves
outputs by more than 1e-2 of the last stage's plain A, in exact bf16
arithmetic too. A second, tighter comparison is against the oracle's bf16
operand model (X and W rounded to bf16, exact products and sums): what remains
there is fp32 accumulation order, and for the FFN the bf16 rounding of H
computed from fp32 rather than exact G and U.

Shapes are chosen so that every workgroup shape of the kernel (1..8 tiles of
16 weight rows, K split or not), ragged rows / tokens and the largest
reduction length (cols = 65536) are exercised.
"""
import numpy as np
import pytest
import torch

from quantized_decode_q4_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-2          # bound for bf16 operands with fp32 accumulation
TOL_BF16_MM = 1e-4  # against the bf16 operand model, matmul
TOL_BF16_FFN = 5e-4 # against the bf16 operand model, gated FFN


@pytest.fixture(scope="module")
def q4k():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_decode_q4_amd import q4k as mod
    return mod


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def ratio(got, ref, A):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(A > 0, err / A, np.where(err == 0, 0.0, np.inf))
    return float(r.max()) if r.size else 0.0


def check(got, ref, A, tol, what):
    r = ratio(got, ref, A)
    print(f"{what}: max |err|/A = {r:.3e} (bound {tol:g})", flush=True)
    assert np.all(np.isfinite(got)), what
    assert r <= tol, f"{what}: max |err|/A = {r:.3e} > {tol}"


def gpu_matmul(q4k, W, X, rows, cols):
    seq = X.shape[0]
    Y = torch.full((seq, rows), float("nan"), device="cuda")
    ws = q4k.workspace(q4k.q4k_matmul_workspace_bytes(rows, cols, seq))
    q4k.q4k_matmul(dev(W), dev(X), Y, rows, cols, seq, ws)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def gpu_ffn_prefill(q4k, Wg, Wu, Wd, X, hidden, inter, act):
    seq = X.shape[0]
    Y = torch.full((seq, hidden), float("nan"), device="cuda")
    ws = q4k.workspace(q4k.q4k_ffn_prefill_workspace_bytes(seq, hidden, inter))
    q4k.q4k_ffn_prefill(dev(Wg), dev(Wu), dev(Wd), dev(X), Y, seq, hidden, inter, act, ws)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


# (rows, cols, seq): tiles per workgroup 1..8 at 256 CUs, K splits for the
# short-and-wide shapes, ragged rows (not a multiple of 16) and ragged tokens.
MATMUL_SHAPES = [
    (64, 256, 64),
    (200, 512, 64),
    (37, 1024, 100),
    (1000, 2560, 64),
    (4800, 256, 64),
    (11200, 256, 65),
    (14400, 256, 64),
    (17600, 256, 64),
    (22400, 256, 64),
    (27203, 256, 64),
    (30400, 256, 64),
    (9700, 256, 130),
    (300, 10240, 64),
    (2560, 2560, 128),
    (40, 65536, 64),       # the largest cols: K split 256 ways, one super-block each
    (300, 65536, 70),      # ... 32 ways, with two token groups
    (1000, 2560, 520),     # nine token groups, the last ragged
]


@pytest.mark.parametrize("rows,cols,seq", MATMUL_SHAPES)
def test_matmul_mfma_shapes(q4k, orc, rows, cols, seq):
    print(f"matmul rows={rows} cols={cols} seq={seq}", flush=True)
    rng = np.random.default_rng(rows * 7 + cols + seq)
    W = inputs.q4k_random(rng, rows, cols)
    X = inputs.normal_f32(rng, (seq, cols))
    Y = gpu_matmul(q4k, W, X, rows, cols)
    ref, A = orc.matmul(W, X, rows, cols)
    check(Y, ref, A, TOL, f"matmul {rows}x{cols} seq={seq} vs exact")
    refb, Ab = orc.matmul_bf16(W, X, rows, cols)
    check(Y, refb, Ab, TOL_BF16_MM, f"matmul {rows}x{cols} seq={seq} vs bf16 model")


def test_matmul_mfma_one_hot_tokens_recover_bf16_weights(q4k, orc):
    """Token t = e_j reads column j of W: the result is the weight rounded
    (binary32, then bf16), element for element."""
    rng = np.random.default_rng(71)
    rows, cols, seq = 48, 512, 64
    W = inputs.q4k_random(rng, rows, cols)
    cols_probe = rng.choice(cols, seq, replace=False)
    X = np.zeros((seq, cols), np.float32)
    X[np.arange(seq), cols_probe] = 1.0
    Y = gpu_matmul(q4k, W, X, rows, cols)
    dense = orc.dequant(W, rows, cols)
    want = np.array([[orc.round_bf16(float(np.float32(dense[i, j]))) for i in range(rows)]
                     for j in cols_probe])
    assert np.array_equal(Y.astype(np.float64), want)


def test_matmul_mfma_deterministic(q4k):
    rng = np.random.default_rng(72)
    rows, cols, seq = 1000, 2560, 64
    W, X = dev(inputs.q4k_random(rng, rows, cols)), dev(inputs.normal_f32(rng, (seq, cols)))
    ws = q4k.workspace(q4k.q4k_matmul_workspace_bytes(rows, cols, seq))
    outs = []
    for _ in range(2):
        Y = torch.full((seq, rows), float("nan"), device="cuda")
        q4k.q4k_matmul(W, X, Y, rows, cols, seq, ws)
        torch.cuda.synchronize()
        outs.append(Y.clone())
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


def test_matmul_mfma_split_any_workspace_contents(q4k):
    """A K-split launch keeps its bf16 activations and partial sums in the
    workspace; whatever the workspace held before (zeros, garbage, the
    previous call's data) the result is the same, bit for bit."""
    rng = np.random.default_rng(74)
    rows, cols, seq = 300, 10240, 64          # 40 splits along K
    W, X = dev(inputs.q4k_random(rng, rows, cols)), dev(inputs.normal_f32(rng, (seq, cols)))
    need = q4k.q4k_matmul_workspace_bytes(rows, cols, seq)
    outs = []
    for fill in (0, 255, 255, 7):
        ws = q4k.workspace(need)
        ws.fill_(fill)
        Y = torch.full((seq, rows), float("nan"), device="cuda")
        q4k.q4k_matmul(W, X, Y, rows, cols, seq, ws)
        q4k.q4k_matmul(W, X, Y, rows, cols, seq, ws)   # again on the same workspace
        torch.cuda.synchronize()
        outs.append(Y.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


def test_matmul_mfma_split_output_alignment(q4k):
    """The K-split sum runs four outputs per thread when Y is 16-byte aligned
    and one otherwise: both give the same bits."""
    rng = np.random.default_rng(75)
    rows, cols, seq = 300, 10240, 64
    W, X = dev(inputs.q4k_random(rng, rows, cols)), dev(inputs.normal_f32(rng, (seq, cols)))
    ws = q4k.workspace(q4k.q4k_matmul_workspace_bytes(rows, cols, seq))
    buf = torch.full((seq * rows + 4,), float("nan"), device="cuda")
    outs = []
    for off in (0, 1):
        Y = buf[off:off + seq * rows]
        q4k.q4k_matmul(W, X, Y, rows, cols, seq, ws)
        torch.cuda.synchronize()
        outs.append(Y.clone())
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


def test_matmul_mfma_workspace_too_small(q4k):
    rows, cols, seq = 64, 256, 64
    need = q4k.q4k_matmul_workspace_bytes(rows, cols, seq)
    assert need >= seq * cols * 2
    W = torch.zeros(rows * 144, dtype=torch.uint8, device="cuda")
    X = torch.zeros(seq, cols, device="cuda")
    Y = torch.full((seq, rows), 3.0, device="cuda")
    ws = q4k.workspace(need - 256)
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q4k_matmul(W, X, Y, rows, cols, seq, ws)
    assert e.value.status == q4k.Q4K_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(Y == 3.0)


# (hidden, inter, seq, act)
FFN_SHAPES = [
    (512, 768, 64, 0),
    (512, 768, 64, 1),
    (256, 2560, 100, 0),
    (1024, 7680, 64, 1),
    (768, 1536, 65, 0),
    (8192, 512, 64, 1),    # gate/up pair split along K (16 splits)
    (4096, 512, 130, 0),   # ... with three token groups
    (256, 65536, 64, 0),   # down reduces over the largest cols (K split 64 ways)
    (65536, 256, 64, 1),   # gate/up over the largest cols, down over the most rows
]


@pytest.mark.parametrize("hidden,inter,seq,act", FFN_SHAPES)
def test_ffn_prefill_mfma_shapes(q4k, orc, hidden, inter, seq, act):
    print(f"ffn_prefill hidden={hidden} inter={inter} seq={seq} act={act}", flush=True)
    rng = np.random.default_rng(hidden + 3 * inter + seq + act)
    Wg = inputs.q4k_random(rng, inter, hidden)
    Wu = inputs.q4k_random(rng, inter, hidden)
    Wd = inputs.q4k_random(rng, hidden, inter)
    X = inputs.normal_f32(rng, (seq, hidden))
    Y = gpu_ffn_prefill(q4k, Wg, Wu, Wd, X, hidden, inter, act)
    ref, A = orc.ffn_prefill(Wg, Wu, Wd, X, hidden, inter, act)
    # bf16 rounding of X alone moves the small-shape outputs by up to ~1.4e-2
    # of the last stage's A (exact bf16 arithmetic included), so the bound
    # uses the FFN's propagated error scale (gate/up magnitudes carried
    # through the activation); the full-size test applies the plain A.
    Ap = orc.ffn_prefill_scale(Wg, Wu, Wd, X, hidden, inter, act)
    check(Y, ref, Ap, TOL, f"ffn_prefill {hidden}/{inter} seq={seq} act={act} vs exact (propagated scale)")
    print(f"  (plain last-stage A: {ratio(Y, ref, A):.3e})", flush=True)
    refb, Ab = orc.ffn_prefill_bf16(Wg, Wu, Wd, X, hidden, inter, act)
    check(Y, refb, Ab, TOL_BF16_FFN, f"ffn_prefill {hidden}/{inter} seq={seq} act={act} vs bf16 model")


@pytest.mark.slow
def test_ffn_prefill_mfma_full_size_layer0(q4k, orc):
    """Gemma-3-4B FFN shape (hidden 2560, inter 10240), 64 tokens, layer-0
    weights of the decode FFN workload with the prefill activations."""
    layer = inputs.ffn_layer(0)
    X = inputs.prefill_x()
    hidden, inter = inputs.HIDDEN, inputs.INTER
    print("ffn_prefill full size, 64 tokens", flush=True)
    Y = gpu_ffn_prefill(q4k, layer["Wg"], layer["Wu"], layer["Wd"], X, hidden, inter, 0)
    ref, A = orc.ffn_prefill(layer["Wg"], layer["Wu"], layer["Wd"], X, hidden, inter, 0)
    check(Y, ref, A, TOL, "ffn_prefill full size vs exact (plain A)")
    Ap = orc.ffn_prefill_scale(layer["Wg"], layer["Wu"], layer["Wd"], X, hidden, inter, 0)
    check(Y, ref, Ap, TOL, "ffn_prefill full size vs exact (propagated scale)")
    sample = np.arange(0, 64, 9)   # the bf16 model is slower: a token sample
    refb, Ab = orc.ffn_prefill_bf16(layer["Wg"], layer["Wu"], layer["Wd"], X[sample], hidden,
                                    inter, 0)
    check(Y[sample], refb, Ab, TOL_BF16_FFN, "ffn_prefill full size vs bf16 model (sampled tokens)")
