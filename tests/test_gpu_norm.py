"""GPU parity of the residual RMSNorm fused into a projection's input
(q4k_rmsnorm_matvec, q4k_rmsnorm_ffn) through the C ABI.

The oracle forms s = h + delta with one f32 addition (the stream is f32),
then x = s / sqrt(mean(s^2) + eps) * w and the projection in f64. Pass rule:
|gpu - oracle| <= 1e-4 * A per output, A = sum_j |w_ij x_j| of the last
stage; the new residual stream h_out must equal s bit for bit.
"""
import numpy as np
import pytest
import torch

from quantized_decode_q4_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def q4k():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_decode_q4_amd import q4k as mod
    return mod


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check(got, ref, A, what):
    err = np.abs(got.astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(A > 0, err / A, np.where(err == 0, 0.0, np.inf))
    worst = float(r.max()) if r.size else 0.0
    print(f"{what}: max |err|/A = {worst:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert worst <= TOL, f"{what}: {worst:.3e} > {TOL}"


def gpu_norm_matvec(q4k, W, h, delta, w, eps, rows, cols, want_h_out=True):
    y = torch.full((rows,), float("nan"), device="cuda")
    h_out = torch.full((cols,), float("nan"), device="cuda") if want_h_out else None
    q4k.q4k_rmsnorm_matvec(dev(W), dev(h), dev(delta), dev(w), eps, h_out, y, rows, cols)
    torch.cuda.synchronize()
    return y.cpu().numpy(), None if h_out is None else h_out.cpu().numpy()


# (rows, cols): few sweeps per workgroup (f32 activations), many sweeps
# (activations converted in LDS), rows wider than the LDS copy (per-thread
# conversion), ragged and tiny shapes.
SHAPES = [(1, 256), (100, 512), (4096, 2560), (2560, 2048), (30000, 1024), (10240, 2560),
          (300, 20480), (777, 768), (3, 65536)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("with_delta", [True, False])
def test_rmsnorm_matvec_shapes(q4k, orc, rows, cols, with_delta):
    print(f"rmsnorm_matvec rows={rows} cols={cols} delta={with_delta}", flush=True)
    rng = np.random.default_rng(rows + 5 * cols + with_delta)
    W = inputs.q4k_random(rng, rows, cols)
    h = inputs.normal_f32(rng, cols, scale=4.0)
    delta = inputs.normal_f32(rng, cols) if with_delta else None
    w = (1 + 0.1 * rng.standard_normal(cols)).astype(np.float32)
    y, h_out = gpu_norm_matvec(q4k, W, h, delta, w, 1e-6, rows, cols)
    s, x = orc.residual_rmsnorm(h, delta, w, 1e-6)
    assert np.array_equal(h_out.view(np.uint32), s.view(np.uint32))
    ref, A = orc.matvec_f64(W, x, rows, cols)
    check(y, ref, A, f"rmsnorm_matvec {rows}x{cols} delta={with_delta}")


def test_rmsnorm_qkv_config(q4k, orc):
    """Fused QKV (4096 x 2560) behind the norm; q, k, v are slices of y."""
    c = inputs.qkv()
    n = inputs.norm_inputs(0)
    rows, cols = c["q_rows"] + 2 * c["kv_rows"], inputs.HIDDEN
    y, h_out = gpu_norm_matvec(q4k, c["W"], n["h"], n["delta"], n["w"], n["eps"], rows, cols)
    s, x = orc.residual_rmsnorm(n["h"], n["delta"], n["w"], n["eps"])
    assert np.array_equal(h_out.view(np.uint32), s.view(np.uint32))
    ref, A = orc.matvec_f64(c["W"], x, rows, cols)
    check(y, ref, A, "rmsnorm + QKV 4096x2560")


def test_rmsnorm_without_h_out_and_zero_stream(q4k, orc):
    rng = np.random.default_rng(81)
    rows, cols = 500, 1024
    W = inputs.q4k_random(rng, rows, cols)
    w = np.ones(cols, np.float32)
    y, _ = gpu_norm_matvec(q4k, W, np.zeros(cols, np.float32), None, w, 1e-6, rows, cols,
                           want_h_out=False)
    assert np.all(y == 0)
    h = inputs.normal_f32(rng, cols)
    y, _ = gpu_norm_matvec(q4k, W, h, None, w, 0.0, rows, cols, want_h_out=False)
    _, x = orc.residual_rmsnorm(h, None, w, 0.0)
    ref, A = orc.matvec_f64(W, x, rows, cols)
    check(y, ref, A, "rmsnorm eps=0, no h_out")


def test_rmsnorm_scale_invariance_on_gpu(q4k, orc):
    """With eps = 0, scaling the stream by 2^k changes nothing but rounding."""
    rng = np.random.default_rng(82)
    rows, cols = 2048, 2560
    W = inputs.q4k_random(rng, rows, cols)
    h = inputs.normal_f32(rng, cols)
    w = np.ones(cols, np.float32)
    y1, _ = gpu_norm_matvec(q4k, W, h, None, w, 0.0, rows, cols, want_h_out=False)
    y2, _ = gpu_norm_matvec(q4k, W, (h * np.float32(2.0 ** 40)).astype(np.float32), None, w,
                            0.0, rows, cols, want_h_out=False)
    _, x = orc.residual_rmsnorm(h, None, w, 0.0)
    ref, A = orc.matvec_f64(W, x, rows, cols)
    check(y1, ref, A, "scale 1")
    check(y2, ref, A, "scale 2^40")


@pytest.mark.parametrize("hidden,inter,act", [(512, 768, 0), (1024, 3072, 1), (2560, 10240, 0),
                                              (65536, 512, 1)])
def test_rmsnorm_ffn(q4k, orc, hidden, inter, act):
    print(f"rmsnorm_ffn hidden={hidden} inter={inter} act={act}", flush=True)
    if hidden == inputs.HIDDEN:
        L = inputs.ffn_layer(0)
        Wg, Wu, Wd = L["Wg"], L["Wu"], L["Wd"]
        n = inputs.norm_inputs(1)
        h, delta, w, eps = n["h"], n["delta"], n["w"], n["eps"]
    else:
        rng = np.random.default_rng(hidden + inter + act)
        Wg = inputs.q4k_random(rng, inter, hidden)
        Wu = inputs.q4k_random(rng, inter, hidden)
        Wd = inputs.q4k_random(rng, hidden, inter)
        h = inputs.normal_f32(rng, hidden, scale=4.0)
        delta = inputs.normal_f32(rng, hidden)
        w = (1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32)
        eps = 1e-6
    y = torch.full((hidden,), float("nan"), device="cuda")
    h_out = torch.full((hidden,), float("nan"), device="cuda")
    ws = q4k.workspace(q4k.q4k_ffn_workspace_bytes(hidden, inter))
    q4k.q4k_rmsnorm_ffn(dev(Wg), dev(Wu), dev(Wd), dev(h), dev(delta), dev(w), eps, h_out, y,
                        hidden, inter, act, ws)
    torch.cuda.synchronize()
    s, x = orc.residual_rmsnorm(h, delta, w, eps)
    assert np.array_equal(h_out.cpu().numpy().view(np.uint32), s.view(np.uint32))
    r = orc.ffn_f64(Wg, Wu, Wd, x, hidden, inter, act)
    check(y.cpu().numpy(), r["y"], r["A"], f"rmsnorm_ffn {hidden}/{inter} act={act}")


def test_rmsnorm_deterministic(q4k):
    rng = np.random.default_rng(83)
    rows, cols = 4096, 2560
    W = dev(inputs.q4k_random(rng, rows, cols))
    h, d = dev(inputs.normal_f32(rng, cols)), dev(inputs.normal_f32(rng, cols))
    w = dev(np.ones(cols, np.float32))
    outs = []
    for _ in range(2):
        y = torch.full((rows,), float("nan"), device="cuda")
        q4k.q4k_rmsnorm_matvec(W, h, d, w, 1e-6, None, y, rows, cols)
        torch.cuda.synchronize()
        outs.append(y.clone())
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
