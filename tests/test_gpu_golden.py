"""The HIP path (through the C ABI) against the stored oracle values under
tests/golden/: the tiny matvec (every row) and the full-size lm_head top-5 with
its probabilities and log-sum-exp. Tolerance per output: 1e-4 * A, A = sum_j
|w_ij x_j| from the fixture."""
import importlib.util
import os

import numpy as np
import pytest
import torch

from quantized_decode_q4_amd import inputs

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-4


def _maker():
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLDEN, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def q4k():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_decode_q4_amd import q4k as mod
    return mod


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_tiny_matvec_equals_golden(q4k):
    fx = _maker().read(_maker().TINY)
    c = inputs.tiny_matvec()
    y = torch.full((256,), float("nan"), device="cuda")
    q4k.q4k_matvec(dev(c["W"]), dev(c["x"]), y, 256, 512)
    torch.cuda.synchronize()
    ref = np.array([float(r[1]) for r in fx["rows"]])
    A = np.array([float(r[2]) for r in fx["rows"]])
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    print(f"tiny golden: max |err|/A = {float((err / A).max()):.3e}", flush=True)
    assert np.all(err <= TOL * A)


def test_lmhead_top5_probs_equal_golden(q4k):
    fx = _maker().read(_maker().LMHEAD)
    rows, cols, k = inputs.VOCAB, inputs.HIDDEN, 5
    c = inputs.lm_head(0)
    logits = torch.empty(rows, device="cuda")
    ti = torch.empty(k, dtype=torch.int32, device="cuda")
    tv = torch.empty(k, device="cuda")
    tp = torch.empty(k, device="cuda")
    lse = torch.empty(1, device="cuda")
    ws = q4k.workspace(q4k.q4k_lmhead_workspace_bytes(rows, cols, k))
    q4k.q4k_lmhead_topk_probs(dev(c["W"]), dev(c["x"]), logits, rows, cols, k, ti, tv, tp, lse, ws)
    torch.cuda.synchronize()
    idx = [int(r[1]) for r in fx["rows"]]
    val = np.array([float(r[2]) for r in fx["rows"]])
    A = np.array([float(r[3]) for r in fx["rows"]])
    prob = np.array([float(r[4]) for r in fx["rows"]])
    print(f"golden top-5 {idx}, GPU {ti.cpu().tolist()}", flush=True)
    assert ti.cpu().tolist() == idx
    assert np.all(np.abs(tv.cpu().numpy().astype(np.float64) - val) <= TOL * A)
    # log-probabilities: an error e in a logit moves log p by at most 2e
    e = TOL * float(A.max())
    assert abs(float(lse.cpu()[0]) - fx["logsumexp"]) <= e + 1e-5
    assert np.all(np.abs(np.log(tp.cpu().numpy().astype(np.float64)) - np.log(prob)) <= 2 * e + 2e-5)
