"""lm_head at the largest vocabulary the library takes for a row width
(q4k_lmhead_rows_max): the launch then produces the most candidate lists the
merge kernel accepts (1024 at cols 256 on any grid). Checked for k = 64 (the
top-k maximum, merged by rounds) and k = 5 (merged by ranks), both with the
softmax: every logit against the oracle to the f32 tolerance (|err| <= 1e-4 * A
per logit, A = sum_j |w_ij x_j|), the top-k against the oracle's selection over
the GPU's own logits, the probabilities and the log-sum-exp against the f64
softmax of those logits. Inputs: seeded Q4_K rows (config 8, tensor 0) and
x ~ N(0,1) (tensor 3)."""
import math

import numpy as np
import pytest
import torch

from quantized_decode_q4_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-4
COLS = 256


@pytest.fixture(scope="module")
def q4k():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_decode_q4_amd import q4k as mod
    return mod


@pytest.fixture(scope="module")
def case(q4k, orc):
    rows = int(q4k.lib.q4k_lmhead_rows_max(COLS))
    assert rows > 0
    W = inputs.q4k_random(inputs.rng_for(8, 0), rows, COLS)
    x = inputs.normal_f32(inputs.rng_for(8, 3), (COLS,))
    ref, A = orc.matvec(W, x, rows, COLS)
    Wd = torch.from_numpy(W).cuda()
    xd = torch.from_numpy(x).cuda()
    return rows, Wd, xd, ref, A


@pytest.mark.parametrize("k", [64, 5])
def test_lmhead_at_the_row_limit(q4k, orc, case, k):
    rows, Wd, xd, ref, A = case
    print(f"lm_head {rows} x {COLS}, k = {k}", flush=True)
    ws = q4k.workspace(q4k.q4k_lmhead_workspace_bytes(rows, COLS, k))
    logits = torch.full((rows,), float("nan"), device="cuda")
    ti = torch.full((k,), -7, dtype=torch.int32, device="cuda")
    tv = torch.full((k,), float("nan"), device="cuda")
    tp = torch.full((k,), float("nan"), device="cuda")
    lse = torch.full((1,), float("nan"), device="cuda")
    q4k.q4k_lmhead_topk_probs(Wd, xd, logits, rows, COLS, k, ti, tv, tp, lse, ws)
    torch.cuda.synchronize()
    logits, ti, tv, tp, lse = (t.cpu().numpy() for t in (logits, ti, tv, tp, lse))

    assert not np.isnan(logits).any(), "rows never written"
    r = float((np.abs(logits.astype(np.float64) - ref) / A).max())
    print(f"max |err|/A = {r:.3e}", flush=True)
    assert r <= TOL
    gidx, _ = orc.topk(logits.astype(np.float64), k)   # the GPU's own ranking
    assert np.array_equal(ti, gidx)
    assert np.array_equal(tv.view(np.uint32), logits[ti].view(np.uint32))
    l64 = logits.astype(np.float64)
    m = l64.max()
    lse_ref = m + math.log(math.fsum(np.exp(l64 - m)))
    assert abs(float(lse[0]) - lse_ref) <= 1e-5 + 1e-6 * abs(lse_ref)
    assert np.allclose(tp, np.exp(tv.astype(np.float64) - float(lse[0])), rtol=1e-5, atol=0)
