"""The path at one GPU's share of a tensor-parallel split, on one GPU.

Every output row of the path is an independent dot product, so a split by
rows (QKV heads, lm_head vocabulary) or by the FFN's inner dimension (Wg/Wu
rows with the matching Wd columns, cut at super-block boundaries) runs the
same kernels at a smaller shape. These tests run the shards of the Gemma-3-4B
shapes one after another and check what the split must preserve:
  * QKV and lm_head shards give the unsplit call's outputs bit for bit (a
    row's reduction order depends only on the column count);
  * the sum of the eight FFN shards' outputs is the unsplit FFN within the
    f32 bound, and each shard matches the oracle at its own shape;
  * the merged per-shard top-k lists give the unsplit top-k.
"""
import numpy as np
import pytest
import torch

from quantized_decode_q4_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-4
NSHARD = 8


@pytest.fixture(scope="module")
def q4k():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_decode_q4_amd import q4k as mod
    return mod


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def ratio(got, ref, A):
    err = np.abs(np.asarray(got, np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(A > 0, err / A, np.where(err == 0, 0.0, np.inf))
    return float(r.max())


def wd_columns(Wd, hidden, inter, s, n):
    """Columns [s*inter/n, (s+1)*inter/n) of a Q4_K matrix (whole super-blocks)."""
    nb = inter // 256
    per = nb // n
    return np.ascontiguousarray(Wd.reshape(hidden, nb, 144)[:, s * per:(s + 1) * per, :]
                                .reshape(hidden, per * 144))


def test_ffn_shards_sum_to_unsplit_ffn(q4k, orc):
    hidden, inter = inputs.HIDDEN, inputs.INTER
    part = inter // NSHARD
    L = inputs.ffn_layer(3)
    full = orc.ffn(L["Wg"], L["Wu"], L["Wd"], L["x"], hidden, inter, 0)
    x = dev(L["x"])
    ws = q4k.workspace(q4k.q4k_ffn_workspace_bytes(hidden, part))
    ys = []
    worst = 0.0
    for s in range(NSHARD):
        print(f"ffn shard {s}: Wg/Wu {part}x{hidden}, Wd {hidden}x{part}", flush=True)
        Wg = L["Wg"][s * part:(s + 1) * part]
        Wu = L["Wu"][s * part:(s + 1) * part]
        Wd = wd_columns(L["Wd"], hidden, inter, s, NSHARD)
        y = torch.full((hidden,), float("nan"), device="cuda")
        q4k.q4k_ffn(dev(Wg), dev(Wu), dev(Wd), x, y, hidden, part, 0, ws)
        torch.cuda.synchronize()
        yn = y.cpu().numpy()
        r = orc.ffn(Wg, Wu, Wd, L["x"], hidden, part, 0)
        worst = max(worst, ratio(yn, r["y"], r["A"]))
        ys.append(yn.astype(np.float64))
    print(f"  worst shard |err|/A = {worst:.3e}", flush=True)
    assert worst <= TOL
    total = np.sum(ys, axis=0)
    rr = ratio(total, full["y"], full["A"])
    print(f"  sum of shards vs unsplit: |err|/A = {rr:.3e}", flush=True)
    assert rr <= TOL


def test_qkv_head_shards_equal_unsplit_slices(q4k):
    c = inputs.qkv(copy=2)
    W, x = c["W"], dev(c["x"])
    qr, kr, cols = c["q_rows"], c["kv_rows"], inputs.HIDDEN
    q, k, v = (torch.empty(n, device="cuda") for n in (qr, kr, kr))
    q4k.q4k_qkv(dev(W), x, q, k, v, qr, kr, cols)
    nsh = 4                                     # 2 q heads and 1 kv head each
    qs, ks = qr // nsh, kr // nsh
    for s in range(nsh):
        Ws = np.concatenate([W[s * qs:(s + 1) * qs], W[qr + s * ks:qr + (s + 1) * ks],
                             W[qr + kr + s * ks:qr + kr + (s + 1) * ks]])
        a, b, d = (torch.empty(n, device="cuda") for n in (qs, ks, ks))
        q4k.q4k_qkv(dev(Ws), x, a, b, d, qs, ks, cols)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), q[s * qs:(s + 1) * qs].view(torch.int32)), s
        assert torch.equal(b.view(torch.int32), k[s * ks:(s + 1) * ks].view(torch.int32)), s
        assert torch.equal(d.view(torch.int32), v[s * ks:(s + 1) * ks].view(torch.int32)), s


def test_lmhead_vocab_shards_merge_to_unsplit_topk(q4k):
    c = inputs.lm_head()
    W, x = c["W"], dev(c["x"])
    rows, cols, kk = inputs.VOCAB, inputs.HIDDEN, 5
    logits = torch.empty(rows, device="cuda")
    ti, tv = torch.empty(kk, dtype=torch.int32, device="cuda"), torch.empty(kk, device="cuda")
    q4k.q4k_lmhead_topk(dev(W), x, logits, rows, cols, kk, ti, tv,
                        q4k.workspace(q4k.q4k_lmhead_workspace_bytes(rows, cols, kk)))
    torch.cuda.synchronize()
    per = rows // NSHARD
    ws = q4k.workspace(q4k.q4k_lmhead_workspace_bytes(per, cols, kk))
    cand = []
    for s in range(NSHARD):
        print(f"lm_head shard {s}: rows {s * per}..{(s + 1) * per - 1}", flush=True)
        ls = torch.empty(per, device="cuda")
        si, sv = torch.empty(kk, dtype=torch.int32, device="cuda"), torch.empty(kk, device="cuda")
        q4k.q4k_lmhead_topk(dev(W[s * per:(s + 1) * per]), x, ls, per, cols, kk, si, sv, ws)
        torch.cuda.synchronize()
        assert torch.equal(ls.view(torch.int32), logits[s * per:(s + 1) * per].view(torch.int32)), s
        cand += [(float(v), s * per + int(i)) for v, i in zip(sv.cpu().tolist(), si.cpu().tolist())]
    # the merge of the shards' lists: value descending, index ascending
    merged = sorted(cand, key=lambda t: (-t[0], t[1]))[:kk]
    assert [i for _, i in merged] == ti.cpu().tolist()
    assert [v for v, _ in merged] == tv.cpu().tolist()
