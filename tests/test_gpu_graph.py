"""HIP-graph capture of the C-ABI calls (what the benchmark replays).

A decode-layer sequence (norm -> QKV, O projection, norm -> FFN), the lm_head
with probabilities, the Q6_K matvec and the 64-token prefill FFN are captured
once into a graph, then replayed several times with unrelated eager work and
synchronisations in between. Every replay must reproduce the eager results bit
for bit (the kernels are deterministic; nothing in them is a memset node).
"""
import numpy as np
import pytest
import torch

from quantized_decode_q4_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4k():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_decode_q4_amd import q4k as mod
    return mod


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_graph_replays_match_eager(q4k):
    rng = np.random.default_rng(91)
    hid, inter, qr, kvr, vocab = 1024, 3072, 512, 256, 20000
    rows_qkv = qr + 2 * kvr
    W = {
        "qkv": dev(inputs.q4k_random(rng, rows_qkv, hid)),
        "o": dev(inputs.q4k_random(rng, hid, qr)),
        "g": dev(inputs.q4k_random(rng, inter, hid)),
        "u": dev(inputs.q4k_random(rng, inter, hid)),
        "d": dev(inputs.q4k_random(rng, hid, inter)),
        "lm": dev(inputs.q4k_random(rng, vocab, hid)),
        "q6": dev(inputs.q6k_random(rng, hid, inter)),
    }
    h0 = dev(inputs.normal_f32(rng, hid, scale=4.0))
    attn = dev(inputs.normal_f32(rng, qr))
    w_attn = dev((1 + 0.1 * rng.standard_normal(hid)).astype(np.float32))
    w_ffn = dev((1 + 0.1 * rng.standard_normal(hid)).astype(np.float32))
    xl = dev(inputs.normal_f32(rng, hid, scale=1 / np.sqrt(hid)))
    x6 = dev(inputs.normal_f32(rng, inter))
    Xp = dev(inputs.normal_f32(rng, (64, hid)))

    out = {
        "qkv": torch.empty(rows_qkv, device="cuda"),
        "h1": torch.empty(hid, device="cuda"),
        "o": torch.empty(hid, device="cuda"),
        "h2": torch.empty(hid, device="cuda"),
        "y": torch.empty(hid, device="cuda"),
        "logits": torch.empty(vocab, device="cuda"),
        "ti": torch.empty(5, dtype=torch.int32, device="cuda"),
        "tv": torch.empty(5, device="cuda"),
        "tp": torch.empty(5, device="cuda"),
        "lse": torch.empty(1, device="cuda"),
        "y6": torch.empty(hid, device="cuda"),
        "Yp": torch.empty((64, hid), device="cuda"),
    }
    ws_ffn = q4k.workspace(q4k.q4k_ffn_workspace_bytes(hid, inter))
    ws_lm = q4k.workspace(q4k.q4k_lmhead_workspace_bytes(vocab, hid, 5))
    ws_pf = q4k.workspace(q4k.q4k_ffn_prefill_workspace_bytes(64, hid, inter))

    def step():
        q4k.q4k_rmsnorm_matvec(W["qkv"], h0, None, w_attn, 1e-6, out["h1"], out["qkv"], rows_qkv, hid)
        q4k.q4k_matvec(W["o"], attn, out["o"], hid, qr)
        q4k.q4k_rmsnorm_ffn(W["g"], W["u"], W["d"], out["h1"], out["o"], w_ffn, 1e-6, out["h2"],
                            out["y"], hid, inter, q4k.Q4K_ACT_GELU_TANH, ws_ffn)
        q4k.q4k_lmhead_topk_probs(W["lm"], xl, out["logits"], vocab, hid, 5, out["ti"], out["tv"],
                                  out["tp"], out["lse"], ws_lm)
        q4k.q6k_matvec(W["q6"], x6, out["y6"], hid, inter)
        q4k.q4k_ffn_prefill(W["g"], W["u"], W["d"], Xp, out["Yp"], 64, hid, inter,
                            q4k.Q4K_ACT_GELU_TANH, ws_pf)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in out.values():
            v.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            a, b = v.view(torch.int32), eager[k].view(torch.int32)
            assert torch.equal(a, b), (rep, k)
        del junk
