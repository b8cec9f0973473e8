"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes a part of the oracle by an independent fact: the binary16
standard as implemented by numpy, blocks packed from known fields (the encoder
direction of the layout), closed forms of the dequantised dot product, brute
force over single set bits, library routines for the activations and bf16
rounding, analytic moments of the random workload, and invariances of top-k.
"""
import math

import numpy as np
import pytest
import torch

from q4k_fields import Fields, pack_block, pack_scales, pack_quants, f16_bits, pack_q6k_block
from quantized_decode_q4_amd import inputs


# ---------------------------------------------------------------- binary16 ---

def test_f16_decoder_matches_numpy_for_every_bit_pattern(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert math.copysign(1.0, orc.f16_to_f64(0x8000)) == -1.0


def test_f16_decoder_special_values(orc):
    assert orc.f16_to_f64(0x3C00) == 1.0
    assert orc.f16_to_f64(0x0001) == 2.0 ** -24          # smallest subnormal
    assert orc.f16_to_f64(0x03FF) == 1023 * 2.0 ** -24   # largest subnormal
    assert orc.f16_to_f64(0x0400) == 2.0 ** -14          # smallest normal
    assert orc.f16_to_f64(0x7BFF) == 65504.0             # largest finite
    assert orc.f16_to_f64(0x7C00) == math.inf
    assert orc.f16_to_f64(0xFC00) == -math.inf


# ------------------------------------------------------- 6-bit scale field ---

def test_scale_unpack_hand_worked_example(orc):
    # Worked by hand from the layout: sub-blocks 0-3 use the low 6 bits of bytes
    # 0-3 (scales) and 4-7 (mins); 4-7 combine the nibbles of bytes 8-11 with the
    # top two bits of bytes 0-3 (scales) and 4-7 (mins).
    s = [0xC1, 0x02, 0x03, 0x04, 0x45, 0x06, 0x07, 0x08, 0x9A, 0xBC, 0xDE, 0xF0]
    sc, mn = orc.unpack_scales(s)
    # sc4 = 0xA | (0xC1>>6)<<4 = 10 + 48; m4 = 0x9 | (0x45>>6)<<4 = 9 + 16
    assert sc == [1, 2, 3, 4, 58, 12, 14, 0]
    assert mn == [5, 6, 7, 8, 25, 11, 13, 15]


def test_scale_unpack_each_bit_used_exactly_once(orc):
    """Setting one of the 96 bits changes exactly one of the 16 fields by one
    power of two, and the 96 bits map one-to-one onto the 16 x 6 field bits."""
    seen = set()
    for byte in range(12):
        for bit in range(8):
            s = np.zeros(12, np.uint8)
            s[byte] = 1 << bit
            sc, mn = orc.unpack_scales(s)
            vals = sc + mn
            nz = [i for i, v in enumerate(vals) if v]
            assert len(nz) == 1, (byte, bit, vals)
            v = vals[nz[0]]
            assert v & (v - 1) == 0
            seen.add((nz[0], v.bit_length() - 1))
    assert len(seen) == 96


def test_scale_unpack_roundtrip_with_packer(orc):
    rng = np.random.default_rng(1)
    for _ in range(500):
        sc = rng.integers(0, 64, 8)
        mn = rng.integers(0, 64, 8)
        got_sc, got_mn = orc.unpack_scales(pack_scales(sc, mn))
        assert got_sc == sc.tolist() and got_mn == mn.tolist()
    # and the other direction: random bytes -> fields -> identical bytes
    for _ in range(500):
        s = rng.integers(0, 256, 12).astype(np.uint8)
        sc, mn = orc.unpack_scales(s)
        assert np.array_equal(pack_scales(sc, mn), s)


# ----------------------------------------------------------- element order ---

def test_element_order_single_nibble_brute_force(orc):
    """d = 1, every scale 1, dmin = 0: one set nibble gives exactly one weight."""
    base = pack_block(1.0, 0.0, [1] * 8, [0] * 8, np.zeros(256, int))
    seen = set()
    for byte in range(128):
        for hi in (0, 1):
            blk = base.copy()
            blk[16 + byte] = 0x10 if hi else 0x01
            w = orc.dequant_block(blk)
            nz = np.flatnonzero(w)
            assert len(nz) == 1 and w[nz[0]] == 1.0
            g, r = divmod(byte, 32)
            assert nz[0] == 64 * g + r + 32 * hi
            seen.add(int(nz[0]))
    assert seen == set(range(256))


def test_dequant_matches_fields(orc):
    rng = np.random.default_rng(2)
    F = Fields(rng, 6, 1024)
    W = F.to_bytes()
    assert np.array_equal(orc.dequant(W, 6, 1024), F.dense())


def test_sub_block_of_each_element(orc):
    """One sub-block scale set at a time isolates 32 elements."""
    q = np.full(256, 3)
    for s in range(8):
        sc = [0] * 8
        sc[s] = 5
        w = orc.dequant_block(pack_block(0.5, 0.0, sc, [0] * 8, q))
        assert np.array_equal(np.flatnonzero(w), np.arange(32 * s, 32 * s + 32))
        assert np.all(w[32 * s:32 * s + 32] == 0.5 * 5 * 3)
        mn = [0] * 8
        mn[s] = 7
        w = orc.dequant_block(pack_block(0.0, 0.25, [0] * 8, mn, q))
        assert np.array_equal(np.flatnonzero(w), np.arange(32 * s, 32 * s + 32))
        assert np.all(w[32 * s:32 * s + 32] == -0.25 * 7)   # the min is subtracted


def test_dequant_f16_extremes_exact(orc):
    """Subnormal and largest-finite d/dmin: the weight is exact in double."""
    for d_bits, m_bits in [(0x0001, 0x7BFF), (0x7BFF, 0x0001), (0x03FF, 0x0400)]:
        sc = list(range(56, 64))
        mn = list(range(1, 9))
        q = np.arange(256) % 16
        blk = pack_block(np.uint16(d_bits), np.uint16(m_bits), sc, mn, q)
        w = orc.dequant_block(blk)
        d = np.uint16(d_bits).view(np.float16).astype(np.float64)
        m = np.uint16(m_bits).view(np.float16).astype(np.float64)
        for e in range(256):
            s = e // 32
            # exact integer arithmetic in units of 2^-24
            exact = (int(d * 2**24) * sc[s] * int(q[e]) - int(m * 2**24) * mn[s])
            assert w[e] * 2**24 == exact


# ------------------------------------------------------------- closed forms ---

def _sub_block_sums(x, nb):
    return np.asarray(x, np.float64).reshape(nb, 8, 32).sum(axis=2)


def test_closed_form_zero_nibbles(orc):
    """All-zero nibbles: y_i = -sum_b dmin_b sum_s m_bs * (sum of x over s)."""
    rng = np.random.default_rng(3)
    rows, cols = 9, 1280
    F = Fields(rng, rows, cols, q=np.zeros(256, int))
    x = rng.standard_normal(cols).astype(np.float32)
    y, A = orc.matvec(F.to_bytes(), x, rows, cols)
    S = _sub_block_sums(x, cols // 256)
    ref = -(F.dmin.astype(np.float64)[:, :, None] * F.mn * S[None]).sum(axis=(1, 2))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * A.max())


def test_closed_form_d_zero(orc):
    """d = 0: the same min-only expression, whatever the nibbles and scales."""
    rng = np.random.default_rng(4)
    rows, cols = 7, 768
    F = Fields(rng, rows, cols, d=0.0)
    x = rng.standard_normal(cols).astype(np.float32)
    y, A = orc.matvec(F.to_bytes(), x, rows, cols)
    S = _sub_block_sums(x, cols // 256)
    ref = -(F.dmin.astype(np.float64)[:, :, None] * F.mn * S[None]).sum(axis=(1, 2))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * A.max())


def test_closed_form_scale_term_ones(orc):
    """dmin = 0, x = 1: y_i = sum_b d_b sum_s sc_bs * (integer sum of nibbles in s)."""
    rng = np.random.default_rng(5)
    rows, cols = 5, 1024
    F = Fields(rng, rows, cols, dmin=0.0)
    y, _ = orc.matvec(F.to_bytes(), np.ones(cols, np.float32), rows, cols)
    Q = F.q.reshape(rows, cols // 256, 8, 32).sum(axis=3)
    ref = (F.d.astype(np.float64)[:, :, None] * F.sc * Q).sum(axis=(1, 2))
    assert np.array_equal(y, ref) or np.allclose(y, ref, rtol=1e-14, atol=0)


def test_closed_form_saturated_block(orc):
    """All nibbles 15, all scales 63, dmin = 0: y_i = 945 sum_b d_b sum_{j in b} x_j."""
    rng = np.random.default_rng(6)
    rows, cols = 4, 2560
    F = Fields(rng, rows, cols, dmin=0.0, sc=np.full(8, 63), q=np.full(256, 15))
    x = rng.standard_normal(cols).astype(np.float32)
    y, A = orc.matvec(F.to_bytes(), x, rows, cols)
    xb = np.asarray(x, np.float64).reshape(cols // 256, 256).sum(axis=1)
    ref = 945.0 * (F.d.astype(np.float64) * xb[None]).sum(axis=1)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * A.max())


def test_matvec_against_dense_fields_and_tolerance_scale(orc):
    rng = np.random.default_rng(7)
    rows, cols = 33, 1536
    F = Fields(rng, rows, cols)
    x = rng.standard_normal(cols).astype(np.float32)
    y, A = orc.matvec(F.to_bytes(), x, rows, cols)
    Wd = F.dense()
    P = Wd * x.astype(np.float64)[None]
    np.testing.assert_allclose(y, P.sum(axis=1), rtol=0, atol=1e-12 * A.max())
    np.testing.assert_allclose(A, np.abs(P).sum(axis=1), rtol=1e-13)


def test_matvec_linearity(orc):
    rng = np.random.default_rng(8)
    rows, cols = 16, 2560
    W = inputs.q4k_random(rng, rows, cols)
    x1 = rng.standard_normal(cols).astype(np.float32)
    x2 = rng.standard_normal(cols).astype(np.float32)
    a, b = 0.5, -2.0            # powers of two keep a*x1 + b*x2 exact in f32? not
    x3 = (a * x1.astype(np.float64) + b * x2.astype(np.float64))
    y1, A1 = orc.matvec(W, x1, rows, cols)
    y2, A2 = orc.matvec(W, x2, rows, cols)
    y3, _ = orc.matvec_f64(W, x3, rows, cols)
    np.testing.assert_allclose(y3, a * y1 + b * y2, rtol=0, atol=1e-12 * (A1 + 2 * A2).max())


def test_single_hot_x_recovers_columns(orc):
    """x = e_j gives column j of W."""
    W = inputs.tiny_matvec()["W"]
    dense = orc.dequant(W, 256, 512)
    for j in [0, 1, 31, 32, 63, 64, 255, 256, 300, 511]:
        x = np.zeros(512, np.float32)
        x[j] = 1.0
        y, _ = orc.matvec(W, x, 256, 512)
        assert np.array_equal(y, dense[:, j])


def test_random_weight_moments_match_analytic(orc):
    """E[w] = E[d] E[sc] E[q] - E[dmin] E[m] and E[w^2] for the random workload
    (independent fields). A dropped or sign-flipped min term moves the mean by
    ~30 standard errors."""
    W = inputs.q4k_random(np.random.default_rng(9), 4096, 2560)
    w = orc.dequant(W, 4096, 2560).ravel()
    # moments of the binary16-rounded uniform d on [1e-4, 2e-3): integrate over
    # the representable values weighted by their rounding cells
    g = np.random.default_rng(10).uniform(1e-4, 2e-3, 2_000_000).astype(np.float16).astype(np.float64)
    Ed, Ed2 = g.mean(), (g * g).mean()
    Esc, Esc2 = 31.5, (63 * 64 * 127 / 6) / 64
    Eq, Eq2 = 7.5, (15 * 16 * 31 / 6) / 16
    mean = Ed * Esc * Eq - Ed * Esc
    # E[w^2] = E[d^2]E[sc^2]E[q^2] - 2 E[d]^2 E[sc]E[q]E[m] + E[dmin^2]E[m^2]
    # (d, dmin independent; sc and m independent within a sub-block)
    second = Ed2 * Esc2 * Eq2 - 2 * Ed * Ed * Esc * Eq * Esc + Ed2 * Esc2
    n = w.size
    # weights within a block share d and dmin: use the number of blocks as the
    # (conservative) effective sample count for the standard error
    se = math.sqrt(second - mean * mean) / math.sqrt(n / 256)
    assert abs(w.mean() - mean) < 5 * se
    assert abs((w * w).mean() - second) / second < 0.02
    assert abs(mean - 0.2149) < 0.002


# ------------------------------------------------------------- activations ---

def test_gelu_tanh_matches_torch_f64(orc):
    z = np.linspace(-12, 12, 4001)
    ref = torch.nn.functional.gelu(torch.tensor(z, dtype=torch.float64), approximate="tanh").numpy()
    got = orc.act_array(z, orc.GELU_TANH)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)


def test_silu_matches_torch_f64(orc):
    z = np.linspace(-40, 40, 4001)
    ref = torch.nn.functional.silu(torch.tensor(z, dtype=torch.float64)).numpy()
    got = orc.act_array(z, orc.SILU)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-300)


def test_activation_identities(orc):
    for f in (orc.gelu_tanh, orc.silu):
        assert f(0.0) == 0.0
        for z in [0.1, 0.7, 1.5, 3.0, 9.0]:
            assert abs(f(-z) - (f(z) - z)) < 1e-14 * max(1, z)
        assert abs(f(30.0) - 30.0) < 1e-9
        assert abs(f(-30.0)) < 1e-9
    # tanh form stays within 1e-3 of the erf form of GELU
    for z in np.linspace(-6, 6, 241):
        erf_gelu = 0.5 * z * (1 + math.erf(z / math.sqrt(2)))
        assert abs(orc.gelu_tanh(z) - erf_gelu) < 1e-3
    # known value: 0.5 (1 + tanh(sqrt(2/pi) * 1.044715)) at z = 1
    assert abs(orc.gelu_tanh(1.0) - 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715))) < 1e-15


# -------------------------------------------------------------------- FFN ---

def test_ffn_is_gate_activation_times_up_then_down(orc):
    rng = np.random.default_rng(11)
    hidden, inter = 512, 768
    Wg = inputs.q4k_random(rng, inter, hidden)
    Wu = inputs.q4k_random(rng, inter, hidden)
    Wd = inputs.q4k_random(rng, hidden, inter)
    x = rng.standard_normal(hidden).astype(np.float32)
    for act in (orc.GELU_TANH, orc.SILU):
        r = orc.ffn(Wg, Wu, Wd, x, hidden, inter, act)
        g, _ = orc.matvec(Wg, x, inter, hidden)
        u, _ = orc.matvec(Wu, x, inter, hidden)
        tg = torch.tensor(g, dtype=torch.float64)
        a = (torch.nn.functional.gelu(tg, approximate="tanh") if act == orc.GELU_TANH
             else torch.nn.functional.silu(tg)).numpy()
        h = a * u
        np.testing.assert_allclose(r["h"], h, rtol=1e-13, atol=1e-13 * np.abs(h).max())
        # down projection against the dense dequantised Wd
        dense = orc.dequant(Wd, hidden, inter)
        np.testing.assert_allclose(r["y"], dense @ h, rtol=0, atol=1e-11 * r["A"].max())
        # the gate carries the activation: swapping gate and up changes h
        swapped = orc.ffn(Wu, Wg, Wd, x, hidden, inter, act)
        assert not np.allclose(swapped["h"], r["h"])


# ------------------------------------------------------------------- top-k ---

def _brute_topk(v, k):
    v = np.asarray(v, np.float64)
    key = np.where(np.isnan(v), np.inf, -v)        # NaN last
    order = np.lexsort((np.arange(v.size), key))   # primary -v, then index
    return order[:k]


def test_topk_matches_brute_force_sort(orc):
    rng = np.random.default_rng(12)
    for n, k in [(1, 1), (10, 3), (1000, 64), (262144, 5)]:
        v = rng.standard_normal(n)
        idx, val = orc.topk(v, k)
        ref = _brute_topk(v, k)
        assert np.array_equal(idx, ref)
        assert np.array_equal(val, v[ref])


def test_topk_tie_break_and_nan(orc):
    v = np.array([1.0, 3.0, 3.0, np.nan, 2.0, 3.0, -np.inf, np.nan])
    idx, val = orc.topk(v, 8)
    assert idx.tolist() == [1, 2, 5, 4, 0, 6, 3, 7]
    idx, _ = orc.topk(np.array([np.nan, 0.0, np.nan]), 2)
    assert idx.tolist() == [1, 0]


def test_topk_row_permutation_invariance(orc):
    """Permuting whole row records permutes logits: the top-k values are kept
    and the indices map through the permutation."""
    rng = np.random.default_rng(13)
    rows, cols = 3000, 512
    W = inputs.q4k_random(rng, rows, cols)
    x = rng.standard_normal(cols).astype(np.float32)
    perm = rng.permutation(rows)
    y, _ = orc.matvec(W, x, rows, cols)
    yp, _ = orc.matvec(W[perm], x, rows, cols)
    assert np.array_equal(yp, y[perm])
    i1, v1 = orc.topk(y, 16)
    i2, v2 = orc.topk(yp, 16)
    assert np.array_equal(v1, v2)
    assert np.array_equal(perm[i2], i1)


def test_topk_duplicated_rows_lower_index_first(orc):
    rng = np.random.default_rng(14)
    rows, cols = 200, 256
    W = inputs.q4k_random(rng, rows, cols)
    x = rng.standard_normal(cols).astype(np.float32)
    y, _ = orc.matvec(W, x, rows, cols)
    best = int(np.argmax(y))
    W2 = W.copy()
    W2[150] = W[best]
    W2[37] = W[best]
    y2, _ = orc.matvec(W2, x, rows, cols)
    idx, _ = orc.topk(y2, 3)
    assert idx.tolist()[:3] == sorted({best, 37, 150})[:3]


# --------------------------------------------------------------------- Q6_K ---

def test_q6k_block_round_trip_from_fields(orc):
    """Blocks packed from random fields decode to d * scale[e // 16] * (q - 32)."""
    rng = np.random.default_rng(51)
    for _ in range(20):
        q = rng.integers(0, 64, 256)
        sc = rng.integers(-128, 128, 16)
        d = float(np.float16(rng.uniform(1e-4, 2e-3)))
        w = orc.q6k_dequant_block(pack_q6k_block(d, sc, q))
        want = np.array([d * sc[e // 16] * (q[e] - 32) for e in range(256)], np.float64)
        assert np.array_equal(w, want)


def test_q6k_every_quant_bit_moves_exactly_one_weight(orc):
    """From the all-zero-weight block (every q = 32, scales 1, d = 1), each of
    the 1536 quant bits (bytes 0-191) changes exactly one weight, by a power of
    two, and together they cover each of the 256 weights' six bits once."""
    base = pack_q6k_block(1.0, np.ones(16, int), np.full(256, 32))
    assert np.all(orc.q6k_dequant_block(base) == 0)
    hits = {}
    for byte in range(192):
        for bit in range(8):
            blk = base.copy()
            blk[byte] ^= 1 << bit
            w = orc.q6k_dequant_block(blk)
            nz = np.flatnonzero(w)
            assert nz.size == 1, (byte, bit)
            e = int(nz[0])
            mag = abs(w[e])
            assert mag in (1, 2, 4, 8, 16, 32), (byte, bit, mag)
            hits.setdefault(e, []).append(int(mag))
    assert sorted(hits) == list(range(256))
    assert all(sorted(v) == [1, 2, 4, 8, 16, 32] for v in hits.values())


def test_q6k_scales_are_signed_and_cover_16_consecutive_weights(orc):
    rng = np.random.default_rng(52)
    q = rng.integers(0, 64, 256)
    sc = np.ones(16, int)
    w0 = orc.q6k_dequant_block(pack_q6k_block(1.0, sc, q))
    for s in range(16):
        for v in (-128, -1, 5, 127):
            sc2 = sc.copy()
            sc2[s] = v
            w = orc.q6k_dequant_block(pack_q6k_block(1.0, sc2, q))
            changed = np.flatnonzero(w != w0)
            assert set(changed.tolist()) <= set(range(16 * s, 16 * s + 16))
            assert np.array_equal(w[16 * s:16 * s + 16], v * w0[16 * s:16 * s + 16])
    blk = pack_q6k_block(1.0, sc, q)
    blk[192] = 0x80          # int8 -128
    assert np.array_equal(orc.q6k_dequant_block(blk)[:16], -128 * w0[:16])


def test_q6k_d_is_the_last_two_bytes(orc):
    q = np.arange(256) % 64
    sc = np.arange(16) - 8
    blk = pack_q6k_block(0.5, sc, q)
    w = orc.q6k_dequant_block(blk)
    blk2 = blk.copy()
    blk2[208:210] = np.array([f16_bits(-2.0) & 0xFF, f16_bits(-2.0) >> 8], np.uint8)
    assert np.array_equal(orc.q6k_dequant_block(blk2), -4.0 * w)
    # binary16 subnormal d
    blk2[208:210] = np.array([0x01, 0x00], np.uint8)
    assert np.array_equal(orc.q6k_dequant_block(blk2), w * (2.0 ** -24) / 0.5)


def test_q6k_closed_forms(orc):
    rows, cols = 3, 512
    nb = cols // 256
    x1 = np.ones(cols, np.float32)
    # q = 32 everywhere: zero
    W = np.stack([np.concatenate([pack_q6k_block(1e-3, np.full(16, 77), np.full(256, 32))
                                  for _ in range(nb)]) for _ in range(rows)])
    y, A = orc.q6k_matvec(W, x1, rows, cols)
    assert np.all(y == 0) and np.all(A == 0)
    # q = 63, scales 127, d = 1: every weight 127 * 31; sum of x = cols
    W = np.stack([np.concatenate([pack_q6k_block(1.0, np.full(16, 127), np.full(256, 63))
                                  for _ in range(nb)]) for _ in range(rows)])
    y, A = orc.q6k_matvec(W, x1, rows, cols)
    assert np.all(y == 127 * 31 * cols) and np.all(A == y)
    # q = 0, scales -128: every weight (-128)(-32) = 4096
    W = np.stack([np.concatenate([pack_q6k_block(0.25, np.full(16, -128), np.zeros(256, int))
                                  for _ in range(nb)]) for _ in range(rows)])
    x = np.random.default_rng(53).standard_normal(cols).astype(np.float32)
    y, _ = orc.q6k_matvec(W, x, rows, cols)
    assert np.allclose(y, 0.25 * 4096 * math.fsum(x.astype(np.float64)), rtol=1e-13, atol=1e-9)


def test_q6k_matvec_one_hot_columns_and_linearity(orc):
    rng = np.random.default_rng(54)
    rows, cols = 40, 768
    W = inputs.q6k_random(rng, rows, cols)
    dense = orc.q6k_dequant(W, rows, cols)
    for j in rng.choice(cols, 12, replace=False):
        x = np.zeros(cols, np.float32)
        x[j] = 1.0
        y, A = orc.q6k_matvec(W, x, rows, cols)
        assert np.array_equal(y, dense[:, j]) and np.array_equal(A, np.abs(dense[:, j]))
    x1 = rng.standard_normal(cols).astype(np.float32)
    x2 = rng.standard_normal(cols).astype(np.float32)
    y1, _ = orc.q6k_matvec(W, x1, rows, cols)
    y2, _ = orc.q6k_matvec(W, x2, rows, cols)
    y12, _ = orc.q6k_matvec(W, (x1 + x2).astype(np.float32), rows, cols)
    x12 = (x1 + x2).astype(np.float32).astype(np.float64)
    assert np.allclose(y12, dense @ x12, rtol=1e-12, atol=1e-9)
    assert np.allclose(y1 + y2, dense @ (x1.astype(np.float64) + x2), rtol=1e-12, atol=1e-9)


def test_q6k_random_weight_moments(orc):
    """Uniform bytes make q and the int8 scales uniform: E[q - 32] = -1/2,
    E[scale] = -1/2, so E[w] = E[d] / 4, and E[w^2] = E[d^2] E[s^2] E[(q-32)^2]
    with E[s^2] = 5461.5 and E[(q-32)^2] = 341.5."""
    rng = np.random.default_rng(55)
    rows, cols = 400, 2560
    W = inputs.q6k_random(rng, rows, cols)
    w = orc.q6k_dequant(W, rows, cols)
    lo, hi = 1e-4, 2e-3
    Ed, Ed2 = (lo + hi) / 2, (hi ** 3 - lo ** 3) / (3 * (hi - lo))
    m1, m2 = w.mean(), (w ** 2).mean()
    assert abs(m1 - Ed / 4) < 4 * math.sqrt(m2 / w.size) * 16    # blocks share d and scales
    assert m2 == pytest.approx(Ed2 * 5461.5 * 341.5, rel=0.03)


# ------------------------------------------------------------------ RMSNorm ---

def test_residual_add_is_one_f32_addition(orc):
    rng = np.random.default_rng(71)
    h = (rng.standard_normal(4096) * 100).astype(np.float32)
    d = (rng.standard_normal(4096) * 1e-3).astype(np.float32)
    h[:4] = [1.0, -1.0, 3e38, 1e-30]
    d[:4] = [2.0 ** -30, 2.0 ** -25, 3e38, -1e-30]
    s, _ = orc.residual_rmsnorm(h, d, np.ones(4096, np.float32), 1e-6)
    with np.errstate(over="ignore"):
        want = h + d      # numpy: IEEE single addition, round to nearest even (3e38 + 3e38 = inf)
    assert np.array_equal(s.view(np.uint32), want.view(np.uint32))
    s0, x0 = orc.residual_rmsnorm(h, None, np.ones(4096, np.float32), 1e-6)
    s1, x1 = orc.residual_rmsnorm(h, np.zeros(4096, np.float32), np.ones(4096, np.float32), 1e-6)
    assert np.array_equal(s0, h) and np.array_equal(x0, x1)


def test_rmsnorm_unit_weight_has_unit_rms(orc):
    rng = np.random.default_rng(72)
    for n in (256, 2560, 10240):
        h = (rng.standard_normal(n) * 7.5).astype(np.float32)
        _, x = orc.residual_rmsnorm(h, None, np.ones(n, np.float32), 0.0)
        assert math.fsum(x * x) / n == pytest.approx(1.0, abs=1e-12)   # f64 sum over n terms
        assert np.all(np.sign(x) == np.sign(h))


def test_rmsnorm_scale_invariance_and_weights(orc):
    """eps = 0: multiplying s by a power of two (exact in f32) leaves x
    unchanged, -1 flips it, and the weight multiplies element by element."""
    rng = np.random.default_rng(73)
    n = 2560
    h = rng.standard_normal(n).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
    _, x = orc.residual_rmsnorm(h, None, w, 0.0)
    for c in (2.0 ** 20, 2.0 ** -20, -1.0):
        _, xc = orc.residual_rmsnorm((h * np.float32(c)).astype(np.float32), None, w, 0.0)
        assert np.allclose(xc, np.sign(c) * x, rtol=1e-14, atol=0)
    _, x1 = orc.residual_rmsnorm(h, None, np.ones(n, np.float32), 0.0)
    assert np.allclose(x, x1 * w.astype(np.float64), rtol=1e-15, atol=0)


def test_rmsnorm_closed_forms(orc):
    n = 1000
    w = np.linspace(0.5, 1.5, n).astype(np.float32)
    # constant vector c: x_j = w_j c / sqrt(c^2 + eps)
    for c, eps in [(3.0, 0.0), (-0.25, 1e-6), (1e-3, 1e-6)]:
        _, x = orc.residual_rmsnorm(np.full(n, c, np.float32), None, w, eps)
        cf = float(np.float32(c))
        want = w.astype(np.float64) * cf / math.sqrt(cf * cf + float(np.float32(eps)))
        assert np.allclose(x, want, rtol=1e-14, atol=0)
    # one nonzero element a at k, eps = 0: x_k = sign(a) sqrt(n) w_k, others 0
    h = np.zeros(n, np.float32)
    h[123] = -7.0
    _, x = orc.residual_rmsnorm(h, None, w, 0.0)
    assert x[123] == pytest.approx(-math.sqrt(n) * float(w[123]), rel=1e-15)
    assert np.count_nonzero(x) == 1
    # zero input with eps > 0 stays zero
    _, x = orc.residual_rmsnorm(np.zeros(n, np.float32), None, w, 1e-6)
    assert np.all(x == 0)


def test_rmsnorm_then_matvec_one_hot(orc):
    """A one-element residual normalises to sqrt(n) e_k (eps = 0, w = 1), so the
    following matvec reads sqrt(n) times column k of the weights."""
    rng = np.random.default_rng(74)
    rows, cols = 64, 512
    W = inputs.q4k_random(rng, rows, cols)
    h = np.zeros(cols, np.float32)
    h[300] = 0.5
    _, x = orc.residual_rmsnorm(h, None, np.ones(cols, np.float32), 0.0)
    y, _ = orc.matvec_f64(W, x, rows, cols)
    col = orc.dequant(W, rows, cols)[:, 300]
    assert np.allclose(y, math.sqrt(cols) * col, rtol=1e-14, atol=1e-300)


def test_ffn_f64_matches_ffn_on_f32_inputs(orc):
    rng = np.random.default_rng(75)
    hidden, inter = 256, 512
    Wg = inputs.q4k_random(rng, inter, hidden)
    Wu = inputs.q4k_random(rng, inter, hidden)
    Wd = inputs.q4k_random(rng, hidden, inter)
    x = rng.standard_normal(hidden).astype(np.float32)
    a = orc.ffn(Wg, Wu, Wd, x, hidden, inter, 0)
    b = orc.ffn_f64(Wg, Wu, Wd, x.astype(np.float64), hidden, inter, 0)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["A"], b["A"])


# ------------------------------------------------------------------ softmax ---

def test_softmax_two_values_is_the_logistic_function(orc):
    """Two classes: p_0 = 1 / (1 + e^(v1 - v0)), lse = v0 + log(1 + e^(v1 - v0))."""
    for v0, v1 in [(0.0, 0.0), (1.5, -0.25), (-3.0, 2.0), (10.0, 10.5)]:
        p = orc.softmax([v0, v1])
        assert p[0] == pytest.approx(1.0 / (1.0 + math.exp(v1 - v0)), rel=1e-15)
        assert p[1] == pytest.approx(1.0 / (1.0 + math.exp(v0 - v1)), rel=1e-15)
        assert orc.logsumexp([v0, v1]) == pytest.approx(v0 + math.log1p(math.exp(v1 - v0)),
                                                        rel=1e-15, abs=1e-15)


def test_softmax_equal_values_are_uniform(orc):
    for n in (1, 3, 262144):
        v = np.full(n, -1.75)
        p = orc.softmax(v)
        assert np.allclose(p, 1.0 / n, rtol=1e-12, atol=0)
        assert orc.logsumexp(v) == pytest.approx(-1.75 + math.log(n), rel=1e-14)


def test_logsumexp_brute_force_on_small_inputs(orc):
    """Without the max shift: log of the exactly rounded sum of exponentials."""
    rng = np.random.default_rng(41)
    for n in (1, 2, 5, 17, 100):
        v = rng.uniform(-5, 5, n)
        want = math.log(math.fsum(math.exp(t) for t in v))
        assert orc.logsumexp(v) == pytest.approx(want, rel=1e-14, abs=1e-14)
        p = orc.softmax(v)
        assert np.allclose(p, [math.exp(t - want) for t in v], rtol=1e-13, atol=0)


def test_softmax_sums_to_one_and_keeps_the_order(orc):
    rng = np.random.default_rng(42)
    v = rng.standard_normal(100000) * 4.0
    p = orc.softmax(v)
    assert math.fsum(p) == pytest.approx(1.0, abs=1e-12)
    order = np.argsort(v, kind="stable")
    assert np.all(np.diff(p[order]) >= 0)
    assert np.all(p > 0)


def test_softmax_shift_invariance_and_large_magnitudes(orc):
    """softmax(v + c) = softmax(v) and lse(v + c) = lse(v) + c, also where
    e^v alone overflows (v ~ 1000) or underflows (v ~ -1000)."""
    v = np.array([0.0, 1.0, -1.0, 0.5])
    p0 = orc.softmax(v)
    lse0 = orc.logsumexp(v)
    for c in (1000.0, -1000.0, 700.25):
        p = orc.softmax(v + c)
        assert np.all(np.isfinite(p))
        assert np.allclose(p, p0, rtol=1e-12, atol=0)
        assert orc.logsumexp(v + c) == pytest.approx(lse0 + c, rel=1e-14)
    assert p0[1] == pytest.approx(math.e / (1 + math.e + 1 / math.e + math.exp(0.5)), rel=1e-15)


def test_softmax_nan_poisons_everything(orc):
    v = np.array([1.0, np.nan, 2.0])
    assert math.isnan(orc.logsumexp(v))
    assert np.all(np.isnan(orc.softmax(v)))


def test_softmax_of_logits_is_shift_invariant_through_the_weights(orc):
    """A row's dmin term m*dmin*sum(x) over a sub-block is a shift: with all
    quants zero and the same dmin/min fields in every row, every logit is the
    same number, so the probabilities are uniform."""
    rows, cols = 7, 256
    blk = pack_block(0.5, 0.25, [1] * 8, [3, 1, 4, 1, 5, 9, 2, 6], [0] * 256)
    W = np.stack([blk] * rows)
    x = np.random.default_rng(43).standard_normal(cols).astype(np.float32)
    y, _ = orc.matvec(W, x, rows, cols)
    assert np.all(y == y[0]) and y[0] != 0
    assert np.allclose(orc.softmax(y), 1.0 / rows, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- prefill ---

def test_matmul_rows_equal_matvec(orc):
    rng = np.random.default_rng(15)
    rows, cols, seq = 40, 512, 5
    W = inputs.q4k_random(rng, rows, cols)
    X = rng.standard_normal((seq, cols)).astype(np.float32)
    Y, A = orc.matmul(W, X, rows, cols)
    for t in range(seq):
        y, a = orc.matvec(W, X[t], rows, cols)
        assert np.array_equal(Y[t], y) and np.array_equal(A[t], a)


def test_ffn_prefill_rows_equal_decode_ffn(orc):
    rng = np.random.default_rng(16)
    hidden, inter, seq = 256, 512, 3
    Wg = inputs.q4k_random(rng, inter, hidden)
    Wu = inputs.q4k_random(rng, inter, hidden)
    Wd = inputs.q4k_random(rng, hidden, inter)
    X = rng.standard_normal((seq, hidden)).astype(np.float32)
    Y, A = orc.ffn_prefill(Wg, Wu, Wd, X, hidden, inter)
    for t in range(seq):
        r = orc.ffn(Wg, Wu, Wd, X[t], hidden, inter)
        assert np.array_equal(Y[t], r["y"]) and np.array_equal(A[t], r["A"])


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(17)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.4e38, 1e-40], np.float32)])
    ref = torch.tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.round_bf16(float(t)) for t in v])
    assert np.array_equal(got, ref)


def test_bf16_prefill_model_close_to_exact(orc):
    """The bf16 operand model differs from the exact prefill by bf16-sized
    relative error, far inside the 1e-2 A bound; with the rounding removed
    (all operands already bf16-exact) it would coincide."""
    rng = np.random.default_rng(18)
    hidden, inter, seq = 256, 512, 2
    Wg = inputs.q4k_random(rng, inter, hidden)
    Wu = inputs.q4k_random(rng, inter, hidden)
    Wd = inputs.q4k_random(rng, hidden, inter)
    X = rng.standard_normal((seq, hidden)).astype(np.float32)
    Y, A = orc.ffn_prefill(Wg, Wu, Wd, X, hidden, inter)
    Yb, _ = orc.ffn_prefill_bf16(Wg, Wu, Wd, X, hidden, inter)
    err = np.abs(Yb - Y) / A
    assert err.max() < 1e-2
    assert err.max() > 1e-7    # the rounding is really applied


def test_bf16_matmul_model_exact_on_bf16_operands(orc):
    """With every weight and activation already bf16-exact (d a power of two,
    dmin 0, scale*quant below 256; activations k/8), the bf16 operand model and
    the exact product coincide bit for bit."""
    rng = np.random.default_rng(19)
    rows, cols, seq = 12, 512, 3
    blocks = []
    for _ in range(rows * cols // 256):
        sc = rng.integers(0, 16, 8)
        q = rng.integers(0, 16, 256)
        blocks.append(pack_block(2.0 ** -10, 0.0, sc, np.zeros(8, int), q))
    W = np.concatenate(blocks).reshape(rows, -1)
    X = (rng.integers(-64, 65, (seq, cols)) / 8.0).astype(np.float32)
    Y, A = orc.matmul(W, X, rows, cols)
    Yb, Ab = orc.matmul_bf16(W, X, rows, cols)
    assert np.array_equal(Y, Yb) and np.array_equal(A, Ab)


def test_bf16_matmul_model_within_rounding_bound(orc):
    """Each bf16 operand carries relative error <= 2^-9 (the weight after its
    binary32 rounding), so every product is off by at most 2^-8 + 2^-17 of its
    magnitude and |Y_bf16 - Y| <= (2^-8 + 2^-17) A."""
    rng = np.random.default_rng(20)
    rows, cols, seq = 50, 1024, 4
    W = inputs.q4k_random(rng, rows, cols)
    X = rng.standard_normal((seq, cols)).astype(np.float32)
    Y, A = orc.matmul(W, X, rows, cols)
    Yb, _ = orc.matmul_bf16(W, X, rows, cols)
    err = np.abs(Yb - Y) / A
    assert err.max() <= 2.0 ** -8 + 2.0 ** -17
    assert err.max() > 1e-6


def _torch_bf16(a):
    """binary64 -> binary32 -> bfloat16 -> binary64, each cast by torch."""
    t = torch.from_numpy(np.asarray(a, dtype=np.float64))
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def _bf16_exact_fields(rng, rows, cols):
    """Fields whose every weight is bf16-exact: d = 2^-10, dmin = 0 and
    sc * q <= 15 * 15 < 2^8 (eight significant bits at most)."""
    nb = cols // 256
    return Fields(rng, rows, cols, d=np.float16(2.0 ** -10), dmin=np.float16(0.0),
                  sc=rng.integers(0, 16, (rows, nb, 8)), mn=np.zeros((rows, nb, 8), np.int64))


def test_bf16_matmul_model_rounds_weights_via_binary32_and_x_to_nearest_even(orc):
    """One-hot bf16-exact activations read back single weights: each must be
    the field value cast f64 -> f32 -> bf16 by torch. Then bf16-exact weights
    times arbitrary f32 activations must equal W times X cast to bf16 by torch."""
    rng = np.random.default_rng(23)
    rows, cols = 16, 512
    F = Fields(rng, rows, cols)
    W = F.to_bytes()
    wref = _torch_bf16(F.dense())                              # rows x cols
    X = np.eye(cols, dtype=np.float32)[::7]                    # one-hot rows, bf16-exact
    Yb, _ = orc.matmul_bf16(W, X, rows, cols)
    assert np.array_equal(Yb, wref[:, ::7].T)
    # the weights above really are rounded (not all bf16-exact already)
    assert not np.array_equal(wref, F.dense())

    G = _bf16_exact_fields(rng, rows, cols)
    Xf = rng.standard_normal((3, cols)).astype(np.float32)
    Yb, _ = orc.matmul_bf16(G.to_bytes(), Xf, rows, cols)
    ref = _torch_bf16(Xf.astype(np.float64)) @ G.dense().T
    A = np.abs(_torch_bf16(Xf.astype(np.float64))) @ np.abs(G.dense()).T
    assert np.all(np.abs(Yb - ref) <= 1e-13 * A)


@pytest.mark.parametrize("act", [0, 1])
def test_bf16_ffn_model_rounds_h_once_after_the_activation(orc, act):
    """Composition of the bf16 FFN model, pinned from outside the oracle.
    Every weight and activation is bf16-exact, so G and U are exact sums
    (multiples of 2^-13 far below 2^40) and the only rounding left is that of
    H = act(G) * U. Expected: the field-level dense weights, torch's f64
    activation, torch's bf16 cast of H, and a numpy f64 product. A model that
    skips the rounding of H, or rounds G and U instead of H, misses by orders
    of magnitude more than the summation-order tolerance used here."""
    rng = np.random.default_rng(24 + act)
    hidden, inter, seq = 512, 768, 3
    Fg = _bf16_exact_fields(rng, inter, hidden)
    Fu = _bf16_exact_fields(rng, inter, hidden)
    Fd = _bf16_exact_fields(rng, hidden, inter)
    X = (rng.integers(-64, 65, (seq, hidden)) / 8.0).astype(np.float32)   # bf16-exact
    Yb, _ = orc.ffn_prefill_bf16(Fg.to_bytes(), Fu.to_bytes(), Fd.to_bytes(), X, hidden, inter,
                                 act)

    xg = X.astype(np.float64)
    G = xg @ Fg.dense().T
    U = xg @ Fu.dense().T
    tg = torch.from_numpy(G)
    a = (torch.nn.functional.gelu(tg, approximate="tanh") if act == 0
         else torch.nn.functional.silu(tg)).numpy()
    Wd = Fd.dense()

    def down(h):
        return h @ Wd.T, np.abs(h) @ np.abs(Wd).T

    Y_ref, A_ref = down(_torch_bf16(a * U))
    tol = 1e-12 * A_ref
    assert np.all(np.abs(Yb - Y_ref) <= tol)

    # the pin discriminates: each plausible slip would fail it
    Y_noround, _ = down(a * U)
    tgu = torch.from_numpy(_torch_bf16(G))
    a_r = (torch.nn.functional.gelu(tgu, approximate="tanh") if act == 0
           else torch.nn.functional.silu(tgu)).numpy()
    Y_gu, _ = down(a_r * _torch_bf16(U))
    for wrong in (Y_noround, Y_gu):
        assert np.max(np.abs(wrong - Y_ref) / tol) > 1e3


@pytest.mark.parametrize("act", [0, 1])
def test_activation_derivative_matches_finite_differences(orc, act):
    f = orc.gelu_tanh if act == 0 else orc.silu
    hstep = 1e-5
    for z in np.linspace(-8.0, 8.0, 161):
        fd = (f(z + hstep) - f(z - hstep)) / (2 * hstep)
        assert abs(orc.act_deriv(z, act) - fd) < 1e-8, (z, act)
    assert orc.act_deriv(0.0, act) == 0.5          # both: f'(0) = 1/2


@pytest.mark.parametrize("act", [0, 1])
def test_ffn_error_scale_bounds_input_perturbations(orc, act):
    """Relative perturbations of X of at most e move y by at most e * Ap (to
    first order), and Ap is never below the last stage's plain A."""
    rng = np.random.default_rng(21 + act)
    hidden, inter, seq = 256, 512, 3
    Wg = inputs.q4k_random(rng, inter, hidden)
    Wu = inputs.q4k_random(rng, inter, hidden)
    Wd = inputs.q4k_random(rng, hidden, inter)
    X = rng.standard_normal((seq, hidden)).astype(np.float32)
    Y, A = orc.ffn_prefill(Wg, Wu, Wd, X, hidden, inter, act)
    Ap = orc.ffn_prefill_scale(Wg, Wu, Wd, X, hidden, inter, act)
    assert np.all(Ap >= A)
    e = 1e-4
    worst = 0.0
    for _ in range(6):
        Xp = (X.astype(np.float64) * (1 + rng.uniform(-e, e, X.shape))).astype(np.float32)
        Yp, _ = orc.ffn_prefill(Wg, Wu, Wd, Xp, hidden, inter, act)
        worst = max(worst, float((np.abs(Yp - Y) / (e * Ap)).max()))
    assert worst <= 1.0, worst
    assert worst > 1e-3                                # the scale is not vacuous


def test_generator_is_deterministic_and_layout_sized():
    a = inputs.tiny_matvec()
    b = inputs.tiny_matvec()
    assert np.array_equal(a["W"], b["W"]) and np.array_equal(a["x"], b["x"])
    assert a["W"].shape == (256, 2 * 144) and a["x"].dtype == np.float32
    d = a["W"].reshape(256, 2, 144)[:, :, 0:2].copy().view("<f2").astype(np.float64)
    assert d.min() >= 1e-4 * (1 - 2**-10) and d.max() <= 2e-3 * (1 + 2**-10)
    q = inputs.qkv()
    assert q["W"].shape == (4096, 1440)
    assert not np.array_equal(inputs.ffn_layer(0)["x"], inputs.ffn_layer(1)["x"])
