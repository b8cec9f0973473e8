"""CPU oracle for the Q4_K decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``q4k_oracle.c`` (plain C, f64,
single-threaded) through ctypes and shares no code with the HIP library.

Parity-unpinned parts: correspondence of the byte layouts to Q4_K and Q6_K
files written by other tools (no such file or decoder exists in this environment; the layout
is pinned by round-trip, single-bit and closed-form tests instead).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "q4k_oracle.c")

GELU_TANH = 0
SILU = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math: IEEE semantics kept)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-D_GNU_SOURCE",
                        "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
                        SRC_PATH, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.q4o_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.q4o_f16_to_f64.restype = ctypes.c_double
        L.q4o_unpack_scales.argtypes = [P, P, P]
        L.q4o_dequant_block.argtypes = [P, P]
        L.q4o_dequant.argtypes = [P, I64, I64, P]
        L.q4o_matvec.argtypes = [P, P, I64, I64, P, P]
        L.q4o_matvec_f64.argtypes = [P, P, I64, I64, P, P]
        L.q4o_gelu_tanh.argtypes = [ctypes.c_double]
        L.q4o_gelu_tanh.restype = ctypes.c_double
        L.q4o_silu.argtypes = [ctypes.c_double]
        L.q4o_silu.restype = ctypes.c_double
        L.q4o_act_array.argtypes = [P, I64, ctypes.c_int, P]
        L.q4o_ffn.argtypes = [P, P, P, P, I64, I64, ctypes.c_int, P, P, P, P, P]
        L.q4o_topk.argtypes = [P, I64, ctypes.c_int, P, P]
        L.q4o_ffn_f64.argtypes = [P, P, P, P, I64, I64, ctypes.c_int, P, P, P, P, P]
        L.q4o_residual_rmsnorm.argtypes = [P, P, P, ctypes.c_float, I64, P, P]
        L.q6o_dequant_block.argtypes = [P, P]
        L.q6o_dequant.argtypes = [P, I64, I64, P]
        L.q6o_matvec.argtypes = [P, P, I64, I64, P, P]
        L.q4o_logsumexp.argtypes = [P, I64]
        L.q4o_logsumexp.restype = ctypes.c_double
        L.q4o_softmax.argtypes = [P, I64, P]
        L.q4o_matmul.argtypes = [P, P, I64, I64, I64, P, P]
        L.q4o_ffn_prefill.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_int, P, P]
        L.q4o_ffn_prefill_bf16.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_int, P, P]
        L.q4o_matmul_bf16.argtypes = [P, P, I64, I64, I64, P, P]
        L.q4o_act_deriv.argtypes = [ctypes.c_double, ctypes.c_int]
        L.q4o_act_deriv.restype = ctypes.c_double
        L.q4o_ffn_prefill_scale.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_int, P]
        L.q4o_round_bf16.argtypes = [ctypes.c_double]
        L.q4o_round_bf16.restype = ctypes.c_double
        _lib = L
    return _lib


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint8)
    return a


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_w(W: np.ndarray, rows: int, cols: int) -> None:
    if cols <= 0 or cols % 256:
        raise ValueError("cols must be a positive multiple of 256")
    if W.size != rows * (cols // 256) * 144:
        raise ValueError(f"W has {W.size} bytes, expected {rows * (cols // 256) * 144}")


def f16_to_f64(h: int) -> float:
    return lib().q4o_f16_to_f64(int(h) & 0xFFFF)


def unpack_scales(s12) -> tuple[list[int], list[int]]:
    s = _u8(s12)
    assert s.size == 12
    sc = np.zeros(8, np.int32)
    mn = np.zeros(8, np.int32)
    lib().q4o_unpack_scales(_ptr(s), _ptr(sc), _ptr(mn))
    return sc.tolist(), mn.tolist()


def dequant_block(blk) -> np.ndarray:
    b = _u8(blk)
    assert b.size == 144
    out = np.zeros(256, np.float64)
    lib().q4o_dequant_block(_ptr(b), _ptr(out))
    return out


def dequant(W, rows: int, cols: int) -> np.ndarray:
    W = _u8(W)
    _check_w(W, rows, cols)
    out = np.zeros((rows, cols), np.float64)
    lib().q4o_dequant(_ptr(W), rows, cols, _ptr(out))
    return out


def matvec(W, x, rows: int, cols: int):
    """(y, A): y = W x in f64, A = sum_j |w_ij x_j|."""
    W = _u8(W)
    _check_w(W, rows, cols)
    x = _f32(x)
    assert x.size == cols
    y = np.zeros(rows, np.float64)
    A = np.zeros(rows, np.float64)
    lib().q4o_matvec(_ptr(W), _ptr(x), rows, cols, _ptr(y), _ptr(A))
    return y, A


def matvec_f64(W, x, rows: int, cols: int):
    W = _u8(W)
    _check_w(W, rows, cols)
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.size == cols
    y = np.zeros(rows, np.float64)
    A = np.zeros(rows, np.float64)
    lib().q4o_matvec_f64(_ptr(W), _ptr(x), rows, cols, _ptr(y), _ptr(A))
    return y, A


def gelu_tanh(z: float) -> float:
    return lib().q4o_gelu_tanh(float(z))


def silu(z: float) -> float:
    return lib().q4o_silu(float(z))


def act_array(z, act: int) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float64)
    out = np.zeros_like(z)
    lib().q4o_act_array(_ptr(z), z.size, int(act), _ptr(out))
    return out


def ffn(Wg, Wu, Wd, x, hidden: int, inter: int, act: int = GELU_TANH):
    """dict(y, A, g, u, h) of the gated FFN h = act(Wg x) * (Wu x), y = Wd h."""
    Wg, Wu, Wd = _u8(Wg), _u8(Wu), _u8(Wd)
    _check_w(Wg, inter, hidden)
    _check_w(Wu, inter, hidden)
    _check_w(Wd, hidden, inter)
    x = _f32(x)
    assert x.size == hidden
    y = np.zeros(hidden, np.float64)
    A = np.zeros(hidden, np.float64)
    g = np.zeros(inter, np.float64)
    u = np.zeros(inter, np.float64)
    h = np.zeros(inter, np.float64)
    lib().q4o_ffn(_ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(x), hidden, inter, int(act),
                  _ptr(y), _ptr(A), _ptr(g), _ptr(u), _ptr(h))
    return {"y": y, "A": A, "g": g, "u": u, "h": h}


def ffn_f64(Wg, Wu, Wd, x, hidden: int, inter: int, act: int = GELU_TANH):
    """q4o_ffn with an f64 activation vector (e.g. a normalised residual)."""
    Wg, Wu, Wd = _u8(Wg), _u8(Wu), _u8(Wd)
    _check_w(Wg, inter, hidden)
    _check_w(Wu, inter, hidden)
    _check_w(Wd, hidden, inter)
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.size == hidden
    y = np.zeros(hidden, np.float64)
    A = np.zeros(hidden, np.float64)
    g = np.zeros(inter, np.float64)
    u = np.zeros(inter, np.float64)
    h = np.zeros(inter, np.float64)
    lib().q4o_ffn_f64(_ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(x), hidden, inter, int(act),
                      _ptr(y), _ptr(A), _ptr(g), _ptr(u), _ptr(h))
    return {"y": y, "A": A, "g": g, "u": u, "h": h}


def residual_rmsnorm(h, delta, w, eps: float):
    """(s f32, x f64): s = h + delta in f32 (delta None: s = h),
    x = s / sqrt(mean(s^2) + eps) * w in f64."""
    h = _f32(h)
    w = _f32(w)
    n = h.size
    assert w.size == n
    d = None if delta is None else _f32(delta)
    s = np.zeros(n, np.float32)
    x = np.zeros(n, np.float64)
    lib().q4o_residual_rmsnorm(_ptr(h), None if d is None else _ptr(d), _ptr(w),
                               ctypes.c_float(eps), n, _ptr(s), _ptr(x))
    return s, x


def topk(v, k: int):
    """(idx int64[k], val f64[k]) -- first k of all entries by (value desc, index asc)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    k = min(int(k), v.size)
    idx = np.zeros(k, np.int64)
    val = np.zeros(k, np.float64)
    lib().q4o_topk(_ptr(v), v.size, k, _ptr(idx), _ptr(val))
    return idx, val


Q6K_BLOCK = 210


def _check_w6(W: np.ndarray, rows: int, cols: int) -> None:
    assert cols % 256 == 0, cols
    assert W.dtype == np.uint8 and W.size == rows * (cols // 256) * Q6K_BLOCK, (W.shape, rows, cols)


def q6k_dequant_block(blk) -> np.ndarray:
    """The 256 weights of one 210-byte Q6_K block, f64."""
    b = _u8(blk)
    assert b.size == Q6K_BLOCK
    w = np.zeros(256, np.float64)
    lib().q6o_dequant_block(_ptr(b), _ptr(w))
    return w


def q6k_dequant(W, rows: int, cols: int) -> np.ndarray:
    """Dense f64 [rows, cols] copy of a Q6_K matrix."""
    W = _u8(W)
    _check_w6(W, rows, cols)
    out = np.zeros((rows, cols), np.float64)
    lib().q6o_dequant(_ptr(W), rows, cols, _ptr(out))
    return out


def q6k_matvec(W, x, rows: int, cols: int):
    """(y, A): y = W x in f64 for a Q6_K matrix, A = sum_j |w_ij x_j|."""
    W = _u8(W)
    _check_w6(W, rows, cols)
    x = _f32(x)
    assert x.size == cols
    y = np.zeros(rows, np.float64)
    A = np.zeros(rows, np.float64)
    lib().q6o_matvec(_ptr(W), _ptr(x), rows, cols, _ptr(y), _ptr(A))
    return y, A


def logsumexp(v) -> float:
    """log sum_i exp(v_i) in f64 (largest value taken out first); NaN if any v_i is NaN."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    return float(lib().q4o_logsumexp(_ptr(v), v.size))


def softmax(v) -> np.ndarray:
    """p_i = exp(v_i - logsumexp(v)) in f64: the probabilities of the top-k predictions."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    p = np.zeros(v.size, np.float64)
    lib().q4o_softmax(_ptr(v), v.size, _ptr(p))
    return p


def matmul(W, X, rows: int, cols: int):
    """(Y, A) for Y[t] = W X[t], shapes [seq, rows]."""
    W = _u8(W)
    _check_w(W, rows, cols)
    X = _f32(X)
    seq = X.size // cols
    assert X.size == seq * cols
    Y = np.zeros((seq, rows), np.float64)
    A = np.zeros((seq, rows), np.float64)
    lib().q4o_matmul(_ptr(W), _ptr(X), seq, rows, cols, _ptr(Y), _ptr(A))
    return Y, A


def matmul_bf16(W, X, rows: int, cols: int):
    """(Y, A) of W X[t] with bf16 operands (X rounded; W formed in binary32, then
    rounded) and exact f64 products and sums: the matrix-core operand model."""
    W = _u8(W)
    _check_w(W, rows, cols)
    X = _f32(X)
    seq = X.size // cols
    assert X.size == seq * cols
    Y = np.zeros((seq, rows), np.float64)
    A = np.zeros((seq, rows), np.float64)
    lib().q4o_matmul_bf16(_ptr(W), _ptr(X), seq, rows, cols, _ptr(Y), _ptr(A))
    return Y, A


def ffn_prefill(Wg, Wu, Wd, X, hidden: int, inter: int, act: int = GELU_TANH):
    Wg, Wu, Wd = _u8(Wg), _u8(Wu), _u8(Wd)
    X = _f32(X)
    seq = X.size // hidden
    Y = np.zeros((seq, hidden), np.float64)
    A = np.zeros((seq, hidden), np.float64)
    lib().q4o_ffn_prefill(_ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(X), seq, hidden, inter, int(act),
                          _ptr(Y), _ptr(A))
    return Y, A


def act_deriv(z: float, act: int) -> float:
    return lib().q4o_act_deriv(float(z), int(act))


def ffn_prefill_scale(Wg, Wu, Wd, X, hidden: int, inter: int, act: int = GELU_TANH):
    """Per-output error scale Ap [seq, hidden] of the gated FFN under relative
    operand rounding: sum_j |wd_ij| (|act'(g_j) u_j| A_g,j + |act(g_j)| A_u,j
    + 2 |h_j|). Never below the last stage's plain A."""
    Wg, Wu, Wd = _u8(Wg), _u8(Wu), _u8(Wd)
    X = _f32(X)
    seq = X.size // hidden
    Ap = np.zeros((seq, hidden), np.float64)
    lib().q4o_ffn_prefill_scale(_ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(X), seq, hidden, inter,
                                int(act), _ptr(Ap))
    return Ap


def ffn_prefill_bf16(Wg, Wu, Wd, X, hidden: int, inter: int, act: int = GELU_TANH):
    Wg, Wu, Wd = _u8(Wg), _u8(Wu), _u8(Wd)
    X = _f32(X)
    seq = X.size // hidden
    Y = np.zeros((seq, hidden), np.float64)
    A = np.zeros((seq, hidden), np.float64)
    lib().q4o_ffn_prefill_bf16(_ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(X), seq, hidden, inter,
                               int(act), _ptr(Y), _ptr(A))
    return Y, A


def round_bf16(v: float) -> float:
    return lib().q4o_round_bf16(float(v))
