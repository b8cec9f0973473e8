"""Thin ctypes binding of libq4k.so (include/q4k.h): argument marshalling only.

Each function takes torch tensors (device memory) or raw integer device
pointers, passes their addresses, sizes and the current HIP stream to the C
call of the same name, and raises Q4KError on a nonzero status. Every step of
the computation runs in the library's HIP kernels. There is no fallback: if
libq4k.so is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libq4k.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "q4k.h")

Q4K_OK = 0
Q4K_ERR_NULL = -1
Q4K_ERR_SHAPE = -2
Q4K_ERR_ALIGN = -3
Q4K_ERR_K = -4
Q4K_ERR_ACT = -5
Q4K_ERR_WORKSPACE = -6
Q4K_ERR_ALIAS = -7
Q4K_ERR_HIP = -8
Q4K_ERR_EPS = -9
Q4K_ERR_SCRATCH = -10
Q4K_NOALLOC_INTER_MAX = 32768
Q4K_ACT_GELU_TANH = 0
Q4K_ACT_SILU = 1
Q4K_TOPK_MAX = 64
Q4K_COLS_MAX = 65536

# torch brings its own HIP runtime (same soname, libamdhip64.so.7). Loading it
# first makes this library bind to that runtime instead of a second copy from
# /opt/rocm: one process must use one HIP runtime, or tensors allocated by torch
# are invisible to our launches.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                      "or python -m quantized_decode_q4_amd.build")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
_INT = ctypes.c_int

lib = ctypes.CDLL(LIB_PATH)
_SIGS = {
    "q4k_matvec": ([_P, _P, _P, _I64, _I64, _P], _INT),
    "q4k_qkv": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], _INT),
    "q4k_gate_up": ([_P, _P, _P, _P, _I64, _I64, _INT, _P], _INT),
    "q4k_ffn_workspace_bytes": ([_I64, _I64], _SZ),
    "q4k_ffn": ([_P, _P, _P, _P, _P, _I64, _I64, _INT, _P, _SZ, _P], _INT),
    "q4k_ffn_noalloc": ([_P, _P, _P, _P, _P, _I64, _I64, _INT, _P], _INT),
    "q4k_lmhead_workspace_bytes": ([_I64, _I64, _INT], _SZ),
    "q4k_lmhead_rows_max": ([_I64], _I64),
    "q4k_lmhead_topk": ([_P, _P, _P, _I64, _I64, _INT, _P, _P, _P, _SZ, _P], _INT),
    "q6k_matvec": ([_P, _P, _P, _I64, _I64, _P], _INT),
    "q4k_rmsnorm_matvec": ([_P, _P, _P, _P, _F32, _P, _P, _I64, _I64, _P], _INT),
    "q4k_rmsnorm_ffn": ([_P, _P, _P, _P, _P, _P, _F32, _P, _P, _I64, _I64, _INT, _P, _SZ, _P],
                        _INT),
    "q4k_lmhead_topk_probs": ([_P, _P, _P, _I64, _I64, _INT, _P, _P, _P, _P, _P, _SZ, _P], _INT),
    "q4k_matmul_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "q4k_matmul": ([_P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "q4k_ffn_prefill_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "q4k_ffn_prefill": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _SZ, _P], _INT),
    "q4k_probe_read": ([_P, _I64, _INT, _INT, _INT, _INT, _P, _P], _INT),
    "q4k_probe_empty": ([_INT, _INT, _P, _P], _INT),
    "q4k_status_string": ([_INT], ctypes.c_char_p),
    "q4k_last_hip_error": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _res


class Q4KError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.q4k_status_string(status).decode()
        if status == Q4K_ERR_HIP:
            msg += " -- " + lib.q4k_last_hip_error().decode()
        super().__init__(f"{where}: {msg}")
        self.status = status


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _arg(t, name: str, nbytes: int, dtype=None, optional: bool = False) -> int | None:
    """Address of a tensor argument after checking what the C call cannot:
    that it is a contiguous device tensor of the expected dtype holding at
    least `nbytes` bytes. Raw integer pointers are passed through unchecked
    (the caller vouches for them); None is allowed only for optional ones."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor, got device {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call reads or writes {nbytes}")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check(status: int, where: str) -> None:
    if status != Q4K_OK:
        raise Q4KError(status, where)


def _blocks(n: int) -> int:
    """Super-blocks per row (0 for a length the library will reject)."""
    return n // 256 if n > 0 and n % 256 == 0 else 0


def _wq4(rows: int, cols: int) -> int:
    return max(rows, 0) * _blocks(cols) * 144


def _wq6(rows: int, cols: int) -> int:
    return max(rows, 0) * _blocks(cols) * 210


def _f32(n: int) -> int:
    return 4 * max(n, 0)


def _colv(n: int) -> int:
    """Bytes of an f32 vector whose length must be a positive multiple of 256
    (0 when it is not: the C call reports the shape error itself)."""
    return 4 * n if _blocks(n) else 0


_U8, _FLOAT, _INT32 = torch.uint8, torch.float32, torch.int32


def q4k_matvec(W, x, y, rows: int, cols: int, stream=None) -> None:
    _check(lib.q4k_matvec(_arg(W, "W", _wq4(rows, cols), _U8), _arg(x, "x", _colv(cols), _FLOAT),
                          _arg(y, "y", _f32(rows), _FLOAT), rows, cols, _stream(stream)),
           "q4k_matvec")


def q6k_matvec(W, x, y, rows: int, cols: int, stream=None) -> None:
    _check(lib.q6k_matvec(_arg(W, "W", _wq6(rows, cols), _U8), _arg(x, "x", _colv(cols), _FLOAT),
                          _arg(y, "y", _f32(rows), _FLOAT), rows, cols, _stream(stream)),
           "q6k_matvec")


def q4k_rmsnorm_matvec(W, h, delta, norm_w, eps: float, h_out, y, rows: int, cols: int,
                       stream=None) -> None:
    _check(lib.q4k_rmsnorm_matvec(_arg(W, "W", _wq4(rows, cols), _U8),
                                  _arg(h, "h", _colv(cols), _FLOAT),
                                  _arg(delta, "delta", _colv(cols), _FLOAT, optional=True),
                                  _arg(norm_w, "norm_w", _colv(cols), _FLOAT), float(eps),
                                  _arg(h_out, "h_out", _colv(cols), _FLOAT, optional=True),
                                  _arg(y, "y", _f32(rows), _FLOAT), rows, cols, _stream(stream)),
           "q4k_rmsnorm_matvec")


def q4k_rmsnorm_ffn(Wg, Wu, Wd, h, delta, norm_w, eps: float, h_out, y, hidden: int, inter: int,
                    act: int, ws, ws_bytes: int | None = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    _check(lib.q4k_rmsnorm_ffn(_arg(Wg, "Wg", _wq4(inter, hidden), _U8),
                               _arg(Wu, "Wu", _wq4(inter, hidden), _U8),
                               _arg(Wd, "Wd", _wq4(hidden, inter), _U8),
                               _arg(h, "h", _colv(hidden), _FLOAT),
                               _arg(delta, "delta", _colv(hidden), _FLOAT, optional=True),
                               _arg(norm_w, "norm_w", _colv(hidden), _FLOAT), float(eps),
                               _arg(h_out, "h_out", _colv(hidden), _FLOAT, optional=True),
                               _arg(y, "y", _colv(hidden), _FLOAT), hidden, inter, act,
                               _arg(ws, "ws", ws_bytes), ws_bytes, _stream(stream)),
           "q4k_rmsnorm_ffn")


def q4k_qkv(Wqkv, x, q, k, v, q_rows: int, kv_rows: int, cols: int, stream=None) -> None:
    rows = q_rows + 2 * kv_rows
    _check(lib.q4k_qkv(_arg(Wqkv, "Wqkv", _wq4(rows, cols), _U8), _arg(x, "x", _colv(cols), _FLOAT),
                       _arg(q, "q", _f32(q_rows), _FLOAT), _arg(k, "k", _f32(kv_rows), _FLOAT),
                       _arg(v, "v", _f32(kv_rows), _FLOAT), q_rows, kv_rows, cols,
                       _stream(stream)), "q4k_qkv")


def q4k_gate_up(Wg, Wu, x, h, inter: int, hidden: int, act: int = Q4K_ACT_GELU_TANH,
                stream=None) -> None:
    _check(lib.q4k_gate_up(_arg(Wg, "Wg", _wq4(inter, hidden), _U8),
                           _arg(Wu, "Wu", _wq4(inter, hidden), _U8),
                           _arg(x, "x", _colv(hidden), _FLOAT), _arg(h, "h", _f32(inter), _FLOAT),
                           inter, hidden, act, _stream(stream)), "q4k_gate_up")


def q4k_ffn_workspace_bytes(hidden: int, inter: int) -> int:
    return lib.q4k_ffn_workspace_bytes(hidden, inter)


def q4k_ffn(Wg, Wu, Wd, x, y, hidden: int, inter: int, act: int, ws, ws_bytes: int | None = None,
            stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    _check(lib.q4k_ffn(_arg(Wg, "Wg", _wq4(inter, hidden), _U8),
                       _arg(Wu, "Wu", _wq4(inter, hidden), _U8),
                       _arg(Wd, "Wd", _wq4(hidden, inter), _U8),
                       _arg(x, "x", _colv(hidden), _FLOAT), _arg(y, "y", _colv(hidden), _FLOAT),
                       hidden, inter, act, _arg(ws, "ws", ws_bytes), ws_bytes, _stream(stream)),
           "q4k_ffn")


def q4k_ffn_noalloc(Wg, Wu, Wd, x, y, hidden: int, inter: int, act: int, stream=None) -> None:
    """q4k_ffn without a workspace: h lives in the library's per-device scratch."""
    _check(lib.q4k_ffn_noalloc(_arg(Wg, "Wg", _wq4(inter, hidden), _U8),
                               _arg(Wu, "Wu", _wq4(inter, hidden), _U8),
                               _arg(Wd, "Wd", _wq4(hidden, inter), _U8),
                               _arg(x, "x", _colv(hidden), _FLOAT),
                               _arg(y, "y", _colv(hidden), _FLOAT), hidden, inter, act,
                               _stream(stream)), "q4k_ffn_noalloc")


def q4k_lmhead_workspace_bytes(rows: int, cols: int, k: int) -> int:
    return lib.q4k_lmhead_workspace_bytes(rows, cols, k)


def q4k_lmhead_topk(W, x, logits, rows: int, cols: int, k: int, top_idx, top_val, ws,
                    ws_bytes: int | None = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    kk = max(k, 0)
    _check(lib.q4k_lmhead_topk(_arg(W, "W", _wq4(rows, cols), _U8), _arg(x, "x", _colv(cols), _FLOAT),
                               _arg(logits, "logits", _f32(rows), _FLOAT), rows, cols, k,
                               _arg(top_idx, "top_idx", 4 * kk, _INT32),
                               _arg(top_val, "top_val", _f32(kk), _FLOAT),
                               _arg(ws, "ws", ws_bytes), ws_bytes, _stream(stream)),
           "q4k_lmhead_topk")


def q4k_lmhead_topk_probs(W, x, logits, rows: int, cols: int, k: int, top_idx, top_val, top_prob,
                          lse, ws, ws_bytes: int | None = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    kk = max(k, 0)
    _check(lib.q4k_lmhead_topk_probs(_arg(W, "W", _wq4(rows, cols), _U8),
                                     _arg(x, "x", _colv(cols), _FLOAT),
                                     _arg(logits, "logits", _f32(rows), _FLOAT), rows, cols, k,
                                     _arg(top_idx, "top_idx", 4 * kk, _INT32),
                                     _arg(top_val, "top_val", _f32(kk), _FLOAT),
                                     _arg(top_prob, "top_prob", _f32(kk), _FLOAT),
                                     _arg(lse, "lse", 4, _FLOAT), _arg(ws, "ws", ws_bytes),
                                     ws_bytes, _stream(stream)), "q4k_lmhead_topk_probs")


def q4k_matmul_workspace_bytes(rows: int, cols: int, seq: int) -> int:
    return lib.q4k_matmul_workspace_bytes(rows, cols, seq)


def q4k_matmul(W, X, Y, rows: int, cols: int, seq: int, ws=None, ws_bytes: int | None = None,
               stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else _nbytes(ws)
    _check(lib.q4k_matmul(_arg(W, "W", _wq4(rows, cols), _U8),
                          _arg(X, "X", _colv(cols) * max(seq, 0), _FLOAT),
                          _arg(Y, "Y", _f32(rows) * max(seq, 0), _FLOAT), rows, cols, seq,
                          _arg(ws, "ws", ws_bytes, optional=True), ws_bytes, _stream(stream)),
           "q4k_matmul")


def q4k_ffn_prefill_workspace_bytes(seq: int, hidden: int, inter: int) -> int:
    return lib.q4k_ffn_prefill_workspace_bytes(seq, hidden, inter)


def q4k_ffn_prefill(Wg, Wu, Wd, X, Y, seq: int, hidden: int, inter: int, act: int, ws,
                    ws_bytes: int | None = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    _check(lib.q4k_ffn_prefill(_arg(Wg, "Wg", _wq4(inter, hidden), _U8),
                               _arg(Wu, "Wu", _wq4(inter, hidden), _U8),
                               _arg(Wd, "Wd", _wq4(hidden, inter), _U8),
                               _arg(X, "X", _colv(hidden) * max(seq, 0), _FLOAT),
                               _arg(Y, "Y", _colv(hidden) * max(seq, 0), _FLOAT), seq, hidden,
                               inter, act, _arg(ws, "ws", ws_bytes), ws_bytes, _stream(stream)),
           "q4k_ffn_prefill")


def q4k_status_string(status: int) -> str:
    return lib.q4k_status_string(status).decode()


def q4k_last_hip_error() -> str:
    return lib.q4k_last_hip_error().decode()


def q4k_probe_read(buf, nbytes: int, grid: int, threads: int, depth: int, contiguous: bool,
                   sink, stream=None) -> None:
    """Streaming read of the first nbytes of buf (measurement helper)."""
    _check(lib.q4k_probe_read(_arg(buf, "buf", nbytes), nbytes, grid, threads, depth,
                              1 if contiguous else 0, _arg(sink, "sink", 4), _stream(stream)),
           "q4k_probe_read")


def q4k_probe_empty(grid: int, threads: int, sink, stream=None) -> None:
    """An empty kernel of grid x threads (measurement helper)."""
    _check(lib.q4k_probe_empty(grid, threads, _arg(sink, "sink", 4), _stream(stream)),
           "q4k_probe_empty")


def workspace(nbytes: int, device="cuda"):
    """A caller-owned device workspace of nbytes (uint8, 256-byte aligned by torch)."""
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
