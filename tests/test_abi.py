"""The C-ABI library: loads, exports every declared symbol, and rejects bad
arguments before touching the device (CPU only: no call here reaches a launch;
pointers are fake, never dereferenced, because every call fails validation)."""
import ctypes
import re

import pytest

from quantized_decode_q4_amd import q4k

# Fake device addresses: 256-byte aligned and far apart (never dereferenced).
A = 0x7F0000000000
B = 0x7F1000000000
C = 0x7F2000000000
D = 0x7F3000000000
E = 0x7F4000000000
F = 0x7F5000000000
S = None  # stream


def declared_functions():
    text = open(q4k.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q[46]k_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["q4k_matvec", "q4k_qkv", "q4k_ffn", "q4k_gate_up", "q4k_lmhead_topk",
              "q4k_lmhead_topk_probs", "q6k_matvec", "q4k_rmsnorm_matvec", "q4k_rmsnorm_ffn",
              "q4k_matmul",
              "q4k_ffn_prefill", "q4k_status_string", "q4k_last_hip_error",
              "q4k_ffn_workspace_bytes", "q4k_lmhead_workspace_bytes", "q4k_lmhead_rows_max",
              "q4k_matmul_workspace_bytes", "q4k_ffn_prefill_workspace_bytes"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q4k.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_library_exports_nothing_else():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", q4k.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_status_strings():
    for s in range(-9, 1):
        assert q4k.q4k_status_string(s)
    assert "unknown" in q4k.q4k_status_string(-99)
    assert q4k.q4k_last_hip_error() == ""


L = q4k.lib


def test_matvec_validation():
    assert L.q4k_matvec(A, B, C, 10, 300, S) == q4k.Q4K_ERR_SHAPE
    assert L.q4k_matvec(A, B, C, 10, 0, S) == q4k.Q4K_ERR_SHAPE
    assert L.q4k_matvec(A, B, C, -1, 256, S) == q4k.Q4K_ERR_SHAPE
    assert L.q4k_matvec(A, B, C, 10, 65536 + 256, S) == q4k.Q4K_ERR_SHAPE
    assert L.q4k_matvec(A, B, C, 0, 256, S) == q4k.Q4K_OK            # empty: no-op
    assert L.q4k_matvec(None, B, C, 0, 256, S) == q4k.Q4K_OK
    assert L.q4k_matvec(None, B, C, 10, 256, S) == q4k.Q4K_ERR_NULL
    assert L.q4k_matvec(A, None, C, 10, 256, S) == q4k.Q4K_ERR_NULL
    assert L.q4k_matvec(A, B, None, 10, 256, S) == q4k.Q4K_ERR_NULL
    assert L.q4k_matvec(A + 8, B, C, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    assert L.q4k_matvec(A, B + 4, C, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    assert L.q4k_matvec(A, B, C + 2, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    # y inside W, y overlapping x
    assert L.q4k_matvec(A, B, A + 144, 10, 256, S) == q4k.Q4K_ERR_ALIAS
    assert L.q4k_matvec(A, B, B + 1020, 10, 256, S) == q4k.Q4K_ERR_ALIAS
    # y just past the end of W: no overlap, but do not launch (fake pointers);
    # check only that the boundary computation is half-open via qkv below.


def test_qkv_validation():
    assert L.q4k_qkv(A, B, C, D, E, -1, 2, 256, S) == q4k.Q4K_ERR_SHAPE
    assert L.q4k_qkv(A, B, C, D, E, 0, 0, 256, S) == q4k.Q4K_OK
    assert L.q4k_qkv(A, B, None, D, E, 4, 2, 256, S) == q4k.Q4K_ERR_NULL
    assert L.q4k_qkv(A, B, C, None, E, 4, 2, 256, S) == q4k.Q4K_ERR_NULL
    assert L.q4k_qkv(A, B, C, D, E + 2, 4, 2, 256, S) == q4k.Q4K_ERR_ALIGN
    assert L.q4k_qkv(A, B, C, C + 8, E, 4, 2, 256, S) == q4k.Q4K_ERR_ALIAS   # k inside q
    assert L.q4k_qkv(A, B, C, D, D + 4, 4, 2, 256, S) == q4k.Q4K_ERR_ALIAS   # v overlaps k


def test_gate_up_and_ffn_validation():
    assert L.q4k_gate_up(A, B, C, D, 8, 256, 2, S) == q4k.Q4K_ERR_ACT
    assert L.q4k_gate_up(A, B, C, D, 8, 200, 0, S) == q4k.Q4K_ERR_SHAPE
    assert L.q4k_gate_up(A, B, C, D, 0, 256, 0, S) == q4k.Q4K_OK
    assert L.q4k_gate_up(A, None, C, D, 8, 256, 0, S) == q4k.Q4K_ERR_NULL
    assert L.q4k_gate_up(A, B, C, B + 16, 8, 256, 1, S) == q4k.Q4K_ERR_ALIAS
    need = q4k.q4k_ffn_workspace_bytes(256, 512)
    assert need >= 512 * 4 and need % 256 == 0
    assert q4k.q4k_ffn_workspace_bytes(256, 100) == 0
    assert L.q4k_ffn(A, B, C, D, E, 256, 512, 0, F, need - 1, S) == q4k.Q4K_ERR_WORKSPACE
    assert L.q4k_ffn(A, B, C, D, E, 256, 512, 0, None, need, S) == q4k.Q4K_ERR_WORKSPACE
    assert L.q4k_ffn(A, B, C, D, E, 256, 512, 0, F + 8, need, S) == q4k.Q4K_ERR_ALIGN
    assert L.q4k_ffn(A, B, C, D, E, 256, 512, 5, F, need, S) == q4k.Q4K_ERR_ACT
    assert L.q4k_ffn(A, B, C, D, F, 256, 512, 0, F, need, S) == q4k.Q4K_ERR_ALIAS   # y in ws
    assert L.q4k_ffn(A, B, C, D, E, 256, 512, 0, D, need, S) == q4k.Q4K_ERR_ALIAS   # ws on x


def test_ffn_noalloc_validation():
    L = q4k.lib
    F_ = L.q4k_ffn_noalloc
    assert F_(A, B, C, D, E, 256, q4k.Q4K_NOALLOC_INTER_MAX + 256, 0, S) == q4k.Q4K_ERR_SCRATCH
    assert F_(A, B, C, D, E, 256, 300, 0, S) == q4k.Q4K_ERR_SHAPE
    assert F_(A, B, C, D, E, 256, 512, 7, S) == q4k.Q4K_ERR_ACT
    assert F_(None, B, C, D, E, 256, 512, 0, S) == q4k.Q4K_ERR_NULL
    assert F_(A + 4, B, C, D, E, 256, 512, 0, S) == q4k.Q4K_ERR_ALIGN
    assert F_(A, B, C, D, D, 256, 512, 0, S) == q4k.Q4K_ERR_ALIAS
    assert "Q4K_NOALLOC_INTER_MAX" in L.q4k_status_string(q4k.Q4K_ERR_SCRATCH).decode()


def test_q6k_matvec_validation():
    P = L.q6k_matvec
    assert P(A, B, C, 10, 300, S) == q4k.Q4K_ERR_SHAPE
    assert P(A, B, C, -1, 256, S) == q4k.Q4K_ERR_SHAPE
    assert P(A, B, C, 10, 65536 + 256, S) == q4k.Q4K_ERR_SHAPE
    assert P(None, B, C, 10, 256, S) == q4k.Q4K_ERR_NULL
    assert P(A + 2, B, C, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    assert P(A, B + 4, C, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    assert P(A, B, C + 2, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    assert P(A, B, A + 2096, 10, 256, S) == q4k.Q4K_ERR_ALIAS   # y inside W (10 x 210 B)
    assert P(A, B, B + 512, 10, 256, S) == q4k.Q4K_ERR_ALIAS    # y inside x
    assert P(None, None, None, 0, 256, S) == q4k.Q4K_OK         # rows = 0: nothing to do


def test_rmsnorm_validation():
    G = 0x7F6000000000
    H = 0x7F7000000000
    M = L.q4k_rmsnorm_matvec
    # W, h, delta, w, eps, h_out, y, rows, cols
    assert M(A, B, C, D, 1e-6, E, F, 0, 256, S) == q4k.Q4K_ERR_SHAPE
    assert M(A, B, C, D, 1e-6, E, F, 10, 100, S) == q4k.Q4K_ERR_SHAPE
    assert M(A, None, C, D, 1e-6, E, F, 10, 256, S) == q4k.Q4K_ERR_NULL
    assert M(A, B, C, None, 1e-6, E, F, 10, 256, S) == q4k.Q4K_ERR_NULL
    assert M(A, B, C, D, -1.0, E, F, 10, 256, S) == q4k.Q4K_ERR_EPS
    assert M(A, B, C, D, float("nan"), E, F, 10, 256, S) == q4k.Q4K_ERR_EPS
    assert M(A, B, C, D, float("inf"), E, F, 10, 256, S) == q4k.Q4K_ERR_EPS
    assert M(A, B + 4, C, D, 1e-6, E, F, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    assert M(A, B, C + 8, D, 1e-6, E, F, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    assert M(A, B, C, D, 1e-6, E + 4, F, 10, 256, S) == q4k.Q4K_ERR_ALIGN
    assert M(A, B, C, D, 1e-6, B, F, 10, 256, S) == q4k.Q4K_ERR_ALIAS        # h_out on h
    assert M(A, B, C, D, 1e-6, C + 512, F, 10, 256, S) == q4k.Q4K_ERR_ALIAS  # h_out in delta
    assert M(A, B, C, D, 1e-6, A + 32, F, 10, 256, S) == q4k.Q4K_ERR_ALIAS   # h_out in W
    assert M(A, B, C, D, 1e-6, F + 16, F, 10, 256, S) == q4k.Q4K_ERR_ALIAS   # h_out on y
    assert M(A, B, C, D, 1e-6, E, D + 4, 10, 256, S) == q4k.Q4K_ERR_ALIAS    # y in norm_w
    assert M(A, B, C, D, 1e-6, E, A + 8, 10, 256, S) == q4k.Q4K_ERR_ALIAS    # y in W
    Fn = L.q4k_rmsnorm_ffn
    need = q4k.q4k_ffn_workspace_bytes(256, 512)
    # Wg, Wu, Wd, h, delta, w, eps, h_out, y, hidden, inter, act, ws, ws_bytes
    assert Fn(A, B, C, D, None, E, 1e-6, None, F, 256, 512, 7, G, need, S) == q4k.Q4K_ERR_ACT
    assert Fn(A, B, C, D, None, E, -2.0, None, F, 256, 512, 0, G, need, S) == q4k.Q4K_ERR_EPS
    assert Fn(A, B, C, D, None, E, 1e-6, None, F, 256, 512, 0, G, need - 4, S) == q4k.Q4K_ERR_WORKSPACE
    assert Fn(A, B, C, None, None, E, 1e-6, None, F, 256, 512, 0, G, need, S) == q4k.Q4K_ERR_NULL
    assert Fn(A, B, C, D, None, E, 1e-6, G + 64, F, 256, 512, 0, G, need, S) == q4k.Q4K_ERR_ALIAS  # h_out in ws
    assert Fn(A, B, C, D, None, E, 1e-6, H, D + 16, 256, 512, 0, G, need, S) == q4k.Q4K_ERR_ALIAS  # y on h


def test_lmhead_validation():
    need = q4k.q4k_lmhead_workspace_bytes(1000, 256, 5)
    assert need > 0 and need % 256 == 0
    assert q4k.q4k_lmhead_workspace_bytes(1000, 256, 0) == 0
    assert L.q4k_lmhead_topk(A, B, C, 1000, 256, 0, D, E, F, need, S) == q4k.Q4K_ERR_K
    assert L.q4k_lmhead_topk(A, B, C, 1000, 256, 65, D, E, F, need, S) == q4k.Q4K_ERR_K
    assert L.q4k_lmhead_topk(A, B, C, 4, 256, 5, D, E, F, need, S) == q4k.Q4K_ERR_K
    assert L.q4k_lmhead_topk(A, B, C, 0, 256, 1, D, E, F, need, S) == q4k.Q4K_ERR_K
    assert L.q4k_lmhead_topk(A, B, C, 1000, 256, 5, D, E, F, need - 8, S) == q4k.Q4K_ERR_WORKSPACE
    assert L.q4k_lmhead_topk(A, B, C, 1000, 256, 5, None, E, F, need, S) == q4k.Q4K_ERR_NULL
    assert L.q4k_lmhead_topk(A, B, C, 1000, 256, 5, D, D + 8, F, need, S) == q4k.Q4K_ERR_ALIAS
    assert L.q4k_lmhead_topk(A, B, C, 1000, 256, 5, D, E, C + 64, need, S) == q4k.Q4K_ERR_ALIAS
    # a vocabulary too large for the single-workgroup merge at k = 64
    assert L.q4k_lmhead_topk(A, B, C, 5_000_000, 256, 64, D, E, F, 1 << 40, S) == q4k.Q4K_ERR_SHAPE


def test_lmhead_row_limit():
    """The vocabulary limit the header states: rows up to q4k_lmhead_rows_max
    size a workspace, one more is refused by the calls before any launch."""
    L = q4k.lib
    rup = lambda n: (n + 255) // 256 * 256
    for cols in (256, 512, 2560, 4096, 16384, 65536):
        rmax = L.q4k_lmhead_rows_max(cols)
        assert rmax >= 4_000_000, (cols, rmax)
        # the workspace and the calls share one test; at the limit the grid is
        # exactly the 1024 candidate lists the merge takes (k keys and one
        # softmax partial each)
        for rows in (rmax, rmax - 1, rmax - 63, rmax // 2 + 1):
            assert L.q4k_lmhead_workspace_bytes(rows, cols, 5) > 0, (cols, rows)
        assert L.q4k_lmhead_workspace_bytes(rmax, cols, 5) == rup(1024 * 5 * 8) + rup(1024 * 8)
        assert L.q4k_lmhead_workspace_bytes(rmax, cols, 64) == rup(1024 * 64 * 8) + rup(1024 * 8)
        assert L.q4k_lmhead_workspace_bytes(rmax + 1, cols, 5) == 0
        assert L.q4k_lmhead_topk(A, B, C, rmax + 1, cols, 5, D, E, F, 1 << 40, S) == \
            q4k.Q4K_ERR_SHAPE
        assert L.q4k_lmhead_topk_probs(A, B, C, rmax + 1, cols, 5, D, E, D + 4096, E + 4096, F,
                                       1 << 40, S) == q4k.Q4K_ERR_SHAPE
    assert L.q4k_lmhead_rows_max(2560) == 1024 * (4096 - 16)
    assert L.q4k_lmhead_rows_max(100) == 0 and L.q4k_lmhead_rows_max(0) == 0


def test_probe_validation():
    """The measurement helpers reject bad sizes, launch shapes, pointers and an
    overlapping sink before any launch."""
    L = q4k.lib
    R = L.q4k_probe_read
    assert R(A, 0, 256, 512, 4, 0, F, S) == q4k.Q4K_ERR_SHAPE
    assert R(A, 4100, 256, 512, 4, 0, F, S) == q4k.Q4K_ERR_SHAPE          # not a multiple of 16
    assert R(A, 1 << 31, 256, 512, 4, 0, F, S) == q4k.Q4K_ERR_SHAPE
    assert R(A, 4096, 0, 512, 4, 0, F, S) == q4k.Q4K_ERR_SHAPE
    assert R(A, 4096, 65537, 512, 4, 0, F, S) == q4k.Q4K_ERR_SHAPE
    assert R(A, 4096, 256, 500, 4, 0, F, S) == q4k.Q4K_ERR_SHAPE
    assert R(A, 4096, 256, 2048, 4, 0, F, S) == q4k.Q4K_ERR_SHAPE
    assert R(A, 4096, 256, 512, 3, 0, F, S) == q4k.Q4K_ERR_SHAPE
    assert R(A, 4096, 256, 512, 32, 0, F, S) == q4k.Q4K_ERR_SHAPE
    assert R(None, 4096, 256, 512, 4, 0, F, S) == q4k.Q4K_ERR_NULL
    assert R(A, 4096, 256, 512, 4, 0, None, S) == q4k.Q4K_ERR_NULL
    assert R(A + 8, 4096, 256, 512, 4, 0, F, S) == q4k.Q4K_ERR_ALIGN
    assert R(A, 4096, 256, 512, 4, 0, F + 2, S) == q4k.Q4K_ERR_ALIGN
    assert R(A, 4096, 256, 512, 4, 1, A + 1024, S) == q4k.Q4K_ERR_ALIAS
    E_ = L.q4k_probe_empty
    assert E_(0, 256, F, S) == q4k.Q4K_ERR_SHAPE
    assert E_(256, 100, F, S) == q4k.Q4K_ERR_SHAPE
    assert E_(256, 256, None, S) == q4k.Q4K_ERR_NULL
    assert E_(256, 256, F + 1, S) == q4k.Q4K_ERR_ALIGN


def test_lmhead_probs_validation():
    G = 0x7F6000000000
    H = 0x7F7000000000
    P = L.q4k_lmhead_topk_probs
    need = q4k.q4k_lmhead_workspace_bytes(1000, 256, 5)
    assert P(A, B, C, 1000, 256, 0, D, E, G, H, F, need, S) == q4k.Q4K_ERR_K
    assert P(A, B, C, 1000, 256, 5, D, E, None, H, F, need, S) == q4k.Q4K_ERR_NULL
    assert P(A, B, C, 1000, 256, 5, D, E, G, None, F, need, S) == q4k.Q4K_ERR_NULL
    assert P(A, B, C, 1000, 256, 5, D, E, G + 2, H, F, need, S) == q4k.Q4K_ERR_ALIGN
    assert P(A, B, C, 1000, 256, 5, D, E, G, H + 1, F, need, S) == q4k.Q4K_ERR_ALIGN
    assert P(A, B, C, 1000, 256, 5, D, E, G, H, F, need - 8, S) == q4k.Q4K_ERR_WORKSPACE
    assert P(A, B, C, 1000, 256, 5, D, E, G, G + 16, F, need, S) == q4k.Q4K_ERR_ALIAS  # lse in probs
    assert P(A, B, C, 1000, 256, 5, D, E, E, H, F, need, S) == q4k.Q4K_ERR_ALIAS      # probs on vals
    assert P(A, B, C, 1000, 256, 5, D, E, G, F + 64, F, need, S) == q4k.Q4K_ERR_ALIAS  # lse in ws
    assert P(A, B, C, 1000, 256, 5, D, E, G, A + 4, F, need, S) == q4k.Q4K_ERR_ALIAS   # lse on W
    assert P(A, B, C, 1000, 256, 5, D, E, B, H, F, need, S) == q4k.Q4K_ERR_ALIAS       # probs on x
    assert P(A, B, C, 5_000_000, 256, 64, D, E, G, H, F, 1 << 40, S) == q4k.Q4K_ERR_SHAPE


def test_prefill_validation():
    assert q4k.q4k_matmul_workspace_bytes(512, 2560, 63) == 0
    assert q4k.q4k_matmul_workspace_bytes(512, 2560, 64) >= 64 * 2560 * 2
    assert L.q4k_matmul(A, B, C, 10, 256, -1, None, 0, S) == q4k.Q4K_ERR_SHAPE
    assert L.q4k_matmul(A, B, C, 10, 256, 0, None, 0, S) == q4k.Q4K_OK
    assert L.q4k_matmul(A, B, C, 10, 256, 64, None, 0, S) == q4k.Q4K_ERR_WORKSPACE
    assert L.q4k_matmul(A, B, B + 64, 10, 256, 2, None, 0, S) == q4k.Q4K_ERR_ALIAS
    need = q4k.q4k_ffn_prefill_workspace_bytes(64, 256, 512)
    assert need >= 64 * 256 * 2 + 64 * 512 * 2
    assert q4k.q4k_ffn_prefill_workspace_bytes(3, 256, 512) >= 512 * 4
    # below 64 tokens h is kept for every token
    assert q4k.q4k_ffn_prefill_workspace_bytes(5, 256, 512) == 5 * 512 * 4
    assert q4k.q4k_ffn_prefill_workspace_bytes(63, 256, 1024) == 63 * 1024 * 4
    assert L.q4k_ffn_prefill(A, B, C, D, E, 64, 256, 512, 3, F, need, S) == q4k.Q4K_ERR_ACT
    assert L.q4k_ffn_prefill(A, B, C, D, E, 64, 256, 512, 0, F, need - 1, S) == q4k.Q4K_ERR_WORKSPACE
    assert L.q4k_ffn_prefill(A, B, C, D, E, 0, 256, 512, 0, None, 0, S) == q4k.Q4K_OK
    assert L.q4k_ffn_prefill(A, B, C, D, F + 256, 64, 256, 512, 0, F, need, S) == q4k.Q4K_ERR_ALIAS


def test_debug_sync_variant_compiles(tmp_path):
    """The Q4K_DEBUG_SYNC build (every call waits for its stream and reports a
    failed kernel as Q4K_ERR_HIP) compiles: host pass of the ABI source."""
    import os
    import subprocess
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([hipcc, "--offload-arch=gfx950", "--cuda-host-only", "-std=c++17", "-fsyntax-only",
                          "-DQ4K_DEBUG_SYNC", f"-I{root}/include", f"-I{root}/quantized_decode_q4_amd/csrc",
                          f"{root}/quantized_decode_q4_amd/csrc/q4k_api.hip"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
