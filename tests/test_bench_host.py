"""CPU checks of bench.py's reporting logic (no GPU): the algorithmic byte
counts it divides by, and the rule that HBM traffic from the committed counter
summary is reported only while the decode kernels' source is the one it was
measured on."""
import json
import os
import shutil

import bench


def test_algorithmic_bytes_from_the_block_format():
    # 144 bytes per 256 weights; activations and outputs f32, once each
    w = lambda rows, cols: rows * cols // 256 * 144
    assert bench.QKV_BYTES == w(4096, 2560) + 2560 * 4 + 4096 * 4 == 5_924_864
    assert bench.GATE_UP_BYTES == 2 * w(10240, 2560) + 2560 * 4 + 10240 * 4 == 29_542_400
    assert bench.DOWN_BYTES == w(2560, 10240) + 10240 * 4 + 2560 * 4 == 14_796_800
    # lm_head: weights, x, logits, and k winners as index + value + probability, plus lse
    assert bench.LMHEAD_BYTES == w(262144, 2560) + 2560 * 4 + 262144 * 4 + 5 * 12 + 4
    assert bench.STEP_BYTES == 34 * (5_924_864 + 29_542_400 + 14_796_800) + bench.LMHEAD_BYTES
    assert bench.STEP_BYTES == 2_087_524_416
    # prefill: 64 tokens x 2 flops per weight
    assert bench.PREFILL_FLOPS == 2 * 64 * 3 * 10240 * 2560 == 10_066_329_600


def test_traffic_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    csrc = tmp_path / "quantized_decode_q4_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = os.path.join(bench.ROOT, "quantized_decode_q4_amd", "csrc", "q4k_rows.hip")
    shutil.copy(src, csrc / "q4k_rows.hip")
    (tmp_path / "profiles").mkdir()
    rec = json.load(open(os.path.join(bench.ROOT, "profiles", "pmc_traffic.json")))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec["source_digest"] = bench.source_digest()
    (tmp_path / "profiles" / "pmc_traffic.json").write_text(json.dumps(rec))
    assert bench.counters_traffic("gate_up") == rec["kernels"]["gate_up"]["hbm_bytes_per_launch"]
    assert bench.counters_traffic("no_such_kernel") is None
    # any change to the kernel source makes the stored counters stale
    with open(csrc / "q4k_rows.hip", "a") as f:
        f.write("\n// edited\n")
    assert bench.counters_traffic("gate_up") is None

