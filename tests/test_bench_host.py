"""Host-side logic of bench.py (no GPU): algorithmic byte accounting, the traffic record's
staleness check, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_long1d():
    w = synth.WORKLOADS["long1d"]
    acc, total_bytes, _ = bench.kernel_accounting(w, 4)
    tok = 16 * 65536
    assert acc["summary"]["bytes"] == tok * 128 * 2 * 2          # K and V, bf16
    assert acc["readout"]["bytes"] == tok * 128 * (2 + 4)        # Q bf16 in, O fp32 out
    assert acc["mix"]["bytes"] == 256 * 256 * 4                  # M_c, fp32
    assert acc["mix"]["bound"] == "mfma"
    assert total_bytes == tok * 128 * (3 * 2 + 4) + 256 * 256 * 4
    acc_b, total_b, _ = bench.kernel_accounting(w, 2)
    assert total_b == tok * 128 * 8 + 256 * 256 * 4               # the all-bf16 figure


def test_fused_kernel_accounting_and_mala():
    w = synth.WORKLOADS["image_mala"]
    acc, total_bytes, _ = bench.kernel_accounting(w, 4, split=True)
    assert acc["mix"]["bytes"] == 0 and acc["mix"]["bound"] == "alu"
    assert acc["mix+readout"]["bytes"] == acc["readout"]["bytes"]
    assert total_bytes == 16 * 8 * 4096 * 64 * (3 * 2 + 4)


def test_traffic_record_requires_current_digest(tmp_path, monkeypatch):
    d = bench.source_digest()
    assert d == bench.source_digest() and len(d) == 16
    rec = {"workload": "long1d", "kernel": "readout", "out_dtype": "fp32",
           "hbm_bytes_per_launch": 123, "source_digest": d}
    f = tmp_path / "traffic.md"
    f.write_text("# x\n" + bench.TRAFFIC_TAG + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("long1d", "readout", "fp32") == 123
    assert bench.measured_traffic("long1d", "readout", "bf16") is None
    assert bench.measured_traffic("image", "readout", "fp32") is None
    rec["source_digest"] = "0" * 16
    f.write_text(bench.TRAFFIC_TAG + json.dumps(rec) + "\n")
    assert bench.measured_traffic("long1d", "readout", "fp32") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_decode_accounting_by_hand():
    """Decode bytes: 12 d^2 + 12 d + 3 d s_in + d s_out per call and (batch, head), plus
    4 d^2 (i + 3) + 12 d at the first position of block i > 0."""
    d, nb = 128, 256
    per = 12 * d * d + 12 * d + 3 * d * 2 + d * 2
    # positions 0 .. 255: block 0 only, no block start after the first
    assert bench.decode_accounting(1, d, nb, 0, 256, 2, 2) == 256 * per
    # positions 0 .. 767: blocks 1 and 2 start inside
    extra = (4 * d * d * 4 + 12 * d) + (4 * d * d * 5 + 12 * d)
    assert bench.decode_accounting(1, d, nb, 0, 768, 2, 2) == 768 * per + extra
    # a window that starts at a block start counts it; (batch, head) pairs scale linearly
    assert bench.decode_accounting(3, d, nb, 256, 512, 2, 2) == 3 * (256 * per + 4 * d * d * 4 + 12 * d)


def test_digest_ignores_the_peak_probe(tmp_path, monkeypatch):
    """The measured-peak probe is outside the MHLA path: editing it leaves the digest alone, while
    any kernel source changes it."""
    import shutil
    root = tmp_path / "r"
    for d in bench.SOURCE_DIRS:
        shutil.copytree(os.path.join(ROOT, d), root / d)
    monkeypatch.setattr(bench, "ROOT", str(root))
    d0 = bench.source_digest()
    (root / "token_blocked_linear_amd/csrc/peak_probe.hip").write_text("// changed\n")
    assert bench.source_digest() == d0
    with open(root / "token_blocked_linear_amd/csrc/decode.hip", "a") as f:
        f.write("\n// changed\n")
    assert bench.source_digest() != d0
