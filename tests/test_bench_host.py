"""Host-side checks of bench.py's bookkeeping (no GPU): the byte counts its
value and roofline divide by, the hash that decides whether a committed
counter summary still describes the kernels, and the one-GPU refusal."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_byte_counts_follow_the_layout(cfg):
    """27/16 * I * H bytes per active expert (NVFP4: 9/16 per weight, three
    I x H matrices); gate+up moves two of them plus x once and h once."""
    shape = synth.config(cfg)
    ids, _ = synth.gen_routing(cfg, shape)
    act = np.unique(ids).size
    assert synth.expert_bytes(shape) == 27 * shape.I * shape.H // 16
    assert synth.expert_bytes(shape, 32) == 3 * shape.I * shape.H // 2 + 3 * shape.I * shape.H // 32
    assert bench.active_weight_bytes(shape, ids) == act * 27 * shape.I * shape.H // 16
    gu = bench.gate_up_bytes(shape, ids)
    assert gu == act * 2 * (9 * shape.I * shape.H // 16 + 4) + shape.T * shape.H * 2 + shape.P * shape.I * 4
    # ids outside [0, E) move no weights
    bad = ids.copy()
    bad.reshape(-1)[0] = -1
    bad.reshape(-1)[1] = shape.E
    act_bad = np.unique(bad[(bad >= 0) & (bad < shape.E)]).size
    assert bench.active_weight_bytes(shape, bad) == act_bad * synth.expert_bytes(shape)


def test_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n    return x + 1;  // add one\n}\n/* block\ncomment */\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", (str(src),))
    h0 = bench.kernel_source_hash()
    src.write_text("int f(int x) { return x + 1; }   // other words\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_summary_is_used_only_while_the_hash_matches(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(tmp_path / "bench.py"))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    assert bench.measured_traffic("w") is None  # no summary
    (prof / "traffic_w.txt").write_text("hbm_bytes_per_launch: 1234567\nkernel_source_sha256_16: 0123456789abcdef\n")
    assert bench.measured_traffic("w") == 1234567
    (prof / "traffic_w.txt").write_text("hbm_bytes_per_launch: 1234567\nkernel_source_sha256_16: ffffffffffffffff\n")
    assert bench.measured_traffic("w") is None  # the kernels changed since


def test_committed_traffic_summaries_parse():
    """Every committed gate+up traffic summary carries the fields bench.py
    reads, and its bytes are within a small factor of the algorithmic ones."""
    prof = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.startswith("traffic_")]
    assert names
    for f in names:
        fields = {}
        for ln in open(os.path.join(prof, f)):
            if ":" in ln:
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
        hbm = float(fields["hbm_bytes_per_launch"])
        alg = float(fields["algorithmic_bytes_per_launch"])
        assert len(fields["kernel_source_sha256_16"]) == 16
        assert 0.9 < hbm / alg < 2.0, f


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
