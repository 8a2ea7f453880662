"""The benchmark's host logic (CPU): the one-GPU refusal, the algorithmic bytes behind the roofline fraction
(written out from the weight formats), the counter record's staleness check and the step statistics."""
import os
import shutil
import subprocess
import sys

import pytest

import bench
from expert_ffn_canvas_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert '"error"' in r.stdout and '"n_gpus": 2' in r.stdout


def test_expert_bytes_per_format():
    # d_model 2816, d_ff 704: gate_up is [2 F, D], down [D, F]
    D, F = 2816, 704
    w = {k: synth.WORKLOADS[k] for k in ("canvas256", "int4", "q8", "mxfp4", "mxfp8")}
    assert bench.expert_bytes(w["canvas256"]) == (2 * F * D * 2, D * F * 2)                       # bf16
    # int4: half a byte per weight, an fp16 scale per 128 inputs (the last down group 64 wide)
    assert bench.expert_bytes(w["int4"]) == (2 * F * D // 2 + 2 * F * 22 * 2, D * F // 2 + D * 6 * 2)
    assert bench.expert_bytes(w["q8"]) == (2 * F * (D // 32) * 34, D * (F // 32) * 34)           # 34 B / 32
    assert bench.expert_bytes(w["mxfp4"]) == (2 * F * (D // 32) * 17, D * (F // 32) * 17)        # 17 B / 32
    assert bench.expert_bytes(w["mxfp8"]) == (2 * F * (D // 32) * 33, D * (F // 32) * 33)        # 33 B / 32


def test_canvas256_launch_bytes():
    # the fused launch's algorithmic bytes at canvas256: the 82 experts the batch touches (bf16 weights) and
    # the 256 input rows; the layer adds the router weight, the two norms, the bias and the output rows
    wl = synth.WORKLOADS["canvas256"]
    layer, flops, gemm, gate_up = bench.algorithmic(wl, 256, 82)
    assert gemm == 82 * (3 * 704 * 2816 * 2) + 256 * 2816 * 2 == 976814080
    assert layer == gemm + 128 * 2816 * 2 + 2 * 2816 * 4 + 128 * 4 + 256 * 2816 * 2
    assert flops == 256 * 8 * 2 * 3 * 2816 * 704 + 256 * 2 * 128 * 2816


def _record(tmp_path, digest):
    src = os.path.join(ROOT, "profiles", "canvas256_gemm_counters.txt")
    text = open(src).read()
    lines = [("source_digest = " + digest) if ln.startswith("source_digest") else ln for ln in text.splitlines()]
    (tmp_path / "canvas256_gemm_counters.txt").write_text("\n".join(lines) + "\n")


def test_counter_record_only_for_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    _record(tmp_path, bench.kernel_sources_digest())
    rec = bench.read_counters("canvas256", "gate_up+down")
    assert rec is not None and rec["traffic_bytes_per_launch"] > 0 and rec["rocprof_avg_us"] > 0
    assert bench.read_counters("encode2304", "gate_up+down") is None      # no record for that workload here
    assert bench.read_counters("canvas256", "router") is None             # another kernel's
    _record(tmp_path, "0" * 16)
    assert bench.read_counters("canvas256", "gate_up+down") is None       # taken on other sources


def test_digest_ignores_comments_only(tmp_path, monkeypatch):
    csrc = tmp_path / "expert_ffn_canvas_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "expert_ffn_canvas_amd", "csrc"), csrc,
                    ignore=shutil.ignore_patterns("*.o", "*.so"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_sources_digest()
    f = csrc / "permute.hip"
    f.write_text(f.read_text() + "\n// a comment\n")
    assert bench.kernel_sources_digest() == d0
    f.write_text(f.read_text().replace("constexpr int kStage = 20480;", "constexpr int kStage = 20000;"))
    assert bench.kernel_sources_digest() != d0


def test_percentiles():
    p = bench.percentiles([float(v) for v in range(1, 12)])  # 1 .. 11
    assert p["median"] == 6 and p["min"] == 1 and p["max"] == 11 and p["n"] == 11
    assert p["p10"] == 2 and p["p90"] == 10 and p["spread_p90_p10"] == pytest.approx(5.0)
