"""bench.py's contract pieces that run without a GPU: the one-GPU refusal,
the kernel it names for each workload agrees with the kernel the library's
plan says it will launch, the roofline arithmetic, and the staleness guard
of the committed counter figures."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import bench
import lm_synth
import stft_log_mel_amd as lm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", sorted(lm_synth.WORKLOADS))
def test_bench_names_the_kernel_the_plan_launches(name):
    w = lm_synth.WORKLOADS[name]
    if w.entry == "stft":
        text = lm.Plan(400, 160, w.NM).describe()
        line = [l for l in text.splitlines() if l.startswith("lm_from_stft:")][0]
    else:
        p = lm.Plan(w.n_fft, w.hop, w.n_mels, w.center, w.pad_mode, w.power, w.out_dtype)
        p.set_mel(w.sample_rate, w.f_min, w.f_max)
        line = [l for l in p.describe().splitlines() if l.startswith("lm_from_pcm:")][0]
    assert bench.main_kernel_name(w) in line, (bench.main_kernel_name(w), line)


def test_roofline_arithmetic():
    w = lm_synth.WORKLOADS["pcm_i16_b64"]
    r = bench.roofline_of(w, 0.1)                       # 0.1 ms per launch
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["algorithmic_bytes_per_launch"] == 64 * 480000 * 2 + 64 * 128 * 3001 * 4
    assert abs(r["achieved"] - r["algorithmic_bytes_per_launch"] / 1e-4 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4
    big = lm_synth.WORKLOADS["pcm_f32_nfft16384"]
    r = bench.roofline_of(big, 0.1)
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s" and r["peak"] == 157.3
    frames = 16 * 108
    assert r["algorithmic_flops_per_launch"] == round(frames * bench.flops_per_frame(big))
    assert abs(r["frac"] - r["achieved"] / 157.3) < 1e-4


def test_counter_figures_are_reported_only_for_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    rec = {"pcm_i16_b64": {"source_hash": bench.kernel_source_hash(), "bytes_per_launch": 123}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.counter_traffic("pcm_i16_b64") == 123
    rec["pcm_i16_b64"]["source_hash"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.counter_traffic("pcm_i16_b64") is None
    assert bench.counter_traffic("no_such_workload") is None


def test_committed_counter_records_name_their_kernel():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        rec = json.load(fh)
    for name, r in rec.items():
        if name.startswith("_"):
            continue
        assert name in lm_synth.WORKLOADS
        assert r["kernel"] == bench.main_kernel_name(lm_synth.WORKLOADS[name])
        assert r["bytes_per_launch"] == r["fetch_bytes"] + r["write_bytes"]
        assert len(r["source_hash"]) == 16


def test_floored_share_counts_values_and_regions_at_the_clip_floor():
    import numpy as np
    w = lm_synth.WORKLOADS["pcm_f32_b8"]          # n_fft 400: regions of 16 frames x 4 bands
    got = np.full((2, 8, 40), 1.0, dtype=np.float32)
    got[0, 0, 0] = 3.0                             # clip 0: largest output 3, floor 1
    got[1, 0, 0] = 2.5                             # clip 1: floor 0.5, nothing at it
    got[0, 5, 33] = 1.5
    r = bench.floored_share(w, got)
    assert r["values_at_floor"] == round((8 * 40 - 2) / (2 * 8 * 40), 7)
    # clip 0: 2 band groups x 3 frame groups, all hold a floored value; clip 1: none
    assert r["regions"] == 12 and r["regions_holding_floored_values"] == 0.5
    big = lm_synth.WORKLOADS["pcm_f32_nfft16384"]  # one frame x all bands
    g2 = np.zeros((1, 4, 3), dtype=np.float32)
    g2[0, :, 1] = 2.0
    r2 = bench.floored_share(big, g2)
    assert r2["regions"] == 3 and abs(r2["regions_holding_floored_values"] - 2 / 3) < 1e-6
