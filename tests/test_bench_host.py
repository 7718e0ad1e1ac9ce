"""Host-side logic of bench.py, without a GPU: the algorithmic byte counts per
expert against the layouts' sizes, the roofline class of every workload the
line reports, the rescaling of derived figures when a step time is replaced,
the counter record's source-hash check, and the one-GPU refusal."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

import moe_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
B = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(B)


def test_packed_bytes_per_expert_match_the_layouts():
    # NF4: codes [2I, H/2] u8 + fp32 absmax [2I, H/64]; down [H, I/2] + [H, I/64]
    g, d = B.packed_bytes_per_expert(S.WORKLOADS["olmoe_decode"])
    assert (g, d) == (2 * 1024 * (2048 // 2 + 4 * 2048 // 64), 2048 * (1024 // 2 + 4 * 1024 // 64))
    assert (g, d) == (2_359_296, 1_179_648)
    # MXFP4: e8m0 bytes per 32
    g, d = B.packed_bytes_per_expert(S.WORKLOADS["gptoss_mxfp4"])
    assert (g, d) == (8_812_800, 4_406_400)
    # bf16 absmax: 2 bytes per 64 (the page's 5.6 % fewer bytes per NF4 row)
    g2, _ = B.packed_bytes_per_expert(B.workload("olmoe_decode", absmax_bf16=True))
    assert g2 == 2 * 1024 * (1024 + 2 * 32)
    assert abs(1 - g2 / 2_359_296 - 0.0556) < 1e-3


@pytest.mark.parametrize("name,T,active,bound", [
    ("olmoe_decode", 1, 8, "hbm"),         # 3.6 flop/B
    ("olmoe_prefill", 4096, 64, "mfma"),   # 1820 flop/B
    ("qwen3_zipf", 512, 66.9, "hbm"),      # ~210 flop/B
    ("gptoss_mxfp4", 2048, 128, "hbm"),    # ~241 flop/B
])
def test_roofline_class_follows_intensity(name, T, active, bound):
    wl = S.WORKLOADS[name]
    got, intensity = B.roofline_class(wl, T, active)
    assert got == bound
    g, d = B.packed_bytes_per_expert(wl)
    assert intensity == pytest.approx(6.0 * T * wl.top_k * wl.H * wl.I / (active * (g + d)))
    assert (intensity > B.RIDGE_FLOP_PER_BYTE) == (bound == "mfma")
    assert B.RIDGE_FLOP_PER_BYTE == pytest.approx(312.5)


def test_retime_rescales_every_derived_figure():
    res = {"ms_per_step": 2.0, "tokens_per_s": 500.0, "effective_packed_GBps": 10.0,
           "algorithmic_TFLOPs": 3.0, "layer_roofline_frac": 0.25}
    B.retime(res, 4.0, T=1)
    assert res == {"ms_per_step": 4.0, "tokens_per_s": 250.0, "effective_packed_GBps": 5.0,
                   "algorithmic_TFLOPs": 1.5, "layer_roofline_frac": 0.125}


def test_traffic_record_is_tied_to_the_kernel_sources(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for key, kind in (("olmoe_decode", "small"), ("olmoe_prefill", "mfma")):
        fresh = rec[key]["source_hash"] == B.kernel_source_hash(kind)
        want = float(rec[key]["hbm_bytes_per_launch"]) if fresh else None
        assert B.measured_traffic(key, kind) == want
    # a record whose hash does not match the sources reads as absent
    bad = dict(rec)
    bad["olmoe_decode"] = dict(rec["olmoe_decode"], source_hash="0" * 16)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(bad))
    real = B.kernel_source_hash("small")
    monkeypatch.setattr(B, "kernel_source_hash", lambda kind: real)
    monkeypatch.setattr(B, "ROOT", str(tmp_path))
    assert B.measured_traffic("olmoe_decode", "small") is None
    assert B.measured_traffic("no_such_workload", "small") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
