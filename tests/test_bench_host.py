"""Host-side checks of bench.py: the one-GPU guard, the source-hash guard on committed
counter summaries, and the arithmetic of a measured leg.  No GPU is touched."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def _summary(tmp_path, name, tag, payload):
    (tmp_path / name).write_text("# summary\n\n%s: %s\n" % (tag, json.dumps(payload)))


def test_counter_summaries_are_used_only_for_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    good = bench._source_hash(bench.QMV_SOURCES)
    _summary(tmp_path, "t_ok.md", "traffic-json", {"source_hash": good, "hbm_bytes_per_launch": 123})
    _summary(tmp_path, "t_old.md", "traffic-json", {"source_hash": "0" * 16, "hbm_bytes_per_launch": 456})
    assert bench._traffic("t_ok.md", bench.QMV_SOURCES) == 123
    assert bench._traffic("t_old.md", bench.QMV_SOURCES) is None
    assert bench._traffic("missing.md", bench.QMV_SOURCES) is None
    # the decode and prefill kernels hash different source sets
    assert bench._traffic("t_ok.md", bench.QMM_T_SOURCES) is None
    _summary(tmp_path, "u.md", "mfma-util-json", {"source_hash": bench._source_hash(bench.QMM_T_SOURCES),
                                                  "mfma_util": 0.5})
    assert bench._profile_field("u.md", "mfma-util-json", bench.QMM_T_SOURCES, "mfma_util") == 0.5
    assert bench._profile_field("u.md", "traffic-json", bench.QMM_T_SOURCES, "mfma_util") is None


def test_committed_summaries_carry_a_hash_and_positive_figures():
    for name, tag, field in (("qmv_stream_kernel_lm_head_traffic.md", "traffic-json", "hbm_bytes_per_launch"),
                             ("qmm_prefill_dma_kernel_prefill_traffic.md", "traffic-json", "hbm_bytes_per_launch"),
                             ("qmm_prefill_dma_kernel_prefill_mfma_util.md", "mfma-util-json", "mfma_util")):
        lines = [ln for ln in open(os.path.join(ROOT, "profiles", name)) if ln.startswith(tag + ":")]
        assert len(lines) == 1, name
        d = json.loads(lines[0].split(":", 1)[1])
        assert len(d["source_hash"]) == 16 and d[field] > 0


def test_leg_divides_algorithmic_amount_by_the_two_times():
    t = {"wall_ms": 0.5, "kernel_ms": 0.4}
    leg = bench._leg("m", 2.0e9, t, "hbm", "GB/s", 8000.0, "k", {"workload": "w"})
    assert leg["value"] == pytest.approx(4000.0)            # 2 GB over 0.5 ms
    roof = leg["roofline"]
    assert roof["achieved"] == pytest.approx(5000.0)        # 2 GB over 0.4 ms
    assert roof["frac"] == pytest.approx(5000.0 / 8000.0)
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["kernel_ms"] == pytest.approx(0.4)
    flops = bench._leg("m", 2.5e12, t, "mfma", "TFLOP/s", 2500.0, "k", {"workload": "w"})
    assert flops["value"] == pytest.approx(5000.0)          # 2.5 TFLOP over 0.5 ms
    assert flops["roofline"]["frac"] == pytest.approx(6250.0 / 2500.0)


def test_host_info_names_the_cpu_and_blas():
    info = bench._host_info()
    assert info["nproc"] >= 1 and isinstance(info["cpu_model"], str) and info["numpy"]
