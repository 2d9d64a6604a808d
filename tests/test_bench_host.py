"""Host-side logic of bench.py, on the CPU: the one-GPU contract, the
roofline arithmetic of the JSON line, and the rule that profiled counters
are reported only for the GEMM sources they were taken on."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_padded_ratio_rounds_each_group_up_to_128():
    assert bench._padded_ratio({}) is None
    # 1 -> 128, 128 -> 128, 129 -> 256, 0 -> 0
    assert bench._padded_ratio({"group_sizes": [1, 128, 129, 0]}) == pytest.approx(512 / 258)


class _Stage:
    def __init__(self, kernel, flops=0.0, nbytes=0.0, name=""):
        self.kernel, self.flops, self.bytes, self.name = kernel, flops, nbytes, name


def test_kernel_table_and_gemm_roofline():
    # two GEMM launches of 2 and 4 TFLOP taking 1 ms and 2 ms, one 3 GB
    # bandwidth launch taking 1 ms; the second GEMM moves 16 GB (HBM-bound:
    # 2 ms at 8 TB/s against 0.8 ms of MFMA)
    stages = [_Stage("g", 2e12, name="a"), _Stage("q", 0.0, 3e9), _Stage("g", 4e12, name="b")]
    out, table = bench._kernel_table(stages, [1e-3, 1e-3, 2e-3], {"a": 1e9, "b": 16e9})
    assert out["g"] == {"launches_per_step": 2, "ms_per_step": 3.0, "avg_launch_us": 1500.0,
                        "useful_tflops": 2000.0, "mfma_floor_us": 600.0, "hbm_floor_us": 1062.5,
                        "roofline_frac": round((0.4e-3 + 2e-3) / 3e-3, 4)}
    assert out["q"]["gbps"] == 3000.0 and "useful_tflops" not in out["q"]
    r = bench._roofline_gemm(table, "g", 5.0e15, traffic=123.0, padded_ratio=1.25,
                             mfma={"mfma_busy": 0.6, "sclk_ghz": 2.0})
    assert r["achieved"] == 2000.0 and r["peak"] == 5000.0 and r["frac"] == 0.4
    assert r["per_launch_flops"] == 3e12 and r["avg_launch_us"] == 1500.0
    assert r["padded_tflops"] == 2500.0 and r["traffic"] == 123.0
    assert r["mfma_busy_profiled"] == 0.6 and r["sclk_ghz_profiled"] == 2.0
    assert bench._roofline_gemm(table, "g", 5.0e15)["traffic"] is None


def test_profile_values_only_for_matching_sources(tmp_path):
    body = "# title\n\n| a | b |\n- note: ignored\ntraffic_bytes_per_launch: 42\n"
    good = tmp_path / "good.md"
    good.write_text(body + f"source_sha256: {bench.gemm_source_hash()}\n")
    stale = tmp_path / "stale.md"
    stale.write_text(body + "source_sha256: " + "0" * 64 + "\n")
    kv = bench._profile_values(str(good))
    assert kv["traffic_bytes_per_launch"] == "42" and "- note" not in kv
    assert bench._profile_values(str(stale)) is None
    assert bench._profile_values(str(tmp_path / "missing.md")) is None


def test_source_hash_covers_the_gemm_sources():
    for rel in bench.GEMM_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, rel)), rel
    assert len(bench.gemm_source_hash()) == 64


def test_gemm_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    """Counters stay valid across comment edits of the GEMM sources and are
    dropped when their code changes."""
    import shutil
    for rel in bench.GEMM_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.gemm_source_hash()
    assert base == bench.gemm_source_hash()
    src = tmp_path / "quantize_grouped_gemm_amd/csrc/mx_gemm.hip"
    text = src.read_text()
    src.write_text(text.replace("#include \"mx_device.h\"",
                                "// a new comment line\n\n#include \"mx_device.h\"  /* and a block comment */", 1))
    assert bench.gemm_source_hash() == base
    src.write_text(text.replace("constexpr int kPfOps = 2;", "constexpr int kPfOps = 3;", 1))
    assert "constexpr int kPfOps = 2;" in text
    assert bench.gemm_source_hash() != base
