"""bench.py's bookkeeping, on the CPU: which sources key a kernel's counter
figures, when a committed traffic figure is used (it must have been counted
on the current sources, at the same block_m), and that every committed
traffic summary names a kernel, workload and tile size the bench can match."""
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_sources_follow_the_gemm_family():
    assert bench.kernel_sources("gemm_gate_up", 16)[0] == "gemm.hip"
    assert bench.kernel_sources("gemm_down", 32)[0] == "gemm.hip"
    for bm in (64, 128, 192, 256):
        assert bench.kernel_sources("gemm_gate_up", bm)[:2] == ["gemm_dma.hip", "gemm_expand.h"]
    for stage in ("gemm_gate_up", "shrink_down", "align", "route", "combine"):
        for name in bench.kernel_sources(stage, 256):
            assert os.path.exists(os.path.join(ROOT, "lora_moe_amd", "csrc", name)), name


def test_kernel_source_sha_changes_with_the_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "lora_moe_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("gemm_dma.hip", "gemm_expand.h", "device_util.h", "internal.h"):
        (csrc / name).write_text("// " + name + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    a = bench.kernel_source_sha("gemm_gate_up", 256)
    assert a == bench.kernel_source_sha("gemm_down", 128)  # same family, same files
    (csrc / "gemm_expand.h").write_text("// changed\n")
    assert bench.kernel_source_sha("gemm_gate_up", 256) != a


def _profile(path, sha, block_m, traffic=123456789):
    path.write_text("# HBM traffic of gemm_gate_up, workload w\n\n"
                    "Values read by bench.py:\n\n"
                    f"kernel: gemm_gate_up\nworkload: w\nblock_m: {block_m}\n"
                    f"kernel_source_sha: {sha}\ntraffic_bytes_per_launch: {traffic}\n")


def test_measured_traffic_only_while_current(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda stage, bm: "cafe0123")
    f = tmp_path / "profiles" / "traffic_gemm_gate_up_w.txt"
    assert bench.measured_traffic("gemm_gate_up", "w", 256) is None  # no summary
    _profile(f, "cafe0123", 256)
    assert bench.measured_traffic("gemm_gate_up", "w", 256) == 123456789.0
    assert bench.measured_traffic("gemm_gate_up", "w", 192) is None  # counted at another tile size
    _profile(f, "beef4567", 256)
    assert bench.measured_traffic("gemm_gate_up", "w", 256) is None  # sources changed since


@pytest.mark.parametrize("name", sorted(n for n in os.listdir(os.path.join(ROOT, "profiles"))
                                        if n.startswith("traffic_")))
def test_committed_traffic_summaries_are_well_formed(name):
    vals = {}
    for line in open(os.path.join(ROOT, "profiles", name)):
        if ":" in line and not line.startswith(("#", " ", "`")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    assert name == f"traffic_{vals['kernel']}_{vals['workload']}.txt"
    assert int(vals["block_m"]) in (16, 32, 64, 128, 192, 256)
    assert len(vals["kernel_source_sha"]) == 16
    assert float(vals["traffic_bytes_per_launch"]) > 0
