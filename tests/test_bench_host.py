"""Host logic of bench.py's roofline: the counter-derived HBM traffic it reports
comes from the committed rocprofv3 summary of the same precision's kernels, and
only while the GEMM source is the one the counters were taken on."""
import glob
import os

import bench


def _fields(path):
    out = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def test_traffic_file_is_per_precision():
    names = {p: os.path.basename(bench.traffic_file("gpt96l-tp8", "fc1_bwd", p)) for p in ("bf16", "fp8", "mxfp4")}
    assert names["bf16"] == "gemm_fc1_bwd_gpt96l-tp8_traffic.txt"
    assert names["fp8"] == "gemm_fc1_bwd_fp8_gpt96l-tp8_traffic.txt"
    assert names["mxfp4"] == "gemm_fc1_bwd_mxfp4_gpt96l-tp8_traffic.txt"


def test_committed_traffic_summaries_are_consistent():
    paths = sorted(glob.glob(os.path.join(bench.HERE, "profiles", "gemm_*_traffic.txt")))
    assert paths
    for p in paths:
        f = _fields(p)
        traffic, alg = float(f["traffic_bytes_per_launch"]), float(f["algorithmic_bytes_per_launch"])
        assert traffic > 0 and alg > 0, p
        assert abs(traffic / alg - float(f["traffic_over_algorithmic"])) < 2e-3, p
        assert len(f["gemm_source_sha256_16"]) == 16, p


def test_stored_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    src = bench.traffic_file("gpt96l-tp8", "fc1_bwd", "bf16")
    if not os.path.exists(src):
        return
    f = _fields(src)
    profiles = tmp_path / "profiles"
    profiles.mkdir()
    text = open(src).read()
    (profiles / os.path.basename(src)).write_text(text)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: f["gemm_source_sha256_16"])
    assert bench.stored_traffic("gpt96l-tp8", "fc1_bwd", "bf16") == float(f["traffic_bytes_per_launch"])
    # another precision's kernels have no summary here, so no figure
    assert bench.stored_traffic("gpt96l-tp8", "fc1_bwd", "mxfp4") is None
    # once the GEMM source changes, the counters no longer describe it
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "0" * 16)
    assert bench.stored_traffic("gpt96l-tp8", "fc1_bwd", "bf16") is None
