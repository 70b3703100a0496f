"""bench.py reads counter values from committed rocprofv3 summaries only while the kernel
sources they name are unchanged (host logic, no GPU): a summary whose recorded sha256 matches
the sources is used, one whose sha256 or sources differ is ignored (the bench line then says
null), and the VALU figure follows from the three SQ_INSTS counts and the launch time.
"""

import hashlib
import os

import bench

SOURCES = ["continuous_softmax_attention_amd/csrc/attn16.hpp", "continuous_softmax_attention_amd/build.py"]


def _sha(paths):
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(bench.ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _write(tmp_path, sha, sources=SOURCES, extra=""):
    p = tmp_path / "summary.md"
    p.write_text("# a summary\n| table | W = 1 |\n"
                 f"kernel_sources = {' '.join(sources)}\n"
                 f"kernel_source_sha256 = {sha}\n"
                 "csa_insts_valu = 1200\ncsa_insts_mfma = 200\ncsa_insts_trans = 100\n"
                 "csa_fetch_bytes = 1000\ncsa_write_bytes = 24\n" + extra)
    return str(p)


def test_matching_sources_are_used(tmp_path, monkeypatch):
    path = _write(tmp_path, _sha(SOURCES))
    kv = bench._profile_values(path)
    assert kv is not None and kv["csa_insts_valu"] == "1200"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    monkeypatch.setattr(bench, "ISSUE_FILE", path)
    assert bench.measured_traffic("lm") == 1024
    v = bench.measured_valu("lm", 1e-3)  # 1 us
    ops = 64.0 * 1000 / 1e-6
    assert abs(v["achieved"] - round(ops / 1e12, 2)) < 1e-9
    assert abs(v["frac"] - round(ops / bench.VALU_PEAK_LANE_OPS, 4)) < 1e-12
    weighted = 64.0 * (1000 + (bench.TRANS_ISSUE_WEIGHT - 1) * 100) / 1e-6
    assert abs(v["frac_trans_weighted"] - round(weighted / bench.VALU_PEAK_LANE_OPS, 4)) < 1e-12
    # other workloads have no committed counters
    assert bench.measured_traffic("long") is None and bench.measured_valu("stress", 1.0) is None


def test_changed_sources_are_ignored(tmp_path, monkeypatch):
    path = _write(tmp_path, "0" * 64)
    assert bench._profile_values(path) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    monkeypatch.setattr(bench, "ISSUE_FILE", path)
    assert bench.measured_traffic("lm") is None and bench.measured_valu("lm", 1.0) is None
    # a named source that does not exist
    path2 = _write(tmp_path, _sha(SOURCES), sources=SOURCES + ["no/such/file.hpp"])
    assert bench._profile_values(path2) is None
    # a missing summary
    assert bench._profile_values(str(tmp_path / "absent.md")) is None


def test_valu_peak_is_the_chip_unit_count():
    # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: one unpacked fp32 lane operation per cycle
    assert bench.VALU_PEAK_LANE_OPS == 256 * 4 * 16 * 2.4e9
