"""Host-side logic of bench.py: the stored HBM counter summaries and the
kernel-source hash that decides whether a summary still applies.  No GPU."""
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _fields(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip().split()[0]
    return kv


def test_every_traffic_summary_is_consistent():
    for cfg, (name, sources) in bench.TRAFFIC_FILES.items():
        path = os.path.join(ROOT, "profiles", name)
        assert os.path.exists(path), name
        kv = _fields(path)
        # read and write bytes are the counter readings times the copy-calibrated scale
        rd = float(kv["fetch_size_kib_per_dispatch"]) * 1024 * float(kv["fetch_scale"])
        wr = float(kv["write_size_kib_per_dispatch"]) * 1024 * float(kv["write_scale"])
        assert abs(rd - float(kv["hbm_read_bytes_per_launch"])) < 1e-4 * rd, name
        assert abs(rd + wr - float(kv["traffic_bytes_per_launch"])) < 1e-4 * (rd + wr), name
        # a kernel cannot read less than the K/V bytes it attends over
        assert float(kv["hbm_read_bytes_per_launch"]) >= 0.999 * float(kv["algorithmic_kv_bytes_per_launch"]), name
        assert re.fullmatch(r"[0-9a-f]{16}", kv["kernel_source_sha256_16"]), name
        got = bench.read_traffic(cfg)
        if kv["kernel_source_sha256_16"] == bench.kernel_source_hash(sources):
            assert got == float(kv["traffic_bytes_per_launch"])
        else:  # taken on other kernel code: reported as unknown
            assert got is None


def test_configs_without_a_summary_report_no_traffic():
    # the tiny fp32 workload (a launch-latency case) has no counter summary
    assert 1 not in bench.TRAFFIC_FILES
    assert bench.read_traffic(1) is None
    assert set(bench.TRAFFIC_FILES) == {2, 3, 4, 5}


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) { return x + 1; }  // one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash(["a.hip"])
    a.write_text("/* doc */\nint f(int x)\n{\n  return x + 1;  // another comment\n}\n")
    assert bench.kernel_source_hash(["a.hip"]) == h0
    a.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash(["a.hip"]) != h0


def test_every_counter_summary_is_consistent():
    """The MFMA busy fraction is the MFMA busy cycles over active cycles x
    1024 SIMDs, and the busy cycles are the MFMA instructions times their
    cycles (32 for 32x32x16, 16 for 16x16x32)."""
    for cfg, (name, sources) in bench.COUNTER_FILES.items():
        path = os.path.join(ROOT, "profiles", name)
        assert os.path.exists(path), name
        kv = _fields(path)
        cyc = float(kv["GRBM_GUI_ACTIVE"]) / 8
        assert abs(cyc - float(kv["active_cycles_per_xcd"])) < 1, name
        frac = float(kv["SQ_VALU_MFMA_BUSY_CYCLES"]) / (cyc * 1024)
        assert abs(frac - float(kv["mfma_busy_frac"])) < 1e-4, name
        per = float(kv["SQ_VALU_MFMA_BUSY_CYCLES"]) / float(kv["SQ_INSTS_MFMA"])
        assert per in (16.0, 32.0), name
        assert 0 < frac < 1 and 0 < float(kv["valu_issue_frac"]) < 1, name
        got = bench.read_counters(cfg)
        if kv["kernel_source_sha256_16"] == bench.kernel_source_hash(sources):
            assert got["mfma_busy_frac"] == float(kv["mfma_busy_frac"])
        else:
            assert got is None
