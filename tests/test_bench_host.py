"""Host-side arithmetic of the benchmark: the algorithmic bytes per scored
position that the roofline figures rest on, the cold-input rotation, and the
rule that a counter record counts only for the kernel sources it was taken
on."""
import json

import bench


def test_bytes_per_scored_position():
    # bf16 rows of V = 152064: p and q rows (2 * V * 2 B), the drafted token,
    # the 16-byte statistics record and the 4-byte alpha; greedy reads p only
    assert bench.bytes_per_row_pair(152064, 2) == 2 * 152064 * 2 + 24 == 608280
    assert bench.bytes_per_row_pair(152064, 2, "greedy") == 152064 * 2 + 24 == 304152
    assert bench.bytes_per_row_pair(32, 4) == 2 * 32 * 4 + 24


def test_batched_serving_launch_bytes():
    # 2048 scored positions per launch: 1.2458 GB
    assert abs(bench.bytes_per_row_pair(152064, 2) * 2048 / 1e9 - 1.2458) < 1e-4


def test_cold_input_copies():
    gib = 1 << 30
    assert bench.input_copies(2 * gib) == 1          # larger than the rotation target
    assert bench.input_copies(gib) == 1
    assert bench.input_copies(gib // 2) == 2
    assert bench.input_copies(17 * 304128) == 208    # single stream: 9 p rows and 8 q rows
    assert bench.input_copies(1) == 512              # capped


def test_counter_record_needs_matching_sources(tmp_path, monkeypatch):
    # a record counts only while the kernel's sources hash to its kernel_hash
    # and it was taken on the same workload
    rec = {"kernel": "kr_rowstats", "workload": "batched_serving", "mode": "standard",
           "kernel_hash": bench.kernel_hash("rowstats"), "hbm_bytes_per_launch": 123.0}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "kr_rowstats_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # kernel_hash reads the sources under ROOT: point it back at the repository
    monkeypatch.setattr(bench, "kernel_hash", lambda k, h=rec["kernel_hash"]: h)
    assert bench.measured_traffic("rowstats", "batched_serving") == 123.0
    assert bench.measured_traffic("rowstats", "self_selection") is None
    rec["kernel_hash"] = "0" * 16
    (tmp_path / "profiles" / "kr_rowstats_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("rowstats", "batched_serving") is None


def test_committed_records_match_their_kernels():
    # the committed counter records were taken on the committed kernel sources
    for kern, mode in (("rowstats", "standard"), ("rowstats", "greedy"),
                       ("pool_stats", "standard"), ("pool_stats", "greedy"),
                       ("lattice", "standard")):
        with open(bench.traffic_file(kern, mode)) as f:
            rec = json.load(f)
        assert rec["kernel_hash"] == bench.kernel_hash(kern), (kern, mode)
        assert 1.0 <= rec["traffic_over_algorithmic"] < 1.01, (kern, mode)


def test_lattice_algorithmic_bytes():
    # one read of each of the 256 drafter rows, plus the 15 candidates (token and
    # log-probability) and the count written per row
    rec = json.load(open(bench.traffic_file("lattice")))
    assert rec["algorithmic_bytes_per_launch"] == 256 * (152064 * 2 + 15 * 8 + 8)
    assert rec["workload"] == "cps_shared_marginal"
