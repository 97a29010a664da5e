"""bench.py's host logic, on the CPU: ring sizing and its labels, the
kernel-trace reduction that the committed profiles come from, and the
source digests that tie those profiles to the kernels they measured."""
import csv
import os

import pytest

import bench as B


def test_ring_slots_cover_the_ring_or_raise():
    # a prefill launch: enough buffer sets to cover the ring bytes
    r = B.ring_slots(59_261_952)
    assert r * 59_261_952 >= B.RING_BYTES and (r - 1) * 59_261_952 < B.RING_BYTES
    assert B.ring_mode(59_261_952, r) == "cold"
    assert B.ring_slots(10**12) == 8                     # never fewer than 8 sets
    # a decode-width call would need more sets than one captured graph may hold
    with pytest.raises(ValueError):
        B.ring_slots(10_240)
    r = B.ring_slots(10_240, cache_resident_ok=True)
    assert r == B.MAX_SLOTS
    assert B.ring_mode(10_240, r) == "cache-resident"
    assert B.ring_mode(150_000, B.MAX_SLOTS) == "partly cache-resident"


def _trace(path, rows):
    cols = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
            "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for name, grid, t0, dur in rows:
            w.writerow([name, grid, 1, 1, t0, t0 + dur])


def test_trace_stats_groups_and_runs(tmp_path):
    qa = "void mbt::(anonymous namespace)::qknorm_rope_vec<2, 8, 4, 0, false, 1>(mbt::QkParams)"
    qb = "void mbt::(anonymous namespace)::qknorm_rope_vec<2, 16, 2, 0, false, 0>(mbt::QkParams)"
    cp = "__amd_rocclr_copyBuffer"
    # out of order in the file: the reduction sorts by start time
    rows = [(qa, 100, 3000, 10), (qa, 100, 1000, 10), (cp, 7, 2000, 5), (qa, 100, 2500, 30),
            (qb, 50, 4000, 4), (qb, 50, 5000, 6), (qa, 100, 6000, 20)]
    src, dst = tmp_path / "t.csv", tmp_path / "s.csv"
    _trace(src, rows)
    B.trace_stats(str(src), str(dst))
    groups, runs, us = B._read_stats(str(dst))
    g = groups[("qknorm_rope_vec<2, 8, 4, 0, false, 1>", "100x1x1")]
    assert int(g["Calls"]) == 4 and float(g["AverageNs"]) == 17.5
    assert int(groups[("__amd_rocclr_copyBuffer", "7x1x1")]["Calls"]) == 1
    # runs: consecutive prologue launches of one (kernel, grid), copies ignored
    assert [(r["Name"][:20], int(r["Calls"])) for r in runs] == [
        ("qknorm_rope_vec<2, 8", 3), ("qknorm_rope_vec<2, 1", 2), ("qknorm_rope_vec<2, 8", 1)]
    assert us(runs[1], "AverageNs") == 0.005


def test_source_digest_ignores_comments(tmp_path):
    a = "int f() { return 1; } // one\n/* block\n comment */\n"
    b = "int f() { return 1; }\n\n// another comment\n"
    assert B._code_only(a, False) == B._code_only(b, False)
    assert B._code_only("x = 1\n# note\n", True) == B._code_only("x = 1\n", True)
    assert B._code_only("int f() { return 2; }", False) != B._code_only(a, False)
    d = B.source_digest("qknorm_rope")
    assert len(d) == 64 and d != B.source_digest("rmsnorm")


def test_profile_records_follow_the_sources():
    """The committed profiles carry the digest of the kernels they measured;
    bench.py reports their figures only while the digest matches."""
    rec = B._profile_record("traffic.json", "prologue_prefill", "qknorm_rope")
    if rec is None:
        pytest.skip("profiles/traffic.json predates the current prologue source")
    assert rec["hbm_bytes_per_launch"] > rec["algorithmic_bytes_per_launch"] * 0.99
    assert B.traffic_for("prologue_prefill", "qknorm_rope") == rec["hbm_bytes_per_launch"]
    avg, med = B.rocprof_us_for(B.prefill_cell(__import__("workloads")).name)
    assert avg is not None and 5.0 < avg < 20.0
    # the headline's figure comes from the default run under the tracer
    avg, med = B.headline_rocprof_us()
    assert avg is not None and 5.0 < avg < 20.0 and 5.0 < med < 20.0


def test_multi_gpu_request_exits(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        B.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("threads", [1, 2])
def test_cpu_baseline_fields_and_affinity(threads):
    # the oracle leg on a tiny sample (two tokens per thread and call): the
    # fields the JSON line carries, quartiles around the median, and the
    # process's CPU affinity restored after the pinned single-thread leg
    import workloads as W
    before = os.sched_getaffinity(0)
    r = B.cpu_baseline(W, B.prefill_cell(W), threads=threads, tokens_per_call=2)
    assert os.sched_getaffinity(0) == before
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["cores"] == threads
    assert 0 < r["p25"] <= r["value"] <= r["p75"]
    assert r["cores_visible"] == len(before)
    assert f"on {2 * threads} of the headline cell's 2048 tokens" in r["sample"]
