"""Host logic of bench.py (no GPU): the one-GPU rule, the scaling of the
rocprofv3 counters by the calibration copy, the source-hash check that keeps
a stale traffic record out of the JSON line, and the committed records."""
import glob
import json
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def _counter_csv(d, counter, rows):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f'"{name}",{counter},{value}\n')


def test_pmc_summary_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    split = "void fd::(anonymous namespace)::split_valu_kernel<128>(fd::SplitParams)"
    copy = "__amd_rocclr_copyBuffer"
    copy_kib = bench.COPY_BYTES / 1024 / 2          # the counter reads half of a known copy
    _counter_csv(str(tmp_path / "f"), "FETCH_SIZE",
                 [(split, 1000.0), (split, 1002.0), (copy, 10.0), (copy, copy_kib)])
    _counter_csv(str(tmp_path / "w"), "WRITE_SIZE", [(split, 8.0), (copy, bench.COPY_BYTES / 1024)])
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel="mfma": f"hash-{kernel}")
    bench.pmc_summary("wl", str(tmp_path / "f"), str(tmp_path / "w"))
    rec = json.load(open(tmp_path / "profiles" / "traffic_split_wl.json"))
    assert rec["kernel"] == "valu" and rec["kernel_source_hash"] == "hash-valu"
    assert rec["fetch"]["scale"] == pytest.approx(2.0)
    assert rec["fetch"]["bytes_per_launch"] == pytest.approx(1001.0 * 1024 * 2)
    assert rec["write"]["bytes_per_launch"] == pytest.approx(8.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(1001.0 * 2048 + 8.0 * 1024)
    # the record is used only while the sources it was taken on are unchanged
    assert bench.traffic_from_profile("wl", "hash-valu") == pytest.approx(rec["bytes_per_launch"])
    assert bench.traffic_from_profile("wl", "hash-mfma") is None
    assert bench.traffic_from_profile("other", "hash-valu") is None


def test_source_hash_names_its_kernel():
    assert bench.kernel_source_hash("mfma") != bench.kernel_source_hash("valu")
    assert bench.kernel_source_hash("mfma") == bench.kernel_source_hash()


def test_committed_traffic_records_are_consistent():
    paths = glob.glob(os.path.join(ROOT, "profiles", "traffic_split_*.json"))
    assert any(p.endswith("traffic_split_gqa64x8_f16_L128000.json") for p in paths)
    for p in paths:
        rec = json.load(open(p))
        assert os.path.basename(p) == f"traffic_split_{rec['workload']}.json"
        assert rec["workload"] in bench.WORKLOADS
        assert rec.get("kernel", "mfma") in ("mfma", "valu")
        assert len(rec["kernel_source_hash"]) == 16
        assert rec["bytes_per_launch"] == pytest.approx(rec["fetch"]["bytes_per_launch"] +
                                                        rec["write"]["bytes_per_launch"])
        for key in ("fetch", "write"):
            c = rec[key]
            assert c["scale"] == pytest.approx(rec["copy_bytes"] / (c["copy_kib_per_dispatch"] * 1024))
            assert c["bytes_per_launch"] == pytest.approx(c["split_kib_per_dispatch"] * 1024 * c["scale"])


def test_cpu_baseline_leg_on_the_tiny_workload():
    w = bench.make_workload("tiny_mha_f32_L1000", "cpu")
    cb, ref, pairs = bench.cpu_baseline(w, 64)
    assert cb["kind"] == "oracle" and cb["unit"] == "TB/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert len(pairs) == 4 and len(ref) == 4
    assert "passes" in cb["sample"] and "(1.000)" in cb["sample"]


def _profile_commands():
    """The bench.py arguments of every command the profile summaries print."""
    import re

    cmds = []
    for md in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        text = open(md).read().replace("\\\n", " ")
        for line in text.splitlines():
            m = re.search(r"bench\.py((?: --?[\w-]+(?: [\w./<>-]+)*)*)\s*$", line.strip())
            if m and "bench.py" in line and "`" not in line:
                cmds.append((os.path.basename(md), m.group(1).split()))
    return cmds


def test_profile_commands_parse_with_this_bench():
    cmds = _profile_commands()
    assert len(cmds) >= 12                      # trace, counter passes and summaries of four workloads
    parser = bench.build_parser()
    for md, argv in cmds:
        args = parser.parse_args(argv)
        assert args.workload in bench.WORKLOADS, (md, argv)


def test_trace_follow_reads_kernels_by_their_predecessor(tmp_path, capsys):
    """--trace-follow: each kernel's traced duration and the gap before it,
    keyed by the kernel that ran before it on the same queue."""
    import csv as _csv
    import json as _json

    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    rows = [  # queue, name, start, end (ns)
        (1, "fd::split_mfma_kernel", 0, 80_000), (1, "fd::merge_kernel<128>", 80_000, 84_500),
        (1, "fd::split_mfma_kernel", 84_500, 164_500), (1, "at::elementwise_kernel", 164_500, 169_100),
        (1, "at::elementwise_kernel", 169_100, 173_700), (2, "fd::split_mfma_kernel", 0, 70_000),
        (1, "fd::split_mfma_kernel", 174_700, 254_700), (1, "fd::merge_kernel<128>", 254_700, 259_500),
    ]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        wr = _csv.writer(f)
        wr.writerow(["Queue_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writerows(rows)
    bench.trace_follow(str(tmp_path / "trace"))
    out = _json.loads(capsys.readouterr().out)
    assert out["merge_kernel after split_mfma"] == {"n": 2, "us_p10_p50_p90": [4.53, 4.65, 4.77], "gap_us_p50": 0.0}
    assert out["elementwise after split_mfma"]["n"] == 1 and out["elementwise after elementwise"]["n"] == 1
    assert out["split_mfma after elementwise"]["gap_us_p50"] == 1.0          # 173.7 -> 174.7 us
    assert all("queue" not in k for k in out) and sum(v["n"] for v in out.values()) == 6
