"""Host logic of bench.py that runs without a GPU: the HBM-counter and utilisation
summaries built from rocprofv3 CSV output, their source-hash check, and the refusal of
more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

bench = pytest.importorskip("bench")


def write_counter_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, value in rows:
            w.writerow([name, counter, value])


def test_counter_summary_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    copy = bench.COPY_KERNEL + "(void*)"
    copy_bytes = 512 * (1 << 20)
    # The copy's counters read half its bytes (fetch) and all of them (write): scales 2 and 1.
    fetch = [(copy, copy_bytes / 1024 / 2), (copy, copy_bytes / 1024 / 2 * 1.001), (copy, 10.0)]
    write = [(copy, copy_bytes / 1024), (copy, 20.0)]
    for i, (name, prefix, _) in enumerate(bench.COUNTED):
        kname = "void " + prefix + "<1>(int, int)"
        fetch += [(kname, 1000.0 * (i + 1)), (kname, 1000.0 * (i + 1)), (kname, 5000.0 * (i + 1))]
        write += [(kname, 100.0 * (i + 1))] * 3
    write_counter_csv(tmp_path / "fetch", "FETCH_SIZE", fetch)
    write_counter_csv(tmp_path / "write", "WRITE_SIZE", write)
    bench.summarize_counters(str(tmp_path / "fetch"), str(tmp_path / "write"), "cmd")
    for i, (name, _, src) in enumerate(bench.COUNTED):
        with open(tmp_path / "profiles" / f"{name}_counters.txt") as f:
            c = json.load(f)
        assert c["dispatches"] == [3, 3]
        assert c["fetch_kib_median"] == 1000.0 * (i + 1)            # the median, not the outlier
        assert abs(c["fetch_scale"] - 2.0) < 0.01 and c["write_scale"] == 1.0
        assert abs(c["fetch_bytes_scaled"] - 1000.0 * (i + 1) * 1024 * c["fetch_scale"]) < 1e-6
        assert c["kernel_src_sha"] == bench.src_digest(*src)
        # traffic is fetched + written bytes while the sources are unchanged ...
        t = bench.traffic_of(name)
        assert t == pytest.approx(c["fetch_bytes_scaled"] + c["write_bytes_scaled"])
    # ... and null once they differ
    name = bench.COUNTED[0][0]
    path = tmp_path / "profiles" / f"{name}_counters.txt"
    c = json.loads(path.read_text())
    c["kernel_src_sha"] = "0" * 16
    path.write_text(json.dumps(c))
    assert bench.traffic_of(name) is None


def test_counter_summary_needs_every_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    copy = bench.COPY_KERNEL
    write_counter_csv(tmp_path / "fetch", "FETCH_SIZE", [(copy, 1.0)])
    write_counter_csv(tmp_path / "write", "WRITE_SIZE", [(copy, 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(tmp_path / "fetch"), str(tmp_path / "write"), "cmd")


def test_util_summary_and_hash(tmp_path, monkeypatch):
    util_file = str(tmp_path / "utilisation_counters.txt")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "UTIL_FILE", util_file)
    d = tmp_path / "util"
    os.makedirs(d)
    key, prefix, _ = bench.UTIL_KERNELS[0]
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for v in (40.0, 50.0, 60.0):
            w.writerow(["void fp4g::(anonymous namespace)::" + prefix + "(int)", "MfmaUtil", v])
            w.writerow(["void fp4g::(anonymous namespace)::" + prefix + "(int)", "VALUBusy", v / 2])
    bench.summarize_util(str(d), "cmd")
    got = bench.util_from_profile(key)
    assert got["mfma_util_pct"] == 50.0 and got["valu_busy_pct"] == 25.0 and got["lds_util_pct"] is None
    assert bench.util_from_profile(bench.UTIL_KERNELS[1][0]) is None      # not in the run


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
