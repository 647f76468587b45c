"""Host checks of the measurement record: every committed profile summary under
profiles/ was taken on the current kernel sources, its derived figures follow
from its own raw fields, and the summariser turns rocprofv3 CSV output into
those figures as stated (run on small synthetic CSV files, no GPU)."""
import csv
import glob
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.json")))


def _sources_of(spec):
    if spec.startswith("gemm:") or spec == "fp16mm":
        return bench.GEMM_SOURCES
    if spec.startswith("encode:"):
        return bench.ENCODE_SOURCES
    return bench.GEMV_SOURCES


def test_there_are_profiles():
    assert len(PROFILES) >= 10


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_profile_taken_on_current_sources(path):
    rec = json.load(open(path))
    assert rec["kernel_sources_hash"] == bench.kernel_sources_hash(_sources_of(rec["launch"])), (
        f"{os.path.basename(path)} was taken on other kernel sources: profile again")


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_profile_figures_follow_from_raw_fields(path):
    rec = json.load(open(path))
    med_s = rec["median_ns"] * 1e-9
    assert rec["min_ns"] <= rec["median_ns"] <= rec["max_ns"]
    assert rec["dispatches"] >= 1 and len(rec["commands"]) >= 2
    if "algorithmic_bytes_per_launch" in rec:
        gbs = rec["algorithmic_bytes_per_launch"] / med_s / 1e9
        assert rec["median_gbs"] == pytest.approx(gbs, abs=0.1)
        assert rec["frac_of_hbm_peak"] == pytest.approx(gbs / bench.HBM_PEAK_GBS, abs=1e-4)
        lc = bench._spec_launch(rec["launch"])
        assert rec["algorithmic_bytes_per_launch"] == bench.launch_bytes(lc)
    if "flops" in rec:
        tf = rec["flops"] / med_s / 1e12
        assert rec["median_tflops"] == pytest.approx(tf, abs=0.1)
        assert rec["frac_of_mfma_f16_peak"] == pytest.approx(tf / bench.MFMA_F16_PEAK_TFLOPS, abs=1e-4)
    t = rec.get("traffic")
    if t:
        hbm = (t["fetch_size_kib_median"] * 1024 * t["copy_fetch_scale"]
               + t["write_size_kib_median"] * 1024 * t["copy_write_scale"])
        assert t["hbm_bytes_per_launch"] == pytest.approx(hbm, rel=1e-3)
        assert t["traffic_over_algorithmic"] == pytest.approx(hbm / rec["algorithmic_bytes_per_launch"], abs=1e-3)
    i = rec.get("issue")
    if i:
        # the encoder's counters belong to its timed launch (the longest; a short
        # warm-up launch precedes it), the others' to the median dispatch
        med_s = rec.get("timed_launch_ns", rec["median_ns"]) * 1e-9
        assert i["valu_insts_without_mfma"] == pytest.approx(i["sq_insts_valu"] - i["sq_insts_mfma"])
        se = i["sq_busy_cycles_per_se"]
        assert i["clock_ghz_est"] == pytest.approx(se / med_s / 1e9, abs=2e-3)
        assert i["mfma_busy_frac_at_est_clock"] == pytest.approx(i["mfma_busy_cycles_per_simd"] / se, abs=1e-4)


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_kernel_stats_agree_with_profile(path):
    # the rocprofv3 --stats summary committed beside each profile: the same
    # kernel, dispatch count and average duration as the trace summary
    rec = json.load(open(path))
    stats = path[:-len(".json")] + "_kernel_stats.txt"
    assert os.path.exists(stats), f"{os.path.basename(stats)} missing"
    lines = [ln for ln in open(stats) if not ln.startswith("#")]
    rows = {r["Name"]: r for r in csv.DictReader(lines)}
    row = rows[rec["kernel"]]
    assert int(row["Calls"]) == rec["dispatches"]
    assert float(row["AverageNs"]) == pytest.approx(rec["mean_ns"], abs=1.0)
    assert int(row["MinNs"]) == rec["min_ns"] and int(row["MaxNs"]) == rec["max_ns"]


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_make_profile_from_synthetic_rocprof_output(tmp_path, capsys):
    # one GEMV launch shape: a kernel trace of 5 dispatches, FETCH_SIZE and
    # WRITE_SIZE of the launch and of the 256 MiB copy, and the SQ counters
    spec, tag = "mlp1:down_k4", "t"
    name = "void exl3::gemv_kernel<4, 4, 0, false>(exl3::GemvParams)"
    durs = [12000, 11000, 13000, 12500, 11500]
    _write_csv(tmp_path / f"{tag}_trace_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [{"Kernel_Name": name, "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + d}
                for i, d in enumerate(durs)])
    cc = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    copy = "__amd_rocclr_copyBuffer"
    _write_csv(tmp_path / "copy_fetch_counter_collection.csv", cc,
               [{"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 131072.0}])
    _write_csv(tmp_path / "copy_write_counter_collection.csv", cc,
               [{"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 262144.0}])
    _write_csv(tmp_path / f"{tag}_fetch_counter_collection.csv", cc,
               [{"Kernel_Name": name, "Counter_Name": "FETCH_SIZE", "Counter_Value": v} for v in (14000.0, 15000.0, 16000.0)])
    _write_csv(tmp_path / f"{tag}_write_counter_collection.csv", cc,
               [{"Kernel_Name": name, "Counter_Name": "WRITE_SIZE", "Counter_Value": 8.0}])
    sq = {"SQ_INSTS_VALU": 3.6e6, "SQ_INSTS_MFMA": 1.0e5, "SQ_INSTS_SALU": 1.0e5,
          "SQ_VALU_MFMA_BUSY_CYCLES": 1.024e6, "SQ_VALU_MFMA_COEXEC_CYCLES": 5.12e5,
          "SQ_BUSY_CYCLES": 32 * 25000.0, "GRBM_GUI_ACTIVE": 3.0e5}
    _write_csv(tmp_path / f"{tag}_sq_counter_collection.csv", cc,
               [{"Kernel_Name": name, "Counter_Name": k, "Counter_Value": v} for k, v in sq.items()])
    bench.make_profile(str(tmp_path), tag, spec)
    rec = json.loads(capsys.readouterr().out)
    assert rec["kernel"] == name and rec["dispatches"] == 5 and rec["median_ns"] == 12000
    b = bench.launch_bytes(bench._spec_launch(spec))
    assert rec["algorithmic_bytes_per_launch"] == b
    assert rec["median_gbs"] == pytest.approx(b / 12000e-9 / 1e9, abs=0.1)
    # the copy moved 256 MiB for 128 MiB of FETCH_SIZE and 256 MiB of WRITE_SIZE
    tr = rec["traffic"]
    assert tr["copy_fetch_scale"] == pytest.approx(2.0) and tr["copy_write_scale"] == pytest.approx(1.0)
    assert tr["fetch_size_kib_median"] == 15000.0
    assert tr["hbm_bytes_per_launch"] == int(15000.0 * 1024 * 2.0 + 8.0 * 1024)
    i = rec["issue"]
    assert i["valu_insts_without_mfma"] == pytest.approx(3.5e6)
    assert i["clock_ghz_est"] == pytest.approx(25000 / 12000e-9 / 1e9, abs=1e-3)
    assert i["mfma_busy_cycles_per_simd"] == pytest.approx(1000.0)
    assert i["valu_coexec_frac_of_mfma_busy"] == pytest.approx(0.5)


def test_sources_hash_ignores_comments_only(tmp_path, monkeypatch):
    a = tmp_path / "k.hip"
    a.write_text("int f() { return 1; }  // one\n/* block\n comment */\n\nint g();\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "decode_gemm_exl3_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text(a.read_text())
    h1 = bench.kernel_sources_hash(("k.hip",))
    (csrc / "k.hip").write_text("int f() { return 1; }  // another comment\n\nint g();\n")
    assert bench.kernel_sources_hash(("k.hip",)) == h1
    (csrc / "k.hip").write_text("int f() { return 2; }\nint g();\n")
    assert bench.kernel_sources_hash(("k.hip",)) != h1


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_trace_summary_of_synthetic_trace(tmp_path, capsys):
    path = tmp_path / "k_kernel_trace.csv"
    _write_csv(path, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [{"Kernel_Name": "a", "Start_Timestamp": 0, "End_Timestamp": 300},
                {"Kernel_Name": "a", "Start_Timestamp": 400, "End_Timestamp": 500},
                {"Kernel_Name": "b", "Start_Timestamp": 600, "End_Timestamp": 700}])
    bench.trace_summary(str(path))
    lines = capsys.readouterr().out.strip().splitlines()
    assert lines[0].startswith("# columns")
    # kernels by total time: a (2 calls, median 200 ns, 80 %), then b
    assert lines[1] == "a | 2 | 200 | 200 | 100 | 300 | 80.00"
    assert lines[2] == "b | 1 | 100 | 100 | 100 | 100 | 20.00"
