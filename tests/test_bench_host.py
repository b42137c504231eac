"""Host-side logic of bench.py, on the CPU: the rocprofv3 summaries that the
reported HBM traffic comes from (counter scaling by the calibration copy,
per-launch medians), the kernel-source check that keeps a stale traffic
figure out of the bench line, and the one-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counter_run(directory, ours_kib, copy_kib):
    """A counter_collection.csv as rocprofv3 writes it: three dispatches of the
    dominant kernel and three of the calibration copy, plus an unrelated small
    kernel."""
    ours = f"void attnres::(anonymous namespace)::{bench.DOMINANT_KERNEL}(attnres::KParams)"
    copy = "void at::native::vectorized_elementwise_kernel<4, copy>(...)"
    other = "void at::native::fill_kernel(...)"
    rows = []
    for k, v in enumerate(ours_kib):
        rows.append([k, ours, 458752, v])
    for k in range(3):
        rows.append([10 + k, copy, 1 << 20, copy_kib])
        rows.append([20 + k, other, 4096, 3.0])
    _write_csv(os.path.join(directory, "x", "run_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Value"], rows)


@pytest.fixture
def profiles_dir(tmp_path, monkeypatch):
    d = tmp_path / "profiles"
    monkeypatch.setattr(bench, "PROFILES", str(d))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(d / "traffic.json"))
    return d


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path, profiles_dir):
    copy_kib = bench.CALIBRATION_BYTES / 1024
    # FETCH_SIZE reads half of a copy's bytes (scale 2), WRITE_SIZE all of them.
    _counter_run(tmp_path / "fetch", [70000.0, 71000.0, 72000.0], copy_kib / 2)
    _counter_run(tmp_path / "write", [30000.0, 30500.0, 29000.0], copy_kib)
    _write_csv(str(tmp_path / "trace" / "a" / "mid_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [[bench.DOMINANT_KERNEL, 10, 33600.0, 33000.0, 34000.0, 99.9]])
    bench.summarize_profile(str(tmp_path / "trace"), str(tmp_path / "fetch"),
                            str(tmp_path / "write"), {"trace": "cmd"})
    t = json.load(open(profiles_dir / "traffic.json"))
    assert t["counters"]["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert t["counters"]["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    want = 71000.0 * 1024 * 2.0 + 30000.0 * 1024 * 1.0   # medians, scaled
    assert t["bytes_per_launch"] == round(want)
    assert t["ratio_to_algorithmic"] == pytest.approx(
        round(want / bench.W.mid_prefill().algorithmic_bytes(), 4))
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
    stats = (profiles_dir / "attnres_row_kernel_mid_prefill_T1024_kernel_stats.txt").read_text()
    assert "# command: cmd" in stats and "33.600" in stats


def test_source_hash_ignores_comments_and_layout_only():
    src = (b'#define N 4  // rows\n'
           b'__device__ int f(int x) { /* twice */ return x * 2; }\n'
           b'const char *s = "a // b"; char c = \'"\';\n')
    same = (b'// a note\n#define N 4\n\n'
            b'__device__   int f(int x)   {  return x * 2; } // done\n'
            b'const char *s = "a // b";   char c = \'"\';\n')
    assert bench.code_only(src) == bench.code_only(same)
    # code, string contents and line structure still count
    for other in (src.replace(b"x * 2", b"x * 3"), src.replace(b'"a // b"', b'"a b"'),
                  src.replace(b"4  // rows\n", b"4 ")):
        assert bench.code_only(other) != bench.code_only(src)
    assert bench.code_only(b"int a; /* unterminated") == b"int a;"


def test_stale_traffic_is_not_reported(profiles_dir):
    os.makedirs(profiles_dir)
    with open(bench.TRAFFIC_FILE, "w") as f:
        json.dump({"kernel_source_hash": bench.kernel_source_hash(), "bytes_per_launch": 123}, f)
    assert bench.load_traffic() == 123
    with open(bench.TRAFFIC_FILE, "w") as f:
        json.dump({"kernel_source_hash": "not-this-source", "bytes_per_launch": 123}, f)
    assert bench.load_traffic() is None
    os.remove(bench.TRAFFIC_FILE)
    assert bench.load_traffic() is None


def test_committed_traffic_matches_the_current_kernel_source():
    """The traffic summary in profiles/ was taken on the kernels as they are."""
    assert bench.load_traffic() is not None


def test_kernel_stats_group_dispatches_by_launch_shape(tmp_path, profiles_dir):
    rows = []
    for k, (wg, grid, dur) in enumerate([(448, 458752, 30000), (448, 458752, 40000),
                                         (256, 262144, 10000)]):
        rows.append([f"void attnres::(anonymous namespace)::attnres_anyh_kernel<2, false, 8, true, "
                     f"true>(attnres::KParams)", wg, grid, 0, 1000, 1000 + dur])
    rows.append(["void other_kernel()", 64, 64, 0, 0, 5])
    _write_csv(str(tmp_path / "t" / "k_kernel_trace.csv"),
               ["Kernel_Name", "Workgroup_Size_X", "Grid_Size_X", "Scratch_Size",
                "Start_Timestamp", "End_Timestamp"], rows)
    bench.write_kernel_stats(str(tmp_path / "t"), "x.txt", "title", "the command")
    text = (profiles_dir / "x.txt").read_text().splitlines()
    shapes = [l for l in text if l.startswith("attnres_anyh_kernel")]
    assert len(shapes) == 2
    assert any("| 448 | 458752 | 0 | 2 | 35.000 |" in l for l in shapes)
    assert any("| 256 | 262144 | 0 | 1 | 10.000 |" in l for l in shapes)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_graph_repeats_cover_the_minimum_calls():
    # The driver's --steps 20 and the default 300 both time >= MIN_TIMED_CALLS calls.
    for steps in (1, 20, 300, 599, 600, 601, 5000):
        r = bench.graph_repeats(steps, bench.MIN_TIMED_CALLS)
        assert r * steps >= bench.MIN_TIMED_CALLS
        assert (r - 1) * steps < bench.MIN_TIMED_CALLS
    assert bench.graph_repeats(20, 0) == 1


def test_kernel_trace_average_read_only_for_current_source(profiles_dir, monkeypatch):
    f = profiles_dir / "stats.txt"
    monkeypatch.setattr(bench, "KERNEL_STATS_FILE", str(f))
    os.makedirs(profiles_dir)
    body = ["# rocprofv3 kernel statistics, x", "# command: c",
            f"# kernel source hash: {bench.kernel_source_hash()}",
            f"{bench.DOMINANT_KERNEL} | 448 | 458752 | 0 | 2720 | 32.902 | 32.557"]
    f.write_text("\n".join(body) + "\n")
    assert bench.load_kernel_trace_us() == pytest.approx(32.902)
    e = bench.kernel_trace_entry(190883840)
    assert e["frac"] == pytest.approx(190883840 / 32.902 / 1e3 / bench.HBM_PEAK_GBPS, abs=1e-4)
    body[2] = "# kernel source hash: other"
    f.write_text("\n".join(body) + "\n")
    assert bench.load_kernel_trace_us() is None


def test_counter_summary_medians_and_ratios(tmp_path, profiles_dir):
    """Per-dispatch medians by kernel, and the derived ratios from them."""
    ours = f"void attnres::(anonymous namespace)::{bench.DOMINANT_KERNEL}(attnres::KParams)"
    probe = "void (anonymous namespace)::mid_kernel<true>(u32x4*, u32x4*, u32x4 const*, u32x4*, long)"
    rows = []
    for k, (w, c) in enumerate([(100.0, 5000.0), (100.0, 7000.0), (100.0, 6000.0)]):
        rows += [[k, ours, "SQ_WAVES", w, 0, 1000], [k, ours, "SQ_WAVE_CYCLES", c, 0, 1000]]
    rows += [[9, probe, "SQ_WAVES", 50.0, 0, 2000], [9, probe, "SQ_WAVE_CYCLES", 1000.0, 0, 2000]]
    _write_csv(str(tmp_path / "run" / "a_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                "End_Timestamp"], rows)
    bench.write_counter_summary("c.txt", "t", ["cmd1"], {"k": str(tmp_path / "run")})
    text = (profiles_dir / "c.txt").read_text()
    assert "# command: cmd1" in text
    kernels = [bench.DOMINANT_KERNEL, "mid_kernel<true>"]
    assert text.count(" | ".join(["# per-dispatch medians; counter"] + kernels)) == 1
    assert "SQ_WAVE_CYCLES | 6000 | 1000" in text
    assert "wave lifetime, cycles (SQ_WAVE_CYCLES / SQ_WAVES) | 60 | 20" in text
    assert "duration | 1.000 | 2.000" in text
