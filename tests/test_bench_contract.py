"""CPU: the parts of bench.py's contract that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "--gpus 2 is not supported" in (r.stdout + r.stderr)


def test_counter_summary_is_machine_readable():
    """The committed HBM-counter summary carries the sources digest and per-kernel bytes the
    bench reads back (the value is reported only while the digest matches the sources)."""
    sys.path.insert(0, ROOT)
    import bench
    lines = open(bench.TRAFFIC_FILE).read().splitlines()
    vals = dict(l.strip("` ").split(" = ", 1) for l in lines if l.startswith("`") and " = " in l)
    assert len(vals["sources"]) == 16
    assert int(vals["traffic_bytes[score_pass2_merge]"]) > 0
    got = bench.recorded_traffic("score_pass2_merge")
    assert got is None or got == int(vals["traffic_bytes[score_pass2_merge]"])


def test_ranking_ignores_a_cold_first_launch():
    """A first launch that loads its code object (ten times its steady time) must not make
    its kernel the dominant one: the ranking uses the median launch time per step."""
    sys.path.insert(0, ROOT)
    import bench
    marks = []
    for s in range(3):
        marks.append(("score_pass1", 0.41 if s == 0 else 0.044))
        marks.append(("combine", 0.11 if s == 0 else 0.006))
        marks.append(("score_pass2_merge", 0.051))
        marks.append(("decode", 0.22 if s == 0 else 0.0145))
        marks.append(("combine", 0.005))
    ranked = bench.rank_kernels(marks, 3)
    assert bench.dominant_kernel(ranked) == "score_pass2_merge"
    assert ranked["combine"]["launches_per_step"] == 2
    assert abs(ranked["score_pass1"]["median_ms"] - 0.044) < 1e-12


def test_cpu_model_and_machine_fields():
    sys.path.insert(0, ROOT)
    import bench
    m = bench.cpu_model()
    assert m is None or isinstance(m, str)
    info = bench.gpu_clock_info()
    assert set(info) >= {"gpu_peak_sclk_MHz", "gpu_sclk_now", "rocm_version", "hip_runtime"}
