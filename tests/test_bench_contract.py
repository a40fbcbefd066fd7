"""CPU: the parts of bench.py's contract that need no GPU."""
import json
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


def test_cpu_oracle_config_on_c1_and_its_summary(tmp_path):
    """The per-config oracle timing on C1 (every slice measured, plus a small decode) and
    the per-config summary's CPU table."""
    import torch
    import bench
    from long_context_kv_kvslimmer_amd import configs, pipeline, synth
    cfg = configs.CONFIGS[1]
    K0, V0, _ = pipeline.config_cache(cfg, 0, "cpu")
    Qws = [torch.stack([synth.window_queries(cfg, 0, b, r, "cpu") for b in range(cfg.batch)])
           for r in range(len(cfg.rounds))]
    N = K0.shape[2]
    n = torch.ones(K0.shape[0], K0.shape[1], N, dtype=torch.int32)
    qs = [torch.randn(1, cfg.q_heads, cfg.head_dim) for _ in range(2)]
    res = bench.cpu_oracle_config(cfg, K0, V0, Qws, (K0, V0, n, qs, [N - 1, N]))
    assert res["kind"] == "oracle" and res["merge"] == "measured" and res["slices"].startswith("1 of 1")
    assert res["merge_s_per_layer"] > 0 and res["cores"] >= 1 and res["cpu_model"]
    assert res["decode"] == "measured" and res["decode_steps"] == 2
    line = {"config": "C1 x", "batch": 1, "layers": 1, "rounds": list(cfg.rounds), "merge_ms_per_layer": 0.07,
            "merge_ms_all_layers": 0.07, "merge_tokens_per_s": 7e6, "merge_algorithmic_MB_per_layer": 0.66,
            "merge_GBps": 9.0, "kernel_us_per_layer": {}, "cpu_oracle": res}
    many = {"config": "C3 y", "batch": 1, "layers": 32, "rounds": [38011], "merge_ms_per_layer": 0.44,
            "merge_ms_all_layers": 11.7, "merge_ms_all_layers_one_stream": 12.3, "merge_ms_all_layers_two_streams": 11.7,
            "merge_ms_all_layers_scaled": 14.08, "merge_tokens_per_s": 2.98e8, "merge_tokens_per_s_all_layers": 3.58e8,
            "merge_algorithmic_MB_per_layer": 1460.88, "merge_GBps": 3320.0, "merge_GBps_all_layers": 3995.5,
            "all_layers_outputs_equal": True, "kernel_us_per_layer": {}}
    f = tmp_path / "pc.jsonl"
    f.write_text(json.dumps(line) + "\n" + json.dumps(many) + "\n")
    out = bench.summarize_per_config(str(f), "cmd")
    assert "CPU oracle on the same layer" in out and "| C1 x | 1 of 1" in out and "CPU oracle decode" in out
    # several layers: measured whole-model time (one stream / two streams) and the per-layer share of the faster
    assert "| C3 y | 1 x 32 | [38011] | 0.44 | 12.3 / 11.7 | 0.3656 | 3.58e+08 | 1460.88 | 3995.5 |" in out
    assert "| C1 x | 1 x 1 | [256] | 0.07 | 0.07 | 0.07 | 7e+06 | 0.66 | 9.0 |" in out
