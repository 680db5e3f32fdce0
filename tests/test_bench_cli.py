"""Command-line contract of bench.py that holds without a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    # One stage on one GPU is what the benchmark measures; N > 1 exits non-zero
    # before touching any device, with a message saying so.
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""


def test_pipeline_model_from_measured_times():
    # The bench's P-stage timeline from per-role times: every kind the
    # schedule allows for the workload, the interleaved one marked not
    # applicable when M is not a multiple of P (c2: P = 4, M = 6).
    import importlib.util
    from pipeline_schedules_amd.configs import PRESETS
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    times = {"gemm_gateup_swiglu": 2.0, "gemm_down_residual": 1.0, "gemm_dh_swiglu_bwd": 1.0, "gemm_dn": 2.0,
             "gemm_wgrad_down": 1.0, "gemm_wgrad_gateup": 2.0}
    for name, interleaved in (("c2_swiglu_p4m6", False), ("c3_80layer_p8_stage0", True)):
        cfg = PRESETS[name]
        kernels = {k: {"total_ms_per_step": v * cfg.M} for k, v in times.items()}
        m = bench.pipeline_model_from_times(cfg, kernels)
        assert (m["t_f_ms"], m["t_b_input_ms"], m["t_w_ms"]) == (3.0, 3.0, 3.0)
        for kind in ("gpipe", "1f1b", "zb1p", "zb2p"):
            assert m[kind]["step_ms"] > 0 and 0 <= m[kind]["bubble"] < 1
        # equal F, B and W costs: 1F1B's bubble is (P-1)/(M+P-1), ZB2P removes it for M >= 2P-1
        assert abs(m["1f1b"]["bubble"] - (cfg.P - 1) / (cfg.M + cfg.P - 1)) < 1e-3
        assert m["zb2p"]["bubble"] <= m["zb1p"]["bubble"] <= m["1f1b"]["bubble"]
        if interleaved:
            assert m["interleaved_v2"]["bubble"] < m["1f1b"]["bubble"]
        else:
            assert "not_applicable" in m["interleaved_v2"]
