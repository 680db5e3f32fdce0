"""Benchmark: one pipeline stage's F+B throughput on one MI355X.

Workload (default): stage k=0 of an 8-stage, 16-micro-batch 1F1B pipeline of
an 80-layer model -- 10 residual SwiGLU blocks, d=8192, ffn=28672, micro-batch
2x4096 = 8192 tokens, bf16 -- i.e. the stage's 32-op list F0..F7, then
(B_j, F_{8+j}) pairs, then B8..B15.  One step = one full pass of that op list
over 16 micro-batches with the inputs resident in HBM.  Inputs are seeded
synthetic data (weights N(0,0.02), x N(0,1), output gradients N(0,0.01)).

Prints one JSON line: stage F+B TFLOP/s (algorithmic 18*T*d*ffn per block per
micro-batch), its fraction of the bf16 dense MFMA peak, peak stash bytes, the
dominant kernel's roofline from HIP events recorded around every launch in
the timed region, and the float64 CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0

# L2-to-memory bytes per launch of each GEMM role at the c3 workload, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs (bytes = 2.0 x FETCH_SIZE KiB + 1.0 x WRITE_SIZE KiB, scales taken from a plain 1 GiB
# copy kernel measured in the same runs).  Valid only for the GEMM source they were taken on.
TRAFFIC = {
    "config": "c3_80layer_p8_stage0",
    "gemm_source_sha1": "a32cc5eebafb6b1c281edeb35e850212196bf1d7",
    "bytes_per_launch": {
        "gemm_gateup_swiglu": 13.666e9, "gemm_down_residual": 6.052e9, "gemm_dh_swiglu_bwd": 9.170e9,
        "gemm_dn": 12.631e9, "gemm_wgrad_down": 8.151e9, "gemm_wgrad_gateup": 8.151e9,
    },
}


def _measured_traffic(config_name, kernel_name):
    """The counter-measured bytes per launch, or None once the GEMM source has changed since."""
    import hashlib
    src = os.path.join(ROOT, "pipeline_schedules_amd", "csrc", "gemm_bf16.hip")
    try:
        with open(src, "rb") as f:
            sha = hashlib.sha1(f.read()).hexdigest()
    except OSError:
        return None
    if sha != TRAFFIC["gemm_source_sha1"] or config_name != TRAFFIC["config"]:
        return None
    return TRAFFIC["bytes_per_launch"].get(kernel_name)


def _sig(x):
    """x to two decimals, or to four significant digits when that would round it to zero."""
    return round(x, 2) if abs(x) >= 1.0 else float(f"{x:.4g}")


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(cfg, params_dev, budget_s=20.0):
    """Time the float64 oracle (numpy/OpenBLAS, all host cores it is given) on
    one SwiGLU block of this workload's width, forward + backward on a sample
    of tokens sized to take roughly ``budget_s`` seconds."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import numerics as N

    p = params_dev[0]
    host = {k: p[k].float().cpu().numpy().astype(np.float64) for k in ("Wg", "Wu", "Wd")}
    host["gamma"] = p["gamma"].float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(0)

    def run(ts):
        x = rng.normal(0, 1, (ts, cfg.d))
        dy = rng.normal(0, 0.01, (ts, cfg.d))
        t0 = time.perf_counter()
        y, s = N.swiglu_forward(x, host, cfg.eps)
        N.swiglu_backward(s, dy, host)
        return time.perf_counter() - t0

    ts = 64
    dt = run(ts)
    while dt < budget_s / 2 and ts < 8192:
        ts *= 2
        dt = run(ts)
    flops = 18.0 * ts * cfg.d * cfg.f
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    del host
    torch.cuda.synchronize()
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"one SwiGLU block (d={cfg.d}, ffn={cfg.f}) forward+backward on {ts} tokens in float64 "
                  f"({flops / 1e12:.2f} TFLOP, {dt:.1f} s); weights = block 0 of the benchmark inputs",
    }


def vendor_reference(cfg, reps=10):
    """hipBLASLt (through torch.mm / torch.addmm) on the stage's six GEMM shapes, both operands
    K-contiguous as the stage's own kernel reads them: plain bf16 products with nothing fused, and
    the weight-gradient shapes also as fp32 C += A B.  A comparison point for the stage's fused
    kernels, not part of the stage."""
    import torch
    T, d, f = cfg.T, cfg.d, cfg.f
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed + 7)
    # small check that addmm with an fp32 out_dtype really computes C + A B
    a = torch.randn(256, 512, generator=gen, device=dev).to(torch.bfloat16)
    b = torch.randn(384, 512, generator=gen, device=dev).to(torch.bfloat16)
    c = torch.randn(256, 384, generator=gen, device=dev)
    got = torch.addmm(c, a, b.t(), out_dtype=torch.float32)
    want = c + a.float() @ b.float().t()
    check = float((got - want).norm() / want.norm())
    shapes = [("gemm_gateup", T, 2 * f, d, False), ("gemm_down", T, d, f, False), ("gemm_dh", T, f, d, False),
              ("gemm_dn", T, d, 2 * f, False), ("gemm_wgrad_down", f, d, T, True), ("gemm_wgrad_gateup", d, 2 * f, T, True)]
    out = {}
    for name, M, N, K, acc in shapes:
        a = torch.randn(M, K, generator=gen, device=dev).to(torch.bfloat16)
        b = (0.02 * torch.randn(N, K, generator=gen, device=dev)).to(torch.bfloat16)
        fl = 2.0 * M * N * K
        runs = [("bf16_out", lambda: torch.mm(a, b.t()))]
        if acc:
            c = torch.zeros(M, N, device=dev)
            runs.append(("fp32_accumulate", lambda: torch.addmm(c, a, b.t(), out_dtype=torch.float32, out=c)))
        for kind, fn in runs:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out[f"{name}.{kind}"] = {"M": M, "N": N, "K": K, "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1)}
            _log(f"vendor {name} {kind}: {ms:.3f} ms, {fl / ms / 1e9:.1f} TFLOP/s")
        del a, b
        torch.cuda.empty_cache()
    return {"library": "hipBLASLt via torch.mm / torch.addmm(out_dtype=float32)", "reps": reps,
            "addmm_fp32_check_rel_l2": check, "gemms": out}


def pipeline_model_from_times(cfg, kernels):
    """The P-stage timeline this stage's measured per-op times imply (no
    transfer time): every stage is assumed to cost what this one does.
    ``kernels`` maps kernel-role names to {"total_ms_per_step": ...}."""
    from pipeline_schedules_amd import pps
    per_mb = lambda names: sum(kernels[n]["total_ms_per_step"] for n in names if n in kernels) / cfg.M
    t_f = per_mb(["rmsnorm_fwd", "gemm_gateup_swiglu", "gemm_down_residual"])
    t_bx = per_mb(["gemm_dh_swiglu_bwd", "gemm_dn", "rmsnorm_bwd_residual", "dgamma_reduce"])
    # "copy" also holds the once-per-pass weight refresh; it is charged to W
    t_w = per_mb(["prep_w", "gemm_wgrad_down", "gemm_wgrad_gateup", "copy"])
    model = {"P": cfg.P, "M": cfg.M, "t_f_ms": round(t_f, 3), "t_b_ms": round(t_bx + t_w, 3),
             "t_b_input_ms": round(t_bx, 3), "t_w_ms": round(t_w, 3), "transfer_ms": 0.0}
    for name, kind, v, tf, tb, tw in (("gpipe", pps.GPIPE, 1, t_f, t_bx + t_w, 0.0),
                                      ("1f1b", pps.ONE_F_ONE_B, 1, t_f, t_bx + t_w, 0.0),
                                      ("interleaved_v2", pps.ONE_F_ONE_B, 2, t_f / 2, (t_bx + t_w) / 2, 0.0),
                                      ("zb1p", pps.ZB1P, 1, t_f, t_bx, t_w),
                                      ("zb2p", pps.ZB2P, 1, t_f, t_bx, t_w)):
        if v > 1 and cfg.M % cfg.P:
            # the interleaved order takes micro-batches in groups of P
            model[name] = {"not_applicable": f"M = {cfg.M} is not a multiple of P = {cfg.P}"}
            continue
        mk, bubble = pps.simulate_pipeline(cfg.P, cfg.M, v, kind, tf, tb, tw)
        model[name] = {"step_ms": round(mk, 1), "bubble": round(bubble, 4)}
    return model


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3_80layer_p8_stage0")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--profile-stride", type=int, default=7,
                    help="HIP events on every Nth launch of each kernel (1: all; an odd N cycles through the "
                         "blocks and roles that share a kernel id)")
    ap.add_argument("--recompute", action="store_true",
                    help="activation-recompute mode: a stash entry is the stage input alone and every "
                         "backward re-runs the forward; value stays the algorithmic rate")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain fp32 copy kernel (pps_scale by 1.0) three times over this many MiB: "
                         "a reference of known size for the HBM byte counters")
    ap.add_argument("--vendor-reference", action="store_true",
                    help="instead of the stage pass, time hipBLASLt on the workload's six GEMM shapes "
                         "(plain bf16 products; fp32 accumulate for the weight gradients) and print them as JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one pipeline stage on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU transport between stages is not implemented)", file=sys.stderr)
        sys.exit(1)

    import torch

    from pipeline_schedules_amd import pps
    from pipeline_schedules_amd.configs import PRESETS
    from pipeline_schedules_amd.inputs import make_device_inputs

    cfg = PRESETS[args.config]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.vendor_reference:
        if cfg.block != "swiglu":
            sys.exit("--vendor-reference needs a SwiGLU workload")
        res = vendor_reference(cfg)
        res["workload"] = cfg.name
        print(json.dumps(res), flush=True)
        return
    stream = torch.cuda.current_stream()
    dtype_id = pps.DTYPE_BY_NAME[cfg.dtype]
    kind_id = pps.KIND_BY_NAME[cfg.kind]

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            pps.scale(dst, src, n, 1.0, pps.DTYPE_FP32, stream)
        torch.cuda.synchronize()
        _log(f"copy probe: 3 x {n * 4} bytes read and written")
        del src, dst

    _log(f"workload {cfg.name}: drawing inputs on the device")
    inp = make_device_inputs(cfg, dev)
    weights = []
    for p in inp["params"]:
        weights += [p["Wg"], p["Wu"], p["Wd"], p["gamma"]] if cfg.block == "swiglu" else [p["W"], p["b"]]
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k, cfg.v, kind_id)
    launches_per_pass = 0
    per_block_f = 3 if cfg.block == "swiglu" else 2
    per_block_b = 12 if cfg.block == "swiglu" else 5   # bf16 SwiGLU: 4 transposed copies, dW_g and dW_u apart
    launches_per_pass = cfg.M * cfg.v * cfg.L * (per_block_f + per_block_b) + 2 * cfg.M * cfg.v
    flags = 0 if args.no_profile else pps.FLAG_PROFILE
    if args.recompute:
        if cfg.block != "swiglu" or cfg.kind not in ("1f1b", "gpipe"):
            print("--recompute needs SwiGLU blocks and a 1f1b or gpipe schedule", file=sys.stderr)
            sys.exit(1)
        flags |= pps.FLAG_RECOMPUTE
        launches_per_pass += cfg.M * cfg.v * cfg.L * per_block_f
    st = pps.stage_from_config(cfg, weights=weights, stream=stream, flags=flags,
                               profile_capacity=launches_per_pass * (args.steps + 1),
                               profile_stride=args.profile_stride)
    T, d = cfg.T, cfg.d
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    xs = inp["xs"]
    if cfg.v > 1:   # later chunks take their own synthetic inputs on one device
        xs2 = make_device_inputs(cfg.with_(seed=cfg.seed + 1), dev, with_G=True)
        chunk_x = [xs] + [xs2["xs"]] * (cfg.v - 1)
        chunk_g = [inp["Gs"]] + [xs2["Gs"]] * (cfg.v - 1)
    else:
        chunk_x, chunk_g = [xs], [inp["Gs"]]
    y = torch.empty((T, d), dtype=tdt, device=dev)
    dx = torch.empty((T, d), dtype=tdt, device=dev)

    def one_pass():
        st.zero_grad()   # a pass starts from zero gradients, as a training step would
        for op, mb, c, *_ in ops:
            if op == pps.OP_F:
                st.forward(mb, c, chunk_x[c][mb], y)
            elif op == pps.OP_B:
                st.backward(mb, c, chunk_g[c][mb], dx)
            else:
                st.backward_weight(mb, c)

    _log(f"warmup: {args.warmup} pass(es) of {len(ops)} ops")
    for _ in range(args.warmup):
        one_pass()
    st.sync()
    if not args.no_profile:
        st.kernel_times()   # drop warm-up timings
    torch.cuda.synchronize()
    _log(f"timed: {args.steps} pass(es)")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        one_pass()
    e1.record(stream)
    st.sync()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / args.steps
    flops_per_pass = cfg.flops_per_microbatch() * cfg.M
    tflops = flops_per_pass / (ms_per_step * 1e-3) / 1e12
    # recompute: each backward re-runs the chunk's forward except the last down GEMM
    extra = cfg.M * cfg.v * (6 * cfg.L - 2) * T * d * cfg.f if args.recompute else 0
    executed_tflops = (flops_per_pass + extra) / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    stats = st.stats()

    roofline = None
    kernels = {}
    if not args.no_profile:
        kt = st.kernel_times()
        # every profile_stride-th launch of each kernel carries HIP events:
        # averages over the timed launches, totals scaled to all launches
        kt = [k for k in kt if k["timed"] > 0]
        for k in kt:
            avg = k["total_ms"] / k["timed"]
            kernels[k["name"]] = {
                "launches": k["launches"], "timed": k["timed"], "avg_ms": avg,
                "total_ms_per_step": avg * k["launches"] / args.steps,
                "tflops": (k["flops"] / (k["total_ms"] * 1e-3) / 1e12) if k["flops"] else None,
                "gbs": (k["bytes"] / (k["total_ms"] * 1e-3) / 1e9) if k["bytes"] else None,
            }
        dom = max(kt, key=lambda k: k["total_ms"] / k["timed"] * k["launches"])
        if dom["flops"]:
            ach = dom["flops"] / (dom["total_ms"] * 1e-3) / 1e12
            # bf16 GEMMs run on the matrix cores; the fp32 path on the vector ALUs
            roofline = {"bound": "mfma" if cfg.dtype == "bf16" else "alu", "achieved": _sig(ach), "peak": peak,
                        "unit": "TFLOP/s",
                        "frac": round(ach / peak, 4), "traffic": _measured_traffic(cfg.name, dom["name"]),
                        "kernel": dom["name"], "avg_launch_ms": dom["total_ms"] / dom["timed"],
                        "flops_per_launch": dom["flops"] / dom["timed"]}
        else:
            ach = dom["bytes"] / (dom["total_ms"] * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None, "kernel": dom["name"],
                        "avg_launch_ms": dom["total_ms"] / dom["timed"],
                        "bytes_per_launch": dom["bytes"] / dom["timed"]}

    pipeline_model = None
    if kernels and cfg.block == "swiglu" and cfg.v == 1 and not args.recompute:
        pipeline_model = pipeline_model_from_times(cfg, kernels)

    cpu = None
    if not args.no_cpu_baseline and cfg.block == "swiglu":
        _log("cpu baseline: float64 oracle on a token sample")
        cpu = cpu_baseline(cfg, inp["params"])
    st.close()

    out = {
        "metric": "stage F+B TFLOP/s & MFMA-peak fraction at P=8 slice; peak stash bytes",
        "value": _sig(tflops),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: stage k={cfg.k} of P={cfg.P}, M={cfg.M} micro-batches, "
                               f"{cfg.kind}{' v=' + str(cfg.v) if cfg.v > 1 else ''}, {cfg.L * cfg.v} "
                               + (f"SwiGLU blocks d={cfg.d} ffn={cfg.f}" if cfg.block == "swiglu"
                                  else f"Linear+GELU blocks d={cfg.d}")
                               + f", {cfg.T} tokens/micro-batch",
                   "P": cfg.P, "M": cfg.M, "k": cfg.k, "v": cfg.v, "schedule": cfg.kind, "blocks": cfg.L * cfg.v,
                   "d": cfg.d, "ffn": cfg.f, "tokens_per_microbatch": cfg.T, "ops_per_step": len(ops),
                   "recompute": bool(args.recompute)},
        "peak_fraction": round(tflops / peak, 4),
        "peak_stash_bytes": stats["peak_live_bytes"],
        "peak_stash_entries": stats["peak_live_entries"],
        "stash_bound_entries": max(o[4] for o in ops),
        "flops_per_step": flops_per_pass,
        "executed_flops_per_step": flops_per_pass + extra,
        "executed_tflops": _sig(executed_tflops),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "pipeline_model": pipeline_model,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
