"""GPU parity of one stage through the C ABI against the float64 oracle.

Shapes span several 256-wide tiles with ragged tails in every GEMM dimension
(T=600, d=520, ffn=776).  Tolerances: rel-L2 <= 2e-2 for bf16 and <= 1e-5 for
fp32, per tensor (outputs and input gradients per micro-batch, every weight
gradient).  Schedules and stash bookkeeping are compared exactly.
"""

import numpy as np
import pytest

from oracle import numerics as N
from oracle import schedule as S

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-5}


@pytest.fixture(scope="module")
def env():
    import torch
    from pipeline_schedules_amd import pps
    from tests import gpu_util as G
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pps.lib()
    return torch, pps, G


def _swiglu_cfg(dtype, T=600, d=520, f=776, L=2, M=3, P=2, k=0, v=1, kind="1f1b"):
    from pipeline_schedules_amd.configs import StageConfig
    return StageConfig("test", P=P, M=M, k=k, v=v, kind=kind, block="swiglu", dtype=dtype, L=L, d=d, f=f, T=T)


def _oracle_kind(name):
    return {"1f1b": S.ONE_F_ONE_B, "gpipe": S.GPIPE, "zb1p": S.ZB1P, "zb2p": S.ZB2P}[name]


def _run_single(env, cfg, inp, kind, flags=0):
    torch, pps, G = env
    w = G.upload_params(inp.params[0], cfg.block, cfg.dtype)
    st = pps.stage_from_config(cfg, weights=w, kind=kind, stream=torch.cuda.current_stream(), flags=flags)
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k, cfg.v, pps.KIND_BY_NAME[kind])
    assert ops == [tuple(o) for o in S.stage_ops(cfg.P, cfg.M, cfg.k, cfg.v, _oracle_kind(kind))]
    xs = [[G.to_dev(x, cfg.dtype) for x in inp.xs]]
    dys = [[G.to_dev(g, cfg.dtype) for g in inp.Gs]]
    ys, dxs = G.run_stage(st, ops, xs, dys, cfg.T, cfg.d, cfg.dtype)
    assert st.oplog() == ops
    grads = G.stage_grads(st, cfg.L, cfg.block, cfg.d, cfg.f)
    ys = [G.to_host(y) for y in ys[0]]
    dxs = [G.to_host(x) for x in dxs[0]]
    stats = st.stats()
    st.close()
    return ys, dxs, grads, stats


def _check(cfg, got, inp, tol):
    ys, dxs, grads, _ = got
    ry, rdx, rg = N.full_batch_step(inp.xs, inp.Gs, inp.params[0], cfg.block, cfg.eps)
    errs = {}
    for i in range(cfg.M):
        errs[f"y{i}"] = N.rel_l2(ys[i], ry[i])
        errs[f"dx{i}"] = N.rel_l2(dxs[i], rdx[i])
    for b in range(cfg.L):
        for key in rg[b]:
            errs[f"d{key}{b}"] = N.rel_l2(grads[b][key], rg[b][key])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert not bad, bad
    return errs


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["1f1b", "gpipe", "zb1p", "zb2p"])
def test_swiglu_stage_parity(env, dtype, kind):
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg(dtype, kind=kind)
    inp = make_inputs(cfg, gamma="random")
    got = _run_single(env, cfg, inp, kind)
    _check(cfg, got, inp, TOL[dtype])


@pytest.mark.parametrize("shape", ["ragged", "full_tiles"])
def test_split_is_bit_identical_to_unsplit(env, shape):
    # full tiles: both runs take dg|du T-contiguous from the dh epilogue (the
    # split keeps it in the entry until W), ragged: both copy it
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", M=5, P=3) if shape == "ragged" else _swiglu_cfg("bf16", T=512, d=264, f=512, M=5, P=3)
    inp = make_inputs(cfg, gamma="random")
    a = _run_single(env, cfg, inp, "1f1b")
    b = _run_single(env, cfg, inp, "zb1p")
    for i in range(cfg.M):
        assert np.array_equal(a[0][i], b[0][i])
        assert np.array_equal(a[1][i], b[1][i])
    for blk in range(cfg.L):
        for key in a[2][blk]:
            assert np.array_equal(a[2][blk][key], b[2][blk][key]), key
    # the split keeps dg|du and dy per block until W: more bytes at the peak
    assert b[3]["peak_live_bytes"] > a[3]["peak_live_bytes"]


@pytest.mark.parametrize("kind", ["zb1p", "zb2p"])
def test_zero_bubble_stage0_extra_warmup(env, kind):
    # P=4, M=8, stage 0: ZB2P runs 7 forwards before its first backward and
    # holds up to 8 entries until their W; ZB1P holds 4.  Same kernels in the
    # same per-micro-batch order as the unsplit 1F1B run, so the results are
    # bit-identical to it, and within tolerance of the oracle.
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=1, M=8, P=4)
    inp = make_inputs(cfg, gamma="random")
    a = _run_single(env, cfg, inp, "1f1b")
    b = _run_single(env, cfg, inp, kind)
    _check(cfg, b, inp, TOL["bf16"])
    assert b[3]["peak_live_entries"] == (8 if kind == "zb2p" else 4)
    for i in range(cfg.M):
        assert np.array_equal(a[0][i], b[0][i])
        assert np.array_equal(a[1][i], b[1][i])
    for blk in range(cfg.L):
        for key in a[2][blk]:
            assert np.array_equal(a[2][blk][key], b[2][blk][key]), key


def test_fused_hT_full_tiles(env):
    # T and ffn multiples of the 256 x 256 GEMM tile: the dh epilogue writes
    # h transposed for dW_d (no recompute, no copy).  Parity with the oracle,
    # and bit-identical results to the split run, which recomputes h from the
    # stash at W and copies it transposed.
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=512, d=264, f=512, M=3, P=2)
    inp = make_inputs(cfg, gamma="random")
    a = _run_single(env, cfg, inp, "1f1b")
    _check(cfg, a, inp, TOL["bf16"])
    b = _run_single(env, cfg, inp, "zb1p")
    for i in range(cfg.M):
        assert np.array_equal(a[0][i], b[0][i])
        assert np.array_equal(a[1][i], b[1][i])
    for blk in range(cfg.L):
        for key in a[2][blk]:
            assert np.array_equal(a[2][blk][key], b[2][blk][key]), key


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["1f1b", "gpipe"])
def test_recompute_mode(env, dtype, kind):
    # Recompute mode: parity with the oracle, bit-identical to the run that
    # keeps the forward's tensors, and a stash entry of x [T, d] alone.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg(dtype, M=5, P=3, L=3, kind=kind)
    inp = make_inputs(cfg, gamma="random")
    a = _run_single(env, cfg, inp, kind)
    r = _run_single(env, cfg, inp, kind, flags=pps.FLAG_RECOMPUTE)
    _check(cfg, r, inp, TOL[dtype])
    for i in range(cfg.M):
        assert np.array_equal(a[0][i], r[0][i]) and np.array_equal(a[1][i], r[1][i]), i
    for blk in range(cfg.L):
        for key in a[2][blk]:
            assert np.array_equal(a[2][blk][key], r[2][blk][key]), (blk, key)
    es = 2 if dtype == "bf16" else 4
    entry = (cfg.T * cfg.d * es + 255) // 256 * 256
    peak = cfg.P - cfg.k if kind == "1f1b" else cfg.M
    assert r[3]["slot_bytes"] == entry and r[3]["peak_live_bytes"] == peak * entry
    assert a[3]["peak_live_bytes"] > cfg.L * r[3]["peak_live_bytes"]


def test_orders_agree_with_full_batch(env):
    # 1F1B order, GPipe order and the full-batch oracle give the same result
    # ([1F1B §4.5]: synchronous 1F1B equals one large-batch step).
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", M=4, P=4, k=1)
    inp = make_inputs(cfg, gamma="random")
    a = _run_single(env, cfg, inp, "1f1b")
    g = _run_single(env, cfg, inp, "gpipe")
    _check(cfg, a, inp, TOL["bf16"])
    _check(cfg, g, inp, TOL["bf16"])
    for i in range(cfg.M):
        assert np.array_equal(a[0][i], g[0][i]) and np.array_equal(a[1][i], g[1][i])
    for blk in range(cfg.L):
        for key in a[2][blk]:
            # same per-micro-batch terms, summed in a different order
            assert N.rel_l2(a[2][blk][key], g[2][blk][key]) < 1e-5
    assert a[3]["peak_live_entries"] == 3 and g[3]["peak_live_entries"] == 4


@pytest.mark.parametrize("kind", ["1f1b", "gpipe", "zb1p", "zb2p"])
def test_toy_stage_parity(env, kind):
    from pipeline_schedules_amd.configs import C1_TOY
    from pipeline_schedules_amd.inputs import make_inputs
    inp = make_inputs(C1_TOY, bias="random")
    got = _run_single(env, C1_TOY, inp, kind)
    _check(C1_TOY, got, inp, TOL["fp32"])


@pytest.mark.parametrize("shape,v,k", [("ragged", 2, 0), ("full_tiles", 2, 0), ("ragged", 3, 0), ("ragged", 3, 1),
                                       ("ragged", 4, 1)])
@pytest.mark.parametrize("recompute", [False, True])
def test_interleaved_stage_parity(env, recompute, shape, v, k):
    # "full_tiles": T and ffn multiples of the 256 x 256 GEMM tile, so the dh
    # epilogue writes h transposed for dW_d under chunked stashing.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    if shape == "ragged":
        cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=1, M=4, P=2, k=k, v=v)
    else:
        cfg = _swiglu_cfg("bf16", T=512, d=264, f=512, L=2, M=4, P=2, k=k, v=v)
    inp = make_inputs(cfg, gamma="random")
    # independent seeded inputs for chunks c > 0 (their real input comes from another device)
    cin = [(inp.xs, inp.Gs)] + [([np.asarray(x) for x in make_inputs(cfg, rng_seed=2 * c - 1).xs],
                                 [np.asarray(g) for g in make_inputs(cfg, rng_seed=2 * c).Gs]) for c in range(1, v)]
    w = G.upload_params(inp.params[0], "swiglu", "bf16")
    st = pps.stage_from_config(cfg, weights=w, stream=torch.cuda.current_stream(),
                               flags=pps.FLAG_RECOMPUTE if recompute else 0)
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k, v, pps.ONE_F_ONE_B)
    assert ops == [tuple(o) for o in S.stage_ops(cfg.P, cfg.M, cfg.k, v, S.ONE_F_ONE_B)]
    xs = [[G.to_dev(x, "bf16") for x in cx] for cx, _ in cin]
    dys = [[G.to_dev(g, "bf16") for g in cg] for _, cg in cin]
    ys, dxs = G.run_stage(st, ops, xs, dys, cfg.T, cfg.d, "bf16")
    assert st.oplog() == ops
    assert st.stats()["peak_live_entries"] == max(o[4] for o in ops)
    for c, (cx, cg) in enumerate(cin):
        ry, rdx, rg = N.full_batch_step(cx, cg, inp.params[0][c * cfg.L:(c + 1) * cfg.L], "swiglu", cfg.eps)
        for i in range(cfg.M):
            assert N.rel_l2(G.to_host(ys[c][i]), ry[i]) <= TOL["bf16"]
            assert N.rel_l2(G.to_host(dxs[c][i]), rdx[i]) <= TOL["bf16"]
        got = G.stage_grads(st, cfg.L, "swiglu", cfg.d, cfg.f, chunk=c)
        for b in range(cfg.L):
            for key in rg[b]:
                assert N.rel_l2(got[b][key], rg[b][key]) <= TOL["bf16"], (c, b, key)
    st.close()


def test_zero_down_projection_closed_form(env):
    # Wd = 0: y = x and dx = dy exactly; dWg = dWu = dgamma = 0 exactly.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", M=2, P=1)
    inp = make_inputs(cfg, gamma="random")
    for p in inp.params[0]:
        p["Wd"] = np.zeros_like(p["Wd"])
    ys, dxs, grads, _ = _run_single(env, cfg, inp, "1f1b")
    for i in range(cfg.M):
        assert np.array_equal(ys[i], inp.xs[i].astype(np.float64))
        assert np.array_equal(dxs[i], inp.Gs[i].astype(np.float64))
    for b in range(cfg.L):
        assert not grads[b]["Wg"].any() and not grads[b]["Wu"].any() and not grads[b]["gamma"].any()


# Degenerate and extreme widths: one token per micro-batch (every GEMM has a
# single row, the weight gradients reduce over one token padded to 8), the
# smallest widths the ABI accepts (d = ffn = 8: every K is a partial tile), and
# the largest model width (d = 16384: the widest RMSNorm kernels, full tiles
# with the fused T-contiguous outputs).
@pytest.mark.parametrize("name,dtype,T,d,f,L,kind,flags", [
    ("one_token", "bf16", 1, 264, 392, 2, "1f1b", 0), ("one_token", "fp32", 1, 264, 392, 2, "1f1b", 0),
    ("one_token", "bf16", 1, 264, 392, 2, "zb1p", 0), ("odd_tokens", "bf16", 77, 264, 392, 2, "1f1b", "recompute"),
    ("minimum_width", "bf16", 37, 8, 8, 2, "1f1b", 0), ("minimum_width", "fp32", 37, 8, 8, 2, "1f1b", 0),
    ("maximum_width", "bf16", 256, 16384, 512, 1, "1f1b", 0)])
def test_extreme_shapes(env, name, dtype, T, d, f, L, kind, flags):
    _, pps, _ = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg(dtype, T=T, d=d, f=f, L=L, M=3, P=2)
    inp = make_inputs(cfg, gamma="random")
    got = _run_single(env, cfg, inp, kind, flags=pps.FLAG_RECOMPUTE if flags == "recompute" else 0)
    _check(cfg, got, inp, TOL[dtype])


# Degenerate pipelines: a single stage (P = 1: F and B alternate, one stash
# slot), a single micro-batch, and the last stage of a deeper pipeline
# (k = P-1: warmup of one), under 1F1B and the Zero-Bubble split.
@pytest.mark.parametrize("P,M,k,kind", [(1, 3, 0, "1f1b"), (2, 1, 0, "1f1b"), (4, 5, 3, "1f1b"),
                                        (4, 5, 3, "zb1p"), (1, 2, 0, "zb2p")])
def test_degenerate_pipelines(env, P, M, k, kind):
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=136, d=264, f=392, L=2, M=M, P=P, k=k)
    inp = make_inputs(cfg, gamma="random")
    got = _run_single(env, cfg, inp, kind)
    _check(cfg, got, inp, TOL["bf16"])
    ops = S.stage_ops(P, M, k, 1, _oracle_kind(kind))
    assert got[3]["peak_live_entries"] == max(o[4] for o in ops)


def test_side_stream_bit_identical(env):
    # Every launch goes to the stream the stage was created with: the same
    # pass on a separate (non-default, default-priority) stream gives the same
    # bits as on the current one.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=2, M=4, P=2)
    inp = make_inputs(cfg, gamma="random")
    a = _run_single(env, cfg, inp, "zb1p")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        b = _run_single(env, cfg, inp, "zb1p")
    torch.cuda.synchronize()
    for i in range(cfg.M):
        assert np.array_equal(a[0][i], b[0][i]) and np.array_equal(a[1][i], b[1][i])
    for blk in range(cfg.L):
        for key in a[2][blk]:
            assert np.array_equal(a[2][blk][key], b[2][blk][key]), key


def test_weights_changed_between_passes_take_effect(env):
    # The library's K-contiguous weight copies are refreshed at the first F of
    # each pass, so weights the caller changes between passes are used.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=2, M=2, P=2)
    inp = make_inputs(cfg, gamma="random")
    w = G.upload_params(inp.params[0], "swiglu", "bf16")
    st = pps.stage_from_config(cfg, weights=w, stream=torch.cuda.current_stream())
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k)
    xs = [[G.to_dev(x, "bf16") for x in inp.xs]]
    dys = [[G.to_dev(g, "bf16") for g in inp.Gs]]
    G.run_stage(st, ops, xs, dys, cfg.T, cfg.d, "bf16")
    # in place, exactly representable: matrices x 0.5 (bf16), gamma x 1.5 (fp32)
    params2 = []
    for b, p in enumerate(inp.params[0]):
        for j, key in enumerate(("Wg", "Wu", "Wd")):
            w[4 * b + j].mul_(0.5)
        w[4 * b + 3].mul_(1.5)
        params2.append({"Wg": p["Wg"] * 0.5, "Wu": p["Wu"] * 0.5, "Wd": p["Wd"] * 0.5,
                        "gamma": (p["gamma"].astype(np.float32) * np.float32(1.5))})
    st.zero_grad()
    ys, dxs = G.run_stage(st, ops, xs, dys, cfg.T, cfg.d, "bf16")
    ry, rdx, rg = N.full_batch_step(inp.xs, inp.Gs, params2, "swiglu", cfg.eps)
    for i in range(cfg.M):
        assert N.rel_l2(G.to_host(ys[0][i]), ry[i]) <= TOL["bf16"]
        assert N.rel_l2(G.to_host(dxs[0][i]), rdx[i]) <= TOL["bf16"]
    got = G.stage_grads(st, cfg.L, "swiglu", cfg.d, cfg.f)
    for b in range(cfg.L):
        for key in rg[b]:
            assert N.rel_l2(got[b][key], rg[b][key]) <= TOL["bf16"], (b, key)
    st.close()


def test_two_stages_on_two_streams(env):
    # Two handles, each on its own stream, their ops issued interleaved: each
    # gives the bits it gives alone (no state shared between handles).
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfgs = [_swiglu_cfg("bf16", T=264, d=264, f=392, L=2, M=4, P=2),
            _swiglu_cfg("bf16", T=256, d=256, f=512, L=1, M=3, P=3, k=1)]
    kinds = ["1f1b", "zb1p"]
    inps = [make_inputs(c, gamma="random") for c in cfgs]
    alone = [_run_single(env, c, i, k) for c, i, k in zip(cfgs, inps, kinds)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for cfg, inp, kind, s in zip(cfgs, inps, kinds, streams):
        with torch.cuda.stream(s):
            w = G.upload_params(inp.params[0], "swiglu", "bf16")
            st = pps.stage_from_config(cfg, weights=w, kind=kind, stream=s)
            xs = [G.to_dev(x, "bf16") for x in inp.xs]
            dys = [G.to_dev(g, "bf16") for g in inp.Gs]
            ys = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.M)]
            dxs = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.M)]
        ops = pps.make_schedule(cfg.P, cfg.M, cfg.k, 1, pps.KIND_BY_NAME[kind])
        runs.append({"st": st, "w": w, "xs": xs, "dys": dys, "ys": ys, "dxs": dxs, "ops": list(ops), "s": s})
    while any(r["ops"] for r in runs):
        for r in runs:
            if r["ops"]:
                op, mb, c, *_ = r["ops"].pop(0)
                if op == pps.OP_F:
                    r["st"].forward(mb, c, r["xs"][mb], r["ys"][mb])
                elif op == pps.OP_B:
                    r["st"].backward(mb, c, r["dys"][mb], r["dxs"][mb])
                else:
                    r["st"].backward_weight(mb, c)
    for r, cfg, ref in zip(runs, cfgs, alone):
        with torch.cuda.stream(r["s"]):
            r["st"].sync()
            grads = G.stage_grads(r["st"], cfg.L, "swiglu", cfg.d, cfg.f)
            ys = [G.to_host(y) for y in r["ys"]]
            dxs = [G.to_host(x) for x in r["dxs"]]
        for i in range(cfg.M):
            assert np.array_equal(ys[i], ref[0][i]) and np.array_equal(dxs[i], ref[1][i])
        for blk in range(cfg.L):
            for key in ref[2][blk]:
                assert np.array_equal(grads[blk][key], ref[2][blk][key]), key
        r["st"].close()
    torch.cuda.synchronize()


def test_pass_captured_in_a_hip_graph(env):
    # A whole pass (gradient zeroing and the op list) recorded into a HIP graph
    # and replayed: the library launches only kernels on the stage's stream
    # during ops (zeroing by a fill kernel, no allocation, no memset), so every
    # replay reproduces the eager pass bit for bit.  Eager work and
    # synchronisation run between the replays.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=2, M=4, P=2)
    inp = make_inputs(cfg, gamma="random")
    ref = _run_single(env, cfg, inp, "zb1p")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        w = G.upload_params(inp.params[0], "swiglu", "bf16")
        st = pps.stage_from_config(cfg, weights=w, kind="zb1p", stream=s)
        xs = [G.to_dev(x, "bf16") for x in inp.xs]
        dys = [G.to_dev(g, "bf16") for g in inp.Gs]
        ys = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.M)]
        dxs = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.M)]
    s.synchronize()
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k, 1, pps.ZB1P)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        st.zero_grad()
        for op, mb, c, *_ in ops:
            if op == pps.OP_F:
                st.forward(mb, c, xs[mb], ys[mb])
            elif op == pps.OP_B:
                st.backward(mb, c, dys[mb], dxs[mb])
            else:
                st.backward_weight(mb, c)
    for rep in range(3):
        for t in ys + dxs:   # clobber the outputs between replays
            t.fill_(rep + 1.0)
        junk = torch.randn((1024, 1024), device="cuda") @ torch.randn((1024, 1024), device="cuda")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            grads = G.stage_grads(st, cfg.L, "swiglu", cfg.d, cfg.f)
            got_y = [G.to_host(y) for y in ys]
            got_dx = [G.to_host(x) for x in dxs]
        s.synchronize()
        for i in range(cfg.M):
            assert np.array_equal(got_y[i], ref[0][i]) and np.array_equal(got_dx[i], ref[1][i]), (rep, i)
        for blk in range(cfg.L):
            for key in ref[2][blk]:
                assert np.array_equal(grads[blk][key], ref[2][blk][key]), (rep, blk, key)
        del junk
    st.close()


def test_misaligned_buffers_rejected_before_any_work(env):
    # Caller buffers must be 16-byte aligned: a misaligned one is rejected with
    # EINVAL before anything is enqueued, the handle stays usable, and the
    # pass then gives the same bits as a run that never saw the bad calls.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=2, M=2, P=2)
    inp = make_inputs(cfg, gamma="random")
    ref = _run_single(env, cfg, inp, "1f1b")
    w = G.upload_params(inp.params[0], "swiglu", "bf16")
    st = pps.stage_from_config(cfg, weights=w, stream=torch.cuda.current_stream())
    xs = [G.to_dev(x, "bf16") for x in inp.xs]
    dys = [G.to_dev(g, "bf16") for g in inp.Gs]
    ys = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.M)]
    dxs = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.M)]
    spare = torch.empty(cfg.T * cfg.d + 8, dtype=torch.bfloat16, device="cuda")
    bad = spare.data_ptr() + 2
    assert st.forward_status(0, 0, bad, ys[0]) == pps.EINVAL
    assert st.forward_status(0, 0, xs[0], bad) == pps.EINVAL
    assert st.oplog() == []
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k)
    for i, (op, mb, c, *_) in enumerate(ops):
        if op == pps.OP_F:
            st.forward(mb, c, xs[mb], ys[mb])
        else:
            if i == 2:   # first backward: try the misaligned buffers first
                assert st.backward_status(mb, c, bad, dxs[mb]) == pps.EINVAL
                assert st.backward_status(mb, c, dys[mb], bad) == pps.EINVAL
                assert len(st.oplog()) == i
            st.backward(mb, c, dys[mb], dxs[mb])
    st.sync()
    assert st.oplog() == ops
    grads = G.stage_grads(st, cfg.L, "swiglu", cfg.d, cfg.f)
    for i in range(cfg.M):
        assert np.array_equal(G.to_host(ys[i]), ref[0][i]) and np.array_equal(G.to_host(dxs[i]), ref[1][i])
    for blk in range(cfg.L):
        for key in ref[2][blk]:
            assert np.array_equal(grads[blk][key], ref[2][blk][key]), key
    st.close()


@pytest.mark.parametrize("L", [1, 2])
def test_forward_in_place_and_backward_overlap(env, L):
    # y_out may be x_in itself (same bits as separate buffers); dy_in and dx_out
    # must not overlap (the first block's weight gradient reads dy_in after
    # dx_out is written): EINVAL, nothing enqueued.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=L, M=2, P=2)
    inp = make_inputs(cfg, gamma="random")
    ref = _run_single(env, cfg, inp, "1f1b")
    w = G.upload_params(inp.params[0], "swiglu", "bf16")
    st = pps.stage_from_config(cfg, weights=w, stream=torch.cuda.current_stream())
    xs = [G.to_dev(x, "bf16") for x in inp.xs]       # overwritten by y in place
    dys = [G.to_dev(g, "bf16") for g in inp.Gs]
    dxs = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.M)]
    for op, mb, c, *_ in pps.make_schedule(cfg.P, cfg.M, cfg.k):
        if op == pps.OP_F:
            st.forward(mb, c, xs[mb], xs[mb])
        else:
            n = len(st.oplog())
            assert st.backward_status(mb, c, dys[mb], dys[mb]) == pps.EINVAL
            half = dys[mb].view(-1)[cfg.T * cfg.d // 2:]   # overlapping, 16-byte aligned
            assert st.backward_status(mb, c, dys[mb], half) == pps.EINVAL
            assert len(st.oplog()) == n
            st.backward(mb, c, dys[mb], dxs[mb])
    st.sync()
    grads = G.stage_grads(st, cfg.L, "swiglu", cfg.d, cfg.f)
    for i in range(cfg.M):
        assert np.array_equal(G.to_host(xs[i]), ref[0][i]) and np.array_equal(G.to_host(dxs[i]), ref[1][i])
    for blk in range(cfg.L):
        for key in ref[2][blk]:
            assert np.array_equal(grads[blk][key], ref[2][blk][key]), key
    st.close()


def test_empty_microbatch(env):
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=0, M=2, P=2)
    inp = make_inputs(_swiglu_cfg("bf16", M=2, P=2))
    w = G.upload_params(inp.params[0], "swiglu", "bf16")
    st = pps.stage_from_config(cfg, weights=w, stream=torch.cuda.current_stream())
    x = torch.empty((0, cfg.d), dtype=torch.bfloat16, device="cuda")
    ops = pps.make_schedule(2, 2, 0)
    # zero-size buffers still need non-NULL pointers
    buf = torch.empty((8,), dtype=torch.bfloat16, device="cuda")
    for op, mb, c, *_ in ops:
        if op == pps.OP_F:
            st.forward(mb, c, buf, buf)
        else:
            st.backward(mb, c, buf, buf)
    st.sync()
    g = G.stage_grads(st, cfg.L, "swiglu", cfg.d, cfg.f)
    assert all(not v.any() for blk in g for v in blk.values())
    del x
    st.close()


def test_pass_repeats_and_zero_grad(env):
    # Two passes accumulate twice the gradient; zero_grad clears it.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=1, M=2, P=2)
    inp = make_inputs(cfg)
    w = G.upload_params(inp.params[0], "swiglu", "bf16")
    st = pps.stage_from_config(cfg, weights=w, stream=torch.cuda.current_stream())
    ops = pps.make_schedule(2, 2, 0)
    xs = [[G.to_dev(x, "bf16") for x in inp.xs]]
    dys = [[G.to_dev(g, "bf16") for g in inp.Gs]]
    G.run_stage(st, ops, xs, dys, cfg.T, cfg.d, "bf16")
    one = G.stage_grads(st, 1, "swiglu", cfg.d, cfg.f)
    G.run_stage(st, ops, xs, dys, cfg.T, cfg.d, "bf16")
    two = G.stage_grads(st, 1, "swiglu", cfg.d, cfg.f)
    for key in one[0]:
        assert N.rel_l2(two[0][key], 2 * one[0][key]) < 1e-6
    st.zero_grad()
    z = G.stage_grads(st, 1, "swiglu", cfg.d, cfg.f)
    assert all(not v.any() for v in z[0].values())
    assert st.stats()["passes_completed"] == 2
    st.close()


def test_profile_stride_times_every_nth_launch(env):
    # PPS_FLAG_PROFILE with profile_stride 3: launches 0, 3, 6, ... of each
    # kernel id carry HIP events; every launch is counted; the results are the
    # bits of an unprofiled run.
    torch, pps, G = env
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _swiglu_cfg("bf16", T=264, d=264, f=392, L=2, M=3, P=2)
    inp = make_inputs(cfg, gamma="random")
    ref = _run_single(env, cfg, inp, "1f1b")
    w = G.upload_params(inp.params[0], "swiglu", "bf16")
    st = pps.stage_from_config(cfg, weights=w, stream=torch.cuda.current_stream(), flags=pps.FLAG_PROFILE,
                               profile_capacity=1000, profile_stride=3)
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k)
    xs = [[G.to_dev(x, "bf16") for x in inp.xs]]
    dys = [[G.to_dev(g, "bf16") for g in inp.Gs]]
    ys, dxs = G.run_stage(st, ops, xs, dys, cfg.T, cfg.d, "bf16")
    kt = {k["name"]: k for k in st.kernel_times()}
    assert kt["gemm_dh_swiglu_bwd"]["launches"] == cfg.M * cfg.L
    assert kt["gemm_gateup_swiglu"]["launches"] == cfg.M * cfg.L
    for name, k in kt.items():
        assert k["timed"] == -(-k["launches"] // 3), (name, k)
        assert k["timed"] == 0 or k["total_ms"] > 0, (name, k)
    again = {k["name"]: k for k in st.kernel_times()}
    assert again == {}   # totals reset by the report
    grads = G.stage_grads(st, cfg.L, "swiglu", cfg.d, cfg.f)
    for i in range(cfg.M):
        assert np.array_equal(G.to_host(ys[0][i]), ref[0][i]) and np.array_equal(G.to_host(dxs[0][i]), ref[1][i])
    for blk in range(cfg.L):
        for key in ref[2][blk]:
            assert np.array_equal(grads[blk][key], ref[2][blk][key]), key
    st.close()
