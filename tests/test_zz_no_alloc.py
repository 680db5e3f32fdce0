"""GPU test of pps_stage_create_noalloc: a stage whose device memory comes
from the library's fixed per-GPU array gives the same results as one created
with pps_stage_create, on two handles in a row (the second with fewer
tokens), and both match the float64 oracle.

The two entry points run the same kernels on the same inputs in the same
order, so outputs, input gradients and weight gradients must be equal
element for element; the oracle comparison uses the bf16 tolerance.
"""

import numpy as np
import pytest

from oracle import numerics as N

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def env():
    import torch
    from pipeline_schedules_amd import pps
    from tests import gpu_util as G
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pps.lib()
    return torch, pps, G


def _cfg(T):
    from pipeline_schedules_amd.configs import StageConfig
    return StageConfig("noalloc", P=2, M=3, k=0, v=1, kind="1f1b", block="swiglu", dtype="bf16", L=2, d=264, f=392, T=T)


def _run(env, cfg, inp, noalloc):
    torch, pps, G = env
    w = G.upload_params(inp.params[0], cfg.block, cfg.dtype)
    st = pps.stage_from_config(cfg, weights=w, stream=torch.cuda.current_stream(), noalloc=noalloc)
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k, cfg.v, pps.KIND_BY_NAME[cfg.kind])
    xs = [[G.to_dev(x, cfg.dtype) for x in inp.xs]]
    dys = [[G.to_dev(g, cfg.dtype) for g in inp.Gs]]
    ys, dxs = G.run_stage(st, ops, xs, dys, cfg.T, cfg.d, cfg.dtype)
    assert st.oplog() == ops
    grads = G.stage_grads(st, cfg.L, cfg.block, cfg.d, cfg.f)
    out = ([G.to_host(y) for y in ys[0]], [G.to_host(x) for x in dxs[0]], grads)
    st.close()
    return out


@pytest.mark.parametrize("T", [600, 264])   # second call: a smaller input
def test_noalloc_matches_allocating_create(env, T):
    from pipeline_schedules_amd.inputs import make_inputs
    cfg = _cfg(T)
    inp = make_inputs(cfg, gamma="random")
    ref = _run(env, cfg, inp, noalloc=False)
    got = _run(env, cfg, inp, noalloc=True)
    for i in range(cfg.M):
        assert np.array_equal(got[0][i], ref[0][i]), f"y{i}"
        assert np.array_equal(got[1][i], ref[1][i]), f"dx{i}"
    for b in range(cfg.L):
        for key in ref[2][b]:
            assert np.array_equal(got[2][b][key], ref[2][b][key]), (b, key)
    ry, rdx, rg = N.full_batch_step(inp.xs, inp.Gs, inp.params[0], cfg.block, cfg.eps)
    errs = [N.rel_l2(got[0][i], ry[i]) for i in range(cfg.M)] + [N.rel_l2(got[1][i], rdx[i]) for i in range(cfg.M)]
    errs += [N.rel_l2(got[2][b][k], rg[b][k]) for b in range(cfg.L) for k in rg[b]]
    assert max(errs) <= TOL, max(errs)


def test_noalloc_rejects_a_stage_larger_than_the_array(env):
    torch, pps, G = env
    from pipeline_schedules_amd.configs import StageConfig
    from pipeline_schedules_amd.inputs import make_device_inputs
    cfg = StageConfig("big", P=4, M=8, k=0, v=1, kind="1f1b", block="swiglu", dtype="bf16", L=1, d=1024, f=2816,
                      T=2048)
    inp = make_device_inputs(cfg, torch.device("cuda:0"), M=1)
    p = inp["params"][0]
    with pytest.raises(pps.PpsError) as e:
        pps.stage_from_config(cfg, weights=[p["Wg"], p["Wu"], p["Wd"], p["gamma"]],
                              stream=torch.cuda.current_stream(), noalloc=True)
    assert e.value.status == pps.ETOOBIG
