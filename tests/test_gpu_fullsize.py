"""GPU parity at the benchmark's full shapes, in the launch configuration the
benchmark times, on outputs the float64 oracle can compute row by row.

The 80-layer-slice stage (T=8192 tokens, d=8192, ffn=28672, bf16) and the
Zero-Bubble stage (T=8192, d=4096, ffn=14336, bf16, dX now / dW later) run
their real GEMM grids; only the number of blocks (2) and micro-batches (2)
is cut, which changes no launch.  Inputs are sparse in tokens: x and the
output gradient are non-zero on a few sampled rows of each micro-batch and
exactly 0 elsewhere (the last row is always sampled, so the ragged end of
every tile row is covered).  Every block is token-local, so:

* the sampled rows of y and dx must match the oracle run on those rows alone
  (rel-L2 <= 2e-2, bf16), and every other row must be exactly 0;
* dW (a sum over tokens) only sees the sampled rows, so the oracle's dW from
  those rows is the full answer; it is compared on 4096 sampled entries of
  every weight gradient, and dgamma on its whole length.
"""

import numpy as np
import pytest

from oracle import numerics as N

pytestmark = pytest.mark.gpu

TOL = 2e-2
ROWS_PER_MB = 4
N_SAMPLES = 4096


@pytest.fixture(scope="module")
def env():
    import torch
    from pipeline_schedules_amd import pps
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pps.lib()
    return torch, pps


def _cfg(name, d, f, kind, P):
    from pipeline_schedules_amd.configs import StageConfig
    return StageConfig(name, P=P, M=2, k=0, v=1, kind=kind, block="swiglu", dtype="bf16", L=2, d=d, f=f, T=8192)


def _run(env, cfg, flags=0):
    torch, pps = env
    from pipeline_schedules_amd.inputs import make_device_inputs

    dev = torch.device("cuda:0")
    inp = make_device_inputs(cfg, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed + 101)
    for p in inp["params"]:      # non-trivial gamma so dgamma and the norm scale are exercised
        p["gamma"] = (1.0 + 0.1 * torch.randn((cfg.d,), generator=gen, device=dev)).float()
    rng = np.random.default_rng(cfg.seed + 7919)
    rows = []
    for i in range(cfg.M):
        r = np.sort(np.concatenate([rng.choice(cfg.T - 1, ROWS_PER_MB - 1, replace=False), [cfg.T - 1]]))
        mask = torch.zeros((cfg.T, 1), device=dev, dtype=inp["xs"][i].dtype)
        mask[torch.from_numpy(r).to(dev)] = 1
        inp["xs"][i] = inp["xs"][i] * mask
        inp["Gs"][i] = inp["Gs"][i] * mask
        rows.append(r)

    weights = []
    for p in inp["params"]:
        weights += [p["Wg"], p["Wu"], p["Wd"], p["gamma"]]
    stream = torch.cuda.current_stream()
    st = pps.stage_from_config(cfg, weights=weights, stream=stream, flags=flags)
    ops = pps.make_schedule(cfg.P, cfg.M, cfg.k, cfg.v, pps.KIND_BY_NAME[cfg.kind])
    ys = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=dev) for _ in range(cfg.M)]
    dxs = [torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=dev) for _ in range(cfg.M)]
    st.zero_grad()
    for op, mb, c, *_ in ops:
        if op == pps.OP_F:
            st.forward(mb, c, inp["xs"][mb], ys[mb])
        elif op == pps.OP_B:
            st.backward(mb, c, inp["Gs"][mb], dxs[mb])
        else:
            st.backward_weight(mb, c)
    st.sync()
    assert st.oplog() == ops
    return inp, rows, st, ys, dxs


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(env, cfg, flags=0):
    torch, pps = env
    inp, rows, st, ys, dxs = _run(env, cfg, flags)

    # the oracle on the sampled rows only (token-local blocks; pipelined order = full batch)
    xs_h = [_host(inp["xs"][i][torch.from_numpy(rows[i]).cuda()]) for i in range(cfg.M)]
    gs_h = [_host(inp["Gs"][i][torch.from_numpy(rows[i]).cuda()]) for i in range(cfg.M)]
    params_h = [{k: _host(v) for k, v in p.items()} for p in inp["params"]]
    ry, rdx, rg = N.full_batch_step(xs_h, gs_h, params_h, "swiglu", cfg.eps)
    del params_h

    errs = {}
    for i in range(cfg.M):
        idx = torch.from_numpy(rows[i]).cuda()
        for name, t, ref in (("y", ys[i], ry[i]), ("dx", dxs[i], rdx[i])):
            got = _host(t[idx])
            errs[f"{name}{i}"] = N.rel_l2(got, ref)
            nz = torch.nonzero(t.float().abs().amax(dim=1)).flatten().cpu().numpy()
            assert set(nz.tolist()) <= set(rows[i].tolist()), f"{name}{i}: non-zero outside the sampled rows"

    srng = np.random.default_rng(cfg.seed + 31)
    for b in range(cfg.L):
        for key, which, shape in (("Wg", 0, (cfg.d, cfg.f)), ("Wu", 1, (cfg.d, cfg.f)), ("Wd", 2, (cfg.f, cfg.d))):
            flat = srng.choice(shape[0] * shape[1], N_SAMPLES, replace=False)
            g = st.grad(0, b, which, shape).reshape(-1)
            got = _host(g[torch.from_numpy(flat).cuda()])
            ref = rg[b][key].reshape(-1)[flat]
            errs[f"{key}{b}"] = N.rel_l2(got, ref)
        got = _host(st.grad(0, b, 3, (cfg.d,)))
        errs[f"gamma{b}"] = N.rel_l2(got, rg[b]["gamma"])
    st.close()
    print(cfg.name, " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, f"rel-L2 above {TOL}: {bad} (all: {errs})"


def test_80layer_slice_shapes_1f1b(env):
    """T=8192, d=8192, ffn=28672, 1F1B, stage 0 of 8."""
    _check(env, _cfg("c3-shapes", 8192, 28672, "1f1b", 8))


def test_zero_bubble_shapes_split(env):
    """T=8192, d=4096, ffn=14336, ZB1P: dX in B, dW deferred to W."""
    _check(env, _cfg("c5-shapes", 4096, 14336, "zb1p", 4))


def test_80layer_slice_shapes_recompute(env):
    """The same stage in recompute mode (each B re-runs the forward from x)."""
    _check(env, _cfg("c3-shapes-recompute", 8192, 28672, "1f1b", 8), flags=env[1].FLAG_RECOMPUTE)
